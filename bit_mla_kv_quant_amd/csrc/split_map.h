// Which sequence and split a decode workgroup works on, and where each
// sequence's split partials lie in the workspace (split-KV across compute
// units [QuantMLA App. C.5, F.1]).
//
// The host plan fixes W = nsplit * B split slots (grid x * grid y) from
// max_seq_len.  With one pages-per-split count for every sequence, a
// ragged batch leaves the splits of short sequences empty while the longest
// sequence's splits set the kernel's duration.  For batches of at most 64
// sequences with the automatic plan (DecodeArgs::balance) the slots are
// instead dealt by length on the device: pages per split pps is the smallest
// value with sum_b max(1, ceil(P_b / pps)) <= W (P_b: pages of sequence b,
// as the kernels clamp its length), sequence b owns n_b = max(1, ceil(P_b /
// pps)) consecutive slots from first_b = sum_{c<b} n_c, and slots past
// sum_b n_b stay idle.  Equal lengths keep the uniform plan.  One wave
// evaluates the plan (lane b holds sequence b), the same way in the decode
// kernels and in the combine, so both see the same layout.
#pragma once
#include "common.h"
#include "internal.h"

namespace mlb {

struct SplitSlot {
  int b;       // sequence (-1: idle slot)
  int j;       // split of the sequence
  int pps;     // pages per split
  int first;   // workspace slot of the sequence's split 0
  int count;   // splits of the sequence
  int L;       // tokens of sequence b, clamped as the decode kernels do
  int sq;      // protection-buffer slot of sequence b
};

namespace splitmap {

constexpr int XOR1 = 0xB1, XOR2 = 0x4E, HALF_MIRROR = 0x141, MIRROR = 0x140;
template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, true);
}
template <typename Op>
__device__ __forceinline__ int wave_reduce_i(int v, Op op) {
  v = op(v, dpp_i<XOR1>(v));
  v = op(v, dpp_i<XOR2>(v));
  v = op(v, dpp_i<HALF_MIRROR>(v));
  v = op(v, dpp_i<MIRROR>(v));
  const auto r16 = __builtin_amdgcn_permlane16_swap((uint32_t)v, (uint32_t)v, false, false);
  v = op((int)r16[0], (int)r16[1]);
  const auto r32 = __builtin_amdgcn_permlane32_swap((uint32_t)v, (uint32_t)v, false, false);
  return __builtin_amdgcn_readfirstlane(op((int)r32[0], (int)r32[1]));
}
struct Add { __device__ int operator()(int x, int y) const { return x + y; } };
struct Max { __device__ int operator()(int x, int y) const { return x > y ? x : y; } };
struct Min { __device__ int operator()(int x, int y) const { return x < y ? x : y; } };

// inclusive prefix sum over the 64 lanes
__device__ __forceinline__ int wave_scan_i(int v, int lane) {
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int u = __shfl_up(v, d, 64);
    if (lane >= d) v += u;
  }
  return v;
}

// tokens of sequence i as the decode kernels clamp its length (0 for an
// unusable sequence slot)
__device__ __forceinline__ int seq_len_clamped(const DecodeArgs& a, int i, int sq) {
  int L = a.seq_lens[i];
  L = L < 0 ? 0 : (L > a.max_seq_len ? a.max_seq_len : L);
  if (sq < 0 || sq >= a.num_seq_slots) L = 0;
  return L;
}

// the balanced plan: pps, and per lane b < B its slot count n and first slot;
// uniform = true when every sequence has the same page count (nothing else
// is then filled in); Lc / sq: lane b's clamped length and sequence slot
struct Dealt {
  bool uniform;
  int pps, n, first, total;
  int Lc, sq;
};
__device__ __forceinline__ Dealt deal(const DecodeArgs& a, int lane) {
  Dealt d;
  const bool in = lane < a.B;
  d.sq = in ? a.seq_slot[lane] : 0;
  d.Lc = in ? seq_len_clamped(a, lane, d.sq) : 0;
  const int P = (d.Lc + PAGE - 1) / PAGE;
  const int pmax = wave_reduce_i(in ? P : 0, Max{});
  const int pmin = wave_reduce_i(in ? P : 0x7fffffff, Min{});
  d.uniform = pmax == pmin;
  if (d.uniform) return d;
  const int64_t W = (int64_t)a.B * a.nsplit;
  const int64_t sum = wave_reduce_i(P, Add{});
  // smallest pps in [lo, hi] with sum_b max(1, ceil(P_b / pps)) <= W; hi
  // always satisfies it (each term is below P_b / pps + 1, or n_b = 1 for all)
  int lo = (int)((sum + W - 1) / W);
  lo = lo < 1 ? 1 : lo;
  int hi = pmax < 1 ? 1 : pmax;
  if (W > a.B) {
    const int h2 = (int)((sum + (W - a.B) - 1) / (W - a.B));
    hi = h2 < hi ? h2 : hi;
  }
  if (hi < lo) hi = lo;
  while (lo < hi) {                              // uniform loop: lo, hi in SGPRs
    const int mid = lo + (hi - lo) / 2;
    const int n = in ? (P > mid ? (P + mid - 1) / mid : 1) : 0;
    if (wave_reduce_i(n, Add{}) <= W) hi = mid;
    else lo = mid + 1;
  }
  d.pps = lo;
  d.n = in ? (P > lo ? (P + lo - 1) / lo : 1) : 0;
  const int cum = wave_scan_i(d.n, lane);
  d.first = cum - d.n;
  d.total = __builtin_amdgcn_readlane(cum, 63);
  return d;
}

}  // namespace splitmap

// The workgroup of grid slot `slot` (= blockIdx.y * nsplit + blockIdx.x).
// Wave-uniform result; lane = the caller's lane in its wave.
__device__ __forceinline__ SplitSlot split_slot(const DecodeArgs& a, int slot, int lane) {
  SplitSlot s;
  const int bu = slot / a.nsplit;
  s.b = bu;
  s.j = slot - bu * a.nsplit;
  s.pps = a.pps;
  s.first = bu * a.nsplit;
  s.count = a.nsplit;
  if (!a.balance) {
    s.sq = a.seq_slot[bu];
    s.L = splitmap::seq_len_clamped(a, bu, s.sq);
    return s;
  }
  const splitmap::Dealt d = splitmap::deal(a, lane);
  if (d.uniform) {
    s.L = __builtin_amdgcn_readlane(d.Lc, bu);
    s.sq = __builtin_amdgcn_readlane(d.sq, bu);
    return s;
  }
  s.pps = d.pps;
  if (slot >= d.total) {
    s.b = -1;
    return s;
  }
  // the sequence whose slot range holds `slot`: the lowest lane with
  // first + n > slot
  const uint64_t owners = __ballot(lane < a.B && d.first + d.n > slot);
  const int b = __builtin_amdgcn_readfirstlane(__builtin_ctzll(owners));
  s.b = b;
  s.first = __builtin_amdgcn_readlane(d.first, b);
  s.count = __builtin_amdgcn_readlane(d.n, b);
  s.j = slot - s.first;
  s.L = __builtin_amdgcn_readlane(d.Lc, b);
  s.sq = __builtin_amdgcn_readlane(d.sq, b);
  return s;
}

// The workspace slots of sequence b's partials: first .. first + count - 1.
__device__ __forceinline__ void split_range(const DecodeArgs& a, int b, int lane, int& first,
                                            int& count) {
  first = b * a.nsplit;
  count = a.nsplit;
  if (!a.balance) return;
  const splitmap::Dealt d = splitmap::deal(a, lane);
  if (d.uniform) return;
  first = __builtin_amdgcn_readlane(d.first, b);
  count = __builtin_amdgcn_readlane(d.n, b);
}

}  // namespace mlb
