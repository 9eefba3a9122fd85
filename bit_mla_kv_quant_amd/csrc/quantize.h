// The cache writer's per-group step [QuantMLA §4.1, App. C.4, App. C.5],
// shared by the writer kernel and by the decode kernels' fused writer (so the
// two write identical bytes).
//
// A 64-lane wave holds one 64-value group of one token, one value per lane.
// The wave reduces min/max, every lane derives the same scale and zero,
// computes its code with IEEE fp32 subtract/divide and round-to-nearest-even,
// and the codes are OR-reduced across 8 (INT4) or 16 (INT2) lanes into the
// 32-bit words of the page layout (include/mla_lowbit.h), which one lane per
// word stores.  Floating-point contraction is off in every function here: the
// quantizer's subtract and divide must round exactly as specified.
#pragma once
#include "common.h"
#include "internal.h"

namespace mlb {

// Cross-lane steps use DPP within each row of 16 lanes and the gfx950 row
// swaps across rows, so a reduction never waits on the LDS crossbar.
constexpr int DPP_XOR1 = 0xB1;          // quad_perm [1,0,3,2]
constexpr int DPP_XOR2 = 0x4E;          // quad_perm [2,3,0,1]
constexpr int DPP_HALF_MIRROR = 0x141;  // lane i <-> 7-i within each 8
constexpr int DPP_MIRROR = 0x140;       // lane i <-> 15-i within each 16

template <int CTRL>
__device__ __forceinline__ uint32_t dpp(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, true);
}
template <int CTRL>
__device__ __forceinline__ float dppf(float v) {
  return __uint_as_float(dpp<CTRL>(__float_as_uint(v)));
}

// Combine the lane's value with its partners in the other three rows of 16
// (the value is already uniform within each row).
template <typename Op>
__device__ __forceinline__ float across_rows(float x, Op op) {
  const auto r16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x),
                                                    false, false);
  x = op(__uint_as_float(r16[0]), __uint_as_float(r16[1]));
  const auto r32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                    false, false);
  return op(__uint_as_float(r32[0]), __uint_as_float(r32[1]));
}

struct MinOp {
  __device__ float operator()(float a, float b) const { return fminf(a, b); }
};
struct MaxOp {
  __device__ float operator()(float a, float b) const { return fmaxf(a, b); }
};

template <typename Op>
__device__ __forceinline__ float wave_reduce(float v, Op op) {
  v = op(v, dppf<DPP_XOR1>(v));
  v = op(v, dppf<DPP_XOR2>(v));
  v = op(v, dppf<DPP_HALF_MIRROR>(v));
  v = op(v, dppf<DPP_MIRROR>(v));
  return across_rows(v, op);
}
__device__ __forceinline__ float wave_min(float v) { return wave_reduce(v, MinOp{}); }
__device__ __forceinline__ float wave_max(float v) { return wave_reduce(v, MaxOp{}); }

// OR over aligned runs of 8 or 16 lanes (every lane of the run gets it).
template <int WIDTH>
__device__ __forceinline__ uint32_t or_reduce(uint32_t v) {
  v |= dpp<DPP_XOR1>(v);
  v |= dpp<DPP_XOR2>(v);
  v |= dpp<DPP_HALF_MIRROR>(v);
  if constexpr (WIDTH == 16) v |= dpp<DPP_MIRROR>(v);
  return v;
}

// Quantize one group held one element per lane.  Returns the lane's code and
// the group's (scale, zero) bf16 bits.
__device__ __forceinline__ uint32_t quantize_lane(float x, int bits, uint32_t& s_bits,
                                                  uint32_t& z_bits) {
#pragma clang fp contract(off)
  const float m = (float)((1 << bits) - 1);
  const float lo = wave_min(x);
  const float hi = wave_max(x);
  const float rng = hi - lo;                      // fl32(hi - lo)
  s_bits = f32_to_bf16_bits(rng / m);             // bf16(fl32(rng / m))
  z_bits = __float_as_uint(lo) >> 16;             // lo is bf16-exact
  const float s = bf16_bits_to_f32(s_bits);
  if (!(s > 0.0f)) return 0u;                     // constant group: all codes 0
  const float t = (x - lo) / s;                   // fl32(fl32(x - z) / s)
  float q = rintf(t);                             // ties to even
  q = fminf(fmaxf(q, 0.0f), m);
  return (uint32_t)q;
}

// The same with the group's (scale, zero) kept in fp32 (the RoPE group of
// format C4R4F [QuantMLA App. C.4/C.5]): s = fl32(fl32(hi - lo) / m), z = lo.
__device__ __forceinline__ uint32_t quantize_lane_f32(float x, int bits, float& s, float& z) {
#pragma clang fp contract(off)
  const float m = (float)((1 << bits) - 1);
  const float lo = wave_min(x);
  const float hi = wave_max(x);
  s = (hi - lo) / m;                              // fl32(fl32(hi - lo) / m)
  z = lo;
  if (!(s > 0.0f)) return 0u;                     // constant group: all codes 0
  const float t = (x - lo) / s;                   // fl32(fl32(x - z) / s)
  float q = rintf(t);                             // ties to even
  q = fminf(fmaxf(q, 0.0f), m);
  return (uint32_t)q;
}

// Quantize group g of one token (g < 8: content dims 64g .. 64g+63; g == 8:
// the RoPE key) held as bf16 bits x, one value per lane, and store its codes
// and metadata into slot `off` of the page at `pg`.
template <int F>
__device__ __forceinline__ void write_group(uint8_t* pg, int off, int g, uint16_t x, int lane) {
  using FM = Fmt<F>;
  if (g < NGC) {
    uint32_t sb, zb;
    const uint32_t q = quantize_lane(bf16_bits_to_f32(x), FM::CBITS, sb, zb);
    const int d = 64 * g + lane;                   // content dim
    const int blk = d / FM::DPB;
    const int dib = d % FM::DPB;                   // dim within block
    if constexpr (FM::CBITS == 4) {
      // byte k = dims 2k (lo), 2k+1 (hi): dword = dims 8w..8w+7, nibble d%8
      const uint32_t w = or_reduce<8>(q << (4 * (lane & 7)));
      if ((lane & 7) == 0)
        *(uint32_t*)(pg + (blk * PAGE + off) * 64 + (dib / 8) * 4) = w;
    } else {
      // dword = dims 16w..16w+15: dim 16w+2m at bits 2m, dim 16w+2m+1 at
      // bits 16+2m
      const int e = lane & 15;
      const uint32_t w = or_reduce<16>(q << (16 * (e & 1) + 2 * (e >> 1)));
      if ((lane & 15) == 0)
        *(uint32_t*)(pg + (blk * PAGE + off) * 64 + (dib / 16) * 4) = w;
    }
    if (lane == 0) *(uint32_t*)(pg + FM::OFF_MC + off * 32 + g * 4) = sb | (zb << 16);
  } else if constexpr (FM::F32R) {                 // RoPE group, fp32 metadata
    float s32, z32;
    const uint32_t q = quantize_lane_f32(bf16_bits_to_f32(x), 4, s32, z32);
    const uint32_t w = or_reduce<8>(q << (4 * (lane & 7)));
    if ((lane & 7) == 0) *(uint32_t*)(pg + FM::OFF_R + off * 32 + (lane / 8) * 4) = w;
    if (lane == 0)
      *(u32x2*)(pg + FM::OFF_MR + off * 8) = u32x2{__float_as_uint(s32), __float_as_uint(z32)};
  } else {                                         // RoPE group, bf16 metadata
    uint32_t sb, zb;
    const uint32_t q = quantize_lane(bf16_bits_to_f32(x), 4, sb, zb);
    const uint32_t w = or_reduce<8>(q << (4 * (lane & 7)));
    if ((lane & 7) == 0) *(uint32_t*)(pg + FM::OFF_R + off * 32 + (lane / 8) * 4) = w;
    if (lane == 0) *(uint32_t*)(pg + FM::OFF_MR + off * 4) = sb | (zb << 16);
  }
}

// Fused writer of a decode step: token pos = L-1 of sequence b (bf16 rows
// a.new_c[b], a.new_r[b]) goes into its slot of the page the block table
// names, and into its protection-buffer row (the newest token is always in
// the recent window).  The nw waves of the calling workgroup share the nine
// groups: wave w takes groups w, w + nw, ...  `wave` is wave-uniform.
// fused_load fetches the wave's values early (so their latency overlaps the
// decode work); fused_store quantizes and stores them.
struct FusedRow {
  uint16_t x[3];                                   // groups wave, wave+nw, wave+2nw
};
__device__ __forceinline__ FusedRow fused_load(const DecodeArgs& a, int b, int wave, int nw,
                                               int lane) {
  FusedRow r{};
#pragma unroll
  for (int k = 0; k < 3; ++k) {
    const int g = wave + k * nw;
    if (g <= NGC)
      r.x[k] = g < NGC ? a.new_c[(int64_t)b * DC + 64 * g + lane] : a.new_r[(int64_t)b * DR + lane];
  }
  return r;
}
template <int F>
__device__ __forceinline__ void fused_store(const DecodeArgs& a, const FusedRow& r, int b, int L,
                                            int sq, int wave, int nw, int lane) {
  const int pos = L - 1;
  const int phys = a.block_table[(int64_t)b * a.max_blocks + pos / PAGE];
  if (phys < 0 || phys >= a.num_pages) return;     // unusable table entry: nothing stored
  uint8_t* pg = a.wpages + (int64_t)phys * Fmt<F>::PAGE_BYTES;
  const int off = pos % PAGE;
  uint16_t* dst = a.wprot + ((int64_t)sq * PROT_ROWS + prot_row(pos)) * DROW;
#pragma unroll
  for (int k = 0; k < 3; ++k) {
    const int g = wave + k * nw;
    if (g <= NGC) {
      write_group<F>(pg, off, g, r.x[k], lane);
      dst[64 * g + lane] = r.x[k];                 // g == 8: RoPE dims 512 + lane
    }
  }
}

}  // namespace mlb
