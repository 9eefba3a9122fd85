// mla_decode_lowbit for 16-head groups: native low-bit MLA decode attention
// [QuantMLA §3.3, App. C.5] in the absorbed form [MLA blog §4], for gfx950.
//
// At 16 heads the path moves ~107 FLOP per byte, so a page's reconstruction
// (vector ALU work) must keep pace with HBM while the matrix cores stay
// mostly idle.  decode16w_kernel<F>: one 512-thread workgroup (8 waves, two
// per SIMD) per (split j, sequence b, 16-head group).  The query sits once in
// LDS; after that the waves work independently -- no workgroup barrier until
// the end of the split -- each on its own 16-token quarter pages (wave w
// takes quarters w, w+8, ...; a fixed assignment keeps results reproducible):
//   * lane (n16, g) reconstructs token n16 of the quarter, content groups
//     2g, 2g+1 and RoPE dims 16g .. 16g+15, from packed codes loaded one
//     quarter earlier;
//   * each reconstructed 8-dim slice is at once the A operand of
//     v_mfma_f32_16x16x32_bf16 for the transposed scores
//     S^T[tokens][heads] = K . Q^T (query slices read from LDS in the same
//     dim order), and its content part is stored to the wave's own LDS tile
//     [16 tokens][512];
//   * lane (head n16, g) then holds its head's scores for tokens 4g .. 4g+3.
//     Each weight is split into bf16 hi + lo terms, and one MFMA per 16 dims
//     aggregates both: K index 8g + j carries hi of token 4g + j for j < 4
//     and lo of token 4g + j - 4 for j >= 4, against the C^T operand holding
//     those tokens' values twice (one ds_read_b64_tr_b16 per operand).  The
//     softmax [QuantMLA §3.3] moves no data between lanes except a head
//     maximum over the head's four lanes.
// Every value is reconstructed once and used for both products
// [QuantMLA App. C.5].  The 128 accumulators per lane are never rescaled in
// the loop: a head's reference maximum is fixed by its first live quarter,
// later weights may exceed 1 by up to 2^REF_HEADROOM_LOG2 (carried exactly by
// fp32 sums and the hi/lo split), and a score beyond that makes the wave
// raise the head's reference and redo its quarters from zero -- the same
// single softmax; each redo raises a reference by more than the headroom, so
// redos are bounded.  At the end the eight waves' (max, weight
// sum, O) are merged through LDS by the log-sum-exp rule; the split writes
// the result to the output (single split) or to the workspace for
// combine_kernel.
#include <type_traits>

#include "common.h"
#include "dequant.h"
#include "internal.h"
#include "quantize.h"
#include "split_map.h"

namespace mlb {

namespace {

typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

constexpr int NW = 8;                 // waves per workgroup
constexpr int QT = 16;                // tokens per quarter page
constexpr int VT_PITCH = DC + 8;      // LDS tile row pitch (bf16 elements)
constexpr int Q_PITCH = DROW + 8;     // LDS query row pitch (bf16 elements)
constexpr float REF_HEADROOM_LOG2 = 64.0f;
constexpr float FP8_PATH_MAX_SCALE9 = 3.4028234663852886e38f;

// max over the four lanes n16, n16+16, n16+32, n16+48 (the lanes of a head)
__device__ __forceinline__ float head_max4(float x) {
  const auto r16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x),
                                                    false, false);
  x = fmaxf(__uint_as_float(r16[0]), __uint_as_float(r16[1]));
  const auto r32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                    false, false);
  return fmaxf(__uint_as_float(r32[0]), __uint_as_float(r32[1]));
}

}  // namespace

template <int F>
__global__ __launch_bounds__(512, 1) void decode16w_kernel(DecodeArgs a) {
  // one LDS block: the waves' content tiles [NW][16][VT_PITCH], then the
  // query [16][Q_PITCH]; the end-of-split merge reuses all of it
  constexpr int LDS_ELEMS = NW * QT * VT_PITCH + 16 * Q_PITCH;
  __shared__ __attribute__((aligned(16))) uint16_t lds[LDS_ELEMS];
  uint16_t* const qtile = lds + NW * QT * VT_PITCH;

  const int hg = blockIdx.z;
  // wave index as a uniform value, so quarter indices and page ids stay in
  // scalar registers
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  // the sequence and split of this workgroup's slot
  const SplitSlot ss = split_slot(a, blockIdx.y * a.nsplit + blockIdx.x, lane);
  if (ss.b < 0) return;                            // idle slot of a balanced plan
  const int j = ss.j, b = ss.b;
  const int n16 = lane & 15, g = lane >> 4;
  const int H = a.H;

  const int L = ss.L, sq = ss.sq;
  const int npages = (L + PAGE - 1) / PAGE;
  const int p0 = j * ss.pps;
  const int p1 = min(p0 + ss.pps, npages);
  const bool single = a.nsplit == 1;
  if (p0 >= p1) {
    if (single && j == 0) {                        // empty sequence: out 0, lse -inf
      float* o = a.out + ((int64_t)b * H + 16 * hg) * DC;
      for (int idx = threadIdx.x; idx < 16 * DC / 4; idx += 512)
        *(f32x4*)(o + 4 * idx) = f32x4{0.f, 0.f, 0.f, 0.f};
      if (threadIdx.x < 16) a.lse[(int64_t)b * H + 16 * hg + threadIdx.x] = -INFINITY;
    } else if (!single && threadIdx.x < 16) {      // no tokens: m = -inf for the merge
      const int64_t base = ((int64_t)ss.first + j) * H + 16 * hg + threadIdx.x;
      *(f32x4*)(a.ws_ml + base * 4) = f32x4{-INFINITY, 0.f, 0.f, 0.f};
    }
    return;
  }
  const int nquart = 4 * (p1 - p0);                // quarter pages of the split
  // tokens the lane's row (query row 16hg + n16) attends to: the causal
  // prefix of its query, all L when there is one query per sequence
  const int L_row = L - (a.nq - 1 - (16 * hg + n16) / a.hq);
  // fused writer: token L-1 of a sequence whose length is within bounds (a
  // clamped length names a token the cache already holds: nothing is stored
  // or substituted, and the call decodes as mla_decode_lowbit)
  const bool fused = a.new_c != nullptr && a.seq_lens[b] <= a.max_seq_len;
  // fused writer: the middle split of the sequence (first head block)
  // fetches the newest token now and stores it once its own work is done.
  // A middle split holds neither the sink tokens nor the recent window, so
  // it finishes ahead of the splits that do and the writer hides behind them.
  const int nsplit_b = (npages + ss.pps - 1) / ss.pps;
  const bool writer = fused && j == nsplit_b / 2 && hg == 0;
  FusedRow fresh_row{};
  if (writer) fresh_row = fused_load(a, b, wave, NW, lane);

  // physical page ids of the split (-1 = unusable table entry)
  PageWindow pw{a.block_table + (int64_t)b * a.max_blocks + p0, p1 - p0, a.num_pages, 0, 0, 0};
  auto page_ptr = [&](int phys) -> const uint8_t* {
    return a.pages + (int64_t)(phys >= 0 ? phys : 0) * Fmt<F>::PAGE_BYTES;
  };

  // ---- the group's query [16 heads][576] into LDS, once
  for (int idx = threadIdx.x; idx < 16 * DROW / 8; idx += 512) {
    const int hh = idx / (DROW / 8), c8 = 8 * (idx % (DROW / 8));
    const int64_t hrow = (int64_t)b * H + 16 * hg + hh;
    *(bf16x8*)(qtile + hh * Q_PITCH + c8) =
        c8 < DC ? *(const bf16x8*)(a.q_lat + hrow * DC + c8)
                : *(const bf16x8*)(a.q_rope + hrow * DR + (c8 - DC));
  }
  __syncthreads();
  // B operand of the transposed score product: slice s < 16 is content dims
  // 128g + 8s .. +7, slices 16 and 17 the RoPE dims 16g + 8(s-16) .. +7 --
  // the dims this lane reconstructs
  const uint16_t* qrow = qtile + n16 * Q_PITCH;
  auto qslice = [&](const int s) -> bf16x8 {
    return *(const bf16x8*)(qrow + (s < 16 ? 128 * g + 8 * s : DC + 16 * g + 8 * (s - 16)));
  };
  const uint16_t* prot_seq = a.prot + (int64_t)sq * PROT_ROWS * DROW;
  uint16_t* vt = lds + wave * QT * VT_PITCH;

  // ---- attention state of lane (head n16, g): m_ref reference maximum
  // (log2 units), f_run sum of the fp32 weights of this lane's tokens,
  // acc[nb][v] = O[head][16nb + 4g + v]; m_need: the reference a redo needs.
  f32x4 acc[32];
  float m_ref = -INFINITY, f_run = 0.f, m_need = -INFINITY;

  // ---- scores of one quarter page: q = quarter index in the split, sl the
  // packed codes of token n16 of it; also stores its content rows to the
  // wave's tile
  auto quarter = [&](auto ordinary_tag, const int q, const int phys, const LaneSlot<F>& sl) {
    constexpr bool ORDINARY = decltype(ordinary_tag)::value;
    const int i0 = (p0 + (q >> 2)) * PAGE + QT * (q & 3);   // first token of the quarter
    uint16_t* rw = vt + n16 * VT_PITCH + 128 * g;
    f32x4 se = {0.f, 0.f, 0.f, 0.f}, so = {0.f, 0.f, 0.f, 0.f};   // even / odd slices
    // query slices are read QPF slices ahead of their MFMA (LDS latency)
    constexpr int QPF = 3;
    bf16x8 qn[QPF];
#pragma unroll
    for (int s = 0; s < QPF; ++s) qn[s] = qslice(s);
    auto qk = [&](const int s, const bf16x8 kv) {
      const bf16x8 qs = qn[s % QPF];
      if (s + QPF < 18) qn[s % QPF] = qslice(s + QPF);
      if (s & 1) so = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kv, qs, so, 0, 0, 0);
      else se = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kv, qs, se, 0, 0, 0);
    };
    if constexpr (ORDINARY) {
#pragma unroll
      for (int grp = 0; grp < 2; ++grp) {
        if constexpr (Fmt<F>::CBITS == 4) {
          const float s9 = meta_scale(sl.mc[grp]) * 512.0f, z = meta_zero(sl.mc[grp]);
#pragma unroll
          for (int t = 0; t < 8; ++t) {
            const bf16x8 kv = deq_int4x8_fp8(sl.c[2 * grp + (t >> 2)][t & 3], s9, z);
            qk(8 * grp + t, kv);
            *(bf16x8*)(rw + 64 * grp + 8 * t) = kv;
          }
        } else {
          const Lut2 lut = make_lut2(meta_scale(sl.mc[grp]), meta_zero(sl.mc[grp]));
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            bf16x8 ka, kb;
            deq_int2x16(sl.c[grp][w], lut, ka, kb);
            qk(8 * grp + 2 * w, ka);
            qk(8 * grp + 2 * w + 1, kb);
            *(bf16x8*)(rw + 64 * grp + 16 * w) = ka;
            *(bf16x8*)(rw + 64 * grp + 16 * w + 8) = kb;
          }
        }
      }
      const float s9 = meta_scale(sl.mr) * 512.0f, z = meta_zero(sl.mr);
      qk(16, deq_rope8_fp8<F>(sl.r[0], s9, z));
      qk(17, deq_rope8_fp8<F>(sl.r[1], s9, z));
    } else {
      // a quarter holding a sink or recent-window token, unusable slots, or
      // a scale beyond the fp8 path: per-lane substitutions.  The BF16 rows
      // of protected tokens are requested in batches before any is used
      // (one memory latency per batch, not one per slice).
      const int i = i0 + n16;
      const bool valid = phys >= 0 && i < L;
      const bool prot = valid && is_protected(i, L);
      // bf16 row of a protected token: its protection-buffer row, or for the
      // token the fused writer stores in this call, the new row itself
      const bool fresh = fused && i == L - 1;
      const uint16_t* prow = prot_seq + (int64_t)(prot ? prot_row(i) : 0) * DROW;
      const uint16_t* pc = fresh ? a.new_c + (int64_t)b * DC : prow;
      const uint16_t* pr = fresh ? a.new_r + (int64_t)b * DR : prow + DC;
      auto prot_at = [&](const int off) -> bf16x8 {  // dims off .. off+7 of the row
        return off < DC ? *(const bf16x8*)(pc + off) : *(const bf16x8*)(pr + (off - DC));
      };
      auto slice_off = [&](const int s) {            // row offset of slice s
        return s < 16 ? 128 * g + 8 * s : DC + 16 * g + 8 * (s - 16);
      };
      auto prot_slice = [&](const int s) -> bf16x8 {
        return prot ? prot_at(slice_off(s)) : bitcast<bf16x8>(u32x4{0u, 0u, 0u, 0u});
      };
      if (__all(prot)) {
        // a quarter of the recent window: nothing to reconstruct, so slice s
        // of lane g is dims 32s + 8g (s < 16) or 512 + 32(s-16) + 8g -- the
        // four lanes of a token read 64 contiguous bytes of its row
        auto off_p = [&](const int s) { return (s < 16 ? 32 * s : DC + 32 * (s - 16)) + 8 * g; };
        bf16x8 pr[18];
#pragma unroll
        for (int s = 0; s < 18; ++s) pr[s] = prot_at(off_p(s));
#pragma unroll
        for (int s = 0; s < 18; ++s) {
          const bf16x8 qs = *(const bf16x8*)(qrow + off_p(s));
          if (s & 1) so = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pr[s], qs, so, 0, 0, 0);
          else se = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pr[s], qs, se, 0, 0, 0);
          if (s < 16) *(bf16x8*)(vt + n16 * VT_PITCH + off_p(s)) = pr[s];
        }
      } else {
        bf16x8 pr[8];
        auto fix = [&](const bf16x8 v, const int s) -> bf16x8 {
          if (prot) return pr[s & 7];
          return valid ? v : bitcast<bf16x8>(u32x4{0u, 0u, 0u, 0u});
        };
#pragma unroll
        for (int grp = 0; grp < 2; ++grp) {
#pragma unroll
          for (int t = 0; t < 8; ++t) pr[t] = prot_slice(8 * grp + t);
          if constexpr (Fmt<F>::CBITS == 4) {
#pragma unroll
            for (int t = 0; t < 8; ++t) {
              const bf16x8 kv = fix(deq_int4x8(sl.c[2 * grp + (t >> 2)][t & 3], sl.mc[grp]), 8 * grp + t);
              qk(8 * grp + t, kv);
              *(bf16x8*)(rw + 64 * grp + 8 * t) = kv;
            }
          } else {
            const Lut2 lut = make_lut2(meta_scale(sl.mc[grp]), meta_zero(sl.mc[grp]));
#pragma unroll
            for (int w = 0; w < 4; ++w) {
              bf16x8 ka, kb;
              deq_int2x16(sl.c[grp][w], lut, ka, kb);
              ka = fix(ka, 8 * grp + 2 * w);
              kb = fix(kb, 8 * grp + 2 * w + 1);
              qk(8 * grp + 2 * w, ka);
              qk(8 * grp + 2 * w + 1, kb);
              *(bf16x8*)(rw + 64 * grp + 16 * w) = ka;
              *(bf16x8*)(rw + 64 * grp + 16 * w + 8) = kb;
            }
          }
        }
        pr[0] = prot_slice(16);
        pr[1] = prot_slice(17);
        qk(16, fix(deq_int4x8(sl.r[0], sl.mr), 16));
        qk(17, fix(deq_int4x8(sl.r[1], sl.mr), 17));
      }
    }

    return se + so;
  };
  // softmax and aggregation of quarter q from its scores sc[v] (token
  // i0 + 4g + v, head n16) and the content rows in the wave's tile
  auto aggregate = [&](const int q, const int phys, const f32x4 sc) {
    const int i0 = (p0 + (q >> 2)) * PAGE + QT * (q & 3);
    // scores in log2 units; tokens past the row's prefix (or an unusable
    // page) then become -inf -- a branch taken only at a prefix's end
    float x[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) x[v] = sc[v] * a.scale_log2;
    if (phys < 0 || !__all(i0 + QT <= L_row)) {
      const int lim = phys >= 0 ? L_row - i0 - 4 * g : 0;        // live offsets < lim
#pragma unroll
      for (int v = 0; v < 4; ++v)
        if (v >= lim) x[v] = -INFINITY;
    }
    const float tm = head_max4(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])));
    // first live quarter of the head sets its reference (all earlier weights
    // were 0); one beyond the headroom asks for a redo
    if (m_ref == -INFINITY) m_ref = tm;
    else if (tm > m_ref + REF_HEADROOM_LOG2) m_need = fmaxf(m_need, tm);
    const float mu = m_ref == -INFINITY ? 0.0f : m_ref;
    float e[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) e[v] = __builtin_amdgcn_exp2f(x[v] - mu);
    f_run += (e[0] + e[1]) + (e[2] + e[3]);
    const uint32_t h01 = pack_bf16x2(e[0], e[1]), h23 = pack_bf16x2(e[2], e[3]);
    const u32x4 pw = {h01, h23,
                      pack_bf16x2(e[0] - __uint_as_float(h01 << 16),
                                  e[1] - __uint_as_float(h01 & 0xffff0000u)),
                      pack_bf16x2(e[2] - __uint_as_float(h23 << 16),
                                  e[3] - __uint_as_float(h23 & 0xffff0000u))};
    const bf16x8 pb = bitcast<bf16x8>(pw);
    // O^T[16nb + 4g + v][head] += C^T . P^T over the quarter's 16 tokens
    const uint16_t* va = vt + (4 * g + (n16 >> 2)) * VT_PITCH + 4 * (n16 & 3);
    // transposed reads run CPF dim tiles ahead of their MFMA (LDS latency)
    constexpr int CPF = 6;
    bf16x4 cn[CPF];
#pragma unroll
    for (int nb = 0; nb < CPF; ++nb)
      cn[nb] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(va + 16 * nb));
#pragma unroll
    for (int nb = 0; nb < 32; ++nb) {
      const bf16x4 c4 = cn[nb % CPF];
      if (nb + CPF < 32)
        cn[nb % CPF] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(va + 16 * (nb + CPF)));
      const bf16x8 ct = __builtin_shufflevector(c4, c4, 0, 1, 2, 3, 0, 1, 2, 3);
      acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ct, pb, acc[nb], 0, 0, 0);
    }
  };

  // Is quarter q ordinary for this wave (position, page id and scales)?
  auto ordinary = [&](const int q, const int phys, const LaneSlot<F>& sl) {
    const int i0 = (p0 + (q >> 2)) * PAGE + QT * (q & 3);
    if (phys < 0 || i0 < NSINK || i0 + QT > L - NRECENT) return false;
    bool fits = meta_scale(sl.mr) * 512.0f <= FP8_PATH_MAX_SCALE9;
    if constexpr (Fmt<F>::CBITS == 4)
      fits = fits && meta_scale(sl.mc[0]) * 512.0f <= FP8_PATH_MAX_SCALE9 &&
             meta_scale(sl.mc[1]) * 512.0f <= FP8_PATH_MAX_SCALE9;
    return !__any(!fits);
  };

  auto load_quarter = [&](const int q) -> LaneSlot<F> {
    return load_lane_slot<F>(page_ptr(pw.id(q >> 2)), QT * (q & 3) + n16, g);
  };

  // ---- this wave's quarters wave, wave+8, ...; the codes of the next one
  // are loaded as soon as the current one's are consumed (its aggregation
  // and the other wave on the SIMD cover the latency)
  for (;;) {
#pragma unroll
    for (int nb = 0; nb < 32; ++nb) acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
    f_run = 0.f;
    pw.init(lane);
    if (wave < nquart) {
      LaneSlot<F> cur = load_quarter(wave);
      for (int q = wave; q < nquart; q += NW) {
        // a wave reconstructing and scoring issues ahead of the other wave on
        // its SIMD; a wave aggregating fills the issue slots that leaves
        __builtin_amdgcn_s_setprio(1);
        const int phys = pw.id(q >> 2);
        pw.advance((q + NW < nquart ? q + NW : q) >> 2, lane);
        const f32x4 sc = ordinary(q, phys, cur) ? quarter(std::true_type{}, q, phys, cur)
                                                : quarter(std::false_type{}, q, phys, cur);
        cur = load_quarter(q + NW < nquart ? q + NW : q);
        __builtin_amdgcn_s_setprio(0);
        aggregate(q, phys, sc);
      }
    }
    __builtin_amdgcn_s_setprio(0);
    // a head beyond the headroom: raise its reference, redo this wave's part
    if (!__any(m_need != -INFINITY)) break;
    if (m_need != -INFINITY) m_ref = m_need;
    m_need = -INFINITY;
  }

  // ---- merge the eight waves through LDS (log-sum-exp rule).  The
  // accumulators are only stored, RD output dims per round; thread t merges
  // head t/32, dims 4(t%32) .. +3 and RD/2 + 4(t%32) .. +3 of the round, so
  // the 32 threads of a head read contiguous 16-byte pieces (no two lanes of
  // a read on one bank).
  float f_tot = f_run + __shfl_xor(f_run, 16, 64);
  f_tot += __shfl_xor(f_tot, 32, 64);              // lane n16: head n16's sum over the wave
  constexpr int RD = 256;                                // output dims per round
  constexpr int MP = RD + 4;                             // row pitch: no bank conflicts
  float* mo = reinterpret_cast<float*>(lds);            // [NW][16 heads][MP]
  float* mm = mo + NW * 16 * MP;                         // [NW][16 heads][2]
  static_assert(sizeof(float) * (NW * 16 * (MP + 2)) <= sizeof(uint16_t) * LDS_ELEMS, "merge");
  __syncthreads();                                 // every wave is done with its tile
  if (g == 0) {
    mm[(wave * 16 + n16) * 2] = m_ref;
    mm[(wave * 16 + n16) * 2 + 1] = f_tot;
  }
  __syncthreads();
  const int hh = threadIdx.x >> 5, d4 = 4 * (threadIdx.x & 31);
  const int head = 16 * hg + hh;
  float M = -INFINITY;
#pragma unroll
  for (int w = 0; w < NW; ++w) M = fmaxf(M, mm[(w * 16 + hh) * 2]);
  float wt[NW], fs = 0.f;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const float mw = mm[(w * 16 + hh) * 2];
    wt[w] = mw == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mw - M);
    fs += wt[w] * mm[(w * 16 + hh) * 2 + 1];
  }
  float* dst;
  float osc;
  if (single) {
    dst = a.out + ((int64_t)b * H + head) * DC;
    osc = fs > 0.f ? 1.0f / fs : 0.f;
    if ((threadIdx.x & 31) == 0)
      a.lse[(int64_t)b * H + head] = fs > 0.f ? (M + __log2f(fs)) * 0.69314718055994531f : -INFINITY;
  } else {
    const int64_t base = ((int64_t)ss.first + j) * H + head;
    dst = a.ws_o + base * DC;
    osc = 1.0f;
    if ((threadIdx.x & 31) == 0) *(f32x4*)(a.ws_ml + base * 4) = f32x4{M, fs, fs, 0.f};
  }
#pragma unroll
  for (int r = 0; r < DC / RD; ++r) {
#pragma unroll
    for (int k = 0; k < RD / 16; ++k)              // dims 16(16r+k) + 4g + v
      *(f32x4*)(mo + (wave * 16 + n16) * MP + 16 * k + 4 * g) = acc[(RD / 16) * r + k];
    __syncthreads();
    f32x4 o0 = {0.f, 0.f, 0.f, 0.f}, o1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      o0 += wt[w] * *(const f32x4*)(mo + (w * 16 + hh) * MP + d4);
      o1 += wt[w] * *(const f32x4*)(mo + (w * 16 + hh) * MP + RD / 2 + d4);
    }
    *(f32x4*)(dst + RD * r + d4) = o0 * osc;
    *(f32x4*)(dst + RD * r + RD / 2 + d4) = o1 * osc;
    __syncthreads();
  }
  if (writer) fused_store<F>(a, fresh_row, b, L, sq, wave, NW, lane);
}

int launch_decode16w(int f, const DecodeArgs& a, hipStream_t stream) {
  const dim3 grid(a.nsplit, a.B, a.H / 16), block(512);
  if (f == 0)
    hipLaunchKernelGGL(decode16w_kernel<0>, grid, block, 0, stream, a);
  else if (f == 1)
    hipLaunchKernelGGL(decode16w_kernel<1>, grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL(decode16w_kernel<2>, grid, block, 0, stream, a);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

}  // namespace mlb
