// mla_decode_lowbit for 128-head blocks: native low-bit MLA decode attention
// [QuantMLA §3.3, App. C.5] in the absorbed form [MLA blog §4], for gfx950.
//
// With 128 heads sharing one latent, the two contractions per 64-token page
// ([128 x 576].[576 x 64] scores, [128 x 64].[64 x 512] aggregation) are
// matrix-core bound, so a page is reconstructed once per workgroup and read
// by all heads from LDS.  decode128_kernel<F>: one 256-thread workgroup
// (4 waves, one per SIMD) per (split j, sequence b, 128-head block), walking
// the split's pages through two LDS tiles [64 tokens][576 dims] of
// reconstructed bf16.  A call whose query rows are not a multiple of 128
// pads its last block: rows past H repeat row 0 of the sequence and write
// nothing.  In step k every wave does two jobs:
//   reconstruct page k+1 -- wave w takes token slots 16w .. 16w+15; lane
//      (n16, g) owns slot 16w + n16 and, in it, content groups 2g and 2g+1
//      (dims 128g .. 128g+127) and RoPE dims 16g .. 16g+15, from packed codes
//      loaded one step earlier.  Protected tokens take their BF16 row
//      instead (a wave whose 16 slots are all protected only copies rows),
//      unusable slots zeros.
//   attend page k -- wave w owns heads 32w .. 32w+31 of the block, with
//      v_mfma_f32_32x32x16_bf16.  Scores are formed transposed,
//      S^T[tokens][heads] = K . Q^T (K slices read from the tile, the query
//      held in registers), so lane (head l%32, h = l/32) ends up with the
//      scores of its own head for tokens 8i + 4h + 0..3 of a 32-token chunk.
//      Those are exactly the weights the lane contributes to the aggregation
//      O^T[dims][heads] += C^T . P^T when the C^T operand is read with
//      ds_read_b64_tr_b16 over the matching token rows, so the softmax
//      [QuantMLA §3.3] moves no data between lanes except one lane swap for
//      a head maximum.  Each weight enters the MFMA as bf16 hi + lo terms, as
//      in the 16-head kernel.
// The 256 accumulators per lane live in AGPRs and are never read inside the
// page loop: a head's reference maximum is fixed by its first live chunk and
// later weights 2^(x - m_ref) may exceed 1 by up to 2^REF_HEADROOM_LOG2,
// which fp32 sums and the bf16 hi/lo split carry exactly.  A score beyond
// that headroom makes the workgroup raise the head's reference to it and
// redo the split from zero accumulators -- the same single softmax, and each
// redo raises a reference by more than the headroom, so redos are bounded
// (realistic scores never trigger one).
// One barrier per step hands a tile over.  A split writes (max, weight sum,
// unnormalised O) to the workspace for the shared combine kernel; with a
// single split the kernel writes the final output itself.
#include <type_traits>

#include "common.h"
#include "dequant.h"
#include "internal.h"
#include "quantize.h"
#include "split_map.h"

namespace mlb {

namespace {

typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int KT_PITCH = DROW + 8;   // LDS tile row pitch (bf16 elements)
constexpr int HB = 128;              // heads per workgroup
constexpr float REF_HEADROOM_LOG2 = 64.0f;   // weights stay below 2^64 (fp32-safe sums)
constexpr float FP8_PATH_MAX_SCALE9 = 3.4028234663852886e38f;

// max over the two lanes of a head (l and l ^ 32)
__device__ __forceinline__ float pair_max(float x) {
  const auto r32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                    false, false);
  return fmaxf(__uint_as_float(r32[0]), __uint_as_float(r32[1]));
}

// The lane's index, recomputed where it is needed: two instructions cost less
// than holding lane-derived offsets across the page loop, where every
// register is taken.  Values hoisted out of the loop spill, and each reload
// waits on the vector memory counter, behind the packed-code loads in
// flight.  The asm is volatile so that it is neither hoisted nor merged.
__device__ __forceinline__ int lane_here() {
  int l;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
  return l;
}

}  // namespace

template <int F>
__global__ __launch_bounds__(256, 1) void decode128_kernel(DecodeArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t ktile[2][PAGE * KT_PITCH];
  __shared__ int redo_flag;

  const int hb = blockIdx.z;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  // the sequence and split of this workgroup's slot
  const SplitSlot ss = split_slot(a, blockIdx.y * a.nsplit + blockIdx.x, lane);
  if (ss.b < 0) return;                            // idle slot of a balanced plan
  const int j = ss.j, b = ss.b;
  const int n16 = lane & 15, g = lane >> 4;        // reconstruction role
  const int tt = 16 * wave + n16;                  // this lane's token slot
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  const int l32 = lane & 31, h = lane >> 5;        // attention role
  const int H = a.H;
  const int head = HB * hb + 32 * wave + l32;      // this lane's head
  // a padding row (past H) repeats row 0 of the sequence, query and causal
  // length both, and writes nothing
  const bool live = head < H;
  const int qrow = live ? head : 0;

  const int L = ss.L, sq = ss.sq;
  const int npages = (L + PAGE - 1) / PAGE;
  const int p0 = j * ss.pps;
  const int p1 = min(p0 + ss.pps, npages);
  const bool single = a.nsplit == 1;
  const int rows_here = min(HB, H - HB * hb);      // rows past H are padding
  if (p0 >= p1) {
    if (single && j == 0) {                        // empty sequence: out 0, lse -inf
      float* o = a.out + ((int64_t)b * H + HB * hb) * DC;
      for (int idx = threadIdx.x; idx < rows_here * DC / 4; idx += 256)
        *(f32x4*)(o + 4 * idx) = f32x4{0.f, 0.f, 0.f, 0.f};
      if (threadIdx.x < rows_here) a.lse[(int64_t)b * H + HB * hb + threadIdx.x] = -INFINITY;
    } else if (!single && threadIdx.x < rows_here) {   // no tokens: m = -inf for the merge
      const int64_t base = ((int64_t)ss.first + j) * H + HB * hb + threadIdx.x;
      *(f32x4*)(a.ws_ml + base * 4) = f32x4{-INFINITY, 0.f, 0.f, 0.f};
    }
    return;
  }
  const int np = p1 - p0;
  // tokens the lane's row attends to: the causal prefix of its query, all L
  // when there is one query per sequence
  const int L_row = L - (a.nq - 1 - qrow / a.hq);
  // fused writer: token L-1 of a sequence whose length is within bounds (a
  // clamped length names a token the cache already holds: nothing is stored
  // or substituted, and the call decodes as mla_decode_lowbit)
  const bool fused = a.new_c != nullptr && a.seq_lens[b] <= a.max_seq_len;
  // fused writer: the middle split of the sequence (first head block)
  // stores the newest token before its page loop.  No workgroup of this
  // launch reads those bytes; a middle split holds neither the sink tokens
  // nor the recent window, so it has time to spare; and this kernel has no
  // registers to spare for holding the row across the loop.
  if (fused && j == (npages + ss.pps - 1) / ss.pps / 2 && hb == 0) {
    fused_store<F>(a, fused_load(a, b, wv, 4, lane), b, L, sq, wv, 4, lane);
  }

  // physical page ids of the split (-1 = unusable table entry)
  PageWindow pw{a.block_table + (int64_t)b * a.max_blocks + p0, np, a.num_pages, 0, 0, 0};
  auto page_ptr = [&](int phys) -> const uint8_t* {
    return a.pages + (int64_t)(phys >= 0 ? phys : 0) * Fmt<F>::PAGE_BYTES;
  };

  // ---- query: B operand of the transposed score product.  Slice s < 32 is
  // content dims 16s + 8h .. +7, slices 32..35 the RoPE dims 16(s-32) + 8h.
  bf16x8 qv[36];
  {
    const uint16_t* ql = a.q_lat + ((int64_t)b * H + qrow) * DC + 8 * h;
#pragma unroll
    for (int s = 0; s < 32; ++s) qv[s] = *(const bf16x8*)(ql + 16 * s);
    const uint16_t* qr = a.q_rope + ((int64_t)b * H + qrow) * DR + 8 * h;
#pragma unroll
    for (int s = 0; s < 4; ++s) qv[32 + s] = *(const bf16x8*)(qr + 16 * s);
  }
  const uint16_t* prot_seq = a.prot + (int64_t)sq * PROT_ROWS * DROW;

  // ---- reconstruct page k (physical id `phys`) from `cur` into tile k & 1:
  // row tt, content dims 128g .. 128g+127 and RoPE dims 16g .. 16g+15.
  auto build = [&](auto ordinary_tag, const LaneSlot<F>& cur, const int k, const int phys) {
    constexpr bool ORDINARY = decltype(ordinary_tag)::value;
    // the lane's slot and group pair, recomputed (see lane_here)
    const int lid = lane_here();
    const int tt = 16 * wv + (lid & 15), g = lid >> 4;
    uint16_t* row = ktile[k & 1] + tt * KT_PITCH;
    uint16_t* rc = row + 128 * g;
    uint16_t* rr = row + DC + 16 * g;
    if constexpr (ORDINARY) {
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        if constexpr (Fmt<F>::CBITS == 4) {
          const float s9 = meta_scale(cur.mc[q]) * 512.0f, z = meta_zero(cur.mc[q]);
#pragma unroll
          for (int t = 0; t < 8; ++t)
            *(bf16x8*)(rc + 64 * q + 8 * t) = deq_int4x8_fp8(cur.c[2 * q + (t >> 2)][t & 3], s9, z);
        } else {
          const Lut2 lut = make_lut2(meta_scale(cur.mc[q]), meta_zero(cur.mc[q]));
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            bf16x8 kv0, kv1;
            deq_int2x16(cur.c[q][u], lut, kv0, kv1);
            *(bf16x8*)(rc + 64 * q + 16 * u) = kv0;
            *(bf16x8*)(rc + 64 * q + 16 * u + 8) = kv1;
          }
        }
      }
      const float s9r = meta_scale(cur.mr) * 512.0f, zr = meta_zero(cur.mr);
      *(bf16x8*)rr = deq_rope8_fp8<F>(cur.r[0], s9r, zr);
      *(bf16x8*)(rr + 8) = deq_rope8_fp8<F>(cur.r[1], s9r, zr);
    } else {
      // a page holding a sink or recent-window token, unusable slots, or a
      // scale beyond the fp8 path: per-lane substitutions, slice by slice
      const int i = (p0 + k) * PAGE + tt;
      const bool valid = phys >= 0 && i < L;
      const bool prot = valid && is_protected(i, L);
      // bf16 row of a protected token: its protection-buffer row, or for the
      // token the fused writer stores in this call, the new row itself
      const bool fresh = fused && i == L - 1;
      const uint16_t* prow = prot_seq + (int64_t)(prot ? prot_row(i) : 0) * DROW;
      const uint16_t* pc = fresh ? a.new_c + (int64_t)b * DC : prow;
      const uint16_t* pr = fresh ? a.new_r + (int64_t)b * DR : prow + DC;
      auto fix = [&](const bf16x8 v, const int off) -> bf16x8 {
        if (prot) return off < DC ? *(const bf16x8*)(pc + off) : *(const bf16x8*)(pr + (off - DC));
        return valid ? v : bitcast<bf16x8>(u32x4{0u, 0u, 0u, 0u});
      };
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        if constexpr (Fmt<F>::CBITS == 4) {
#pragma unroll
          for (int t = 0; t < 8; ++t)
            *(bf16x8*)(rc + 64 * q + 8 * t) =
                fix(deq_int4x8(cur.c[2 * q + (t >> 2)][t & 3], cur.mc[q]), 128 * g + 64 * q + 8 * t);
        } else {
          const Lut2 lut = make_lut2(meta_scale(cur.mc[q]), meta_zero(cur.mc[q]));
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            bf16x8 kv0, kv1;
            deq_int2x16(cur.c[q][u], lut, kv0, kv1);
            *(bf16x8*)(rc + 64 * q + 16 * u) = fix(kv0, 128 * g + 64 * q + 16 * u);
            *(bf16x8*)(rc + 64 * q + 16 * u + 8) = fix(kv1, 128 * g + 64 * q + 16 * u + 8);
          }
        }
      }
      *(bf16x8*)rr = fix(deq_int4x8(cur.r[0], cur.mr), DC + 16 * g);
      *(bf16x8*)(rr + 8) = fix(deq_int4x8(cur.r[1], cur.mr), DC + 16 * g + 8);
    }
  };
  // Is page k ordinary for this wave: are its 16 slots all packed tokens
  // (none a sink, none in the recent window, all within the length) whose
  // scales suit the fp8 path?  Decided per wave, so on the page holding the
  // sinks or the window's start only the waves with such slots leave the
  // fast path.
  auto ordinary = [&](const LaneSlot<F>& cur, const int k, const int phys) -> bool {
    const int i0 = (p0 + k) * PAGE + 16 * wv;
    if (phys < 0 || i0 < NSINK || i0 + 16 > L - NRECENT) return false;
    bool fits = meta_scale(cur.mr) * 512.0f <= FP8_PATH_MAX_SCALE9;
    if constexpr (Fmt<F>::CBITS == 4)
      fits = fits && meta_scale(cur.mc[0]) * 512.0f <= FP8_PATH_MAX_SCALE9 &&
             meta_scale(cur.mc[1]) * 512.0f <= FP8_PATH_MAX_SCALE9;
    return !__any(!fits);
  };
  // Are all of this wave's slots of page k protected (recent-window or sink
  // rows, the fused writer's token among them)?
  auto all_protected = [&](const int k, const int phys) -> bool {
    const int i = (p0 + k) * PAGE + 16 * wv + (lane_here() & 15);
    return __all(phys >= 0 && i < L && is_protected(i, L));
  };
  // such a page has nothing to reconstruct: its BF16 rows are copied with
  // the loads in three batches of six slices (one memory latency per batch,
  // not one per slice)
  auto copy_protected = [&](const int k) {
    const int lid = lane_here();
    const int tt = 16 * wv + (lid & 15), g = lid >> 4;
    const int i = (p0 + k) * PAGE + tt;
    uint16_t* row = ktile[k & 1] + tt * KT_PITCH;
    const bool fresh = fused && i == L - 1;
    const uint16_t* prow = prot_seq + (int64_t)prot_row(i) * DROW;
    const uint16_t* pc = (fresh ? a.new_c + (int64_t)b * DC : prow) + 128 * g;
    const uint16_t* pr = (fresh ? a.new_r + (int64_t)b * DR : prow + DC) + 16 * g;
#pragma unroll
    for (int t0 = 0; t0 < 18; t0 += 6) {
      bf16x8 v[6];
#pragma unroll
      for (int t = 0; t < 6; ++t)
        v[t] = *(const bf16x8*)(t0 + t < 16 ? pc + 8 * (t0 + t) : pr + 8 * (t0 + t - 16));
#pragma unroll
      for (int t = 0; t < 6; ++t)
        *(bf16x8*)(t0 + t < 16 ? row + 128 * g + 8 * (t0 + t) : row + DC + 16 * g + 8 * (t0 + t - 16)) = v[t];
      __builtin_amdgcn_sched_barrier(0);   // the next batch's loads stay below
    }
  };
  auto build_page = [&](const LaneSlot<F>& cur, const int k, const int phys) {
    if (ordinary(cur, k, phys)) build(std::true_type{}, cur, k, phys);
    else if (all_protected(k, phys)) copy_protected(k);
    else build(std::false_type{}, cur, k, phys);
  };

  // ---- attention state of lane (head l32, h): m_ref reference maximum
  // (log2 units), f_run sum of the fp32 weights of this lane's tokens,
  // acc[nt][4i + jj] = O[head][32nt + 8i + 4h + jj]; m_need: the reference a
  // redo would need (-inf: none).
  f32x16 acc[16];
  float m_ref = -INFINITY, f_run = 0.f, m_need = -INFINITY;

  // attend page k in 32-token chunks
  auto attend = [&](const int k, const int phys) {
    const uint16_t* kb = ktile[k & 1];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      // S^T[32c + m][head], m = 8i + 4h + jj in register 4i + jj
      f32x16 sacc;
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[r] = 0.f;
      const uint16_t* ka = kb + (32 * c + l32) * KT_PITCH + 8 * h;
      // K slices are read SPF slices ahead of their MFMA (LDS latency; a
      // fourth slice in flight measured no faster)
      constexpr int SPF = 3;
      bf16x8 kn[SPF];
#pragma unroll
      for (int s = 0; s < SPF; ++s) kn[s] = *(const bf16x8*)(ka + 16 * s);
#pragma unroll
      for (int s = 0; s < 36; ++s) {
        const bf16x8 kv = kn[s % SPF];
        if (s + SPF < 36) kn[s % SPF] = *(const bf16x8*)(ka + 16 * (s + SPF));
        sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kv, qv[s], sacc, 0, 0, 0);
      }
      // scores in log2 units; tokens past the row's prefix (or on an
      // unusable page) are -inf.  Register r holds token offset
      // 8(r/4) + r%4 past lim's origin, a constant, so each score costs one
      // compare against the chunk's limit.
      const int lim = phys >= 0 ? L_row - ((p0 + k) * PAGE + 32 * c + 4 * h) : 0;
#pragma unroll
      for (int r = 0; r < 16; ++r)
        sacc[r] = 8 * (r >> 2) + (r & 3) < lim ? sacc[r] * a.scale_log2 : -INFINITY;
      float tm = sacc[0];
#pragma unroll
      for (int r = 1; r < 16; ++r) tm = fmaxf(tm, sacc[r]);
      tm = pair_max(tm);
      // first live chunk of the head sets its reference (all earlier weights
      // were 0); a chunk beyond the headroom asks for a redo
      if (m_ref == -INFINITY) m_ref = tm;
      else if (tm > m_ref + REF_HEADROOM_LOG2) m_need = fmaxf(m_need, tm);
      const float mu = m_ref == -INFINITY ? 0.0f : m_ref;
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        // weights of half q (tokens 16q .. 16q+15 of the chunk) are registers
        // 8q .. 8q+7: tokens 16q + 4h + 0..3 and 16q + 8 + 4h + 0..3
        u32x4 phi, plo;
        float ft = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float e0 = __builtin_amdgcn_exp2f(sacc[8 * q + 2 * e] - mu);
          const float e1 = __builtin_amdgcn_exp2f(sacc[8 * q + 2 * e + 1] - mu);
          ft += e0 + e1;
          const uint32_t hbits = pack_bf16x2(e0, e1);
          phi[e] = hbits;
          plo[e] = pack_bf16x2(e0 - __uint_as_float(hbits << 16),
                               e1 - __uint_as_float(hbits & 0xffff0000u));
        }
        f_run += ft;
        const bf16x8 pa = bitcast<bf16x8>(phi), pl = bitcast<bf16x8>(plo);
        // C^T operand: dim 32nt + l32, tokens 16q + 4h + 0..3 and
        // 16q + 8 + 4h + 0..3, read one dim tile ahead of its MFMAs
        const uint16_t* va = kb + (32 * c + 16 * q + 4 * h + (n16 >> 2)) * KT_PITCH +
                             16 * ((lane >> 4) & 1) + 4 * (n16 & 3);
        const uint16_t* vb = va + 8 * KT_PITCH;
        bf16x4 cl = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)va);
        bf16x4 ch = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)vb);
#pragma unroll
        for (int nt = 0; nt < 16; ++nt) {
          const bf16x8 ct = __builtin_shufflevector(cl, ch, 0, 1, 2, 3, 4, 5, 6, 7);
          if (nt + 1 < 16) {
            cl = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(va + 32 * (nt + 1)));
            ch = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(vb + 32 * (nt + 1)));
          }
          acc[nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ct, pa, acc[nt], 0, 0, 0);
          acc[nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ct, pl, acc[nt], 0, 0, 0);
        }
      }
    }
  };

  // ---- pipeline: page k+1 is reconstructed while page k is attended; the
  // packed codes of page k+2 are loaded right after page k+1 has consumed
  // its registers (the last page reloads itself, so the wait stays exact).
  for (;;) {
#pragma unroll
    for (int nt = 0; nt < 16; ++nt)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[nt][r] = 0.f;
    f_run = 0.f;
    if (threadIdx.x == 0) redo_flag = 0;
    pw.init(lane);
    int id_k = pw.id(0), id_k1 = pw.id(min(1, np - 1));
    // pages 0 and 1 are requested together: page 1's codes must not wait
    // for page 0's build
    LaneSlot<F> cur = load_lane_slot<F>(page_ptr(id_k), tt, g);
    const LaneSlot<F> cur1 = load_lane_slot<F>(page_ptr(id_k1), tt, g);
    build_page(cur, 0, id_k);
    cur = cur1;
    __syncthreads();
    for (int k = 0; k < np; ++k) {
      pw.advance(min(k + 2, np - 1), lane);
      const int id_k2 = pw.id(min(k + 2, np - 1));
      if (k + 1 < np) {
        build_page(cur, k + 1, id_k1);
        cur = load_lane_slot<F>(page_ptr(id_k2), tt, g);
      }
      attend(k, id_k);
      __syncthreads();
      id_k = id_k1;
      id_k1 = id_k2;
    }
    // a head beyond the headroom: raise its reference, redo the split
    if (__any(m_need != -INFINITY) && lane == 0) redo_flag = 1;
    __syncthreads();
    if (redo_flag == 0) break;
    if (m_need != -INFINITY) m_ref = m_need;
    m_need = -INFINITY;
    __syncthreads();                               // flag read before it is cleared
  }

  // ---- outputs: the weight sum of the head over its two lanes
  const float f_tot = f_run + __shfl_xor(f_run, 32, 64);
  if (!live) return;
  if (single) {
    const float inv = f_tot > 0.f ? 1.0f / f_tot : 0.f;
    float* o = a.out + ((int64_t)b * H + head) * DC + 4 * h;
#pragma unroll
    for (int nt = 0; nt < 16; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        *(f32x4*)(o + 32 * nt + 8 * i) =
            f32x4{acc[nt][4 * i], acc[nt][4 * i + 1], acc[nt][4 * i + 2], acc[nt][4 * i + 3]} * inv;
    if (h == 0)
      a.lse[(int64_t)b * H + head] =
          f_tot > 0.f ? (m_ref + __log2f(f_tot)) * 0.69314718055994531f : -INFINITY;
  } else {
    const int64_t base = ((int64_t)ss.first + j) * H + head;
    float* o = a.ws_o + base * DC + 4 * h;
#pragma unroll
    for (int nt = 0; nt < 16; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        *(f32x4*)(o + 32 * nt + 8 * i) =
            f32x4{acc[nt][4 * i], acc[nt][4 * i + 1], acc[nt][4 * i + 2], acc[nt][4 * i + 3]};
    if (h == 0) *(f32x4*)(a.ws_ml + base * 4) = f32x4{m_ref, f_tot, f_tot, 0.f};
  }
}

int launch_decode128(int f, const DecodeArgs& a, hipStream_t stream) {
  const dim3 grid(a.nsplit, a.B, (a.H + HB - 1) / HB), block(256);
  if (f == 0)
    hipLaunchKernelGGL(decode128_kernel<0>, grid, block, 0, stream, a);
  else if (f == 1)
    hipLaunchKernelGGL(decode128_kernel<1>, grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL(decode128_kernel<2>, grid, block, 0, stream, a);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

}  // namespace mlb
