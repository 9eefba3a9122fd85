// mla_decode_lowbit: native low-bit MLA decode attention [QuantMLA §3.3,
// App. C.5] in the absorbed form [MLA blog §4], for gfx950.
//
// decode16_kernel<F>: one 512-thread workgroup (8 waves, one per CU) per
// (split j, sequence b, 16-head group), walking the split's 64-token pages
// through two LDS page buffers.  In step t every wave does two jobs:
//   build page t -- wave w takes the 16 token slots of block w%4 and dim half
//      w/4.  Lane (n16, g) owns slot 16*(w%4)+n16 and, in that half, one
//      64-dim content group plus 8 RoPE dims.  Its packed codes were loaded
//      one step earlier (two named register buffers), so HBM latency overlaps
//      the previous step.  The reconstructed bf16 slices are directly the B
//      operand of v_mfma_f32_16x16x32_bf16 against the query (dims permuted
//      identically), giving a partial score tile S[16 heads][16 slots] over
//      the half's 288 dims; protected tokens use their BF16 row instead.
//      Content slices also go to the page's LDS tile [64][512], which feeds
//      the aggregation: every value is reconstructed once and used for both
//      products [QuantMLA App. C.5].
//   aggregate page t-1 -- wave w owns token half w%2 and output dims
//      128*(w/2) ..+127.  Lane (head n16, g) sums the two partial scores of
//      its 8 tokens; one online softmax [QuantMLA §3.3] (tile maximum shared
//      by the four lanes of a head through lane swaps) turns them into
//      weights, split into bf16 hi + lo terms that are directly the A operand
//      of the aggregation MFMA: O += P[16][32] . C[32][128], with C read by
//      ds_read_b64_tr_b16 transposed LDS reads.
// The choices a step depends on are made once per step and per wave (is page
// t an ordinary page? does page t-1 raise a head's reference maximum?), so
// the common path has no per-lane branches.
// One barrier per step hands a page buffer over.  The two token halves keep
// separate running maxima and are merged by the log-sum-exp rule once per
// split; a split writes (max, weight sum, unnormalised O) to the workspace and
// combine_kernel merges the splits by the same rule [QuantMLA App. C.5]; with
// a single split the kernel writes the final output itself.
#include <type_traits>

#include "common.h"
#include "dequant.h"
#include "internal.h"

namespace mlb {

typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

constexpr int CT_PITCH = DC + 8;   // LDS content tile row pitch (bf16 elements)
constexpr int SX_PITCH = 64 + 4;   // LDS score tile row pitch (floats)

// Rescale threshold of the online softmax, in log2 units: the reference
// maximum of a head only moves when a tile's maximum exceeds it by more than
// this, so weights exp2(x - m_ref) stay below 2^8 and the common case needs no
// rescaling of the accumulators.  The result is the same single softmax.
constexpr float RESCALE_LOG2 = 8.0f;

// Largest scale whose 2^9 multiple is finite (the fp8 conversion path).
constexpr float FP8_PATH_MAX_SCALE9 = 3.4028234663852886e38f;

template <int F>
__global__ __launch_bounds__(512, 1) void decode16_kernel(DecodeArgs a) {
  // two page buffers: step t fills one while the other is aggregated
  __shared__ __attribute__((aligned(16))) uint16_t ctile[2][PAGE * CT_PITCH];
  __shared__ __attribute__((aligned(16))) float sx[2][2][16 * SX_PITCH];  // [buf][dim half][head][slot]

  const int j = blockIdx.x, b = blockIdx.y, hg = blockIdx.z;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n16 = lane & 15, g = lane >> 4;
  const int tb = wave & 3, dh = wave >> 2;         // build role: token block, dim half
  const int th = wave & 1, dq = wave >> 1;         // aggregate role: token half, dims/128
  const int tt = 16 * tb + n16;                    // this lane's token slot
  const int H = a.H;

  int L = a.seq_lens[b];
  L = L < 0 ? 0 : (L > a.max_seq_len ? a.max_seq_len : L);
  const int sq = a.seq_slot[b];
  if (sq < 0 || sq >= a.num_seq_slots) L = 0;    // unusable sequence slot -> empty
  const int npages = (L + PAGE - 1) / PAGE;
  const int p0 = j * a.pps;
  const int p1 = min(p0 + a.pps, npages);
  const bool single = a.nsplit == 1;
  if (p0 >= p1) {
    if (single && j == 0) {                        // empty sequence: out 0, lse -inf
      for (int idx = threadIdx.x; idx < 16 * DC; idx += 512)
        a.out[((int64_t)b * H + hg * 16) * DC + idx] = 0.0f;
      if (threadIdx.x < 16) a.lse[(int64_t)b * H + hg * 16 + threadIdx.x] = -INFINITY;
    }
    return;
  }
  const int np = p1 - p0;

  // Block-table row of the split, read with scalar loads (uniform address,
  // read-only data): page ids never pass through LDS or vector registers.
  const __attribute__((address_space(4))) int32_t* bt_row =
      (const __attribute__((address_space(4))) int32_t*)(a.block_table +
                                                         (int64_t)b * a.max_blocks + p0);
  auto page_id = [&](int k) -> int {              // -1 = unusable table entry
    const int phys = bt_row[k];
    return (phys >= 0 && phys < a.num_pages) ? phys : -1;
  };
  auto page_ptr = [&](int phys) -> const uint8_t* {
    return a.pages + (int64_t)(phys >= 0 ? phys : 0) * Fmt<F>::PAGE_BYTES;
  };

  // ---- query registers: head 16*hg + n16, the lane's content and RoPE dims
  bf16x8 qc[8], qr;
  {
    const int head = hg * 16 + n16;
    const uint16_t* ql = a.q_lat + ((int64_t)b * H + head) * DC + 256 * dh + 64 * g;
#pragma unroll
    for (int t = 0; t < 8; ++t) qc[t] = *(const bf16x8*)(ql + 8 * t);
    qr = *(const bf16x8*)(a.q_rope + ((int64_t)b * H + head) * DR + 32 * dh + 8 * g);
  }
  const uint16_t* prot_seq = a.prot + (int64_t)sq * PROT_ROWS * DROW;

  // ---- build: reconstruct + score page k (physical id `phys`) from `cur`
  // into buffer k & 1.  ORDINARY: every slot is a cached, unprotected token
  // and every scale takes the fp8 conversion (no per-lane choices at all).
  auto build = [&](auto ordinary_tag, const Packed<F>& cur, const int k, const int phys) {
    constexpr bool ORDINARY = decltype(ordinary_tag)::value;
    uint16_t* ct = ctile[k & 1];
    const int i = (p0 + k) * PAGE + tt;
    const bool valid = phys >= 0 && i < L;
    f32x4 s = {0.f, 0.f, 0.f, 0.f};
    if constexpr (ORDINARY) {
      // slice by slice: reconstruct, score, store
      if constexpr (F == 0) {
        const float s9 = meta_scale(cur.mc) * 512.0f, z = meta_zero(cur.mc);
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const bf16x8 kv = deq_int4x8_fp8(cur.c[t >> 2][t & 3], s9, z);
          s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qc[t], kv, s, 0, 0, 0);
          *(bf16x8*)(ct + tt * CT_PITCH + 256 * dh + 64 * g + 8 * t) = kv;
        }
      } else {
        const Lut2 lut = make_lut2(meta_scale(cur.mc), meta_zero(cur.mc));
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          bf16x8 kv0, kv1;
          deq_int2x16(cur.c[q], lut, kv0, kv1);
          s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qc[2 * q], kv0, s, 0, 0, 0);
          *(bf16x8*)(ct + tt * CT_PITCH + 256 * dh + 64 * g + 16 * q) = kv0;
          s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qc[2 * q + 1], kv1, s, 0, 0, 0);
          *(bf16x8*)(ct + tt * CT_PITCH + 256 * dh + 64 * g + 16 * q + 8) = kv1;
        }
      }
      s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
          qr, deq_int4x8_fp8(cur.rc, meta_scale(cur.mr) * 512.0f, meta_zero(cur.mr)), s, 0, 0, 0);
    } else {
      bf16x8 kv[8], kr;
      // a page holding a sink or recent-window token (at most 3 per
      // sequence), unusable slots, or a scale beyond the fp8 path
      deq_content<F>(cur, kv);
      kr = deq_rope<F>(cur);
      if (valid && is_protected(i, L)) {
        const uint16_t* prow = prot_seq + (int64_t)prot_row(i) * DROW;
#pragma unroll
        for (int t = 0; t < 8; ++t) kv[t] = *(const bf16x8*)(prow + 256 * dh + 64 * g + 8 * t);
        kr = *(const bf16x8*)(prow + DC + 32 * dh + 8 * g);
      } else if (!valid) {
#pragma unroll
        for (int t = 0; t < 8; ++t) kv[t] = bitcast<bf16x8>(u32x4{0u, 0u, 0u, 0u});
        kr = bitcast<bf16x8>(u32x4{0u, 0u, 0u, 0u});
      }
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qc[t], kv[t], s, 0, 0, 0);
        *(bf16x8*)(ct + tt * CT_PITCH + 256 * dh + 64 * g + 8 * t) = kv[t];
      }
      s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qr, kr, s, 0, 0, 0);
    }
    // s[v] = partial score (this dim half) of head 4g+v against slot tt
    float* sxb = sx[k & 1][dh];
#pragma unroll
    for (int v = 0; v < 4; ++v)
      sxb[(4 * g + v) * SX_PITCH + tt] = valid ? s[v] * a.scale_log2 : -INFINITY;
  };
  // Is page k ordinary for this wave (decided from its packed metadata)?
  auto ordinary = [&](const Packed<F>& cur, const int k, const int phys) -> bool {
    const int p = p0 + k;
    if (phys < 0 || p * PAGE < NSINK || (p + 1) * PAGE > L - NRECENT) return false;
    bool fits = meta_scale(cur.mr) * 512.0f <= FP8_PATH_MAX_SCALE9;
    if constexpr (F == 0) fits = fits && meta_scale(cur.mc) * 512.0f <= FP8_PATH_MAX_SCALE9;
    return !__any(!fits);
  };

  // ---- aggregation state.  Lane (head n16, g) of a wave: m_ref reference
  // maximum (log2 units) of head n16 over this token half, f_run sum of its
  // fp32 weights (partial over the lane's tokens; normalises the output and
  // gives the log-sum-exp).  acc[nb][v] = O[head 4g+v][128dq + 16nb + n16].
  // Each weight enters the MFMA as hi = bf16(p) and lo = bf16(p - hi), so the
  // weights multiplying the latent rows match the fp32 weights to ~2^-17.
  f32x4 acc[8];
#pragma unroll
  for (int nb = 0; nb < 8; ++nb) acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_ref = -INFINITY, f_run = 0.f;
  const int arow = 32 * th + 8 * g + (n16 >> 2);
  auto c_operand = [&](const uint16_t* ct, int nb) -> bf16x8 {   // C[32 tok][16 dims] slice nb
    const int col = 128 * dq + 16 * nb + 4 * (n16 & 3);
    const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(ct + arow * CT_PITCH + col));
    const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(ct + (arow + 4) * CT_PITCH + col));
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  };
  // scores of lane (head n16, g): tokens 32th + 8g .. +7, both dim halves summed
  auto read_scores = [&](const int k, f32x4& xa, f32x4& xb) {
    const float* s0 = sx[k & 1][0] + n16 * SX_PITCH + 32 * th + 8 * g;
    const float* s1 = sx[k & 1][1] + n16 * SX_PITCH + 32 * th + 8 * g;
    xa = *(const f32x4*)s0 + *(const f32x4*)s1;
    xb = *(const f32x4*)(s0 + 4) + *(const f32x4*)(s1 + 4);
  };
  // max over the four lanes n16, n16+16, n16+32, n16+48 (the lane groups of
  // one head) with lane-swap instructions (no LDS traffic)
  auto head_max = [](float x) -> float {
    const auto r16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x),
                                                      false, false);
    x = fmaxf(__uint_as_float(r16[0]), __uint_as_float(r16[1]));
    const auto r32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                      false, false);
    return fmaxf(__uint_as_float(r32[0]), __uint_as_float(r32[1]));
  };
  // aggregate page k given its scores and tile maximum tm.  RESCALE: some head
  // of the wave raises its reference maximum (always on the first live tile).
  auto aggregate = [&](auto rescale_tag, const int k, const f32x4 xa, const f32x4 xb,
                       const float tm) {
    constexpr bool RESCALE = decltype(rescale_tag)::value;
    const uint16_t* ct = ctile[k & 1];
    bf16x8 cb[4];
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) cb[nb] = c_operand(ct, nb);
    float alpha = 1.0f;
    if constexpr (RESCALE) {
      if (tm > m_ref + RESCALE_LOG2) {
        alpha = __builtin_amdgcn_exp2f(m_ref - tm);  // 0 while m_ref = -inf
        m_ref = tm;
      }
    }
    const float mu = m_ref == -INFINITY ? 0.0f : m_ref;
    u32x4 phi, plo;
    float ft = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const f32x4& x = e < 2 ? xa : xb;
      const float e0 = __builtin_amdgcn_exp2f(x[(2 * e) & 3] - mu);
      const float e1 = __builtin_amdgcn_exp2f(x[(2 * e + 1) & 3] - mu);
      ft += e0 + e1;
      const uint32_t hb = pack_bf16x2(e0, e1);
      phi[e] = hb;
      plo[e] = pack_bf16x2(e0 - __uint_as_float(hb << 16), e1 - __uint_as_float(hb & 0xffff0000u));
    }
    f_run = f_run * alpha + ft;
    if constexpr (RESCALE) {
      // O rows of this lane are heads 4g+v: rescale by those heads' alpha
      float av[4];
#pragma unroll
      for (int v = 0; v < 4; ++v) av[v] = __shfl(alpha, 4 * g + v, 64);
#pragma unroll
      for (int nb = 0; nb < 8; ++nb)
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[nb][v] *= av[v];
    }
    const bf16x8 pa = bitcast<bf16x8>(phi), pl = bitcast<bf16x8>(plo);
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) {
      const bf16x8 c = cb[nb & 3];
      if (nb < 4) cb[nb] = c_operand(ct, nb + 4);  // second batch of C slices
      acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa, c, acc[nb], 0, 0, 0);
      acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pl, c, acc[nb], 0, 0, 0);
    }
  };
  // does page k raise some head's reference maximum (wave-uniform answer)?
  auto tile_max = [&](const f32x4 xa, const f32x4 xb) -> float {
    return head_max(fmaxf(fmaxf(fmaxf(xa[0], xa[1]), fmaxf(xa[2], xa[3])),
                          fmaxf(fmaxf(xb[0], xb[1]), fmaxf(xb[2], xb[3]))));
  };

  // One step: build page t from `cur`, then aggregate page t-1.  Both
  // choices are wave-uniform branches: ordinary page or not, and (rarely)
  // whether page t-1 raises a head's reference maximum.
  auto step = [&](const Packed<F>& cur, const int t, const int phys) {
    if (ordinary(cur, t, phys)) build(std::true_type{}, cur, t, phys);
    else build(std::false_type{}, cur, t, phys);
    f32x4 xa, xb;
    read_scores(t - 1, xa, xb);
    const float tm = tile_max(xa, xb);
    if (__any(tm > m_ref + RESCALE_LOG2)) aggregate(std::true_type{}, t - 1, xa, xb, tm);
    else aggregate(std::false_type{}, t - 1, xa, xb, tm);
  };

  // ---- pipeline.  Register buffers A/B alternate by step parity (unrolled
  // by two, no copies); the prefetch is unconditional (the last page reloads
  // itself) so the memory counter waits stay exact.  Page ids are read one
  // step ahead.
  int id_cur = page_id(0), id_nxt = page_id(min(1, np - 1)), id_nn = page_id(min(2, np - 1));
  Packed<F> bufA = load_packed<F>(page_ptr(id_cur), tt, dh, g), bufB;
  bufB = load_packed<F>(page_ptr(id_nxt), tt, dh, g);
  if (ordinary(bufA, 0, id_cur)) build(std::true_type{}, bufA, 0, id_cur);
  else build(std::false_type{}, bufA, 0, id_cur);
  __syncthreads();
  for (int t = 1; t < np;) {
    id_cur = id_nxt; id_nxt = id_nn; id_nn = page_id(min(t + 2, np - 1));
    bufA = load_packed<F>(page_ptr(id_nxt), tt, dh, g);
    step(bufB, t, id_cur);
    __syncthreads();
    if (++t == np) break;
    id_cur = id_nxt; id_nxt = id_nn; id_nn = page_id(min(t + 2, np - 1));
    bufB = load_packed<F>(page_ptr(id_nxt), tt, dh, g);
    step(bufA, t, id_cur);
    __syncthreads();
    ++t;
  }
  {
    f32x4 xa, xb;
    read_scores(np - 1, xa, xb);
    const float tm = tile_max(xa, xb);
    if (__any(tm > m_ref + RESCALE_LOG2)) aggregate(std::true_type{}, np - 1, xa, xb, tm);
    else aggregate(std::false_type{}, np - 1, xa, xb, tm);
  }

  // ---- merge the two token halves (log-sum-exp), through LDS
  f_run += __shfl_xor(f_run, 16, 64);
  f_run += __shfl_xor(f_run, 32, 64);              // lane n16: head n16's total
  __syncthreads();                                 // all page reads done
  float* mb = reinterpret_cast<float*>(ctile[0]);  // [4 dq][16 heads][128]
  float* mf = mb + 4 * 16 * 128;                   // [4 dq][16 heads][2]
  if (th == 1) {
#pragma unroll
    for (int nb = 0; nb < 8; ++nb)
#pragma unroll
      for (int v = 0; v < 4; ++v) mb[(dq * 16 + 4 * g + v) * 128 + 16 * nb + n16] = acc[nb][v];
    if (g == 0) {
      mf[(dq * 16 + n16) * 2] = m_ref;
      mf[(dq * 16 + n16) * 2 + 1] = f_run;
    }
  }
  __syncthreads();
  if (th == 1) return;
  const float m1 = mf[(dq * 16 + n16) * 2], f1 = mf[(dq * 16 + n16) * 2 + 1];
  const float m = fmaxf(m_ref, m1);
  const float a0 = m_ref == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_ref - m);
  const float a1 = m1 == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m1 - m);
  const float fh = f_run * a0 + f1 * a1;           // head n16's weight sum
  float a0v[4], a1v[4], fv[4];
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    a0v[v] = __shfl(a0, 4 * g + v, 64);
    a1v[v] = __shfl(a1, 4 * g + v, 64);
    fv[v] = __shfl(fh, 4 * g + v, 64);
  }
#pragma unroll
  for (int nb = 0; nb < 8; ++nb)
#pragma unroll
    for (int v = 0; v < 4; ++v)
      acc[nb][v] = acc[nb][v] * a0v[v] + mb[(dq * 16 + 4 * g + v) * 128 + 16 * nb + n16] * a1v[v];

  if (single) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int h = hg * 16 + 4 * g + v;
      const float inv = 1.0f / fv[v];
      float* o = a.out + ((int64_t)b * H + h) * DC + 128 * dq + n16;
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) o[16 * nb] = acc[nb][v] * inv;
    }
    if (dq == 0 && g == 0)
      a.lse[(int64_t)b * H + hg * 16 + n16] = (m + __log2f(fh)) * 0.69314718055994531f;
  } else {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int h = hg * 16 + 4 * g + v;
      const int64_t base = ((int64_t)b * a.nsplit + j) * H + h;
      float* o = a.ws_o + base * DC + 128 * dq + n16;
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) o[16 * nb] = acc[nb][v];
    }
    if (dq == 0 && g == 0) {
      const int64_t base = ((int64_t)b * a.nsplit + j) * H + hg * 16 + n16;
      *(f32x4*)(a.ws_ml + base * 4) = f32x4{m, fh, fh, 0.f};
    }
  }
}

// ------------------------------------------------------------- combine -----
// grid (8 dim blocks, H/16, B), 256 threads: thread (hh = tid/16, c = tid%16)
// merges head 16*blockIdx.y + hh, dims 64*blockIdx.x + 4c .. +3 over the
// sequence's splits: m* = max m_j, weights e^(m_j - m*), out = sum w_j o_j /
// sum w_j l_j, lse = m* + ln sum w_j f_j  [QuantMLA App. C.5].
__global__ __launch_bounds__(256) void combine_kernel(DecodeArgs a) {
  const int b = blockIdx.z, H = a.H;
  const int hh = threadIdx.x >> 4, c = threadIdx.x & 15;
  const int h = blockIdx.y * 16 + hh;
  const int d0 = 64 * blockIdx.x + 4 * c;
  int L = a.seq_lens[b];
  L = L < 0 ? 0 : (L > a.max_seq_len ? a.max_seq_len : L);
  const int sq = a.seq_slot[b];
  if (sq < 0 || sq >= a.num_seq_slots) L = 0;
  const int npages = (L + PAGE - 1) / PAGE;
  const int ns = (npages + a.pps - 1) / a.pps;
  float* o = a.out + ((int64_t)b * H + h) * DC + d0;
  if (ns == 0) {
    *(f32x4*)o = f32x4{0.f, 0.f, 0.f, 0.f};
    if (blockIdx.x == 0 && c == 0) a.lse[(int64_t)b * H + h] = -INFINITY;
    return;
  }
  const int64_t base = (int64_t)b * a.nsplit * H + h;     // split jj at base + jj*H
  float M = -INFINITY;
  for (int jj = 0; jj < ns; ++jj) M = fmaxf(M, a.ws_ml[(base + (int64_t)jj * H) * 4]);
  f32x4 accv = {0.f, 0.f, 0.f, 0.f};
  float ssum = 0.f, fsum = 0.f;
  int jj = 0;
  for (; jj + 4 <= ns; jj += 4) {
    f32x4 ml[4], ov[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t e = base + (int64_t)(jj + u) * H;
      ml[u] = *(const f32x4*)(a.ws_ml + e * 4);
      ov[u] = *(const f32x4*)(a.ws_o + e * DC + d0);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float wgt = ml[u][0] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(ml[u][0] - M);
      ssum += wgt * ml[u][1];
      fsum += wgt * ml[u][2];
      accv += wgt * ov[u];
    }
  }
  for (; jj < ns; ++jj) {
    const int64_t e = base + (int64_t)jj * H;
    const f32x4 ml = *(const f32x4*)(a.ws_ml + e * 4);
    const float wgt = ml[0] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(ml[0] - M);
    ssum += wgt * ml[1];
    fsum += wgt * ml[2];
    accv += wgt * *(const f32x4*)(a.ws_o + e * DC + d0);
  }
  *(f32x4*)o = accv * (1.0f / ssum);
  if (blockIdx.x == 0 && c == 0)
    a.lse[(int64_t)b * H + h] = (M + __log2f(fsum)) * 0.69314718055994531f;
}

// ---------------------------------------------------------- dequant dump ---
// The bf16 rows the decode kernels reconstruct for all 64 slots of one page,
// through the same load/dequant device functions: out[64][576].
template <int F>
__global__ __launch_bounds__(512) void dequant_dump_kernel(const uint8_t* pages, int64_t page_id,
                                                           uint16_t* out) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, n16 = lane & 15, g = lane >> 4;
  const int tb = wave & 3, dh = wave >> 2, tt = 16 * tb + n16;
  const Packed<F> pk = load_packed<F>(pages + page_id * Fmt<F>::PAGE_BYTES, tt, dh, g);
  uint16_t* row = out + tt * DROW;
  bf16x8 kv[8];
  deq_content<F>(pk, kv);
#pragma unroll
  for (int t = 0; t < 8; ++t) *(bf16x8*)(row + 256 * dh + 64 * g + 8 * t) = kv[t];
  *(bf16x8*)(row + DC + 32 * dh + 8 * g) = deq_rope<F>(pk);
}

int launch_decode(int f, const DecodeArgs& a, hipStream_t stream) {
  if (a.H % 128 == 0) {
    // 128-head blocks: one reconstruction of each page serves all heads
    if (launch_decode128(f, a, stream) != 0) return -5;
  } else {
    const dim3 grid(a.nsplit, a.B, a.H / 16), block(512);
    if (f == 0)
      hipLaunchKernelGGL(decode16_kernel<0>, grid, block, 0, stream, a);
    else
      hipLaunchKernelGGL(decode16_kernel<1>, grid, block, 0, stream, a);
    if (hipGetLastError() != hipSuccess) return -5;
  }
  if (a.nsplit > 1) {
    hipLaunchKernelGGL(combine_kernel, dim3(DC / 64, a.H / 16, a.B), dim3(256), 0, stream, a);
    if (hipGetLastError() != hipSuccess) return -5;
  }
  return 0;
}

int launch_dequant_dump(int f, const uint8_t* pages, int64_t page_id, uint16_t* out,
                        hipStream_t stream) {
  if (f == 0)
    hipLaunchKernelGGL(dequant_dump_kernel<0>, dim3(1), dim3(512), 0, stream, pages, page_id, out);
  else
    hipLaunchKernelGGL(dequant_dump_kernel<1>, dim3(1), dim3(512), 0, stream, pages, page_id, out);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

}  // namespace mlb
