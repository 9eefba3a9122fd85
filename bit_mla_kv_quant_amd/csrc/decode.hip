// mla_decode_lowbit: native low-bit MLA decode attention [QuantMLA §3.3,
// App. C.5] in the absorbed form [MLA blog §4], for gfx950.
//
// decode16_kernel<F>: one 512-thread workgroup (8 waves, one per CU) per
// (split j, sequence b, 16-head group), walking the split's 64-token pages
// with two page buffers in LDS and specialised waves:
//   producers (waves 0-3) -- each takes 16 token slots of page t; lane
//      (n16, g) holds the packed codes of slot 16w+n16 for a quarter of the
//      576 dims, loaded one page earlier (register double buffer) so HBM
//      latency overlaps the previous page.  The lane reconstructs bf16 values
//      in registers; they are directly the B operand of
//      v_mfma_f32_16x16x32_bf16, so the score tile S[16 heads][16 slots] needs
//      no LDS round trip (query dims are permuted identically).  Protected
//      tokens use their BF16 row instead.  The reconstructed 512-d content
//      rows go to the page's LDS tile [64][512], which feeds the aggregation:
//      every value is reconstructed once and used for both products
//      [QuantMLA App. C.5].  Scores go to LDS as well.
//   consumers (waves 4-7) -- meanwhile drain page t-1: every lane (head n16,
//      token quarter g) reads its 16 scores, the four lanes of a head agree on
//      the tile maximum through two lane exchanges, and one global online
//      softmax [QuantMLA §3.3] turns them into weights, split into bf16
//      hi + lo terms held in the registers that are directly the A operand of
//      the aggregation MFMA.  O[16][512] += P[16][64] . C[64][512]: consumer
//      w owns dims 128w..128w+127; the C operand (8 consecutive tokens of one
//      dim per lane) comes from ds_read_b64_tr_b16 transposed LDS reads.
// One barrier per page hands a buffer from producers to consumers.  The
// dequantisation (VALU) of one page and the softmax/aggregation (LDS, MFMA)
// of the previous one run side by side on every SIMD.
// A split writes (max, weight sum, unnormalised O) to the workspace and
// combine_kernel merges the splits by the log-sum-exp rule [QuantMLA
// App. C.5]; with a single split the kernel writes the final output itself.
#include "common.h"
#include "dequant.h"
#include "internal.h"

namespace mlb {

typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

constexpr int CT_PITCH = DC + 8;   // LDS content tile row pitch (bf16 elements)
constexpr int SX_PITCH = 64 + 4;   // LDS score tile row pitch (floats)

// ---------------------------------------------------------- decode main ----
// Rescale threshold of the online softmax, in log2 units: the reference
// maximum of a head only moves when a tile's maximum exceeds it by more than
// this, so weights exp2(x - m_ref) stay below 2^8 and the common case needs no
// rescaling of the accumulators.  The result is the same single softmax.
constexpr float RESCALE_LOG2 = 8.0f;

template <int F>
__global__ __launch_bounds__(512, 1) void decode16_kernel(DecodeArgs a) {
  using FM = Fmt<F>;
  constexpr int NR = FM::NBLK;          // content chunks per lane
  constexpr int NT = FM::DPB / 32;      // 8-dim slices per chunk
  constexpr int SPAN = FM::DPB / 4;     // dims per lane group per chunk

  // two page buffers: producers fill one while consumers drain the other
  __shared__ __attribute__((aligned(16))) uint16_t ctile[2][PAGE * CT_PITCH];
  __shared__ __attribute__((aligned(16))) float sx[2][16 * SX_PITCH];
  __shared__ int32_t pids[MAX_PAGES_PER_SPLIT];
  __shared__ __attribute__((aligned(16))) uint16_t qrope[16 * DR];   // RoPE query rows

  const int j = blockIdx.x, b = blockIdx.y, hg = blockIdx.z;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n16 = lane & 15, g = lane >> 4;
  const bool producer = wave < 4;                  // waves 0-3 produce, 4-7 consume
  const int w = wave & 3;
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
  const int np = p1 - p0;                          // <= MAX_PAGES_PER_SPLIT (host plan)

  // ---- physical page ids of the split (-1 = unusable entry)
  for (int t = threadIdx.x; t < np; t += 512) {
    const int phys = a.block_table[(int64_t)b * a.max_blocks + p0 + t];
    pids[t] = (phys >= 0 && phys < a.num_pages) ? phys : -1;
  }
  // ---- RoPE query rows of the 16 heads (read per page by the producers;
  //      keeping them out of registers leaves room for the page prefetch)
  if (threadIdx.x < 16 * DR / 8)
    *(bf16x8*)(qrope + 8 * threadIdx.x) =
        *(const bf16x8*)(a.q_rope + ((int64_t)b * H + hg * 16) * DR + 8 * threadIdx.x);

  // ================================================================ producer
  // Lane (n16, g) of producer wave w owns token slot 16w+n16 and a quarter of
  // its 576 dims.  Query registers: head 16*hg + n16, dim slices permuted
  // exactly like the key slices the lane reconstructs.
  const int tt = 16 * w + n16;
  bf16x8 qc[NR][NT];
  if (producer) {
    const int head = hg * 16 + n16;
    const uint16_t* ql = a.q_lat + ((int64_t)b * H + head) * DC;
#pragma unroll
    for (int r = 0; r < NR; ++r)
#pragma unroll
      for (int t = 0; t < NT; ++t)
        qc[r][t] = *(const bf16x8*)(ql + r * FM::DPB + g * SPAN + 8 * t);
  }
  __syncthreads();

  const uint16_t* prot_seq = a.prot + (int64_t)sq * PROT_ROWS * DROW;
  auto page_ptr = [&](int k) -> const uint8_t* {
    const int phys = __builtin_amdgcn_readfirstlane(pids[k]);
    return a.pages + (int64_t)(phys >= 0 ? phys : 0) * FM::PAGE_BYTES;
  };

  // Reconstruct page k from `cur` (its packed codes, loaded one page ahead),
  // score it against the 16 heads and publish content rows + scores in
  // buffer k & 1.
  auto produce = [&](const Packed<F>& cur, const int k) {
    uint16_t* ct = ctile[k & 1];
    const int p = p0 + k;
    const bool page_ok = pids[k] >= 0;             // unusable table entry: no tokens
    const int i = p * PAGE + tt;
    const bool valid = page_ok && i < L;
    // pages that hold a sink or a recent-window token (at most 3 per sequence),
    // or no usable tokens at all, take the per-lane path
    const bool prot_page = !page_ok || p * PAGE < NSINK || (p + 1) * PAGE > L - NRECENT;
    f32x4 s = {0.f, 0.f, 0.f, 0.f};
    if (!prot_page) {
      // every slot of the page is a cached, unprotected token
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        bf16x8 kv[NT];
        deq_content<F>(cur, r, kv);
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qc[r][t], kv[t], s, 0, 0, 0);
          *(bf16x8*)(ct + tt * CT_PITCH + r * FM::DPB + g * SPAN + 8 * t) = kv[t];
        }
      }
      bf16x8 kr[2];
      deq_rope<F>(cur, kr);
      s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
          *(const bf16x8*)(qrope + n16 * DR + 16 * g), kr[0], s, 0, 0, 0);
      s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
          *(const bf16x8*)(qrope + n16 * DR + 16 * g + 8), kr[1], s, 0, 0, 0);
    } else {
      // sink / recent-window page: protected slots read their BF16 row, slots
      // past the sequence end contribute zeros (and a -inf score below)
      const bool prot = valid && is_protected(i, L);
      const uint16_t* prow = prot_seq + (int64_t)prot_row(i) * DROW;
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        bf16x8 kv[NT];
        deq_content<F>(cur, r, kv);
        if (prot) {
#pragma unroll
          for (int t = 0; t < NT; ++t)
            kv[t] = *(const bf16x8*)(prow + r * FM::DPB + g * SPAN + 8 * t);
        } else if (!valid) {
#pragma unroll
          for (int t = 0; t < NT; ++t) kv[t] = bitcast<bf16x8>(u32x4{0u, 0u, 0u, 0u});
        }
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qc[r][t], kv[t], s, 0, 0, 0);
          *(bf16x8*)(ct + tt * CT_PITCH + r * FM::DPB + g * SPAN + 8 * t) = kv[t];
        }
      }
      bf16x8 kr[2];
      deq_rope<F>(cur, kr);
      if (prot) {
        kr[0] = *(const bf16x8*)(prow + DC + 16 * g);
        kr[1] = *(const bf16x8*)(prow + DC + 16 * g + 8);
      } else if (!valid) {
        kr[0] = kr[1] = bitcast<bf16x8>(u32x4{0u, 0u, 0u, 0u});
      }
      s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
          *(const bf16x8*)(qrope + n16 * DR + 16 * g), kr[0], s, 0, 0, 0);
      s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
          *(const bf16x8*)(qrope + n16 * DR + 16 * g + 8), kr[1], s, 0, 0, 0);
    }
    // s[v] = raw score of head 4g+v against token slot tt
    float* sxb = sx[k & 1];
#pragma unroll
    for (int v = 0; v < 4; ++v)
      sxb[(4 * g + v) * SX_PITCH + tt] = valid ? s[v] * a.scale_log2 : -INFINITY;
  };

  // ================================================================ consumer
  // Consumer wave w owns output dims 128w..128w+127 of all 16 heads.  Softmax
  // state of head n16 (identical in the four lanes of a head): m_ref reference
  // maximum (log2 units) and f_run, the sum of the fp32 weights (partial over
  // this lane's tokens), which both normalises the output and gives the
  // log-sum-exp.  Each weight enters the aggregation MFMA as two bf16 terms,
  // hi = bf16(p) and lo = bf16(p - hi), so the weights multiplying the latent
  // rows match the fp32 weights to ~2^-17 relative.
  f32x4 acc[8];
#pragma unroll
  for (int nb = 0; nb < 8; ++nb) acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_ref = -INFINITY, f_run = 0.f;

  auto consume = [&](const int k) {
    const uint16_t* ct = ctile[k & 1];
    const float* sxb = sx[k & 1];
    // lane (head n16, quarter g) owns tokens 8g..8g+7 and 32+8g..32+8g+7 --
    // exactly its A-operand columns of the aggregation MFMA
    f32x4 x4[4];
    x4[0] = *(const f32x4*)(sxb + n16 * SX_PITCH + 8 * g);
    x4[1] = *(const f32x4*)(sxb + n16 * SX_PITCH + 8 * g + 4);
    x4[2] = *(const f32x4*)(sxb + n16 * SX_PITCH + 32 + 8 * g);
    x4[3] = *(const f32x4*)(sxb + n16 * SX_PITCH + 32 + 8 * g + 4);
    float tm = -INFINITY;
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int e = 0; e < 4; ++e) tm = fmaxf(tm, x4[q][e]);
    tm = fmaxf(tm, __shfl_xor(tm, 16, 64));
    tm = fmaxf(tm, __shfl_xor(tm, 32, 64));
    float alpha = 1.0f;
    if (tm > m_ref + RESCALE_LOG2) {               // (always true on the first page)
      alpha = __builtin_amdgcn_exp2f(m_ref - tm);  // 0 while m_ref = -inf
      m_ref = tm;
    }
    const float mu = m_ref == -INFINITY ? 0.0f : m_ref;
    u32x4 phi[2], plo[2];
    float ft = 0.f;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
#pragma unroll
      for (int e = 0; e < 4; e += 2) {
        const float e0 = __builtin_amdgcn_exp2f(x4[q][e] - mu);
        const float e1 = __builtin_amdgcn_exp2f(x4[q][e + 1] - mu);
        ft += e0 + e1;
        const uint32_t hb = pack_bf16x2(e0, e1);
        const uint32_t lb = pack_bf16x2(e0 - __uint_as_float(hb << 16),
                                        e1 - __uint_as_float(hb & 0xffff0000u));
        phi[q >> 1][(q & 1) * 2 + (e >> 1)] = hb;
        plo[q >> 1][(q & 1) * 2 + (e >> 1)] = lb;
      }
    }
    f_run = f_run * alpha + ft;
    // O rows of this lane are heads 4g+v: rescale by those heads' alpha
    if (__any(alpha != 1.0f)) {
      float av[4];
#pragma unroll
      for (int v = 0; v < 4; ++v) av[v] = __shfl(alpha, 4 * g + v, 64);
#pragma unroll
      for (int nb = 0; nb < 8; ++nb)
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[nb][v] *= av[v];
    }
    // O[16][128w..128w+127] += (P_hi + P_lo)[16][64] . C[64][...]
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const bf16x8 pa = bitcast<bf16x8>(phi[kb]);
      const bf16x8 pl = bitcast<bf16x8>(plo[kb]);
      const int row = 32 * kb + 8 * g + (n16 >> 2);
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) {
        const int col = 128 * w + 16 * nb + 4 * (n16 & 3);
        const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
            (lds_bf16x4*)(ct + row * CT_PITCH + col));
        const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
            (lds_bf16x4*)(ct + (row + 4) * CT_PITCH + col));
        const bf16x8 cb = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa, cb, acc[nb], 0, 0, 0);
        acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pl, cb, acc[nb], 0, 0, 0);
      }
    }
  };

  // ================================================================ pipeline
  // Step t: producers build page t in buffer t&1 while consumers drain page
  // t-1 from the other buffer; one barrier per step.  Producer register
  // buffers A/B alternate by step parity (unrolled by two, no copies), and the
  // prefetch is unconditional (the last page reloads itself) so the memory
  // counter waits stay exact.
  Packed<F> bufA, bufB;
  if (producer) bufA = load_packed<F>(page_ptr(0), tt, g);
  for (int t = 0;;) {
    if (producer) {
      bufB = load_packed<F>(page_ptr(min(t + 1, np - 1)), tt, g);
      produce(bufA, t);
    } else if (t > 0) {
      consume(t - 1);
    }
    __syncthreads();
    if (++t == np) break;
    if (producer) {
      bufA = load_packed<F>(page_ptr(min(t + 1, np - 1)), tt, g);
      produce(bufB, t);
    } else {
      consume(t - 1);
    }
    __syncthreads();
    if (++t == np) break;
  }
  if (producer) return;                            // no barrier follows
  consume(np - 1);

  // ---- head totals over the four lane groups
  f_run += __shfl_xor(f_run, 16, 64);
  f_run += __shfl_xor(f_run, 32, 64);
  // lane (n16 = h) now holds head h's total; O rows of this lane are 4g+v
  float fv[4];
#pragma unroll
  for (int v = 0; v < 4; ++v) fv[v] = __shfl(f_run, 4 * g + v, 64);

  if (single) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int h = hg * 16 + 4 * g + v;
      const float inv = 1.0f / fv[v];
      float* o = a.out + ((int64_t)b * H + h) * DC + 128 * w + n16;
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) o[16 * nb] = acc[nb][v] * inv;
    }
    if (w == 0 && g == 0)
      a.lse[(int64_t)b * H + hg * 16 + n16] =
          (m_ref + __log2f(f_run)) * 0.69314718055994531f;
  } else {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int h = hg * 16 + 4 * g + v;
      const int64_t base = ((int64_t)b * a.nsplit + j) * H + h;
      float* o = a.ws_o + base * DC + 128 * w + n16;
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) o[16 * nb] = acc[nb][v];
    }
    if (w == 0 && g == 0) {
      const int64_t base = ((int64_t)b * a.nsplit + j) * H + hg * 16 + n16;
      *(f32x4*)(a.ws_ml + base * 4) = f32x4{m_ref, f_run, f_run, 0.f};
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
__global__ __launch_bounds__(256) void dequant_dump_kernel(const uint8_t* pages, int64_t page_id,
                                                           uint16_t* out) {
  using FM = Fmt<F>;
  constexpr int NR = FM::NBLK, NT = FM::DPB / 32, SPAN = FM::DPB / 4;
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63, n16 = lane & 15, g = lane >> 4;
  const int tt = 16 * w + n16;
  const Packed<F> pk = load_packed<F>(pages + page_id * FM::PAGE_BYTES, tt, g);
  uint16_t* row = out + tt * DROW;
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    bf16x8 kv[NT];
    deq_content<F>(pk, r, kv);
#pragma unroll
    for (int t = 0; t < NT; ++t) *(bf16x8*)(row + r * FM::DPB + g * SPAN + 8 * t) = kv[t];
  }
  bf16x8 kr[2];
  deq_rope<F>(pk, kr);
  *(bf16x8*)(row + DC + 16 * g) = kr[0];
  *(bf16x8*)(row + DC + 16 * g + 8) = kr[1];
}

int launch_decode(int f, const DecodeArgs& a, hipStream_t stream) {
  const dim3 grid(a.nsplit, a.B, a.H / 16), block(512);
  if (f == 0)
    hipLaunchKernelGGL(decode16_kernel<0>, grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL(decode16_kernel<1>, grid, block, 0, stream, a);
  if (hipGetLastError() != hipSuccess) return -5;
  if (a.nsplit > 1) {
    hipLaunchKernelGGL(combine_kernel, dim3(DC / 64, a.H / 16, a.B), dim3(256), 0, stream, a);
    if (hipGetLastError() != hipSuccess) return -5;
  }
  return 0;
}

int launch_dequant_dump(int f, const uint8_t* pages, int64_t page_id, uint16_t* out,
                        hipStream_t stream) {
  if (f == 0)
    hipLaunchKernelGGL(dequant_dump_kernel<0>, dim3(1), dim3(256), 0, stream, pages, page_id, out);
  else
    hipLaunchKernelGGL(dequant_dump_kernel<1>, dim3(1), dim3(256), 0, stream, pages, page_id, out);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

}  // namespace mlb
