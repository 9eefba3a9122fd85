// mla_decode_lowbit: native low-bit MLA decode attention [QuantMLA §3.3,
// App. C.5] in the absorbed form [MLA blog §4], for gfx950.
//
// decode_kernel<F>: one 256-thread workgroup (4 waves) per
// (split j, sequence b, 16-head group), iterating over the split's 64-token
// pages.  Per page:
//   1. each wave takes 16 tokens; lane (n = lane%16, g = lane/16) loads the
//      packed codes of token n for 1/4 of the 576 dims (128-bit loads), or the
//      protected bf16 row, and reconstructs bf16 values in registers.  Those
//      registers are directly the B operand of v_mfma_f32_16x16x32_bf16, so
//      the score tile S[16 heads][16 tokens] is formed without an LDS round
//      trip (the contraction dims are permuted identically on the query side).
//   2. the reconstructed 512-d content rows are also stored into an LDS tile
//      [64 tokens][512]; that one tile feeds the aggregation, so each
//      reconstructed value is produced once and used for QK and PV
//      [QuantMLA App. C.5].
//   3. one global online softmax: the tile max per head is exchanged through
//      LDS, P is rounded to bf16 and written to LDS.
//   4. aggregation O[16][512] += P[16][64] . C[64][512]: wave w owns dims
//      128w..128w+127; the C operand (8 consecutive tokens of one dim per lane)
//      is fetched with ds_read_b64_tr_b16 transposed LDS reads.
// A split writes (max, sum, unnormalised O) to the workspace and
// combine_kernel merges them by the log-sum-exp rule [QuantMLA App. C.5];
// with a single split the kernel writes the final output itself.
#include "common.h"
#include "internal.h"

namespace mlb {

typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

constexpr int CT_PITCH = DC + 8;   // LDS content tile row pitch (bf16 elements)
constexpr int PT_PITCH = 64 + 8;   // LDS P tile row pitch

// -------------------------------------------------------------- dequant ----
// x^ = bf16(fl32(q*s + z)); q*s is exact so one FMA rounds exactly once.
__device__ __forceinline__ uint32_t deq2(uint32_t q0, uint32_t q1, float s, float z) {
  return pack_bf16x2(__builtin_fmaf((float)q0, s, z), __builtin_fmaf((float)q1, s, z));
}

// 8 INT4 codes of one 32-bit word (byte k: element 2k low nibble, 2k+1 high)
// -> 8 consecutive reconstructed bf16 values.
__device__ __forceinline__ bf16x8 deq_int4x8(uint32_t w, float s, float z) {
  const uint32_t lo = w & 0x0F0F0F0Fu, hi = (w >> 4) & 0x0F0F0F0Fu;
  u32x4 r;
  r[0] = deq2(lo & 0xff, hi & 0xff, s, z);
  r[1] = deq2((lo >> 8) & 0xff, (hi >> 8) & 0xff, s, z);
  r[2] = deq2((lo >> 16) & 0xff, (hi >> 16) & 0xff, s, z);
  r[3] = deq2(lo >> 24, hi >> 24, s, z);
  return bitcast<bf16x8>(r);
}

// 16 INT2 codes of one 32-bit word (byte k: element 4k+j at bits 2j)
// -> two groups of 8 consecutive bf16 values (elements 0..7 and 8..15).
__device__ __forceinline__ void deq_int2x16(uint32_t w, float s, float z, bf16x8& a, bf16x8& b) {
  const uint32_t c0 = w & 0x03030303u, c1 = (w >> 2) & 0x03030303u;
  const uint32_t c2 = (w >> 4) & 0x03030303u, c3 = (w >> 6) & 0x03030303u;
  u32x4 r, t;
  r[0] = deq2(c0 & 0xff, c1 & 0xff, s, z);
  r[1] = deq2(c2 & 0xff, c3 & 0xff, s, z);
  r[2] = deq2((c0 >> 8) & 0xff, (c1 >> 8) & 0xff, s, z);
  r[3] = deq2((c2 >> 8) & 0xff, (c3 >> 8) & 0xff, s, z);
  t[0] = deq2((c0 >> 16) & 0xff, (c1 >> 16) & 0xff, s, z);
  t[1] = deq2((c2 >> 16) & 0xff, (c3 >> 16) & 0xff, s, z);
  t[2] = deq2(c0 >> 24, c1 >> 24, s, z);
  t[3] = deq2(c2 >> 24, c3 >> 24, s, z);
  a = bitcast<bf16x8>(r);
  b = bitcast<bf16x8>(t);
}

// Content chunk r of token slot `tt` for lane-group g: dims
// r*DPB + g*(DPB/4) + [0, DPB/4), as DPB/32 slices of 8 dims (NT = 4 for C4R4,
// 8 for C2R4).  Reads the token's packed codes and its group metadata.
template <int F>
__device__ __forceinline__ void load_content_packed(const uint8_t* pg, int tt, int g, int r,
                                                    bf16x8* kv) {
  using FM = Fmt<F>;
  const u32x4 w = *(const u32x4*)(pg + (r * PAGE + tt) * 64 + g * 16);
  const int grp = (r * FM::DPB + g * (FM::DPB / 4)) / 64;
  const uint32_t meta = *(const uint32_t*)(pg + FM::OFF_MC + tt * 32 + grp * 4);
  const float s = bf16_bits_to_f32(meta & 0xffffu), z = bf16_bits_to_f32(meta >> 16);
  if (FM::CBITS == 4) {
#pragma unroll
    for (int t = 0; t < 4; ++t) kv[t] = deq_int4x8(w[t], s, z);
  } else {
#pragma unroll
    for (int t = 0; t < 4; ++t) deq_int2x16(w[t], s, z, kv[2 * t], kv[2 * t + 1]);
  }
}

// RoPE dims 16g..16g+15 of token slot `tt` as two slices of 8.
template <int F>
__device__ __forceinline__ void load_rope_packed(const uint8_t* pg, int tt, int g, bf16x8* kv) {
  using FM = Fmt<F>;
  const u32x2 w = *(const u32x2*)(pg + FM::OFF_R + tt * 32 + g * 8);
  const uint32_t meta = *(const uint32_t*)(pg + FM::OFF_MR + tt * 4);
  const float s = bf16_bits_to_f32(meta & 0xffffu), z = bf16_bits_to_f32(meta >> 16);
  kv[0] = deq_int4x8(w[0], s, z);
  kv[1] = deq_int4x8(w[1], s, z);
}

// ---------------------------------------------------------- decode main ----
template <int F>
__global__ __launch_bounds__(256, 2) void decode_kernel(DecodeArgs a) {
  using FM = Fmt<F>;
  constexpr int NR = FM::NBLK;          // content chunks per lane
  constexpr int NT = FM::DPB / 32;      // 8-dim slices per chunk
  constexpr int SPAN = FM::DPB / 4;     // dims per lane-group per chunk

  __shared__ __attribute__((aligned(16))) uint16_t ctile[PAGE * CT_PITCH];
  __shared__ __attribute__((aligned(16))) uint16_t ptile[16 * PT_PITCH];
  __shared__ float red[4][16];
  __shared__ float red2[4][16];

  const int j = blockIdx.x, b = blockIdx.y, hg = blockIdx.z;
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n16 = lane & 15, g = lane >> 4;
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
      for (int idx = threadIdx.x; idx < 16 * DC; idx += 256)
        a.out[((int64_t)b * H + hg * 16) * DC + idx] = 0.0f;
      if (threadIdx.x < 16) a.lse[(int64_t)b * H + hg * 16 + threadIdx.x] = -INFINITY;
    }
    return;
  }

  // ---- query registers: head h = 16*hg + n16, permuted dim slices of lane-group g
  const int head = hg * 16 + n16;
  const uint16_t* ql = a.q_lat + ((int64_t)b * H + head) * DC;
  const uint16_t* qr = a.q_rope + ((int64_t)b * H + head) * DR;
  bf16x8 qc[NR][NT], qrr[2];
#pragma unroll
  for (int r = 0; r < NR; ++r)
#pragma unroll
    for (int t = 0; t < NT; ++t)
      qc[r][t] = *(const bf16x8*)(ql + r * FM::DPB + g * SPAN + 8 * t);
  qrr[0] = *(const bf16x8*)(qr + 16 * g);
  qrr[1] = *(const bf16x8*)(qr + 16 * g + 8);

  f32x4 acc[8];
#pragma unroll
  for (int nb = 0; nb < 8; ++nb) acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
  // l_lane: sum of the bf16-rounded weights used in P.C (normalises out, so
  // the weights applied to the latent rows sum to exactly one); f_lane: sum of
  // the fp32 weights (gives the log-sum-exp).
  float m_run[4], l_lane[4], f_lane[4];
#pragma unroll
  for (int v = 0; v < 4; ++v) { m_run[v] = -INFINITY; l_lane[v] = 0.f; f_lane[v] = 0.f; }

  const uint16_t* prot_seq = a.prot + (int64_t)sq * PROT_ROWS * DROW;
  const int tt = 16 * w + n16;                     // this lane's token slot in the page

  for (int p = p0; p < p1; ++p) {
    const int phys = a.block_table[(int64_t)b * a.max_blocks + p];
    const bool page_ok = phys >= 0 && phys < a.num_pages;
    const int i = p * PAGE + tt;
    const bool valid = page_ok && i < L;
    const bool prot = valid && is_protected(i, L);
    const uint8_t* pg = a.pages + (int64_t)(page_ok ? phys : 0) * FM::PAGE_BYTES;
    const uint16_t* prow = prot_seq + (int64_t)prot_row(i) * DROW;

    // ---- 1+2: reconstruct, score, stage content rows
    f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      bf16x8 kv[NT];
      if (prot) {
#pragma unroll
        for (int t = 0; t < NT; ++t) kv[t] = *(const bf16x8*)(prow + r * FM::DPB + g * SPAN + 8 * t);
      } else if (valid) {
        load_content_packed<F>(pg, tt, g, r, kv);
      } else {
#pragma unroll
        for (int t = 0; t < NT; ++t) kv[t] = bitcast<bf16x8>(u32x4{0u, 0u, 0u, 0u});
      }
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qc[r][t], kv[t], s, 0, 0, 0);
        *(bf16x8*)(ctile + tt * CT_PITCH + r * FM::DPB + g * SPAN + 8 * t) = kv[t];
      }
    }
    {
      bf16x8 kr[2];
      if (prot) {
        kr[0] = *(const bf16x8*)(prow + DC + 16 * g);
        kr[1] = *(const bf16x8*)(prow + DC + 16 * g + 8);
      } else if (valid) {
        load_rope_packed<F>(pg, tt, g, kr);
      } else {
        kr[0] = kr[1] = bitcast<bf16x8>(u32x4{0u, 0u, 0u, 0u});
      }
      s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qrr[0], kr[0], s, 0, 0, 0);
      s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qrr[1], kr[1], s, 0, 0, 0);
    }
    // s[v] = raw score of head 4g+v against token slot tt (column n16 of wave w)

    // ---- 3: tile max per head, exchanged through LDS
    float x[4], mx[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      x[v] = valid ? s[v] * a.scale_log2 : -INFINITY;
      float t = x[v];
      t = fmaxf(t, __shfl_xor(t, 8, 16));
      t = fmaxf(t, __shfl_xor(t, 4, 16));
      t = fmaxf(t, __shfl_xor(t, 2, 16));
      t = fmaxf(t, __shfl_xor(t, 1, 16));
      mx[v] = t;
    }
    if (n16 == 0) {
#pragma unroll
      for (int v = 0; v < 4; ++v) red[w][4 * g + v] = mx[v];
    }
    __syncthreads();
    float alpha[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int h = 4 * g + v;
      const float tm = fmaxf(fmaxf(red[0][h], red[1][h]), fmaxf(red[2][h], red[3][h]));
      const float mn = fmaxf(m_run[v], tm);
      const float mu = mn == -INFINITY ? 0.0f : mn;
      alpha[v] = __builtin_amdgcn_exp2f(m_run[v] - mu);
      const float pv = __builtin_amdgcn_exp2f(x[v] - mu);
      const uint32_t pb = f32_to_bf16_bits(pv);
      l_lane[v] = l_lane[v] * alpha[v] + bf16_bits_to_f32(pb);
      f_lane[v] = f_lane[v] * alpha[v] + pv;
      ptile[h * PT_PITCH + tt] = (uint16_t)pb;
      m_run[v] = mn;
    }
    __syncthreads();

    // ---- 4: O[16][128w..128w+127] += P[16][64] . C[64][...]
#pragma unroll
    for (int nb = 0; nb < 8; ++nb)
#pragma unroll
      for (int v = 0; v < 4; ++v) acc[nb][v] *= alpha[v];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const bf16x8 pa = *(const bf16x8*)(ptile + n16 * PT_PITCH + 32 * kb + 8 * g);
      const int row = 32 * kb + 8 * g + (n16 >> 2);
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) {
        const int col = 128 * w + 16 * nb + 4 * (n16 & 3);
        const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
            (lds_bf16x4*)(ctile + row * CT_PITCH + col));
        const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
            (lds_bf16x4*)(ctile + (row + 4) * CT_PITCH + col));
        const bf16x8 cb = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa, cb, acc[nb], 0, 0, 0);
      }
    }
    __syncthreads();
  }

  // ---- per-head sums over the 64 token columns: 16 lanes x 4 waves
  float lsum[4], fsum[4];
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    float t = l_lane[v], u = f_lane[v];
#pragma unroll
    for (int o = 8; o >= 1; o >>= 1) {
      t += __shfl_xor(t, o, 16);
      u += __shfl_xor(u, o, 16);
    }
    lsum[v] = t;
    fsum[v] = u;
  }
  if (n16 == 0) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      red[w][4 * g + v] = lsum[v];
      red2[w][4 * g + v] = fsum[v];
    }
  }
  __syncthreads();
  float l_tot[4], f_tot[4];
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int h = 4 * g + v;
    l_tot[v] = red[0][h] + red[1][h] + red[2][h] + red[3][h];
    f_tot[v] = red2[0][h] + red2[1][h] + red2[2][h] + red2[3][h];
  }

  if (single) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int h = hg * 16 + 4 * g + v;
      const float inv = 1.0f / l_tot[v];
      float* o = a.out + ((int64_t)b * H + h) * DC + 128 * w + n16;
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) o[16 * nb] = acc[nb][v] * inv;
      if (w == 0 && n16 == 0)
        a.lse[(int64_t)b * H + h] = (m_run[v] + __log2f(f_tot[v])) * 0.69314718055994531f;
    }
  } else {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int h = hg * 16 + 4 * g + v;
      const int64_t base = ((int64_t)b * a.nsplit + j) * H + h;
      float* o = a.ws_o + base * DC + 128 * w + n16;
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) o[16 * nb] = acc[nb][v];
      if (w == 0 && n16 == 0)
        *(f32x4*)(a.ws_ml + base * 4) = f32x4{m_run[v], l_tot[v], f_tot[v], 0.f};
    }
  }
}

// ------------------------------------------------------------- combine -----
// grid (H, B), 128 threads, 4 output dims per thread.
__global__ __launch_bounds__(128) void combine_kernel(DecodeArgs a) {
  const int h = blockIdx.x, b = blockIdx.y, H = a.H;
  int L = a.seq_lens[b];
  L = L < 0 ? 0 : (L > a.max_seq_len ? a.max_seq_len : L);
  const int sq = a.seq_slot[b];
  if (sq < 0 || sq >= a.num_seq_slots) L = 0;
  const int npages = (L + PAGE - 1) / PAGE;
  const int ns = (npages + a.pps - 1) / a.pps;
  float* o = a.out + ((int64_t)b * H + h) * DC + 4 * threadIdx.x;
  if (ns == 0) {
    *(f32x4*)o = f32x4{0.f, 0.f, 0.f, 0.f};
    if (threadIdx.x == 0) a.lse[(int64_t)b * H + h] = -INFINITY;
    return;
  }
  const int64_t base = (int64_t)b * a.nsplit * H + h;     // split jj at base + jj*H
  float M = -INFINITY;
  for (int jj = 0; jj < ns; ++jj) M = fmaxf(M, a.ws_ml[(base + (int64_t)jj * H) * 4]);
  f32x4 accv = {0.f, 0.f, 0.f, 0.f};
  float ssum = 0.f, fsum = 0.f;
  for (int jj = 0; jj < ns; ++jj) {
    const int64_t e = base + (int64_t)jj * H;
    const f32x4 ml = *(const f32x4*)(a.ws_ml + e * 4);   // (max, bf16-weight sum, fp32 sum)
    const float wgt = ml[0] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(ml[0] - M);
    ssum += wgt * ml[1];
    fsum += wgt * ml[2];
    accv += wgt * *(const f32x4*)(a.ws_o + e * DC + 4 * threadIdx.x);
  }
  const float inv = 1.0f / ssum;
  *(f32x4*)o = accv * inv;
  if (threadIdx.x == 0) a.lse[(int64_t)b * H + h] = (M + __log2f(fsum)) * 0.69314718055994531f;
}

// ---------------------------------------------------------- dequant dump ---
// The bf16 rows decode_kernel reconstructs for all 64 slots of one page,
// through the same load/dequant device functions: out[64][576].
template <int F>
__global__ __launch_bounds__(256) void dequant_dump_kernel(const uint8_t* pages, int64_t page_id,
                                                           uint16_t* out) {
  using FM = Fmt<F>;
  constexpr int NR = FM::NBLK, NT = FM::DPB / 32, SPAN = FM::DPB / 4;
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63, n16 = lane & 15, g = lane >> 4;
  const int tt = 16 * w + n16;
  const uint8_t* pg = pages + page_id * FM::PAGE_BYTES;
  uint16_t* row = out + tt * DROW;
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    bf16x8 kv[NT];
    load_content_packed<F>(pg, tt, g, r, kv);
#pragma unroll
    for (int t = 0; t < NT; ++t) *(bf16x8*)(row + r * FM::DPB + g * SPAN + 8 * t) = kv[t];
  }
  bf16x8 kr[2];
  load_rope_packed<F>(pg, tt, g, kr);
  *(bf16x8*)(row + DC + 16 * g) = kr[0];
  *(bf16x8*)(row + DC + 16 * g + 8) = kr[1];
}

int launch_decode(int f, const DecodeArgs& a, hipStream_t stream) {
  const dim3 grid(a.nsplit, a.B, a.H / 16), block(256);
  if (f == 0)
    hipLaunchKernelGGL(decode_kernel<0>, grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL(decode_kernel<1>, grid, block, 0, stream, a);
  if (hipGetLastError() != hipSuccess) return -5;
  if (a.nsplit > 1) {
    hipLaunchKernelGGL(combine_kernel, dim3(a.H, a.B), dim3(128), 0, stream, a);
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
