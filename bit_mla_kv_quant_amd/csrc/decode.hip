// mla_decode_lowbit: native low-bit MLA decode attention [QuantMLA §3.3,
// App. C.5] in the absorbed form [MLA blog §4], for gfx950 -- launch,
// split combine and the reconstruction dump.
//
// The decode kernels live in decode_h16.hip (16-head groups: the
// reconstruction-bound shape) and decode_h128.hip (128-head blocks: the
// matrix-core-bound shape).  Both write, per split, (max, weight sum,
// unnormalised O) to the workspace, and combine_kernel merges the splits by
// the log-sum-exp rule [QuantMLA App. C.5]; with a single split the decode
// kernel writes the final output itself.
#include "common.h"
#include "dequant.h"
#include "internal.h"
#include "split_map.h"

namespace mlb {

// ------------------------------------------------------------- combine -----
// grid (8 dim blocks, H/16, B), 256 threads: thread (hh = tid/16, c = tid%16)
// merges head 16*blockIdx.y + hh, dims 64*blockIdx.x + 4c .. +3 over the
// sequence's splits: m* = max m_j, weights e^(m_j - m*), out = sum w_j o_j /
// sum w_j l_j, lse = m* + ln sum w_j f_j  [QuantMLA App. C.5].
// Every split of the grid has written its (m, l, f): a split past the end of
// its sequence writes m = -inf and no O, so the merge needs no sequence
// length and starts with all its loads in flight.  A split's O is read only
// when its m is finite; a sequence with no finite m gets out 0, lse -inf.
__device__ __forceinline__ void combine_term(const f32x4& ml, const f32x4& ov, float M, f32x4& accv,
                                             float& ssum, float& fsum) {
  if (ml[0] != -INFINITY) {
    const float wgt = __builtin_amdgcn_exp2f(ml[0] - M);
    ssum += wgt * ml[1];
    fsum += wgt * ml[2];
    accv += wgt * ov;
  }
}

// Splits j0 .. j0+N-1 (those below ns) with every partial in flight at once,
// merged into the running (M, sums): the running state is rescaled when this
// round raises the maximum.
template <int N>
__device__ __forceinline__ void combine_round(const DecodeArgs& a, int64_t base, int j0, int ns,
                                              int d0, float& M, f32x4& accv, float& ssum,
                                              float& fsum) {
  f32x4 ml[N], ov[N];
#pragma unroll
  for (int u = 0; u < N; ++u) {
    if (j0 + u < ns) {
      const int64_t e = base + (int64_t)(j0 + u) * a.H;
      ml[u] = *(const f32x4*)(a.ws_ml + e * 4);
      ov[u] = *(const f32x4*)(a.ws_o + e * DC + d0);
    }
  }
  float Mr = M;
#pragma unroll
  for (int u = 0; u < N; ++u)
    if (j0 + u < ns) Mr = fmaxf(Mr, ml[u][0]);
  if (M != -INFINITY && Mr > M) {
    const float r = __builtin_amdgcn_exp2f(M - Mr);
    accv *= r;
    ssum *= r;
    fsum *= r;
  }
  M = Mr;
#pragma unroll
  for (int u = 0; u < N; ++u)
    if (j0 + u < ns) combine_term(ml[u], ov[u], M, accv, ssum, fsum);
}

// NMAX = 8 or 16: plans of at most that many splits, every partial in
// flight at once (one round); NMAX = 0: longer plans, rounds of 16.
// Separate instantiations keep the register count of the short plans low.
template <int NMAX>
__global__ __launch_bounds__(256) void combine_kernel(DecodeArgs a) {
  const int b = blockIdx.z, H = a.H;
  const int hh = threadIdx.x >> 4, c = threadIdx.x & 15;
  const int h = blockIdx.y * 16 + hh;
  const int d0 = 64 * blockIdx.x + 4 * c;
  int first, ns;                                   // the sequence's workspace slots
  split_range(a, b, threadIdx.x & 63, first, ns);
  float* o = a.out + ((int64_t)b * H + h) * DC + d0;
  const int64_t base = (int64_t)first * H + h;     // split jj at base + jj*H
  f32x4 accv = {0.f, 0.f, 0.f, 0.f};
  float ssum = 0.f, fsum = 0.f, M = -INFINITY;
  // rounds of NMAX (16 for NMAX = 0) partials in flight; one round when the
  // sequence has at most NMAX splits (a balanced plan may give it more)
  constexpr int R = NMAX > 0 ? NMAX : 16;
  for (int j0 = 0; j0 < ns; j0 += R) combine_round<R>(a, base, j0, ns, d0, M, accv, ssum, fsum);
  if (M == -INFINITY) {                              // empty sequence
    *(f32x4*)o = f32x4{0.f, 0.f, 0.f, 0.f};
    if (blockIdx.x == 0 && c == 0) a.lse[(int64_t)b * H + h] = -INFINITY;
    return;
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
  if (use_rows128(a.H)) {
    // 128-head blocks: one reconstruction of each page serves all heads
    if (launch_decode128(f, a, stream) != 0) return -5;
  } else {
    if (launch_decode16w(f, a, stream) != 0) return -5;
  }
  if (a.nsplit > 1) {
    const dim3 grid(DC / 64, a.H / 16, a.B), block(256);
    if (a.nsplit <= 8) hipLaunchKernelGGL(combine_kernel<8>, grid, block, 0, stream, a);
    else if (a.nsplit <= 16) hipLaunchKernelGGL(combine_kernel<16>, grid, block, 0, stream, a);
    else hipLaunchKernelGGL(combine_kernel<0>, grid, block, 0, stream, a);
    if (hipGetLastError() != hipSuccess) return -5;
  }
  return 0;
}

int launch_dequant_dump(int f, const uint8_t* pages, int64_t page_id, uint16_t* out,
                        hipStream_t stream) {
  if (f == 0)
    hipLaunchKernelGGL(dequant_dump_kernel<0>, dim3(1), dim3(512), 0, stream, pages, page_id, out);
  else if (f == 1)
    hipLaunchKernelGGL(dequant_dump_kernel<1>, dim3(1), dim3(512), 0, stream, pages, page_id, out);
  else
    hipLaunchKernelGGL(dequant_dump_kernel<2>, dim3(1), dim3(512), 0, stream, pages, page_id, out);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

}  // namespace mlb
