// kv_quant_append: the fused cache writer [QuantMLA App. C.5].
//
// One 64-lane wave per token; lane j owns element j of each of the nine
// 64-wide groups (8 content groups + the RoPE group), each quantized, packed
// and stored by write_group (quantize.h) [QuantMLA §4.1, App. C.4].  The
// token's bf16 row goes to its protection-buffer row when the token is
// protected at the sequence length reached by this call.
//
// This translation unit is compiled with -ffp-contract=off: the quantizer's
// subtract and divide must round exactly as specified.
#include "common.h"
#include "internal.h"
#include "quantize.h"

namespace mlb {

template <int F>
__global__ __launch_bounds__(256) void append_kernel(AppendArgs a) {
  using FM = Fmt<F>;
  const int lane = threadIdx.x & 63;
  // wave-uniform token index: its arguments come in through scalar loads
  const int t = blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (t >= a.T) return;
  const int64_t slot = a.slot_mapping[t];
  const int sq = a.seq_slot[t];
  const int pos = a.pos[t];
  const int new_len = a.new_len[t];
  if (slot < 0 || slot >= a.num_pages * PAGE || sq < 0 || sq >= a.num_seq_slots || pos < 0)
    return;                                        // wave-uniform skip
  const int64_t page = slot / PAGE;
  const int off = (int)(slot % PAGE);
  uint8_t* pg = a.pages + page * FM::PAGE_BYTES;
  const uint16_t* src_c = a.latent + (int64_t)t * DC;
  const uint16_t* src_r = a.k_rope + (int64_t)t * DR;

  uint16_t xc[NGC];
#pragma unroll
  for (int g = 0; g < NGC; ++g) xc[g] = src_c[64 * g + lane];
  const uint16_t xr = src_r[lane];

  // ---- the eight content groups, then the RoPE group
#pragma unroll
  for (int g = 0; g < NGC; ++g) write_group<F>(pg, off, g, xc[g], lane);
  write_group<F>(pg, off, NGC, xr, lane);
  // ---- BF16 protection row, if protected at the length reached by this call
  if (pos < new_len && (pos < NSINK || pos >= new_len - NRECENT)) {
    uint16_t* dst = a.prot + ((int64_t)sq * PROT_ROWS + prot_row(pos)) * DROW;
#pragma unroll
    for (int g = 0; g < NGC; ++g) dst[64 * g + lane] = xc[g];
    dst[DC + lane] = xr;
  }
}

int launch_append(int f, const AppendArgs& a, hipStream_t stream) {
  const dim3 grid((a.T + 3) / 4), block(256);
  if (f == 0)
    hipLaunchKernelGGL(append_kernel<0>, grid, block, 0, stream, a);
  else if (f == 1)
    hipLaunchKernelGGL(append_kernel<1>, grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL(append_kernel<2>, grid, block, 0, stream, a);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

}  // namespace mlb
