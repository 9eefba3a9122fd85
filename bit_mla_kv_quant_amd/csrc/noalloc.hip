// mla_decode_lowbit_noalloc: mla_decode_lowbit without a caller workspace and
// without any allocation, for callers that cannot allocate device memory
// (code under HIP graph capture, tight serving loops, harnesses that forbid
// hipMalloc).  The split partials live in a file-scope device array of fixed
// size instead of a workspace argument; everything else -- validation, plan,
// kernels -- is mla_decode_lowbit's.
//
// Each GPU the library runs on holds one copy of the array until the process
// ends.  Its device address is looked up once per device, with that device
// current, on the first call there (hipGetSymbolAddress); host code uses only
// that address, never the array's name, which in host code is a host-side
// stand-in.  Every call on one GPU shares that GPU's copy, so calls that
// overlap on one GPU (two streams, or two host threads) race on it.  Nothing
// in it needs clearing between calls: every split writes its (max, sums)
// entry and the merge reads a split's partial output only when that split's
// max is finite.
#include <mutex>

#include "../../include/mla_lowbit.h"
#include "internal.h"

namespace mlb {
namespace {

static __device__ __align__(256) uint8_t scratch[MLA_LB_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];   // device address of `scratch`, per device

// Device address of the current device's copy; looked up on first use.
int scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return MLA_LB_EHIP;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) {
      (void)hipGetLastError();
      return MLA_LB_EHIP;
    }
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MLA_LB_OK;
}

}  // namespace
}  // namespace mlb

extern "C" int mla_decode_lowbit_noalloc(int f, const uint16_t* q_lat, const uint16_t* q_rope,
                                         const uint8_t* pages, int64_t num_pages,
                                         const uint16_t* prot, int32_t num_seq_slots,
                                         const int32_t* seq_slot, const int32_t* block_table,
                                         int32_t max_blocks, const int32_t* seq_lens,
                                         int32_t max_seq_len, int32_t B, int32_t H,
                                         float softmax_scale, int32_t num_splits, float* out,
                                         float* lse, void* stream) {
  mlb::DecodeArgs a;
  mlb::Plan plan;
  int rc = mlb::decode_setup(f, q_lat, q_rope, pages, num_pages, prot, num_seq_slots, seq_slot,
                             block_table, max_blocks, seq_lens, max_seq_len, B, H, softmax_scale,
                             num_splits, out, lse, nullptr, nullptr, 1,
                             MLA_LB_NOALLOC_SCRATCH_BYTES, a, plan);
  if (rc != MLA_LB_OK) return rc;
  if (plan.ws_bytes > MLA_LB_NOALLOC_SCRATCH_BYTES) return MLA_LB_EWORKSPACE;
  void* ws = nullptr;
  if (plan.ws_bytes > 0) {
    rc = mlb::scratch_address(&ws);
    if (rc != MLA_LB_OK) return rc;
  }
  mlb::set_workspace(a, plan, ws);
  return mlb::launch_decode(f, a, static_cast<hipStream_t>(stream));
}
