// C-ABI host layer of libmla_lowbit.so: argument validation (pure host code,
// runs before any HIP call), the split plan, and dispatch to the kernels.
#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstddef>
#include <cstdint>
#include <cstring>
#include <vector>

#include "../../include/mla_lowbit.h"
#include "internal.h"

namespace mlb {

static constexpr int kDefaultCUs = 256;   // MI355X compute units (no device visible)
static constexpr int kWavesTarget = 1;    // resident decode workgroups per CU
static constexpr int kMinPagesPerSplit = 2;
static constexpr int kMinPagesPerSplit128 = 8;   // 128-head blocks write 256 KB per split

static size_t page_bytes_of(int f) {
  return f == MLA_LB_C4R4 ? 20736u : (f == MLA_LB_C2R4 ? 12544u : (f == MLA_LB_C4R4F ? 20992u : 0u));
}

// Compute units of the current device (a partitioned MI355X exposes fewer
// than 256), read once per device; kDefaultCUs when no device is visible.
static int device_cu_count() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
    (void)hipGetLastError();
    return kDefaultCUs;
  }
  if (dev < 64) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      n < 1) {
    (void)hipGetLastError();
    return kDefaultCUs;
  }
  if (dev < 64) cache[dev].store(n, std::memory_order_relaxed);
  return n;
}

// Split plan.  A max-length sequence of P pages is cut into nsplit splits of
// pps pages.  Automatic choice: enough (split, sequence, head-block)
// workgroups to keep every CU of the current device busy, but no split
// shorter than a minimum number of pages (each split costs a heads x 512 fp32
// partial write).  Head blocks are 128 rows when use_rows128(H), else 16.

Plan make_plan(int32_t B, int32_t H, int32_t max_seq_len, int32_t num_splits, size_t ws_cap) {
  Plan p{1, 1, 0, false};
  const int64_t P = (static_cast<int64_t>(max_seq_len) + 63) / 64;
  if (P <= 1) return p;
  int64_t ns;
  if (num_splits > 0) {
    ns = num_splits;
  } else {
    const bool h128 = mlb::use_rows128(H);
    const int64_t groups = static_cast<int64_t>(B) * (h128 ? (H + 127) / 128 : H / 16);
    ns = (static_cast<int64_t>(device_cu_count()) * kWavesTarget + groups - 1) / groups;
    const int64_t cap = P / (h128 ? kMinPagesPerSplit128 : kMinPagesPerSplit);
    if (ns > cap) ns = cap;
    if (ws_cap > 0) {              // no more splits than a workspace of ws_cap bytes holds
      const uint64_t per_split = static_cast<uint64_t>(B) * static_cast<uint64_t>(H) *
                                 (512 + 4) * sizeof(float);
      const int64_t fit = static_cast<int64_t>(ws_cap / per_split);
      if (ns > fit) ns = fit < 2 ? 1 : fit;
    }
  }
  if (ns < 1) ns = 1;
  if (ns > P) ns = P;
  const int64_t pps = (P + ns - 1) / ns;
  ns = (P + pps - 1) / pps;
  p.pps = static_cast<int32_t>(pps);
  p.nsplit = static_cast<int32_t>(ns);
  // B x nsplit x rows x (512 + 4) fp32; within the entry points' bounds
  // (B <= 65535, nsplit <= 2^25 pages, rows <= 65536) it can pass 2^64, so
  // it is formed in 128 bits and a plan beyond 2^60 bytes is refused
  if (ns > 1) {
    const unsigned __int128 ws = static_cast<unsigned __int128>(B) * static_cast<uint64_t>(ns) *
                                 static_cast<uint64_t>(H) * ((512 + 4) * sizeof(float));
    if (ws > (static_cast<unsigned __int128>(1) << 60)) p.too_large = true;
    else p.ws_bytes = static_cast<size_t>(ws);
  }
  return p;
}

}  // namespace mlb

extern "C" {

int mla_lb_version(void) { return 1; }

const char* mla_lb_strerror(int code) {
  switch (code) {
    case MLA_LB_OK: return "ok";
    case MLA_LB_EINVAL: return "invalid argument (null pointer or bad scalar)";
    case MLA_LB_ESHAPE: return "unsupported or inconsistent sizes";
    case MLA_LB_EFORMAT: return "unknown cache format";
    case MLA_LB_EWORKSPACE: return "workspace missing or too small";
    case MLA_LB_EHIP: return "HIP runtime error at launch";
    default: return "unknown error code";
  }
}

size_t mla_lb_page_bytes(int f) { return mlb::page_bytes_of(f); }

size_t mla_lb_prot_bytes_per_seq(void) { return 132u * 576u * 2u; }

int kv_quant_append(int f, const uint16_t* latent, const uint16_t* k_rope,
                    const int64_t* slot_mapping, const int32_t* seq_slot, const int32_t* pos,
                    const int32_t* new_len, int32_t T, uint8_t* pages, int64_t num_pages,
                    uint16_t* prot, int32_t num_seq_slots, void* stream) {
  if (mlb::page_bytes_of(f) == 0) return MLA_LB_EFORMAT;
  if (T < 0) return MLA_LB_ESHAPE;
  if (T == 0) return MLA_LB_OK;
  if (!latent || !k_rope || !slot_mapping || !seq_slot || !pos || !new_len || !pages || !prot)
    return MLA_LB_EINVAL;
  if (num_pages < 1 || num_seq_slots < 1) return MLA_LB_ESHAPE;
  if (num_pages > (INT64_MAX / 64)) return MLA_LB_ESHAPE;
  mlb::AppendArgs a{latent, k_rope, slot_mapping, seq_slot, pos, new_len, T,
                    pages,  num_pages, prot, num_seq_slots};
  return mlb::launch_append(f, a, static_cast<hipStream_t>(stream));
}

int mla_decode_lowbit_workspace(int f, int32_t B, int32_t H, int32_t max_seq_len,
                                int32_t num_splits, size_t* bytes) {
  if (mlb::page_bytes_of(f) == 0) return MLA_LB_EFORMAT;
  if (!bytes) return MLA_LB_EINVAL;
  if (B < 1 || H < 16 || H > MLA_LB_MAX_HEADS || H % 16 != 0 || max_seq_len < 0 ||
      num_splits < 0)
    return MLA_LB_ESHAPE;
  if (B > 65535) return MLA_LB_ESHAPE;               // as the decode call
  const mlb::Plan plan = mlb::make_plan(B, H, max_seq_len, num_splits);
  if (plan.too_large) return MLA_LB_ESHAPE;
  *bytes = plan.ws_bytes;
  return MLA_LB_OK;
}

}  // extern "C"

namespace mlb {

// Validation and split plan shared by the decode entry points: host code
// only, no HIP call.  Fills every field of `a` except the workspace
// pointers (set_workspace).  new_c / new_r non-null selects the fused writer
// (pages / prot are then written).  ws_cap > 0 limits the automatic plan to
// that many workspace bytes.
int decode_setup(int f, const uint16_t* q_lat, const uint16_t* q_rope, const uint8_t* pages,
                 int64_t num_pages, const uint16_t* prot, int32_t num_seq_slots,
                 const int32_t* seq_slot, const int32_t* block_table, int32_t max_blocks,
                 const int32_t* seq_lens, int32_t max_seq_len, int32_t B, int32_t H,
                 float softmax_scale, int32_t num_splits, float* out, float* lse,
                 const uint16_t* new_c, const uint16_t* new_r, int32_t nq, size_t ws_cap,
                 DecodeArgs& a, Plan& plan) {
  if (mlb::page_bytes_of(f) == 0) return MLA_LB_EFORMAT;
  if (!q_lat || !q_rope || !pages || !prot || !seq_slot || !block_table || !seq_lens || !out ||
      !lse)
    return MLA_LB_EINVAL;
  if (!(softmax_scale > 0.0f) || !std::isfinite(softmax_scale)) return MLA_LB_EINVAL;
  if (B < 1 || H < 16 || H > MLA_LB_MAX_HEADS || H % 16 != 0) return MLA_LB_ESHAPE;
  if (nq < 1 || static_cast<int64_t>(nq) * H > MLA_LB_MAX_ROWS) return MLA_LB_ESHAPE;
  const int32_t hq = H;
  H = nq * hq;                                       // query rows per sequence
  if (max_seq_len < 0 || max_blocks < 1 || num_pages < 1 || num_seq_slots < 1 || num_splits < 0)
    return MLA_LB_ESHAPE;
  if (static_cast<int64_t>(max_seq_len) > static_cast<int64_t>(max_blocks) * 64)
    return MLA_LB_ESHAPE;
  if (B > 65535) return MLA_LB_ESHAPE;               // grid.y limit
  plan = mlb::make_plan(B, H, max_seq_len, num_splits, ws_cap);
  if (plan.too_large) return MLA_LB_ESHAPE;
  a = mlb::DecodeArgs{};
  a.q_lat = q_lat;
  a.q_rope = q_rope;
  a.pages = pages;
  a.num_pages = num_pages;
  a.prot = prot;
  a.num_seq_slots = num_seq_slots;
  a.seq_slot = seq_slot;
  a.block_table = block_table;
  a.max_blocks = max_blocks;
  a.seq_lens = seq_lens;
  a.max_seq_len = max_seq_len;
  a.B = B;
  a.H = H;
  a.nq = nq;
  a.hq = hq;
  a.scale_log2 = softmax_scale * 1.4426950408889634f;
  a.pps = plan.pps;
  a.nsplit = plan.nsplit;
  // automatic plans of ragged batches of up to 64 sequences are dealt by
  // length on the device (one wave reads every length)
  a.balance = (num_splits == 0 && plan.nsplit > 1 && B <= 64) ? 1 : 0;
  a.out = out;
  a.lse = lse;
  a.new_c = new_c;
  a.new_r = new_r;
  a.wpages = const_cast<uint8_t*>(pages);
  a.wprot = const_cast<uint16_t*>(prot);
  return MLA_LB_OK;
}

// Workspace layout: [B][nsplit][H][512] partial outputs, then [B][nsplit][H][4].
void set_workspace(DecodeArgs& a, const Plan& plan, void* workspace) {
  float* ws = static_cast<float*>(workspace);
  const size_t n_o = static_cast<size_t>(a.B) * plan.nsplit * a.H * 512;
  a.ws_o = plan.nsplit > 1 ? ws : nullptr;
  a.ws_ml = plan.nsplit > 1 ? ws + n_o : nullptr;
}

}  // namespace mlb

namespace {

// The decode entry points with a caller-supplied workspace.
int decode_entry(int f, const uint16_t* q_lat, const uint16_t* q_rope, const uint8_t* pages,
                 int64_t num_pages, const uint16_t* prot, int32_t num_seq_slots,
                 const int32_t* seq_slot, const int32_t* block_table, int32_t max_blocks,
                 const int32_t* seq_lens, int32_t max_seq_len, int32_t B, int32_t H,
                 float softmax_scale, int32_t num_splits, void* workspace,
                 size_t workspace_bytes, float* out, float* lse, void* stream,
                 const uint16_t* new_c, const uint16_t* new_r, int32_t nq = 1) {
  mlb::DecodeArgs a;
  mlb::Plan plan;
  const int rc = mlb::decode_setup(f, q_lat, q_rope, pages, num_pages, prot, num_seq_slots,
                                   seq_slot, block_table, max_blocks, seq_lens, max_seq_len, B, H,
                                   softmax_scale, num_splits, out, lse, new_c, new_r, nq, 0, a,
                                   plan);
  if (rc != MLA_LB_OK) return rc;
  if (plan.ws_bytes > 0 && (!workspace || workspace_bytes < plan.ws_bytes))
    return MLA_LB_EWORKSPACE;
  mlb::set_workspace(a, plan, workspace);
  return mlb::launch_decode(f, a, static_cast<hipStream_t>(stream));
}

}  // namespace

extern "C" {

int mla_decode_lowbit(int f, const uint16_t* q_lat, const uint16_t* q_rope,
                      const uint8_t* pages, int64_t num_pages, const uint16_t* prot,
                      int32_t num_seq_slots, const int32_t* seq_slot,
                      const int32_t* block_table, int32_t max_blocks,
                      const int32_t* seq_lens, int32_t max_seq_len, int32_t B, int32_t H,
                      float softmax_scale, int32_t num_splits, void* workspace,
                      size_t workspace_bytes, float* out, float* lse, void* stream) {
  return decode_entry(f, q_lat, q_rope, pages, num_pages, prot, num_seq_slots, seq_slot,
                      block_table, max_blocks, seq_lens, max_seq_len, B, H, softmax_scale,
                      num_splits, workspace, workspace_bytes, out, lse, stream, nullptr, nullptr);
}

int mla_decode_lowbit_append(int f, const uint16_t* latent, const uint16_t* k_rope,
                             const uint16_t* q_lat, const uint16_t* q_rope, uint8_t* pages,
                             int64_t num_pages, uint16_t* prot, int32_t num_seq_slots,
                             const int32_t* seq_slot, const int32_t* block_table,
                             int32_t max_blocks, const int32_t* seq_lens, int32_t max_seq_len,
                             int32_t B, int32_t H, float softmax_scale, int32_t num_splits,
                             void* workspace, size_t workspace_bytes, float* out, float* lse,
                             void* stream) {
  if (!latent || !k_rope) return mlb::page_bytes_of(f) == 0 ? MLA_LB_EFORMAT : MLA_LB_EINVAL;
  return decode_entry(f, q_lat, q_rope, pages, num_pages, prot, num_seq_slots, seq_slot,
                      block_table, max_blocks, seq_lens, max_seq_len, B, H, softmax_scale,
                      num_splits, workspace, workspace_bytes, out, lse, stream, latent, k_rope);
}

int mla_decode_lowbit_mq_workspace(int f, int32_t B, int32_t nq, int32_t H,
                                   int32_t max_seq_len, int32_t num_splits, size_t* bytes) {
  if (mlb::page_bytes_of(f) == 0) return MLA_LB_EFORMAT;
  if (!bytes) return MLA_LB_EINVAL;
  if (B < 1 || H < 16 || H > MLA_LB_MAX_HEADS || H % 16 != 0 || nq < 1 ||
      static_cast<int64_t>(nq) * H > MLA_LB_MAX_ROWS || max_seq_len < 0 || num_splits < 0)
    return MLA_LB_ESHAPE;
  if (B > 65535) return MLA_LB_ESHAPE;               // as the decode call
  const mlb::Plan plan = mlb::make_plan(B, nq * H, max_seq_len, num_splits);
  if (plan.too_large) return MLA_LB_ESHAPE;
  *bytes = plan.ws_bytes;
  return MLA_LB_OK;
}

int mla_decode_lowbit_mq(int f, const uint16_t* q_lat, const uint16_t* q_rope,
                         const uint8_t* pages, int64_t num_pages, const uint16_t* prot,
                         int32_t num_seq_slots, const int32_t* seq_slot,
                         const int32_t* block_table, int32_t max_blocks,
                         const int32_t* seq_lens, int32_t max_seq_len, int32_t B, int32_t nq,
                         int32_t H, float softmax_scale, int32_t num_splits, void* workspace,
                         size_t workspace_bytes, float* out, float* lse, void* stream) {
  return decode_entry(f, q_lat, q_rope, pages, num_pages, prot, num_seq_slots, seq_slot,
                      block_table, max_blocks, seq_lens, max_seq_len, B, H, softmax_scale,
                      num_splits, workspace, workspace_bytes, out, lse, stream, nullptr, nullptr,
                      nq);
}

int mla_lb_channel_stat(const uint16_t* x, int64_t rows, int32_t n, double pct, float* stat) {
  if (!x || !stat) return MLA_LB_EINVAL;
  if (rows < 1 || n < 1 || !(pct >= 0.0 && pct <= 100.0)) return MLA_LB_ESHAPE;
  std::vector<double> col(static_cast<size_t>(rows));
  // linear interpolation between the order statistics around pct/100*(rows-1)
  const double posn = pct / 100.0 * static_cast<double>(rows - 1);
  const int64_t lo = static_cast<int64_t>(std::floor(posn));
  const int64_t hi = std::min<int64_t>(lo + 1, rows - 1);
  const double frac = posn - static_cast<double>(lo);
  for (int32_t j = 0; j < n; ++j) {
    for (int64_t r = 0; r < rows; ++r) {
      const uint32_t bits = static_cast<uint32_t>(x[r * n + j]) << 16;
      float f;
      std::memcpy(&f, &bits, sizeof f);
      col[static_cast<size_t>(r)] = std::fabs(static_cast<double>(f));
    }
    std::sort(col.begin(), col.end());
    // interpolate from the nearer end (the form numpy's percentile uses)
    const double va = col[static_cast<size_t>(lo)], vb = col[static_cast<size_t>(hi)];
    const double v = frac < 0.5 ? va + (vb - va) * frac : vb - (vb - va) * (1.0 - frac);
    stat[j] = static_cast<float>(v);
  }
  return MLA_LB_OK;
}

int mla_lb_smooth_scales(const float* stat, int32_t n, float alpha, int32_t pair_tied,
                         float* scales) {
  if (!stat || !scales) return MLA_LB_EINVAL;
  if (n < 1 || (pair_tied && n % 2 != 0) || !(alpha >= 0.0f) || !std::isfinite(alpha))
    return MLA_LB_ESHAPE;
  for (int32_t j = 0; j < n; ++j) {
    double a = std::max(static_cast<double>(stat[j]), 1e-8);
    if (pair_tied) {
      const int32_t p = j & ~1;
      a = std::max(std::max(static_cast<double>(stat[p]), 1e-8),
                   std::max(static_cast<double>(stat[p + 1]), 1e-8));
    }
    scales[j] = static_cast<float>(std::pow(a, -static_cast<double>(alpha)));
  }
  return MLA_LB_OK;
}

int mla_lb_hadamard_rows(const float* x, int64_t rows, int32_t n, float* y) {
  if (!x || !y) return MLA_LB_EINVAL;
  if (rows < 1 || n < 1 || n > (1 << 20) || (n & (n - 1)) != 0) return MLA_LB_ESHAPE;
  // y[r] = x[r] H_n with H_n Sylvester's +-1 matrix / sqrt(n): the in-place
  // butterfly over doubling strides builds [[H, H], [H, -H]] at every level;
  // H_n is symmetric, so the row-vector product equals H_n x[r]^T
  std::vector<double> v(static_cast<size_t>(n));
  const double norm = 1.0 / std::sqrt(static_cast<double>(n));
  for (int64_t r = 0; r < rows; ++r) {
    const float* xr = x + r * n;
    for (int32_t i = 0; i < n; ++i) v[static_cast<size_t>(i)] = xr[i];
    for (int32_t len = 1; len < n; len <<= 1)
      for (int32_t i = 0; i < n; i += 2 * len)
        for (int32_t k = i; k < i + len; ++k) {
          const double a = v[static_cast<size_t>(k)], b = v[static_cast<size_t>(k + len)];
          v[static_cast<size_t>(k)] = a + b;
          v[static_cast<size_t>(k + len)] = a - b;
        }
    float* yr = y + r * n;
    for (int32_t i = 0; i < n; ++i) yr[i] = static_cast<float>(v[static_cast<size_t>(i)] * norm);
  }
  return MLA_LB_OK;
}

int mla_lb_dequant_dump(int f, const uint8_t* pages, int64_t num_pages, int64_t page_id,
                        uint16_t* out, void* stream) {
  if (mlb::page_bytes_of(f) == 0) return MLA_LB_EFORMAT;
  if (!pages || !out) return MLA_LB_EINVAL;
  if (num_pages < 1 || page_id < 0 || page_id >= num_pages) return MLA_LB_ESHAPE;
  return mlb::launch_dequant_dump(f, pages, page_id, out, static_cast<hipStream_t>(stream));
}

}  // extern "C"
