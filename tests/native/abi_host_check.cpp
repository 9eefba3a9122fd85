// Host-only driver for the C-ABI layer (abi.cpp) under AddressSanitizer and
// UndefinedBehaviorSanitizer.  The kernel launchers are replaced by stubs
// that record the arguments the host layer hands them, so every validation
// path, the split plan, the workspace sizing and the calibration helpers run
// without a GPU.  Exit status 0 = every check held; the sanitizers abort on
// the first memory or UB error.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "../../include/mla_lowbit.h"
#include "../../bit_mla_kv_quant_amd/csrc/internal.h"

namespace mlb {
static int g_launches = 0;
static DecodeArgs g_last{};
int launch_append(int, const AppendArgs& a, hipStream_t) {
  ++g_launches;
  return a.T > 0 ? 0 : -5;
}
int launch_decode(int, const DecodeArgs& a, hipStream_t) {
  ++g_launches;
  g_last = a;
  return 0;
}
int launch_decode128(int, const DecodeArgs&, hipStream_t) { return 0; }
int launch_decode16w(int, const DecodeArgs&, hipStream_t) { return 0; }
int launch_dequant_dump(int, const uint8_t*, int64_t, uint16_t*, hipStream_t) {
  ++g_launches;
  return 0;
}
}  // namespace mlb

static int failures = 0;
#define CHECK(c)                                                   \
  do {                                                             \
    if (!(c)) {                                                    \
      std::fprintf(stderr, "%s:%d: CHECK failed: %s\n", __FILE__, __LINE__, #c); \
      ++failures;                                                  \
    }                                                              \
  } while (0)

int main() {
  void* P = reinterpret_cast<void*>(0x1000);   // never dereferenced by the host layer
  auto u8 = static_cast<uint8_t*>(P);
  auto u16 = static_cast<uint16_t*>(P);
  auto i32 = static_cast<int32_t*>(P);
  auto i64 = static_cast<int64_t*>(P);
  auto f32 = static_cast<float*>(P);

  // pure queries
  CHECK(mla_lb_version() >= 1);
  for (int c = -7; c <= 1; ++c) CHECK(mla_lb_strerror(c) && std::strlen(mla_lb_strerror(c)) > 0);
  CHECK(mla_lb_page_bytes(0) == 20736 && mla_lb_page_bytes(1) == 12544 &&
        mla_lb_page_bytes(2) == 20992 && mla_lb_page_bytes(3) == 0 && mla_lb_page_bytes(-1) == 0);
  CHECK(mla_lb_prot_bytes_per_seq() == 152064);

  // writer validation
  CHECK(kv_quant_append(5, u16, u16, i64, i32, i32, i32, 4, u8, 1, u16, 1, nullptr) == MLA_LB_EFORMAT);
  CHECK(kv_quant_append(0, u16, u16, i64, i32, i32, i32, -1, u8, 1, u16, 1, nullptr) == MLA_LB_ESHAPE);
  CHECK(kv_quant_append(0, nullptr, u16, i64, i32, i32, i32, 4, u8, 1, u16, 1, nullptr) == MLA_LB_EINVAL);
  CHECK(kv_quant_append(0, u16, u16, i64, i32, i32, i32, 4, u8, 0, u16, 1, nullptr) == MLA_LB_ESHAPE);
  CHECK(kv_quant_append(0, u16, u16, i64, i32, i32, i32, 0, u8, 1, u16, 1, nullptr) == MLA_LB_OK);
  CHECK(kv_quant_append(0, u16, u16, i64, i32, i32, i32, 4, u8, 1, u16, 1, nullptr) == MLA_LB_OK);

  // workspace plans over a grid of shapes; the decode call accepts exactly
  // the size the query returns and refuses one byte less
  const int32_t Hs[] = {16, 32, 48, 64, 96, 112, 128};
  const int32_t Ls[] = {0, 1, 63, 64, 65, 4096, 131072, 1 << 24};
  const int32_t Bs[] = {1, 3, 64, 65535};
  for (int f = 0; f < 3; ++f)
    for (int32_t B : Bs)
      for (int32_t H : Hs)
        for (int32_t L : Ls)
          for (int32_t ns : {0, 1, 7, 64}) {
            size_t need = 1;
            CHECK(mla_decode_lowbit_workspace(f, B, H, L, ns, &need) == MLA_LB_OK);
            const int32_t mb = L > 0 ? (L + 63) / 64 : 1;
            const int before = mlb::g_launches;
            int rc = mla_decode_lowbit(f, u16, u16, u8, 10, u16, 1, i32, i32, mb, i32, L, B, H,
                                       0.07f, ns, need ? P : nullptr, need, f32, f32,
                                       nullptr);
            CHECK(rc == MLA_LB_OK && mlb::g_launches == before + 1);
            if (rc == MLA_LB_OK) {
              CHECK(mlb::g_last.nsplit >= 1 && mlb::g_last.pps >= 1);
              CHECK(static_cast<int64_t>(mlb::g_last.nsplit) * mlb::g_last.pps >= (L + 63) / 64);
              CHECK((mlb::g_last.nsplit > 1) == (need > 0));
            }
            if (need > 0)
              CHECK(mla_decode_lowbit(f, u16, u16, u8, 10, u16, 1, i32, i32, mb, i32, L, B, H,
                                      0.07f, ns, P, need - 1, f32, f32, nullptr) ==
                    MLA_LB_EWORKSPACE);
          }
  size_t n = 0;
  CHECK(mla_decode_lowbit_workspace(0, 65536, 16, 100, 0, &n) == MLA_LB_ESHAPE);
  CHECK(mla_decode_lowbit_workspace(0, 1, 20, 100, 0, &n) == MLA_LB_ESHAPE);
  CHECK(mla_decode_lowbit_workspace(0, 1, 16, 100, 0, nullptr) == MLA_LB_EINVAL);
  CHECK(mla_decode_lowbit_mq_workspace(0, 2, 513, 128, 100, 0, &n) == MLA_LB_ESHAPE);
  CHECK(mla_decode_lowbit_mq_workspace(0, 2, 512, 128, 100, 0, &n) == MLA_LB_OK);
  CHECK(mla_decode_lowbit_mq_workspace(0, 65535, 512, 128, 2147483647, 2147483647, &n) ==
        MLA_LB_ESHAPE);                                 // would pass 2^64 bytes

  // decode validation
  CHECK(mla_decode_lowbit(0, u16, u16, u8, 10, u16, 1, i32, i32, 1, i32, 65, 1, 16, 0.07f, 0,
                          nullptr, 0, f32, f32, nullptr) == MLA_LB_ESHAPE);   // > max_blocks*64
  CHECK(mla_decode_lowbit(0, u16, u16, u8, 10, u16, 1, i32, i32, 1, i32, 64, 1, 16, NAN, 0,
                          nullptr, 0, f32, f32, nullptr) == MLA_LB_EINVAL);
  CHECK(mla_decode_lowbit(0, u16, u16, u8, 10, u16, 1, nullptr, i32, 1, i32, 64, 1, 16, 0.1f, 0,
                          nullptr, 0, f32, f32, nullptr) == MLA_LB_EINVAL);
  CHECK(mla_decode_lowbit_append(0, nullptr, u16, u16, u16, u8, 10, u16, 1, i32, i32, 1, i32, 64,
                                 1, 16, 0.1f, 0, nullptr, 0, f32, f32, nullptr) == MLA_LB_EINVAL);
  CHECK(mla_decode_lowbit_append(0, u16, u16, u16, u16, u8, 10, u16, 1, i32, i32, 1, i32, 64, 1,
                                 16, 0.1f, 0, nullptr, 0, f32, f32, nullptr) == MLA_LB_OK);
  CHECK(mla_decode_lowbit_mq(0, u16, u16, u8, 10, u16, 1, i32, i32, 1, i32, 64, 1, 8, 128, 0.1f,
                             0, nullptr, 0, f32, f32, nullptr) == MLA_LB_OK);
  CHECK(mla_lb_dequant_dump(0, u8, 10, 10, u16, nullptr) == MLA_LB_ESHAPE);
  CHECK(mla_lb_dequant_dump(0, u8, 10, 9, u16, nullptr) == MLA_LB_OK);

  // no-alloc variant: validation and plan limits on the host, before any HIP
  // call (the scratch lookup needs a device; a single-split plan needs none)
  {
    const size_t cap = MLA_LB_NOALLOC_SCRATCH_BYTES;
    const int32_t B = 64, H = 128, L = 2500, mb = (L + 63) / 64;
    const size_t per_split = static_cast<size_t>(B) * H * 516 * 4;
    const mlb::Plan capped = mlb::make_plan(B, H, L, 0, cap);
    const mlb::Plan full = mlb::make_plan(B, H, L, 0);
    CHECK(capped.ws_bytes <= cap && capped.nsplit >= 1);
    CHECK(full.ws_bytes <= cap || capped.nsplit == static_cast<int32_t>(cap / per_split));
    CHECK(mlb::make_plan(1, 16, 100000, 0, cap).nsplit == mlb::make_plan(1, 16, 100000, 0).nsplit);
    CHECK(mlb::make_plan(65535, 128, 100000, 0, cap).nsplit == 1);   // not even two fit
    const int32_t too_many = static_cast<int32_t>(cap / per_split) + 1;
    CHECK(mla_decode_lowbit_noalloc(0, u16, u16, u8, 10, u16, 1, i32, i32, mb, i32, L, B, H, 0.1f,
                                    too_many, f32, f32, nullptr) == MLA_LB_EWORKSPACE);
    CHECK(mla_decode_lowbit_noalloc(0, nullptr, u16, u8, 10, u16, 1, i32, i32, mb, i32, L, B, H,
                                    0.1f, 0, f32, f32, nullptr) == MLA_LB_EINVAL);
    CHECK(mla_decode_lowbit_noalloc(7, u16, u16, u8, 10, u16, 1, i32, i32, mb, i32, L, B, H, 0.1f,
                                    0, f32, f32, nullptr) == MLA_LB_EFORMAT);
    const int before = mlb::g_launches;
    CHECK(mla_decode_lowbit_noalloc(0, u16, u16, u8, 10, u16, 1, i32, i32, mb, i32, L, B, H, 0.1f,
                                    1, f32, f32, nullptr) == MLA_LB_OK);
    CHECK(mlb::g_launches == before + 1 && mlb::g_last.nsplit == 1 && mlb::g_last.ws_o == nullptr);
  }

  // calibration helpers on odd sizes, against a direct computation
  for (int64_t rows : {1, 2, 7, 1000})
    for (int32_t cols : {1, 3, 64}) {
      std::vector<uint16_t> x(static_cast<size_t>(rows) * cols);
      for (size_t i = 0; i < x.size(); ++i) x[i] = static_cast<uint16_t>(0x3F80 + (i * 37) % 200);
      std::vector<float> stat(cols), sc(cols);
      CHECK(mla_lb_channel_stat(x.data(), rows, cols, 100.0, stat.data()) == MLA_LB_OK);
      for (int32_t j = 0; j < cols; ++j) {
        float mx = 0.f;
        for (int64_t r = 0; r < rows; ++r) {
          const uint32_t bits = static_cast<uint32_t>(x[r * cols + j]) << 16;
          float v;
          std::memcpy(&v, &bits, 4);
          mx = std::fmax(mx, std::fabs(v));
        }
        CHECK(stat[j] == mx);
      }
      CHECK(mla_lb_smooth_scales(stat.data(), cols, 0.5f, 0, sc.data()) == MLA_LB_OK);
      for (int32_t j = 0; j < cols; ++j)
        CHECK(std::fabs(sc[j] - std::pow(stat[j], -0.5f)) <= 1e-6f * sc[j]);
    }
  CHECK(mla_lb_channel_stat(u16, 0, 4, 50.0, f32) == MLA_LB_ESHAPE);
  CHECK(mla_lb_smooth_scales(f32, 3, 0.5f, 1, f32) == MLA_LB_ESHAPE);

  // Hadamard rows: H_n H_n = I (apply twice), and n = 2 by hand
  for (int32_t nh : {1, 2, 8, 512}) {
    std::vector<float> x(3 * nh), y(3 * nh), z(3 * nh);
    for (size_t i = 0; i < x.size(); ++i) x[i] = static_cast<float>((i * 7919) % 113) - 56.0f;
    CHECK(mla_lb_hadamard_rows(x.data(), 3, nh, y.data()) == MLA_LB_OK);
    CHECK(mla_lb_hadamard_rows(y.data(), 3, nh, z.data()) == MLA_LB_OK);
    for (size_t i = 0; i < x.size(); ++i) CHECK(std::fabs(z[i] - x[i]) <= 1e-4f);
  }
  {
    float x2[2] = {3.0f, 1.0f}, y2[2];
    CHECK(mla_lb_hadamard_rows(x2, 1, 2, y2) == MLA_LB_OK);
    CHECK(std::fabs(y2[0] - 4.0f / std::sqrt(2.0f)) < 1e-6f && std::fabs(y2[1] - 2.0f / std::sqrt(2.0f)) < 1e-6f);
    CHECK(mla_lb_hadamard_rows(x2, 1, 3, y2) == MLA_LB_ESHAPE);
    CHECK(mla_lb_hadamard_rows(nullptr, 1, 2, y2) == MLA_LB_EINVAL);
  }

  if (failures) std::fprintf(stderr, "%d checks failed\n", failures);
  else std::printf("abi host checks passed\n");
  return failures ? 1 : 0;
}
