// Device-side constants, vector types and small helpers shared by the kernels
// of libmla_lowbit.so (gfx950 / CDNA4 only).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mlb {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int PAGE = 64;        // tokens per page            [QuantMLA App. C.5]
constexpr int DC = 512;         // content latent width        [MLA blog §1]
constexpr int DR = 64;          // decoupled RoPE key width    [MLA blog §3]
constexpr int DROW = DC + DR;   // 576 cached values per token [MLA blog §1]
constexpr int NSINK = 4;        // BF16 sink tokens            [QuantMLA §3.3]
constexpr int NRECENT = 128;    // BF16 recent tokens          [QuantMLA §3.3]
constexpr int PROT_ROWS = NSINK + NRECENT;
constexpr int NGC = DC / 64;    // content groups of 64 per token

// Page geometry per format (byte offsets of the structure-of-arrays regions).
// C4R4:  codes_c [4][64][64] | codes_r [64][32] | meta_c [64][8][2]bf16 | meta_r [64][2]bf16
// C2R4:  codes_c [2][64][64] | ...
// C4R4F: as C4R4, but meta_r [64][2]fp32 (the RoPE group's scale and zero in
//        fp32 [QuantMLA App. C.4/C.5])
template <int F> struct Fmt;
template <> struct Fmt<0> {
  static constexpr int CBITS = 4, NBLK = 4, DPB = 128;   // content dims per block
  static constexpr int OFF_R = 16384, OFF_MC = 18432, OFF_MR = 20480, PAGE_BYTES = 20736;
  static constexpr bool F32R = false;                    // RoPE metadata in fp32
};
template <> struct Fmt<1> {
  static constexpr int CBITS = 2, NBLK = 2, DPB = 256;
  static constexpr int OFF_R = 8192, OFF_MC = 10240, OFF_MR = 12288, PAGE_BYTES = 12544;
  static constexpr bool F32R = false;
};
template <> struct Fmt<2> {
  static constexpr int CBITS = 4, NBLK = 4, DPB = 128;
  static constexpr int OFF_R = 16384, OFF_MC = 18432, OFF_MR = 20480, PAGE_BYTES = 20992;
  static constexpr bool F32R = true;
};

// Protection-buffer row of position i: sinks keep rows 0..3, the recent
// window is a ring over rows 4..131.
__device__ __forceinline__ int prot_row(int i) {
  return i < NSINK ? i : NSINK + (i & (NRECENT - 1));
}
// Membership of position i in the protected set of a length-L sequence:
// the first 4 tokens and the last 128.
__device__ __forceinline__ bool is_protected(int i, int L) {
  return i < NSINK || i >= L - NRECENT;
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b16) {
  return __uint_as_float(b16 << 16);
}

// fp32 -> bf16 bits, round to nearest even (NaN kept quiet).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// Two fp32 -> packed bf16 pair (low half = a), RNE; one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  f32x2 v = {a, b};
  bf16x2 p = __builtin_convertvector(v, bf16x2);
  return __builtin_bit_cast(uint32_t, p);
}

// Physical page ids of one split's pages, read from the block table through
// vector loads into a window held one entry per lane: lane j of `cur` holds
// split page w0 + j, lane j of `nxt` split page w0 + 64 + j, and `nxt` is
// requested as soon as `cur` comes into use, 64 pages ahead of its first
// read.  Entries come out of the window with readlane, so no scalar load (and
// no wait on the counter LDS reads share) sits in a page loop.  Ids outside
// [0, num_pages), and pages past the split, read as -1.  Callers ask for
// page indices that never decrease (advance() before each new maximum) and
// stay below w0 + 128.
struct PageWindow {
  const int32_t* row;   // block-table entries of the split's first page
  int np;               // pages in the split
  int64_t num_pages;
  int w0;
  int cur, nxt;

  __device__ __forceinline__ int fetch(int k, int lane) const {
    const int i = k + lane;
    int v = -1;
    if (i < np) v = row[i];
    return (v >= 0 && v < num_pages) ? v : -1;
  }
  __device__ __forceinline__ void init(int lane) {
    w0 = 0;
    cur = fetch(0, lane);
    nxt = fetch(64, lane);
  }
  // make page k (k >= w0) readable
  __device__ __forceinline__ void advance(int k, int lane) {
    if (k >= w0 + 64) {
      w0 += 64;
      cur = nxt;
      nxt = fetch(w0 + 64, lane);
    }
  }
  __device__ __forceinline__ int id(int k) const {
    const int j = k - w0;
    return j < 64 ? __builtin_amdgcn_readlane(cur, j) : __builtin_amdgcn_readlane(nxt, j - 64);
  }
};

template <typename T, typename S>
__device__ __forceinline__ T bitcast(const S& s) {
  static_assert(sizeof(T) == sizeof(S), "size");
  return __builtin_bit_cast(T, s);
}

}  // namespace mlb
