// Unpack + dequantize of packed cache rows into bf16 MFMA operands, shared by
// the decode kernels and the dequant dump (so the dump shows exactly what the
// decode kernels multiply).  [QuantMLA App. C.4/C.5]
//
// Reconstruction of one code q of a group with stored bf16 (scale s, zero z):
//     x^ = bf16_rne( fl32(q * s + z) )
// q * s is exact in fp32 (q < 16, s has an 8-bit significand), so one fused
// multiply-add rounds exactly once, like the unfused product-then-sum.
//
// Lane geometry (one wave = 16 token slots x 4 lane groups): lane
// (n16 = lane % 16, g = lane / 16) owns token slot `tt` of the page and, per
// content chunk r, a contiguous run of SPAN dims (one 64-dim group or half of
// one); the dims are delivered as slices of 8 consecutive bf16, the unit a
// lane contributes to one v_mfma_f32_16x16x32_bf16 B operand.
#pragma once
#include "common.h"

namespace mlb {

// Keeps the compiler from folding a mask into later byte extractions, so each
// byte of the masked word is converted by one v_cvt_f32_ubyteN.
__device__ __forceinline__ uint32_t opaque(uint32_t x) {
  asm("" : "+v"(x));
  return x;
}

__device__ __forceinline__ float ubyte(uint32_t w, int k) {
  return (float)((w >> (8 * k)) & 0xffu);
}

// 8 INT4 codes of one 32-bit word (byte k: dim 2k in bits 0-3, dim 2k+1 in
// bits 4-7) -> 8 consecutive reconstructed bf16 values.
__device__ __forceinline__ bf16x8 deq_int4x8(uint32_t w, float s, float z) {
  const uint32_t lo = opaque(w & 0x0F0F0F0Fu);          // dims 0,2,4,6
  const uint32_t hi = opaque((w >> 4) & 0x0F0F0F0Fu);   // dims 1,3,5,7
  u32x4 r;
#pragma unroll
  for (int k = 0; k < 4; ++k)
    r[k] = pack_bf16x2(__builtin_fmaf(ubyte(lo, k), s, z), __builtin_fmaf(ubyte(hi, k), s, z));
  return bitcast<bf16x8>(r);
}

// INT2 groups have four possible reconstructions; they are computed once per
// group with the same arithmetic as above and kept as a byte-permute table:
// bytes 0-3 = (x^(0), x^(1)) in `lo`, bytes 4-7 = (x^(2), x^(3)) in `hi`.
struct Lut2 {
  uint32_t lo, hi;
};
__device__ __forceinline__ Lut2 make_lut2(float s, float z) {
  Lut2 t;
  t.lo = pack_bf16x2(__builtin_fmaf(0.0f, s, z), __builtin_fmaf(1.0f, s, z));
  t.hi = pack_bf16x2(__builtin_fmaf(2.0f, s, z), __builtin_fmaf(3.0f, s, z));
  return t;
}

// Two INT2 codes a (bits 0-1) and b (bits 16-17) of `t` -> bf16 pair
// (x^(a), x^(b)).  Selector bytes (2a, 2a+1, 2b, 2b+1) pick the table entries.
__device__ __forceinline__ uint32_t lut2_pair(uint32_t t, const Lut2& lut) {
  const uint32_t sel = t * 0x202u + 0x01000100u;
  return __builtin_amdgcn_perm(lut.hi, lut.lo, sel);
}

// 16 INT2 codes of one 32-bit word (dim 2m in bits 2m, dim 2m+1 in bits
// 16+2m) -> dims 0..7 in `a`, dims 8..15 in `b`.
__device__ __forceinline__ void deq_int2x16(uint32_t w, const Lut2& lut, bf16x8& a, bf16x8& b) {
  u32x4 r, t;
#pragma unroll
  for (int m = 0; m < 4; ++m) r[m] = lut2_pair((w >> (2 * m)) & 0x00030003u, lut);
#pragma unroll
  for (int m = 0; m < 4; ++m) t[m] = lut2_pair((w >> (2 * m + 8)) & 0x00030003u, lut);
  a = bitcast<bf16x8>(r);
  b = bitcast<bf16x8>(t);
}

// ---------------------------------------------------------------- pages ----
// Register image of one lane's share of one token slot of a packed page.
template <int F> struct Packed;
template <> struct Packed<0> {   // C4R4: chunk r = dims 128r + 32g .. +31
  u32x4 c[4];
  uint32_t mc[4];                // (scale, zero) bf16 pair of chunk r's group
  u32x2 rc;                      // RoPE dims 16g .. 16g+15
  uint32_t mr;
};
template <> struct Packed<1> {   // C2R4: chunk r = dims 256r + 64g .. +63
  u32x4 c[2];
  uint32_t mc[2];
  u32x2 rc;
  uint32_t mr;
};

template <int F>
__device__ __forceinline__ Packed<F> load_packed(const uint8_t* pg, int tt, int g) {
  using FM = Fmt<F>;
  Packed<F> p;
#pragma unroll
  for (int r = 0; r < FM::NBLK; ++r) {
    p.c[r] = *(const u32x4*)(pg + (r * PAGE + tt) * 64 + g * 16);
    const int grp = (r * FM::DPB + g * (FM::DPB / 4)) / 64;
    p.mc[r] = *(const uint32_t*)(pg + FM::OFF_MC + tt * 32 + grp * 4);
  }
  p.rc = *(const u32x2*)(pg + FM::OFF_R + tt * 32 + g * 8);
  p.mr = *(const uint32_t*)(pg + FM::OFF_MR + tt * 4);
  return p;
}

__device__ __forceinline__ float meta_scale(uint32_t m) { return bf16_bits_to_f32(m & 0xffffu); }
__device__ __forceinline__ float meta_zero(uint32_t m) { return bf16_bits_to_f32(m >> 16); }

// Content chunk r -> NT slices of 8 bf16 (NT = 4 for C4R4, 8 for C2R4).
template <int F>
__device__ __forceinline__ void deq_content(const Packed<F>& p, int r, bf16x8* kv) {
  const float s = meta_scale(p.mc[r]), z = meta_zero(p.mc[r]);
  if constexpr (F == 0) {
#pragma unroll
    for (int t = 0; t < 4; ++t) kv[t] = deq_int4x8(p.c[r][t], s, z);
  } else {
    const Lut2 lut = make_lut2(s, z);
#pragma unroll
    for (int t = 0; t < 4; ++t) deq_int2x16(p.c[r][t], lut, kv[2 * t], kv[2 * t + 1]);
  }
}

// RoPE dims 16g .. 16g+15 -> two slices of 8 bf16.
template <int F>
__device__ __forceinline__ void deq_rope(const Packed<F>& p, bf16x8* kr) {
  const float s = meta_scale(p.mr), z = meta_zero(p.mr);
  kr[0] = deq_int4x8(p.rc[0], s, z);
  kr[1] = deq_int4x8(p.rc[1], s, z);
}

}  // namespace mlb
