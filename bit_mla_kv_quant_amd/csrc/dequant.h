// Unpack + dequantize of packed cache rows into bf16 MFMA operands, shared by
// the decode kernels and the dequant dump (so the dump shows exactly what the
// decode kernels multiply).  [QuantMLA App. C.4/C.5]
//
// Reconstruction of one code q of a group with stored bf16 (scale s, zero z):
//     x^ = bf16_rne( fl32(q * s + z) )
// q * s is exact in fp32 (q < 16, s has an 8-bit significand), so one fused
// multiply-add rounds exactly once, like the unfused product-then-sum.
// With an fp32 (scale, zero) pair (the RoPE group of format C4R4F) q * s is
// not exact, and the reconstruction rounds the product, then the sum:
//     x^ = bf16_rne( fl32( fl32(q * s) + z ) )
//
// Lane geometry: a lane owns one token slot `tt` of a page and, in dim half
// dh (0 or 1), lane group g (0..3): the 64 content dims 256*dh + 64*g ..+63
// (exactly one quantization group) and the 8 RoPE dims 32*dh + 8*g ..+7.
// Dims are delivered as slices of 8 consecutive bf16, the unit a lane
// contributes to one v_mfma_f32_16x16x32_bf16 operand.
#pragma once
#include "common.h"

namespace mlb {

typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Keeps the compiler from folding a mask into later byte extractions.
__device__ __forceinline__ uint32_t opaque(uint32_t x) {
  asm("" : "+v"(x));
  return x;
}

__device__ __forceinline__ float ubyte(uint32_t w, int k) {
  return (float)((w >> (8 * k)) & 0xffu);
}

// 8 INT4 codes of one 32-bit word (byte k: dim 2k in bits 0-3, dim 2k+1 in
// bits 4-7) -> 8 consecutive reconstructed bf16 values; one byte conversion
// per code.  Valid for every finite scale.
__device__ __forceinline__ bf16x8 deq_int4x8_ubyte(uint32_t w, float s, float z) {
  const uint32_t lo = opaque(w & 0x0F0F0F0Fu);          // dims 0,2,4,6
  const uint32_t hi = opaque((w >> 4) & 0x0F0F0F0Fu);   // dims 1,3,5,7
  u32x4 r;
#pragma unroll
  for (int k = 0; k < 4; ++k)
    r[k] = pack_bf16x2(__builtin_fmaf(ubyte(lo, k), s, z), __builtin_fmaf(ubyte(hi, k), s, z));
  return bitcast<bf16x8>(r);
}

// Same values, two codes per conversion: a byte b in 0..15 read as an OCP
// fp8 e4m3 number is exactly b * 2^-9 (the subnormal range and the first
// normal binade share the spacing 2^-9), so with s9 = s * 2^9 (exact)
// fma(b * 2^-9, s9, z) equals fma(b, s, z) bit for bit.  Needs s9 finite,
// i.e. s < 2^119; callers route larger scales to the byte path.
__device__ __forceinline__ bf16x8 deq_int4x8_fp8(uint32_t w, float s9, float z) {
  const uint32_t lo = w & 0x0F0F0F0Fu;                  // dims 0,2,4,6
  const uint32_t hi = (w >> 4) & 0x0F0F0F0Fu;           // dims 1,3,5,7
  const f32x2_t l01 = __builtin_amdgcn_cvt_pk_f32_fp8(lo, false);   // dims 0,2
  const f32x2_t l23 = __builtin_amdgcn_cvt_pk_f32_fp8(lo, true);    // dims 4,6
  const f32x2_t h01 = __builtin_amdgcn_cvt_pk_f32_fp8(hi, false);   // dims 1,3
  const f32x2_t h23 = __builtin_amdgcn_cvt_pk_f32_fp8(hi, true);    // dims 5,7
  u32x4 r;
  r[0] = pack_bf16x2(__builtin_fmaf(l01[0], s9, z), __builtin_fmaf(h01[0], s9, z));
  r[1] = pack_bf16x2(__builtin_fmaf(l01[1], s9, z), __builtin_fmaf(h01[1], s9, z));
  r[2] = pack_bf16x2(__builtin_fmaf(l23[0], s9, z), __builtin_fmaf(h23[0], s9, z));
  r[3] = pack_bf16x2(__builtin_fmaf(l23[1], s9, z), __builtin_fmaf(h23[1], s9, z));
  return bitcast<bf16x8>(r);
}

// The same 8 codes with an fp32 (scale, zero) pair: the product is rounded
// to fp32 before the zero is added.  (b * 2^-9) * s9 is one rounding of
// b * s, so the fp8 conversion still applies.
__device__ __forceinline__ float mul_then_add(float a, float b, float c) {
#pragma clang fp contract(off)
  const float p = a * b;
  return p + c;
}
__device__ __forceinline__ bf16x8 deq_int4x8_fp8_ma(uint32_t w, float s9, float z) {
  const uint32_t lo = w & 0x0F0F0F0Fu;                  // dims 0,2,4,6
  const uint32_t hi = (w >> 4) & 0x0F0F0F0Fu;           // dims 1,3,5,7
  const f32x2_t l01 = __builtin_amdgcn_cvt_pk_f32_fp8(lo, false);
  const f32x2_t l23 = __builtin_amdgcn_cvt_pk_f32_fp8(lo, true);
  const f32x2_t h01 = __builtin_amdgcn_cvt_pk_f32_fp8(hi, false);
  const f32x2_t h23 = __builtin_amdgcn_cvt_pk_f32_fp8(hi, true);
  u32x4 r;
  r[0] = pack_bf16x2(mul_then_add(l01[0], s9, z), mul_then_add(h01[0], s9, z));
  r[1] = pack_bf16x2(mul_then_add(l01[1], s9, z), mul_then_add(h01[1], s9, z));
  r[2] = pack_bf16x2(mul_then_add(l23[0], s9, z), mul_then_add(h23[0], s9, z));
  r[3] = pack_bf16x2(mul_then_add(l23[1], s9, z), mul_then_add(h23[1], s9, z));
  return bitcast<bf16x8>(r);
}
__device__ __forceinline__ bf16x8 deq_int4x8_ubyte_ma(uint32_t w, float s, float z) {
  const uint32_t lo = opaque(w & 0x0F0F0F0Fu);
  const uint32_t hi = opaque((w >> 4) & 0x0F0F0F0Fu);
  u32x4 r;
#pragma unroll
  for (int k = 0; k < 4; ++k)
    r[k] = pack_bf16x2(mul_then_add(ubyte(lo, k), s, z), mul_then_add(ubyte(hi, k), s, z));
  return bitcast<bf16x8>(r);
}

// INT2 groups have four possible reconstructions; they are computed once per
// group with the same arithmetic as above and kept as a byte-permute table:
// byte q of `lo` is the low byte of x^(q), byte q of `hi` its high byte.
struct Lut2 {
  uint32_t lo, hi;   // byte q: low / high byte of the bf16 value of code q
  uint32_t sel_or;   // 0x04000400 in a vector register (see lut2_pair)
};
__device__ __forceinline__ Lut2 make_lut2(float s, float z) {
  const uint32_t p01 = pack_bf16x2(__builtin_fmaf(0.0f, s, z), __builtin_fmaf(1.0f, s, z));
  const uint32_t p23 = pack_bf16x2(__builtin_fmaf(2.0f, s, z), __builtin_fmaf(3.0f, s, z));
  Lut2 t;
  t.lo = __builtin_amdgcn_perm(p23, p01, 0x06040200u);   // bytes 0, 2, 4, 6 of {p23, p01}
  t.hi = __builtin_amdgcn_perm(p23, p01, 0x07050301u);   // bytes 1, 3, 5, 7
  asm volatile("v_mov_b32 %0, 0x4000400" : "=v"(t.sel_or));
  return t;
}

// Two INT2 codes a (bits 0-1 of bytes 0 and 1 of `d`) and b (same bits of
// bytes 2 and 3) -> bf16 pair (x^(a), x^(b)).  One AND-OR turns d into the
// selector bytes (a, a + 4, b, b + 4): low byte from lut.lo, high byte from
// lut.hi.
// The AND-OR is one v_and_or_b32; its two constants cannot both be literals
// or scalar registers, so the OR constant comes in a vector register.
__device__ __forceinline__ uint32_t lut2_pair(uint32_t d, const Lut2& lut) {
  uint32_t sel;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(sel) : "v"(d), "s"(0x03030303u), "v"(lut.sel_or));
  return __builtin_amdgcn_perm(lut.hi, lut.lo, sel);
}

// 16 INT2 codes of one 32-bit word (dim 2m in bits 2m, dim 2m+1 in bits
// 16+2m) -> dims 0..7 in `a`, dims 8..15 in `b`.  The bytes holding the codes
// are first doubled (byte 0 into bytes 0 and 1, byte 2 into bytes 2 and 3;
// likewise bytes 1 and 3), so one shift brings a code pair into selector
// position.
__device__ __forceinline__ void deq_int2x16(uint32_t w, const Lut2& lut, bf16x8& a, bf16x8& b) {
  const uint32_t dl = __builtin_amdgcn_perm(w, w, 0x02020000u);
  const uint32_t dh = __builtin_amdgcn_perm(w, w, 0x03030101u);
  u32x4 r, t;
#pragma unroll
  for (int m = 0; m < 4; ++m) r[m] = lut2_pair(dl >> (2 * m), lut);
#pragma unroll
  for (int m = 0; m < 4; ++m) t[m] = lut2_pair(dh >> (2 * m), lut);
  a = bitcast<bf16x8>(r);
  b = bitcast<bf16x8>(t);
}

// ---------------------------------------------------------------- pages ----
// Register image of one lane's share of one token slot of a packed page.
template <int F> struct Packed;
template <> struct Packed<0> {   // C4R4
  u32x4 c[2];                    // content dims 256dh+64g .. +63 (2 x 32 dims)
  uint32_t mc;                   // (scale, zero) bf16 pair of that group
  uint32_t rc;                   // RoPE dims 32dh+8g .. +7
  uint32_t mr;                   // RoPE (scale, zero)
};
template <> struct Packed<1> {   // C2R4
  u32x4 c;                       // content dims 256dh+64g .. +63
  uint32_t mc;
  uint32_t rc;
  uint32_t mr;
};
template <> struct Packed<2> {   // C4R4F
  u32x4 c[2];
  uint32_t mc;
  uint32_t rc;
  u32x2 mr;                      // RoPE (scale, zero) fp32 bit patterns
};

template <int F>
__device__ __forceinline__ Packed<F> load_packed(const uint8_t* pg, int tt, int dh, int g) {
  using FM = Fmt<F>;
  Packed<F> p;
  if constexpr (FM::CBITS == 4) {
    // blocks of 128 dims: block 2dh + g/2, bytes 32*(g&1) .. +31 of the row
    const uint8_t* row = pg + ((2 * dh + (g >> 1)) * PAGE + tt) * 64 + 32 * (g & 1);
    p.c[0] = *(const u32x4*)row;
    p.c[1] = *(const u32x4*)(row + 16);
  } else {
    // blocks of 256 dims: block dh, bytes 16g .. +15 of the row
    p.c = *(const u32x4*)(pg + (dh * PAGE + tt) * 64 + 16 * g);
  }
  p.mc = *(const uint32_t*)(pg + FM::OFF_MC + tt * 32 + (4 * dh + g) * 4);
  p.rc = *(const uint32_t*)(pg + FM::OFF_R + tt * 32 + 16 * dh + 4 * g);
  if constexpr (FM::F32R) p.mr = *(const u32x2*)(pg + FM::OFF_MR + tt * 8);
  else p.mr = *(const uint32_t*)(pg + FM::OFF_MR + tt * 4);
  return p;
}

// One lane's share of one token slot when four lanes share a token: lane g
// takes content groups 2g, 2g+1 (dims 128g .. 128g+127) and RoPE dims
// 16g .. 16g+15 (page layout as written by kv_quant_append).
template <int F> struct LaneSlot;
template <> struct LaneSlot<0> {     // C4R4
  u32x4 c[4];                    // dims 128g .. 128g+127 (block g of the page)
  u32x2 r;                       // RoPE dims 16g .. 16g+15
  u32x2 mc;                      // (scale, zero) of groups 2g, 2g+1
  uint32_t mr;                   // RoPE (scale, zero)
};
template <> struct LaneSlot<1> {     // C2R4
  u32x4 c[2];                    // dims 128g .. 128g+127 (half of block g/2)
  u32x2 r;
  u32x2 mc;
  uint32_t mr;
};
template <> struct LaneSlot<2> {     // C4R4F
  u32x4 c[4];
  u32x2 r;
  u32x2 mc;
  u32x2 mr;                      // RoPE (scale, zero) fp32 bit patterns
};

template <int F>
__device__ __forceinline__ LaneSlot<F> load_lane_slot(const uint8_t* pg, int tt, int g) {
  using FM = Fmt<F>;
  LaneSlot<F> p;
  if constexpr (FM::CBITS == 4) {
    const uint8_t* row = pg + (g * PAGE + tt) * 64;
#pragma unroll
    for (int i = 0; i < 4; ++i) p.c[i] = *(const u32x4*)(row + 16 * i);
  } else {
    const uint8_t* row = pg + ((g >> 1) * PAGE + tt) * 64 + 32 * (g & 1);
    p.c[0] = *(const u32x4*)row;
    p.c[1] = *(const u32x4*)(row + 16);
  }
  p.r = *(const u32x2*)(pg + FM::OFF_R + tt * 32 + 8 * g);
  p.mc = *(const u32x2*)(pg + FM::OFF_MC + tt * 32 + 8 * g);
  if constexpr (FM::F32R) p.mr = *(const u32x2*)(pg + FM::OFF_MR + tt * 8);
  else p.mr = *(const uint32_t*)(pg + FM::OFF_MR + tt * 4);
  return p;
}

// (scale, zero) of a group: a bf16 pair in one word, or fp32 bit patterns
__device__ __forceinline__ float meta_scale(uint32_t m) { return bf16_bits_to_f32(m & 0xffffu); }
__device__ __forceinline__ float meta_zero(uint32_t m) { return bf16_bits_to_f32(m >> 16); }
__device__ __forceinline__ float meta_scale(u32x2 m) { return __uint_as_float(m[0]); }
__device__ __forceinline__ float meta_zero(u32x2 m) { return __uint_as_float(m[1]); }

// 8 INT4 codes with the fp8 conversion when the scale allows it.
__device__ __forceinline__ bf16x8 deq_int4x8(uint32_t w, uint32_t meta) {
  const float s = meta_scale(meta), z = meta_zero(meta);
  const float s9 = s * 512.0f;
  if (__builtin_expect(s9 <= 3.4028234663852886e38f, 1)) return deq_int4x8_fp8(w, s9, z);
  return deq_int4x8_ubyte(w, s, z);
}
__device__ __forceinline__ bf16x8 deq_int4x8(uint32_t w, u32x2 meta) {
  const float s = meta_scale(meta), z = meta_zero(meta);
  const float s9 = s * 512.0f;
  if (__builtin_expect(s9 <= 3.4028234663852886e38f, 1)) return deq_int4x8_fp8_ma(w, s9, z);
  return deq_int4x8_ubyte_ma(w, s, z);
}

// The RoPE group's 8 codes on the fp8 path (s9 = s * 2^9 finite), with the
// arithmetic its metadata type asks for.
template <int F>
__device__ __forceinline__ bf16x8 deq_rope8_fp8(uint32_t w, float s9, float z) {
  if constexpr (Fmt<F>::F32R) return deq_int4x8_fp8_ma(w, s9, z);
  else return deq_int4x8_fp8(w, s9, z);
}

// The lane's 64 content dims -> 8 slices of 8 bf16 (dims 8t .. 8t+7 of them).
template <int F>
__device__ __forceinline__ void deq_content(const Packed<F>& p, bf16x8* kv) {
  if constexpr (Fmt<F>::CBITS == 4) {
    const float s = meta_scale(p.mc), z = meta_zero(p.mc);
    const float s9 = s * 512.0f;
    if (__builtin_expect(s9 <= 3.4028234663852886e38f, 1)) {
#pragma unroll
      for (int t = 0; t < 8; ++t) kv[t] = deq_int4x8_fp8(p.c[t >> 2][t & 3], s9, z);
    } else {
#pragma unroll
      for (int t = 0; t < 8; ++t) kv[t] = deq_int4x8_ubyte(p.c[t >> 2][t & 3], s, z);
    }
  } else {
    const Lut2 lut = make_lut2(meta_scale(p.mc), meta_zero(p.mc));
#pragma unroll
    for (int k = 0; k < 4; ++k) deq_int2x16(p.c[k], lut, kv[2 * k], kv[2 * k + 1]);
  }
}

// The lane's 8 RoPE dims -> one slice of 8 bf16.
template <int F>
__device__ __forceinline__ bf16x8 deq_rope(const Packed<F>& p) {
  return deq_int4x8(p.rc, p.mr);
}

}  // namespace mlb
