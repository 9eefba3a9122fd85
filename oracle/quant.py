"""Per-token asymmetric affine group quantizer (oracle).

[QuantMLA §4.1]: every quantized method uses one per-token asymmetric affine
quantizer with groups of 64 coordinates; CxRy names the content-cache and
RoPE-key-cache bit widths (C4R4 primary, C2R4 = INT2 content + INT4 RoPE).

[QuantMLA App. C.4]: each token is quantized on its own in groups of 64; with
bit width b, m = 2^b - 1 and the group extrema x_min, x_max define the
quantizer; rounding is to nearest with ties to even; constant groups get no
special treatment; writer and reader share one rule for scale, zero point,
rounding and clipping, and dequantization uses the stored scale.  The formula
itself is missing from the extracted text.  Reading taken here (the plainest
affine form that makes the zero point exact in bf16 storage):

    lo = min(x), hi = max(x)                       (fp32, exact: x is bf16)
    s  = bf16_rne( fl32( fl32(hi - lo) / m ) )     stored scale
    z  = lo                                        stored zero (bf16-exact)
    q  = clamp( rint_even( fl32( fl32(x - z) / s ) ), 0, m )   if s > 0
    q  = 0                                                     if s == 0
    x^ = bf16_rne( fl32( q * s + z ) )            reconstructed bf16 value

q*s is exact in fp32 (<= 8-bit integer times an 8-bit-mantissa scale), so a
fused multiply-add and a multiply followed by an add round identically.

Metadata dtype: [QuantMLA App. C.4/C.5] store content scales in BF16 and RoPE
scales in FP32.  Formats C4R4 and C2R4 store (scale, zero) in bf16 for all
nine groups (content and RoPE alike).  Format C4R4F follows the pages' split:
content groups as in C4R4, the RoPE group's scale and zero in fp32:

    s  = fl32( fl32(hi - lo) / m )                 stored scale (fp32)
    z  = lo                                        stored zero (fp32, exact)
    q  = clamp( rint_even( fl32( fl32(x - z) / s ) ), 0, m )   if s > 0
    x^ = bf16_rne( fl32( fl32(q * s) + z ) )       reconstructed bf16 value

With an fp32 scale q*s can need more than 24 significant bits, so the
product is rounded to fp32 before the zero is added (two IEEE roundings, the
plain reading of "dequantize with the stored scale" in fp32 arithmetic).

All arrays of bf16 values are carried as uint16 bit patterns.
"""

import numpy as np

GROUP = 64
D_C = 512   # content latent width    [MLA blog §1], [QuantMLA §2.1]
D_R = 64    # decoupled RoPE key width [MLA blog §1,§3]
D_ROW = D_C + D_R
N_GROUPS_C = D_C // GROUP   # 8
N_GROUPS = N_GROUPS_C + 1   # 9 (8 content + 1 RoPE)

# format name -> (content bits, rope bits)   [QuantMLA §4.1]
FORMATS = {"C4R4": (4, 4), "C2R4": (2, 4), "C4R4F": (4, 4)}
# formats whose RoPE group keeps its (scale, zero) in fp32 [QuantMLA App. C.4/C.5]
F32_ROPE = frozenset({"C4R4F"})


# ---------------------------------------------------------------- bf16 -----
def bf16_to_f32(bits):
    """bf16 bit patterns (uint16) -> float32, exact (bf16 is the top half of fp32)."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def f32_to_bf16(x):
    """float32 -> bf16 bit patterns, round to nearest, ties to even.

    Works on the fp32 bit pattern: adding 0x7FFF plus the lowest kept bit and
    truncating the low 16 bits rounds to nearest with ties to the even result;
    a carry out of the mantissa correctly bumps the exponent (and overflows to
    infinity past the largest bf16).  NaN stays NaN (quiet bit forced).
    """
    x = np.asarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    keep_lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = ((u + np.uint64(0x7FFF) + keep_lsb) >> np.uint64(16)).astype(np.uint16)
    nan = np.isnan(x)
    if np.any(nan):
        r = np.where(nan, ((u >> np.uint64(16)).astype(np.uint16) | np.uint16(0x0040)), r)
    return r


# ------------------------------------------------------------ quantizer ----
def quantize_groups(x_bits, bits):
    """Quantize groups of 64 bf16 values.

    x_bits : uint16 [..., 64] bf16 patterns; the last axis is one group.
    bits   : 2 or 4.
    returns (codes uint8 [..., 64], scale_bits uint16 [...], zero_bits uint16 [...]).
    """
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    assert x_bits.shape[-1] == GROUP
    m = np.float32((1 << bits) - 1)
    x = bf16_to_f32(x_bits)
    lo = x.min(axis=-1)
    hi = x.max(axis=-1)
    rng = (hi - lo).astype(np.float32)                    # fl32(hi - lo)
    s_bits = f32_to_bf16((rng / m).astype(np.float32))    # bf16(fl32(rng / m))
    s = bf16_to_f32(s_bits)
    z = lo                                                # bf16-exact
    z_bits = (z.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    pos = s > 0
    with np.errstate(divide="ignore", invalid="ignore"):
        d = (x - z[..., None]).astype(np.float32)         # fl32(x - z)
        t = (d / s[..., None]).astype(np.float32)         # fl32(d / s)
    q = np.rint(t)                                        # ties to even
    q = np.clip(q, 0, m)
    q = np.where(pos[..., None], q, 0).astype(np.uint8)
    return q, s_bits, z_bits


def quantize_groups_f32meta(x_bits, bits):
    """Quantize groups of 64 bf16 values keeping (scale, zero) in fp32.

    returns (codes uint8 [..., 64], scale float32 [...], zero float32 [...]).
    """
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    assert x_bits.shape[-1] == GROUP
    m = np.float32((1 << bits) - 1)
    x = bf16_to_f32(x_bits)
    lo = x.min(axis=-1)
    hi = x.max(axis=-1)
    rng = (hi - lo).astype(np.float32)                    # fl32(hi - lo)
    s = (rng / m).astype(np.float32)                      # fl32(rng / m), kept in fp32
    z = lo.astype(np.float32)
    pos = s > 0
    with np.errstate(divide="ignore", invalid="ignore"):
        d = (x - z[..., None]).astype(np.float32)         # fl32(x - z)
        t = (d / s[..., None]).astype(np.float32)         # fl32(d / s)
    q = np.rint(t)                                        # ties to even
    q = np.clip(q, 0, m)
    q = np.where(pos[..., None], q, 0).astype(np.uint8)
    return q, s, z


def dequantize_groups_f32meta(codes, scale, zero):
    """x^ = bf16(fl32(fl32(q * s) + z)) with fp32 (s, z): [..., 64] -> uint16 [..., 64]."""
    q = np.asarray(codes).astype(np.float32)
    s = np.asarray(scale, dtype=np.float32)[..., None]
    z = np.asarray(zero, dtype=np.float32)[..., None]
    y = (q * s).astype(np.float32)      # one fp32 rounding of the product
    y = (y + z).astype(np.float32)      # one fp32 rounding of the sum
    return f32_to_bf16(y)


def dequantize_groups(codes, scale_bits, zero_bits):
    """x^ = bf16(fl32(q * s + z)); codes [..., 64], scale/zero [...] -> uint16 [..., 64]."""
    q = np.asarray(codes).astype(np.float32)
    s = bf16_to_f32(scale_bits)[..., None]
    z = bf16_to_f32(zero_bits)[..., None]
    y = (q * s).astype(np.float32)      # exact
    y = (y + z).astype(np.float32)      # one fp32 rounding
    return f32_to_bf16(y)


def quantize_tokens(c_bits, kr_bits, fmt):
    """Quantize whole tokens: content c [T,512] and RoPE key k_R [T,64] (bf16 bits).

    returns dict with
      codes_c uint8 [T,512], codes_r uint8 [T,64],
      scale uint16 [T,9], zero uint16 [T,9]   (groups 0..7 content, 8 RoPE)
    and, for formats in F32_ROPE, the RoPE group's fp32 metadata
      scale_r32 float32 [T], zero_r32 float32 [T]   (column 8 of scale/zero is 0)
    """
    bc, br = FORMATS[fmt]
    c_bits = np.asarray(c_bits, dtype=np.uint16)
    kr_bits = np.asarray(kr_bits, dtype=np.uint16)
    T = c_bits.shape[0]
    qc, sc, zc = quantize_groups(c_bits.reshape(T, N_GROUPS_C, GROUP), bc)
    out = {"codes_c": qc.reshape(T, D_C)}
    if fmt in F32_ROPE:
        qr, sr32, zr32 = quantize_groups_f32meta(kr_bits.reshape(T, 1, GROUP), br)
        sr = np.zeros((T, 1), np.uint16)
        zr = np.zeros((T, 1), np.uint16)
        out["scale_r32"] = sr32.reshape(T)
        out["zero_r32"] = zr32.reshape(T)
    else:
        qr, sr, zr = quantize_groups(kr_bits.reshape(T, 1, GROUP), br)
    out["codes_r"] = qr.reshape(T, D_R)
    out["scale"] = np.concatenate([sc, sr], axis=1)
    out["zero"] = np.concatenate([zc, zr], axis=1)
    return out


def dequantize_tokens(qt):
    """Reconstruct bf16 rows [T,576] = [c^ | k^_R] from quantize_tokens' output."""
    T = qt["codes_c"].shape[0]
    c = dequantize_groups(qt["codes_c"].reshape(T, N_GROUPS_C, GROUP),
                          qt["scale"][:, :N_GROUPS_C], qt["zero"][:, :N_GROUPS_C])
    if "scale_r32" in qt:
        r = dequantize_groups_f32meta(qt["codes_r"].reshape(T, 1, GROUP),
                                      qt["scale_r32"].reshape(T, 1), qt["zero_r32"].reshape(T, 1))
    else:
        r = dequantize_groups(qt["codes_r"].reshape(T, 1, GROUP),
                              qt["scale"][:, N_GROUPS_C:], qt["zero"][:, N_GROUPS_C:])
    return np.concatenate([c.reshape(T, D_C), r.reshape(T, D_R)], axis=1)
