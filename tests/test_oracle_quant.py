"""Pins for oracle/quant.py and oracle/layout.py (CPU only).

Each check ties the oracle to something other than itself: torch's bf16
conversion, exact rational arithmetic, brute-force search over all codes,
hand-built byte patterns, and round trips.
"""

from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import quant, layout


def _torch_bf16(x):
    t = torch.from_numpy(np.asarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _exact_round_to_bits(fr, mant_bits):
    """Round a nonzero Fraction to the nearest binary float with `mant_bits`
    significant bits (ties to even); normal range only.  Returns a Fraction."""
    if fr == 0:
        return Fraction(0)
    sign = -1 if fr < 0 else 1
    a = abs(fr)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    ulp = Fraction(2) ** (e - (mant_bits - 1))
    k = a / ulp
    lo = k.numerator // k.denominator
    rem = k - lo
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and lo % 2 == 1):
        lo += 1
    return sign * lo * ulp


# ------------------------------------------------------------------ bf16 ---
def test_bf16_rne_matches_torch_random():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(200000).astype(np.float32) * np.float32(3.0),
        (rng.standard_normal(20000) * 1e-38).astype(np.float32),        # subnormals
        (rng.standard_normal(20000) * 1e30).astype(np.float32),
    ])
    np.testing.assert_array_equal(quant.f32_to_bf16(x), _torch_bf16(x))


def test_bf16_rne_ties_and_specials():
    # exact ties: low 16 bits == 0x8000, both parities of the kept lsb
    hi = np.arange(0x3F00, 0x4100, dtype=np.uint32)
    ties = ((hi << 16) | 0x8000).view(np.float32)
    got = quant.f32_to_bf16(ties)
    np.testing.assert_array_equal(got, _torch_bf16(ties))
    # ties go to the even kept pattern
    assert np.all(got % 2 == 0)
    specials = np.array([0.0, -0.0, np.inf, -np.inf, 3.3895313892515355e38,
                         np.finfo(np.float32).max, 1e-45, -1e-45], dtype=np.float32)
    np.testing.assert_array_equal(quant.f32_to_bf16(specials), _torch_bf16(specials))


def test_bf16_rne_exact_rational():
    rng = np.random.default_rng(1)
    x = (rng.standard_normal(2000) * 10).astype(np.float32)
    got = quant.bf16_to_f32(quant.f32_to_bf16(x))
    for xi, gi in zip(x, got):
        assert Fraction(float(gi)) == _exact_round_to_bits(Fraction(float(xi)), 8)


# ------------------------------------------------------------- quantizer ---
def _groups_small_int(rng, n, bits_range=40, spread=2.0 ** -3):
    """Groups of bf16-exact values (small integers times a power of two): many
    exact ties and exactly representable differences."""
    v = rng.integers(-bits_range, bits_range + 1, size=(n, 64)).astype(np.float32) * np.float32(spread)
    return quant.f32_to_bf16(v)


@pytest.mark.parametrize("bits", [2, 4])
def test_quantizer_brute_force_nearest_code(bits):
    """Each code is the nearest of the 2^b reconstruction points q*s+z
    (exact rational distance), ties to the even code; s and z follow the
    stated rule."""
    rng = np.random.default_rng(10 + bits)
    xb = np.concatenate([_groups_small_int(rng, 300),
                         quant.f32_to_bf16(rng.standard_normal((300, 64)).astype(np.float32))])
    q, sb, zb = quant.quantize_groups(xb, bits)
    m = (1 << bits) - 1
    xf = quant.bf16_to_f32(xb)
    for g in range(xb.shape[0]):
        lo, hi = Fraction(float(xf[g].min())), Fraction(float(xf[g].max()))
        # stated scale: bf16(fl32(fl32(hi-lo)/m)) -- fl32 steps via exact rounding
        rngf = _exact_round_to_bits(hi - lo, 24)
        s = _exact_round_to_bits(_exact_round_to_bits(rngf / m, 24), 8) if rngf != 0 else Fraction(0)
        assert Fraction(float(quant.bf16_to_f32(sb[g]))) == s
        assert Fraction(float(quant.bf16_to_f32(zb[g]))) == lo
        for j in range(64):
            x = Fraction(float(xf[g, j]))
            if s == 0:
                assert q[g, j] == 0
                continue
            d = [abs(x - (k * s + lo)) for k in range(m + 1)]
            best = min(d)
            cands = [k for k in range(m + 1) if d[k] == best]
            want = cands[0] if len(cands) == 1 else [k for k in cands if k % 2 == 0][0]
            assert q[g, j] == want, (g, j, float(x), float(s), float(lo), cands)


@pytest.mark.parametrize("bits", [2, 4])
def test_quantizer_invariants_on_workload_distribution(bits):
    rng = np.random.default_rng(20 + bits)
    a = np.exp(0.5 * rng.standard_normal(64))
    a[:2] *= 16.0
    xb = quant.f32_to_bf16((rng.standard_normal((5000, 64)) * a).astype(np.float32))
    q, sb, zb = quant.quantize_groups(xb, bits)
    m = (1 << bits) - 1
    assert q.max() <= m and q.dtype == np.uint8
    x = quant.bf16_to_f32(xb).astype(np.float64)
    s = quant.bf16_to_f32(sb).astype(np.float64)
    z = quant.bf16_to_f32(zb).astype(np.float64)
    recon = q * s[:, None] + z[:, None]          # exact in float64
    err = np.abs(x - recon)
    assert np.all(err <= 0.5 * s[:, None] * (1 + 1e-6))
    # the group minimum reconstructs exactly (code 0)
    amin = x.argmin(axis=1)
    assert np.all(q[np.arange(len(q)), amin] == 0)
    xh = quant.bf16_to_f32(quant.dequantize_groups(q, sb, zb))
    assert np.all(xh[np.arange(len(q)), amin] == x[np.arange(len(q)), amin])


def test_constant_group_reconstructs_exactly():
    xb = quant.f32_to_bf16(np.full((3, 64), [[1.5], [-7.0], [0.0]], dtype=np.float32))
    for bits in (2, 4):
        q, sb, zb = quant.quantize_groups(xb, bits)
        assert np.all(q == 0) and np.all(sb == 0)
        np.testing.assert_array_equal(quant.dequantize_groups(q, sb, zb), xb)


def test_dequant_is_one_fp32_rounding_then_bf16():
    rng = np.random.default_rng(3)
    xb = quant.f32_to_bf16((rng.standard_normal((200, 64)) * 5).astype(np.float32))
    q, sb, zb = quant.quantize_groups(xb, 4)
    got = quant.bf16_to_f32(quant.dequantize_groups(q, sb, zb))
    for g in range(0, 200, 7):
        s = Fraction(float(quant.bf16_to_f32(sb[g])))
        z = Fraction(float(quant.bf16_to_f32(zb[g])))
        for j in range(64):
            exact = int(q[g, j]) * s + z
            want = _exact_round_to_bits(_exact_round_to_bits(exact, 24), 8)
            assert Fraction(float(got[g, j])) == want


# ----------------------------------------- fp32 RoPE metadata (C4R4F) ---
def _rint_even(fr):
    lo = fr.numerator // fr.denominator
    rem = fr - lo
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and lo % 2 == 1):
        lo += 1
    return lo


def test_quantizer_f32meta_follows_stated_steps_and_is_nearest():
    """fp32 (scale, zero) [QuantMLA App. C.4/C.5]: s = fl32(fl32(hi-lo)/m),
    z = lo, q = clamp(rint(fl32(fl32(x-z)/s))), replayed step by step in exact
    rational arithmetic; every code is also the nearest reconstruction point
    up to the fp32 rounding of the quotient."""
    rng = np.random.default_rng(31)
    xb = np.concatenate([_groups_small_int(rng, 200),
                         quant.f32_to_bf16((rng.standard_normal((200, 64)) * 3).astype(np.float32))])
    q, s32, z32 = quant.quantize_groups_f32meta(xb, 4)
    assert s32.dtype == np.float32 and z32.dtype == np.float32
    m = 15
    xf = quant.bf16_to_f32(xb)
    for g in range(xb.shape[0]):
        lo, hi = Fraction(float(xf[g].min())), Fraction(float(xf[g].max()))
        s = _exact_round_to_bits(_exact_round_to_bits(hi - lo, 24) / m, 24) if hi != lo else Fraction(0)
        assert Fraction(float(s32[g])) == s and Fraction(float(z32[g])) == lo
        for j in range(64):
            x = Fraction(float(xf[g, j]))
            if s == 0:
                assert q[g, j] == 0
                continue
            t = _exact_round_to_bits(_exact_round_to_bits(x - lo, 24) / s, 24)
            assert q[g, j] == min(max(_rint_even(t), 0), m), (g, j)
            d = [abs(x - (k * s + lo)) for k in range(m + 1)]
            assert d[q[g, j]] <= min(d) + s * Fraction(1, 1 << 20), (g, j)


def test_dequant_f32meta_rounds_product_then_sum():
    """x^ = bf16(fl32(fl32(q*s) + z)): checked against exact rationals, and
    the two roundings differ from a single fused rounding on some inputs."""
    rng = np.random.default_rng(32)
    xb = quant.f32_to_bf16((rng.standard_normal((300, 64)) * 7 + 3).astype(np.float32))
    q, s32, z32 = quant.quantize_groups_f32meta(xb, 4)
    got = quant.bf16_to_f32(quant.dequantize_groups_f32meta(q, s32, z32))
    fused_differs = 0
    for g in range(300):
        s, z = Fraction(float(s32[g])), Fraction(float(z32[g]))
        for j in range(64):
            p = int(q[g, j]) * s
            want = _exact_round_to_bits(_exact_round_to_bits(_exact_round_to_bits(p, 24) + z, 24), 8)
            assert Fraction(float(got[g, j])) == want
            fused = _exact_round_to_bits(p + z, 24)
            fused_differs += fused != _exact_round_to_bits(_exact_round_to_bits(p, 24) + z, 24)
    assert fused_differs > 0      # the reading of the two roundings matters


def test_quantizer_f32meta_bound_and_exact_minimum():
    rng = np.random.default_rng(33)
    xb = quant.f32_to_bf16((rng.standard_normal((4000, 64)) * 2.5).astype(np.float32))
    q, s32, z32 = quant.quantize_groups_f32meta(xb, 4)
    x = quant.bf16_to_f32(xb).astype(np.float64)
    s = s32.astype(np.float64)
    recon = q * s[:, None] + z32.astype(np.float64)[:, None]
    assert np.all(np.abs(x - recon) <= 0.5 * s[:, None] * (1 + 1e-6))
    amin = x.argmin(axis=1)
    xh = quant.bf16_to_f32(quant.dequantize_groups_f32meta(q, s32, z32))
    assert np.all(xh[np.arange(len(q)), amin] == x[np.arange(len(q)), amin])
    # a constant group: s = 0, every code 0, exact reconstruction
    cb = quant.f32_to_bf16(np.full((2, 64), [[2.5], [-1.0]], dtype=np.float32))
    qc, sc, zc = quant.quantize_groups_f32meta(cb, 4)
    assert np.all(qc == 0) and np.all(sc == 0)
    np.testing.assert_array_equal(quant.dequantize_groups_f32meta(qc, sc, zc), cb)


def test_c4r4f_tokens_keep_content_as_c4r4():
    rng = np.random.default_rng(34)
    c = quant.f32_to_bf16(rng.standard_normal((16, 512)).astype(np.float32))
    kr = quant.f32_to_bf16(rng.standard_normal((16, 64)).astype(np.float32))
    a, b = quant.quantize_tokens(c, kr, "C4R4"), quant.quantize_tokens(c, kr, "C4R4F")
    np.testing.assert_array_equal(a["codes_c"], b["codes_c"])
    np.testing.assert_array_equal(a["scale"][:, :8], b["scale"][:, :8])
    np.testing.assert_array_equal(a["zero"][:, :8], b["zero"][:, :8])
    ra = quant.dequantize_tokens(a)
    rb = quant.dequantize_tokens(b)
    np.testing.assert_array_equal(ra[:, :512], rb[:, :512])
    # the RoPE rows agree with the fp32-metadata group routines
    q, s32, z32 = quant.quantize_groups_f32meta(kr, 4)
    np.testing.assert_array_equal(b["codes_r"], q)
    np.testing.assert_array_equal(rb[:, 512:], quant.dequantize_groups_f32meta(q, s32, z32))


def test_c4r4f_meta_bytes_known_answer():
    """RoPE dims 0..63 as values 0..63: s = fl32(63/15) = 4.2f, z = 0, stored
    little-endian fp32 at the slot's 8-byte meta_r entry."""
    import struct
    c = quant.f32_to_bf16(np.zeros((1, 512), np.float32))
    kr = quant.f32_to_bf16(np.arange(64, dtype=np.float32)[None, :])
    qt = quant.quantize_tokens(c, kr, "C4R4F")
    pages = np.zeros((1, layout.page_bytes("C4R4F")), np.uint8)
    layout.write_tokens(pages, np.array([5]), qt, "C4R4F")
    off = 16384 + 2048 + 2048 + 5 * 8
    assert bytes(pages[0, off:off + 8]) == struct.pack("<ff", np.float32(63.0) / np.float32(15.0), 0.0)
    assert bytes(pages[0, off:off + 8]).hex() == "6666864000000000"


# --------------------------------------------------------------- packing ---
def test_pack_known_answer_c4():
    codes = np.tile(np.arange(16, dtype=np.uint8), 32)[None, :]      # [1, 512]
    p = layout.pack_content(codes, "C4R4")                              # [1, 4, 64]
    want = np.tile(np.array([0x10, 0x32, 0x54, 0x76, 0x98, 0xBA, 0xDC, 0xFE], np.uint8), 8)
    for b in range(4):
        np.testing.assert_array_equal(p[0, b], want)
    r = layout.pack_rope(np.arange(64, dtype=np.uint8)[None, :] % 16)
    np.testing.assert_array_equal(r[0], want[:32])


def test_pack_known_answer_c2():
    # dim d carries code d % 4: in every 16-dim word the even dims hold
    # 0,2,0,2,... (bits 0..15 = 0x8888) and the odd dims 1,3,1,3,...
    # (bits 16..31 = 0xDDDD); little-endian bytes 88 88 DD DD.
    codes = np.tile(np.array([0, 1, 2, 3], np.uint8), 128)[None, :]
    p = layout.pack_content(codes, "C2R4")
    assert p.shape == (1, 2, 64)
    np.testing.assert_array_equal(p[0, 0], np.tile(np.array([0x88, 0x88, 0xDD, 0xDD], np.uint8), 16))
    np.testing.assert_array_equal(p[0, 1], p[0, 0])
    # one code: blk 1, dim 87 = word 5, odd dim of pair m = 3 -> bits 22-23
    # of word 5 -> byte 4*5 + 2, value 0xC0
    codes = np.zeros((1, 512), np.uint8)
    codes[0, 256 + 87] = 3
    p = layout.pack_content(codes, "C2R4")
    assert p[0, 1, 22] == 0xC0 and int(p.sum()) == 0xC0
    codes = np.zeros((1, 512), np.uint8)
    codes[0, 16 * 3 + 2 * 7] = 2            # blk 0, word 3, even dim m = 7 -> bits 14-15
    p = layout.pack_content(codes, "C2R4")
    assert p[0, 0, 4 * 3 + 1] == 0x80 and int(p.sum()) == 0x80


@pytest.mark.parametrize("fmt", ["C4R4", "C2R4", "C4R4F"])
def test_pack_roundtrip_and_page_roundtrip(fmt):
    rng = np.random.default_rng(4)
    T = 64
    c = quant.f32_to_bf16(rng.standard_normal((T, 512)).astype(np.float32))
    kr = quant.f32_to_bf16(rng.standard_normal((T, 64)).astype(np.float32))
    qt = quant.quantize_tokens(c, kr, fmt)
    np.testing.assert_array_equal(layout.unpack_content(layout.pack_content(qt["codes_c"], fmt), fmt),
                                  qt["codes_c"])
    np.testing.assert_array_equal(layout.unpack_rope(layout.pack_rope(qt["codes_r"])), qt["codes_r"])
    pb = layout.page_bytes(fmt)
    pages = np.zeros((3, pb), np.uint8)
    slots = 2 * 64 + rng.permutation(64)
    layout.write_tokens(pages, slots, qt, fmt)
    assert not pages[:2].any()
    back = layout.read_page(pages[2], fmt)
    inv = np.argsort(slots - 128)
    keys = ("codes_c", "codes_r", "scale", "zero")
    if fmt in quant.F32_ROPE:
        keys += ("scale_r32", "zero_r32")
    for k in keys:
        np.testing.assert_array_equal(back[k][slots - 128], qt[k])
    del inv


def test_page_sizes():
    assert layout.page_bytes("C4R4") == 20736
    assert layout.page_bytes("C2R4") == 12544
    assert layout.page_bytes("C4R4F") == 20992       # 328 B/token against the pages' 320
    assert layout.PROT_ROWS * 576 * 2 == 152064


# ------------------------------------------- page byte placement (known answer) ---
def _hand_token(fmt):
    """One token with hand-chosen codes and metadata (not from the quantizer):
    content code of dim d = (7d + 3) mod 16 (C4R4) or (3d + 1) mod 4 (C2R4),
    RoPE code of dim j = (5j + 1) mod 16, group g (0..7) scale bits 0x3C00+g
    and zero bits 0xBF80+g, RoPE group scale 0x3D11 and zero 0xC022."""
    d = np.arange(512)
    cc = (7 * d + 3) % 16 if fmt == "C4R4" else (3 * d + 1) % 4
    qt = {"codes_c": cc.astype(np.uint8)[None, :],
          "codes_r": ((5 * np.arange(64) + 1) % 16).astype(np.uint8)[None, :],
          "scale": np.array([[0x3C00 + g for g in range(8)] + [0x3D11]], np.uint16),
          "zero": np.array([[0xBF80 + g for g in range(8)] + [0xC022]], np.uint16)}
    return cc, qt


@pytest.mark.parametrize("fmt", ["C4R4", "C2R4"])
def test_page_byte_placement_known_answer(fmt):
    """A token written at slot 5 of page 1 lands at the absolute byte offsets
    the header's layout gives, computed here by hand: content block b at
    (b*64 + 5)*64, codes_r at OFF_R + 5*32, meta_c (scale, zero) of group g at
    OFF_MC + 5*32 + 4g (little-endian bf16 pairs), meta_r at OFF_MR + 5*4; no
    other byte of the pool changes."""
    cc, qt = _hand_token(fmt)
    pb = layout.page_bytes(fmt)
    pages = np.zeros((2, pb), np.uint8)
    layout.write_tokens(pages, np.array([64 + 5]), qt, fmt)
    assert not pages[0].any()
    pg = pages[1]
    want = np.zeros(pb, np.uint8)
    if fmt == "C4R4":
        OFF_R, OFF_MC, OFF_MR = 16384, 18432, 20480
        for b in range(4):                           # byte k: dims 128b+2k (lo), +2k+1 (hi)
            for k in range(64):
                want[(b * 64 + 5) * 64 + k] = cc[128 * b + 2 * k] | (cc[128 * b + 2 * k + 1] << 4)
        # spot values by hand: dims 0, 1 -> codes 3, 10 -> 0xA3; dims 384, 385
        # (block 3, byte 0) -> (2688+3)%16 = 3, (2695+3)%16 = 10 -> 0xA3;
        # dims 130, 131 (block 1, byte 1) -> 1, 8 -> 0x81
        assert pg[320] == 0xA3 and pg[(3 * 64 + 5) * 64] == 0xA3
        assert pg[(1 * 64 + 5) * 64 + 1] == 0x81
    else:
        OFF_R, OFF_MC, OFF_MR = 8192, 10240, 12288
        for b in range(2):                           # 32-bit word k: dims 256b+16k..+15
            for k in range(16):
                w = 0
                for m in range(8):
                    w |= int(cc[256 * b + 16 * k + 2 * m]) << (2 * m)
                    w |= int(cc[256 * b + 16 * k + 2 * m + 1]) << (16 + 2 * m)
                off = (b * 64 + 5) * 64 + 4 * k
                want[off:off + 4] = [w & 0xFF, (w >> 8) & 0xFF, (w >> 16) & 0xFF, w >> 24]
        # by hand: dims 0..15 carry codes 1,0,3,2,...: even dims 1,3,1,3 ->
        # 0xDDDD, odd dims 0,2,0,2 -> 0x8888; word 0x8888DDDD, bytes DD DD 88 88
        assert bytes(pg[320:324]) == bytes([0xDD, 0xDD, 0x88, 0x88])
    for k in range(32):                              # codes_r: dims 2k (lo), 2k+1 (hi)
        r0, r1 = (10 * k + 1) % 16, (10 * k + 6) % 16
        want[OFF_R + 5 * 32 + k] = r0 | (r1 << 4)
    assert pg[OFF_R + 160] == 0x61                   # RoPE dims 0, 1 -> codes 1, 6
    for g in range(8):
        s, z = 0x3C00 + g, 0xBF80 + g
        want[OFF_MC + 5 * 32 + 4 * g:OFF_MC + 5 * 32 + 4 * g + 4] = [s & 0xFF, s >> 8, z & 0xFF, z >> 8]
    want[OFF_MR + 20:OFF_MR + 24] = [0x11, 0x3D, 0x22, 0xC0]
    assert bytes(pg[OFF_MC + 160 + 12:OFF_MC + 160 + 16]) == bytes([0x03, 0x3C, 0x83, 0xBF])
    np.testing.assert_array_equal(pg, want)
    # and read_page, the oracle's inverse, returns the hand-chosen values
    back = layout.read_page(pg, fmt)
    for k in ("codes_c", "codes_r", "scale", "zero"):
        np.testing.assert_array_equal(back[k][5], qt[k][0])


# ------------------------------------- round-trip bounds on what is multiplied ---
@pytest.mark.parametrize("bits", [2, 4])
def test_roundtrip_bound_on_bf16_reconstruction(bits):
    """Two bounds, both asserted.  The quantizer's own round trip (exact
    q*s + z) stays within s/2 of x -- the per-element bound of the
    quantization itself.  The value the decode multiplies is the stored bf16
    reconstruction x^ = bf16(fl32(q*s + z)), which adds at most one fp32 and
    one bf16 rounding: |x - x^| <= s/2 + ulp_bf16(x^)/2 + 2^-24 |x^|.  The
    bf16 step alone can exceed s/2 (lo = 64, x = 64.5, hi = 76: s = 0.80078,
    q = 1, x^ = 65.0, error 0.5 > 0.40), so the first bound is not asserted
    on x^."""
    rng = np.random.default_rng(40 + bits)
    a = np.exp(0.5 * rng.standard_normal(64))
    a[:2] *= 16.0
    x64 = rng.standard_normal((20000, 64)) * a + rng.standard_normal((20000, 1)) * 40.0
    xb = quant.f32_to_bf16(x64.astype(np.float32))
    hand = quant.f32_to_bf16(np.array([[64.0, 64.5, 76.0] + [70.0] * 61], np.float32))
    xb = np.concatenate([hand, xb])
    q, sb, zb = quant.quantize_groups(xb, bits)
    x = quant.bf16_to_f32(xb).astype(np.float64)
    s = quant.bf16_to_f32(sb).astype(np.float64)[:, None]
    exact = q * s + quant.bf16_to_f32(zb).astype(np.float64)[:, None]
    assert np.all(np.abs(x - exact) <= 0.5 * s * (1 + 1e-6))
    xh = quant.bf16_to_f32(quant.dequantize_groups(q, sb, zb)).astype(np.float64)
    ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(xh), 1e-300))) - 7)
    assert np.all(np.abs(x - xh) <= 0.5 * s + 0.5 * ulp + np.abs(xh) * 2.0 ** -24)
    if bits == 4:                                    # the hand case, both ways
        assert xh[0, 1] == 65.0 and abs(x[0, 1] - xh[0, 1]) > 0.5 * s[0, 0]
    assert np.any(np.abs(x - xh)[1:] > 0.5 * s[1:])  # the bf16 step does matter
