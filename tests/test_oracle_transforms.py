"""Pins for oracle/transforms.py (CPU only).

Closed forms and identities: the per-pair rotation/scale commutes with the
positional rotation of the synthetic keys (an independent routine) and keeps
q.k; a dense cross-pair rotation does not (negative control).  Power-of-two
scales make the bf16 cache scaling exact, so the compensated attention
equals the untransformed one to fp64 rounding.  Hand-computed scales.  A
measured property: on outlier channels the held-out search picks alpha > 0
and lowers the attention-output error below plain round-to-nearest.
"""

import numpy as np
import pytest

from bit_mla_kv_quant_amd import synth
from oracle import quant, transforms


def test_pair_transform_commutes_with_rope_and_keeps_scores():
    rng = np.random.default_rng(0)
    n = 40
    k = rng.standard_normal((n, 64))
    q = rng.standard_normal((n, 64))
    pos = rng.integers(0, 100000, n)
    ang = rng.uniform(-np.pi, np.pi, 32)
    sc = np.exp(rng.uniform(-2, 2, 32))
    # transform before or after the positional rotation: same keys
    a = synth.rope_rotate(transforms.pair_transform(k, ang, sc), pos)
    b = transforms.pair_transform(synth.rope_rotate(k, pos), ang, sc)
    np.testing.assert_allclose(a, b, rtol=1e-11, atol=1e-11)
    # reciprocal compensation keeps every positional score
    kp = transforms.pair_transform(k, ang, sc)
    qp = transforms.pair_transform(q, ang, 1.0 / sc)
    np.testing.assert_allclose(qp @ kp.T, q @ k.T, rtol=1e-11, atol=1e-11)
    # negative control: a dense rotation across pairs does not commute
    Q, _ = np.linalg.qr(rng.standard_normal((64, 64)))
    assert np.max(np.abs(synth.rope_rotate(k @ Q, pos) - synth.rope_rotate(k, pos) @ Q)) > 1e-3


def test_smooth_scales_closed_form_and_pair_tying():
    s = transforms.smooth_scales([4.0, 1.0, 0.0, 16.0], 0.5)
    np.testing.assert_allclose(s, [0.5, 1.0, 1e4, 0.25], rtol=1e-12)
    assert np.all(transforms.smooth_scales([4.0, 1.0, 0.0, 16.0], 0.0) == 1.0)
    sp = transforms.smooth_scales([4.0, 1.0, 0.25, 16.0], 1.0, pairs=True)
    np.testing.assert_allclose(sp, [0.25, 0.25, 1 / 16, 1 / 16], rtol=1e-12)
    a = np.abs(np.random.default_rng(1).standard_normal(64)) + 0.1
    st = transforms.channel_stat(np.stack([a, -a, 0.5 * a]))
    np.testing.assert_allclose(st, a, rtol=1e-12)


def test_scaled_decode_preserves_attention_without_quantization():
    """All tokens protected (L <= 132): with power-of-two scales the bf16
    cache scaling is exact, so compensation must give back the untransformed
    attention to fp64 rounding."""
    d = synth.small(fmt="C4R4", batch=1, heads=4, lens=(120,), seed=2)
    rng = np.random.default_rng(2)
    s_c = 2.0 ** rng.integers(-6, 7, 512)
    s_r = np.repeat(2.0 ** rng.integers(-6, 7, 32), 2)
    out, lse = transforms.decode_scaled(d.c[0], d.kr[0], d.q_lat[0], d.q_rope[0], "C4R4",
                                        d.scale, s_c, s_r)
    ref, rl = transforms.exact_decode(d.c[0], d.kr[0], d.q_lat[0], d.q_rope[0], d.scale)
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(lse, rl, rtol=1e-12, atol=1e-12)


def _outlier_draw(seed, L, heads=4):
    d = synth.small(fmt="C4R4", batch=3, heads=heads, lens=(L, L, L), seed=seed,
                    outlier_factor=16.0)
    # RoPE outliers: four frequency pairs x16 in every key
    kr = [quant.bf16_to_f32(x).copy() for x in d.kr]
    for x in kr:
        for p in (3, 10, 17, 29):
            x[:, 2 * p:2 * p + 2] *= 16.0
    d.kr = [quant.f32_to_bf16(x.astype(np.float32)) for x in kr]
    return d


@pytest.mark.parametrize("path", ["content", "rope"])
def test_alpha_search_lowers_error_on_outlier_channels(path):
    d = _outlier_draw(seed=7, L=700)
    calib_c, calib_kr = d.c[0], d.kr[0]                  # statistics from sequence 0
    heldout = [(d.c[b], d.kr[b], d.q_lat[b], d.q_rope[b]) for b in (1, 2)]
    al, errs, s = transforms.select_alpha(calib_c, calib_kr, heldout, "C4R4", d.scale, path)
    assert al > 0.0, errs
    assert errs[al] < 0.9 * errs[0.0], errs
    if path == "rope":
        assert np.all(s[0::2] == s[1::2])


@pytest.mark.parametrize("path", ["content", "rope"])
def test_alpha_search_exact_tie_keeps_smallest_alpha(path):
    """[QuantMLA App. C.4]: a tie favours the smaller alpha.  Calibration rows
    whose every channel has statistic exactly 1 give the scale 1^-alpha = 1
    for every candidate, so all candidates tie exactly; the search must keep
    the smallest (0), not the first or last it tried."""
    rng = np.random.default_rng(5)
    d = synth.small(fmt="C4R4", batch=2, heads=4, lens=(300, 300), seed=5)
    calib_c = quant.f32_to_bf16(rng.choice([-1.0, 1.0], size=(200, 512)).astype(np.float32))
    calib_kr = quant.f32_to_bf16(rng.choice([-1.0, 1.0], size=(200, 64)).astype(np.float32))
    heldout = [(d.c[b], d.kr[b], d.q_lat[b], d.q_rope[b]) for b in (0, 1)]
    order = list(transforms.ALPHAS)
    for alphas in (order, order[::-1]):               # candidate order does not matter
        saved = transforms.ALPHAS
        transforms.ALPHAS = tuple(alphas)
        try:
            al, errs, s = transforms.select_alpha(calib_c, calib_kr, heldout, "C4R4", d.scale, path)
        finally:
            transforms.ALPHAS = saved
        assert len(set(errs.values())) == 1, errs    # an exact tie
        assert al == min(order) == 0.0
        assert np.all(s == 1.0)


# ------------------------------------------------- content-path rotation ---
def test_hadamard_matrix_against_library_and_closed_form():
    """Known answer H_2 = [[1, 1], [1, -1]] / sqrt(2); every order up to 512
    equals scipy's Sylvester Hadamard matrix / sqrt(n); orthogonal and
    symmetric."""
    import scipy.linalg
    np.testing.assert_array_equal(transforms.hadamard(2) * np.sqrt(2), [[1, 1], [1, -1]])
    for n in (1, 2, 4, 8, 64, 512):
        h = transforms.hadamard(n)
        np.testing.assert_allclose(h, scipy.linalg.hadamard(n) / np.sqrt(n), rtol=0, atol=1e-15)
        np.testing.assert_allclose(h @ h.T, np.eye(n), rtol=0, atol=1e-12)
        np.testing.assert_array_equal(h, h.T)
    with pytest.raises(ValueError):
        transforms.hadamard(48)


def _rotation_case(seed, L=300, H=8):
    rng = np.random.default_rng(seed)
    c = rng.standard_normal((L, 512)) * np.exp(0.5 * rng.standard_normal(512))
    kr = rng.standard_normal((L, 64))
    ql = rng.standard_normal((H, 512)) * 0.07
    qr = rng.standard_normal((H, 64)) * 0.07
    return c, kr, ql, qr


def test_content_rotation_preserves_attention_exactly():
    """[QuantMLA §3.1, App. C.1]: with every consumer compensated, an
    orthogonal rotation (the normalized Hadamard, and a random orthogonal
    matrix) times a positive channel scale leaves attention unchanged -- in
    exact arithmetic the transformed decode equals the plain one to fp64
    rounding, output and lse."""
    from oracle import attention
    rng = np.random.default_rng(11)
    c, kr, ql, qr = _rotation_case(11)
    rows = np.concatenate([c, kr], axis=1)
    ref, rl = attention.attend(ql, qr, rows, 0.07)
    Q, _ = np.linalg.qr(rng.standard_normal((512, 512)))
    for R in (transforms.hadamard(512), Q):
        for s_c in (None, np.exp(rng.uniform(-2, 2, 512))):
            out, lse = transforms.attend_rotated_exact(c, kr, ql, qr, 0.07, R, s_c)
            np.testing.assert_allclose(out, ref, rtol=1e-10, atol=1e-12)
            np.testing.assert_allclose(lse, rl, rtol=1e-12, atol=1e-12)


def test_content_rotation_negative_control_non_orthogonal():
    """A matrix that is not orthogonal (the Hadamard with one column scaled by
    1.1, or perturbed by 1e-2) does not preserve attention: the identity above
    is the orthogonality, not the bookkeeping."""
    from oracle import attention
    rng = np.random.default_rng(12)
    c, kr, ql, qr = _rotation_case(12)
    ref, _ = attention.attend(ql, qr, np.concatenate([c, kr], axis=1), 0.07)
    h = transforms.hadamard(512)
    bad1 = h.copy()
    bad1[:, 0] *= 1.1
    bad2 = h + 1e-2 * rng.standard_normal((512, 512))
    for R in (bad1, bad2):
        out, _ = transforms.attend_rotated_exact(c, kr, ql, qr, 0.07, R)
        assert transforms.nmse(out, ref) > 1e-6


def test_hadamard_rotation_lowers_int4_error_on_outlier_channels():
    """On a cache with x16 outlier content channels, the normalized Hadamard
    spreads each token's outliers over all 512 channels, so every 64-group
    has a smaller range and the INT4 attention-output NMSE (against exact
    attention over the original bf16 cache) drops well below plain
    round-to-nearest on the original coordinates."""
    from oracle import attention
    d = _outlier_draw(seed=7, L=700)
    h = transforms.hadamard(512)
    for b in (1, 2):
        ref, _ = transforms.exact_decode(d.c[b], d.kr[b], d.q_lat[b], d.q_rope[b], d.scale)
        o_rtn, _ = attention.decode_sequence(d.c[b], d.kr[b], d.q_lat[b], d.q_rope[b], "C4R4",
                                             d.scale)
        o_rot, _ = transforms.decode_rotated(d.c[b], d.kr[b], d.q_lat[b], d.q_rope[b], "C4R4",
                                             d.scale, h)
        e_rtn, e_rot = transforms.nmse(o_rtn, ref), transforms.nmse(o_rot, ref)
        assert e_rot < e_rtn / 3, (b, e_rtn, e_rot)
