"""Offline cache transformations that preserve full-precision attention (oracle).

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

What is computed, and where it is stated:

* RoPE path [QuantMLA App. C.2]: with R_P = blockdiag(R_i), R_i in SO(2)
  acting on frequency pair i, and S_P = blockdiag(s_i I_2), s_i > 0, keys
  become k R_P S_P and queries q R_P S_P^-1 (row vectors).  The positional
  score q k^T is unchanged, and because R_i, s_i I_2 and the positional
  rotation of pair i are all planar maps of the same plane, the transform
  commutes with RoPE at every position -- so it can be folded into the
  pre-RoPE projections.  Pairs are the interleaved (2i, 2i+1) layout the
  synthetic keys use.
* Statistics-only channel scaling [QuantMLA App. D.2, the SmoothQuant-style
  baseline]: per channel, a_j is the 99.9th-percentile absolute value and
  a~_j = max(a_j, 1e-8).  The candidate formula is missing from the extracted
  text; the reading taken is the SmoothQuant smoothing factor with activation
  statistics only, a~_j^alpha, by which the cached channel is divided:
      s_j = a~_j^(-alpha),  cache x_j * s_j,  compensation 1 / s_j
  (alpha = 0 is plain round-to-nearest).  RoPE statistics and scales are tied
  within each frequency pair: the pair's statistic is the larger of its two
  channels' [QuantMLA App. C.4, App. D.2].  The content cache is compensated
  in every consumer: queries become q / s (scores unchanged) and the
  aggregated latent is divided by s (the value route).  The RoPE key is
  compensated in the query only.
* Content path [QuantMLA §3.1, App. C.1]: the cache holds the latent in
  rotated and scaled coordinates, c' = c R_C S_C (row vectors), with R_C
  orthogonal and S_C = Diag(s_C) positive; every consumer of the latent is
  compensated.  In the absorbed decode form that is q' = q R_C S_C^-1 for the
  content query (so q' . c' = q R S^-1 S R^T c^T = q . c) and
  o = o' S_C^-1 R_C^T for the aggregated latent (o' = sum_i p_i c'_i =
  o R_C S_C).  Both keys and values come from the one shared latent, so the
  one transformed cache serves the score and the aggregation.  The fixed
  rotation taken here is the deterministic normalized Hadamard matrix of the
  QuaRot-style baseline [QuantMLA App. D.2], H_n = Sylvester's +-1 matrix of
  order n divided by sqrt(n); the learned Cayley-parameterised rotation of
  the method itself needs training data and is out of reach.
* Selection [QuantMLA App. D.2]: alpha is chosen from {0, 0.125, 0.25, 0.5,
  0.75, 1} by held-out normalized attention-output MSE, the content and RoPE
  caches calibrated separately with the other kept exact; a tie keeps the
  smaller alpha (the search includes 0 and favours it in a tie,
  [QuantMLA App. C.4]).
"""

import numpy as np

from . import attention, quant

ALPHAS = (0.0, 0.125, 0.25, 0.5, 0.75, 1.0)


def channel_stat(x, pct=99.9):
    """a_j: the pct-th percentile of |x[:, j]| over the calibration rows."""
    return np.percentile(np.abs(np.asarray(x, np.float64)), pct, axis=0)


def smooth_scales(a, alpha, pairs=False):
    """s_j = max(a_j, 1e-8)^(-alpha); with pairs, channels 2i and 2i+1 share
    the statistic max(a~_2i, a~_2i+1)."""
    at = np.maximum(np.asarray(a, np.float64), 1e-8)
    if pairs:
        m = np.maximum(at[0::2], at[1::2])
        at = np.repeat(m, 2)
    return at ** (-float(alpha))


def pair_transform(x, angles, scales):
    """x [n, 2P] row vectors times blockdiag(R_i s_i): pair i = (2i, 2i+1)
    rotated by angles[i] and scaled by scales[i] (one scale per pair)."""
    x = np.asarray(x, np.float64)
    c, s = np.cos(angles), np.sin(angles)
    xe, xo = x[:, 0::2], x[:, 1::2]
    out = np.empty_like(x)
    # row vector [xe, xo] times [[c, s], [-s, c]]
    out[:, 0::2] = (xe * c - xo * s) * scales
    out[:, 1::2] = (xe * s + xo * c) * scales
    return out


def scale_inputs(c_bits, kr_bits, q_lat_bits, q_rope_bits, s_c, s_r):
    """The bf16 cache rows and queries of the transformed model: content
    channels times s_c, RoPE channels times s_r, queries divided by them."""
    c = quant.f32_to_bf16((quant.bf16_to_f32(c_bits) * s_c).astype(np.float32))
    kr = quant.f32_to_bf16((quant.bf16_to_f32(kr_bits) * s_r).astype(np.float32))
    ql = quant.f32_to_bf16((quant.bf16_to_f32(q_lat_bits) / s_c).astype(np.float32))
    qr = quant.f32_to_bf16((quant.bf16_to_f32(q_rope_bits) / s_r).astype(np.float32))
    return c, kr, ql, qr


def decode_scaled(c_bits, kr_bits, q_lat_bits, q_rope_bits, fmt, scale, s_c, s_r,
                  quantized=("content", "rope")):
    """Attention over a cache whose content channels are multiplied by s_c and
    RoPE channels by s_r before storage (bf16), queries compensated by 1/s
    (bf16), output divided by s_c.  Only the paths named in `quantized` are
    read through the low-bit cache; the other keeps its bf16 values for every
    token.  s_c, s_r = 1 with both paths quantized is decode_sequence.

    returns (out [H,512], lse [H]) float64 in the original coordinates.
    """
    c, kr, ql, qr = scale_inputs(c_bits, kr_bits, q_lat_bits, q_rope_bits, s_c, s_r)
    rows = attention.effective_rows(c, kr, fmt)
    orig = quant.bf16_to_f32(np.concatenate([c, kr], 1)).astype(np.float64)
    if "content" not in quantized:
        rows[:, :quant.D_C] = orig[:, :quant.D_C]
    if "rope" not in quantized:
        rows[:, quant.D_C:] = orig[:, quant.D_C:]
    out, lse = attention.attend(quant.bf16_to_f32(ql).astype(np.float64),
                                quant.bf16_to_f32(qr).astype(np.float64), rows, scale)
    return out / s_c, lse


def exact_decode(c_bits, kr_bits, q_lat_bits, q_rope_bits, scale):
    """Attention over the untransformed bf16 cache with no quantization."""
    rows = quant.bf16_to_f32(np.concatenate([c_bits, kr_bits], 1)).astype(np.float64)
    return attention.attend(quant.bf16_to_f32(q_lat_bits).astype(np.float64),
                            quant.bf16_to_f32(q_rope_bits).astype(np.float64), rows, scale)


def nmse(out, ref):
    return float(np.sum((out - ref) ** 2) / np.sum(ref ** 2))


def select_alpha(calib_c, calib_kr, heldout, fmt, scale, path):
    """Choose alpha for one path ('content' or 'rope') from calibration rows'
    statistics, by mean held-out attention-output NMSE with the other path
    exact (scale 1).  heldout: list of (c_bits, kr_bits, q_lat_bits,
    q_rope_bits).  returns (alpha, {alpha: nmse}, scales)."""
    if path == "content":
        a = channel_stat(quant.bf16_to_f32(calib_c))
    else:
        a = channel_stat(quant.bf16_to_f32(calib_kr))
    ones_c, ones_r = np.ones(quant.D_C), np.ones(quant.D_R)
    errs = {}
    for al in ALPHAS:
        s = smooth_scales(a, al, pairs=(path == "rope"))
        s_c, s_r = (s, ones_r) if path == "content" else (ones_c, s)
        e = []
        for (c, kr, ql, qr) in heldout:
            ref, _ = exact_decode(c, kr, ql, qr, scale)
            out, _ = decode_scaled(c, kr, ql, qr, fmt, scale, s_c, s_r, quantized=(path,))
            e.append(nmse(out, ref))
        errs[al] = float(np.mean(e))
    best = min(ALPHAS, key=lambda al: (errs[al], al))
    return best, errs, smooth_scales(a, best, pairs=(path == "rope"))


def hadamard(n):
    """Normalized Hadamard matrix of order n (a power of two) by Sylvester's
    doubling: H_1 = [1], H_2m = [[H_m, H_m], [H_m, -H_m]], then / sqrt(n).
    Symmetric and orthogonal."""
    if n < 1 or n & (n - 1):
        raise ValueError("order must be a power of two")
    h = np.ones((1, 1))
    while h.shape[0] < n:
        h = np.block([[h, h], [h, -h]])
    return h / np.sqrt(n)


def rotate_inputs(c_bits, q_lat_bits, R, s_c=None):
    """The content cache rows and content queries of the transformed model,
    stored in bf16: c' = c R S, q' = q R S^-1 (S = Diag(s_c), identity when
    s_c is None).  RoPE keys and queries are untouched."""
    s_c = np.ones(quant.D_C) if s_c is None else np.asarray(s_c, np.float64)
    c = quant.bf16_to_f32(c_bits).astype(np.float64) @ R * s_c
    q = quant.bf16_to_f32(q_lat_bits).astype(np.float64) @ R / s_c
    return quant.f32_to_bf16(c.astype(np.float32)), quant.f32_to_bf16(q.astype(np.float32))


def unrotate_output(out, R, s_c=None):
    """Aggregated latent back in the original coordinates: o = o' S^-1 R^T."""
    s_c = np.ones(quant.D_C) if s_c is None else np.asarray(s_c, np.float64)
    return (np.asarray(out, np.float64) / s_c) @ R.T


def attend_rotated_exact(c, kr, q_lat, q_rope, scale, R, s_c=None):
    """The transformed cache in exact arithmetic (fp64, no bf16 storage, no
    quantization): attention over c' = c R S with queries q' = q R S^-1,
    output mapped back.  Equals attention over c for orthogonal R."""
    s_c = np.ones(quant.D_C) if s_c is None else np.asarray(s_c, np.float64)
    c2 = np.asarray(c, np.float64) @ R * s_c
    q2 = np.asarray(q_lat, np.float64) @ R / s_c
    rows = np.concatenate([c2, np.asarray(kr, np.float64)], axis=1)
    out, lse = attention.attend(q2, np.asarray(q_rope, np.float64), rows, scale)
    return unrotate_output(out, R, s_c), lse


def decode_rotated(c_bits, kr_bits, q_lat_bits, q_rope_bits, fmt, scale, R, s_c=None):
    """Decode over the low-bit cache of the transformed model: the rotated
    (and scaled) content rows are stored in bf16 and go through the format's
    quantizer like any cache row (protected tokens keep their bf16 rows); the
    output is mapped back to the original coordinates.

    returns (out [H,512], lse [H]) float64."""
    c2, q2 = rotate_inputs(c_bits, q_lat_bits, R, s_c)
    rows = attention.effective_rows(c2, kr_bits, fmt)
    out, lse = attention.attend(quant.bf16_to_f32(q2).astype(np.float64),
                                quant.bf16_to_f32(q_rope_bits).astype(np.float64), rows, scale)
    return unrotate_output(out, R, s_c), lse
