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
