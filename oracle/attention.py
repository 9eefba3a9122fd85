"""Mixed-precision MLA decode attention, float64 (oracle).

What is computed, and where it is stated:

* Cache contents per token: the 512-d content latent c and the 64-d
  post-RoPE key k_R, 576 values [MLA blog §1, §3], [QuantMLA §2.1].
* Absorbed scoring: the content score of head h against token i is
  (W_UK^T q_h) . c_i, so the query is moved into latent space once and the
  RoPE score q_R,h . k_R,i is added separately [MLA blog §4].  The aggregated
  latent sum_i a_hi c_i is what the value/output projections consume
  [MLA blog §4]; those projections sit outside this path [QuantMLA App. C.5].
* Protected set [QuantMLA §3.3, App. C.5]: for a sequence of L tokens with
  zero-based positions, the first four (sink) and the most recent 128 tokens
  are read in their original BF16 form; the union is counted once; every other
  token is read from its packed copy.  The formula is missing from the
  extracted text; the reading taken is
      P_L = [0, min(4, L)) U [max(0, L - 128), L).
  Every token contributes exactly once; none is evicted or masked.
* One global softmax over all L tokens [QuantMLA §3.3].  When regions or
  splits are processed apart, each yields (m_j, s_j, o_j) = (max logit,
  sum of exp(logit - m_j), unnormalised sum of exp(logit - m_j) * value); the
  merge formula is missing from the extracted text and the standard
  log-sum-exp merge is used [QuantMLA App. C.5]:
      m = max_j m_j,  s = sum_j e^(m_j - m) s_j,  o = sum_j e^(m_j - m) o_j / s,
      lse = m + ln s.
  An empty part has m = -inf, s = 0 and contributes nothing.

The current decode token is part of the sequence: L counts it (append first,
then attend over [0, L)).

Several queries per sequence (decode_multi): the last nq tokens of a length-L
sequence each ask a query, the compute-friendly side of MLA attention
[MLA blog §7], and each sees only its causal prefix [MLA blog §8]: query j
(position L - nq + j) attends to [0, L - nq + 1 + j).  The rows every query
reads are those of the cache at length L -- the protected set P_L -- since
the cache holds no other state once the nq tokens are written.  (Reading
taken where the pages are silent; with nq = 1 it is decode_sequence.)
"""

import numpy as np

from . import quant
from .layout import N_SINK, N_RECENT


def protected_mask(L):
    """bool[L]: True where token i is in the protected set P_L."""
    i = np.arange(L)
    return (i < N_SINK) | (i >= L - N_RECENT)


def effective_rows(c_bits, kr_bits, fmt):
    """Rows each token contributes to attention, as float64 [L, 576].

    c_bits [L,512], kr_bits [L,64]: the original bf16 cache rows of one
    sequence in position order.  Protected tokens use these bf16 values;
    the others use the values reconstructed from their packed copy.
    """
    c_bits = np.asarray(c_bits, dtype=np.uint16)
    kr_bits = np.asarray(kr_bits, dtype=np.uint16)
    L = c_bits.shape[0]
    orig = np.concatenate([c_bits, kr_bits], axis=1)
    deq = quant.dequantize_tokens(quant.quantize_tokens(c_bits, kr_bits, fmt))
    rows = np.where(protected_mask(L)[:, None], orig, deq)
    return quant.bf16_to_f32(rows).astype(np.float64)


def scores(q_lat, q_rope, rows, scale):
    """Absorbed logits S[h, i] = scale * (q_lat[h] . c_i + q_rope[h] . k_R,i).

    q_lat [H,512], q_rope [H,64] (float64 or bf16-valued), rows [L,576].
    """
    ql = np.asarray(q_lat, dtype=np.float64)
    qr = np.asarray(q_rope, dtype=np.float64)
    rows = np.asarray(rows, dtype=np.float64)
    return scale * (ql @ rows[:, :quant.D_C].T + qr @ rows[:, quant.D_C:].T)


def attend(q_lat, q_rope, rows, scale):
    """Full softmax attention of H query heads over L rows.

    returns (out [H,512] float64 = sum_i p_hi c_i, lse [H] natural log).
    With L = 0 the output is 0 and lse is -inf.
    """
    H = np.asarray(q_lat).shape[0]
    rows = np.asarray(rows, dtype=np.float64)
    if rows.shape[0] == 0:
        return np.zeros((H, quant.D_C)), np.full(H, -np.inf)
    S = scores(q_lat, q_rope, rows, scale)
    m = S.max(axis=1, keepdims=True)
    e = np.exp(S - m)
    s = e.sum(axis=1, keepdims=True)
    out = (e @ rows[:, :quant.D_C]) / s
    lse = (m + np.log(s))[:, 0]
    return out, lse


def partial(q_lat, q_rope, rows, scale):
    """(m [H], s [H], o [H,512]) for one region/split; empty -> (-inf, 0, 0)."""
    H = np.asarray(q_lat).shape[0]
    rows = np.asarray(rows, dtype=np.float64)
    if rows.shape[0] == 0:
        return np.full(H, -np.inf), np.zeros(H), np.zeros((H, quant.D_C))
    S = scores(q_lat, q_rope, rows, scale)
    m = S.max(axis=1)
    e = np.exp(S - m[:, None])
    return m, e.sum(axis=1), e @ rows[:, :quant.D_C]


def merge(parts):
    """Merge partial triples by the log-sum-exp rule -> (out [H,512], lse [H])."""
    ms = np.stack([p[0] for p in parts])             # [J, H]
    m = ms.max(axis=0)                                # [H]
    H = m.shape[0]
    out = np.zeros((H, quant.D_C))
    s = np.zeros(H)
    finite = np.isfinite(m)
    for (mj, sj, oj) in parts:
        w = np.zeros(H)
        live = np.isfinite(mj)                        # empty parts weigh 0
        w[live] = np.exp(mj[live] - m[live])
        s += w * sj
        out += w[:, None] * oj
    with np.errstate(divide="ignore", invalid="ignore"):
        out = np.where(finite[:, None], out / s[:, None], 0.0)
        lse = np.where(finite, m + np.log(s), -np.inf)
    return out, lse


def decode_sequence(c_bits, kr_bits, q_lat_bits, q_rope_bits, fmt, scale):
    """Decode one sequence: bf16 cache rows [L,...] and bf16 queries [H,...].

    returns (out [H,512] float64, lse [H] float64).
    """
    rows = effective_rows(c_bits, kr_bits, fmt)
    ql = quant.bf16_to_f32(q_lat_bits).astype(np.float64)
    qr = quant.bf16_to_f32(q_rope_bits).astype(np.float64)
    return attend(ql, qr, rows, scale)


def decode_multi(c_bits, kr_bits, q_lat_bits, q_rope_bits, fmt, scale):
    """Attention of the last nq tokens of one sequence, each over its causal
    prefix, on the rows of the length-L cache.

    c_bits [L,512], kr_bits [L,64]; q_lat_bits [nq,H,512], q_rope_bits
    [nq,H,64] (bf16 bits).  returns (out [nq,H,512], lse [nq,H]) float64; a
    query whose prefix is empty gets 0 and -inf.
    """
    rows = effective_rows(c_bits, kr_bits, fmt)
    L = rows.shape[0]
    ql = quant.bf16_to_f32(q_lat_bits).astype(np.float64)
    qr = quant.bf16_to_f32(q_rope_bits).astype(np.float64)
    nq, H = ql.shape[0], ql.shape[1]
    out = np.zeros((nq, H, quant.D_C))
    lse = np.full((nq, H), -np.inf)
    for j in range(nq):
        n = L - nq + 1 + j                            # causal prefix of query j
        if n > 0:
            out[j], lse[j] = attend(ql[j], qr[j], rows[:n], scale)
    return out, lse
