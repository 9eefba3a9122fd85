"""Seeded synthetic workloads for low-bit MLA decode.

This module only draws inputs.  It holds none of the method's arithmetic
(no quantization, packing, protected-set logic or attention) and is shared by
the tests, the benchmark and the smoke check.  bf16 rounding of the drawn
values uses torch's own float32 -> bfloat16 conversion.

Recipe (per workload, numpy PCG64 seeded with 20260 + workload id unless a
seed is given; the draw order is fixed and listed in ``draw``):

* lengths: fixed, or integers uniform on an inclusive range, one per sequence;
* block tables: one random permutation of all physical pages, assigned to
  (sequence, logical block) in order; ``extra_blocks`` spare blocks per
  sequence are reserved for tokens appended later;
* per-channel content scale a_j = exp(0.5 * N(0,1)) for the 512 latent
  channels, then 4 distinct outlier channels whose scale is multiplied by the
  workload's outlier factor (8, or 16 for the 128-head 32K workload);
* content latent c = bf16(N(0,1) * a), drawn sequence by sequence;
* RoPE key: N(0,1) rotated to the token's position with base 10000 and
  interleaved pairs (2p, 2p+1), angle = pos * 10000^(-2p/64), then bf16;
* queries q_lat [H,512] and q_rope [H,64] ~ N(0, sd = 1/sqrt(192)), bf16,
  one set per query of the sequence (queries x H rows, query-major);
* softmax scale 1/sqrt(192).

The named workloads mirror the shapes the method is evaluated on
(DeepSeek-V2-Lite-shaped: 16 heads; DeepSeek-V2-shaped: 128 heads; d_c = 512,
d_R = 64, 64-token pages).  No public dataset is involved.
"""

import dataclasses
import math

import numpy as np

D_C = 512
D_R = 64
PAGE = 64


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    fmt: str                 # "C4R4", "C2R4" or "C4R4F"
    batch: int
    heads: int
    len_lo: int              # inclusive range of context lengths
    len_hi: int
    outlier_factor: float = 8.0
    n_outliers: int = 4
    append_steps: int = 0    # decode steps with one appended token per sequence
    seed: int = 0
    queries: int = 1         # new tokens per sequence that each ask a query

    @property
    def ragged(self):
        return self.len_lo != self.len_hi


WORKLOADS = {
    0: Workload("tiny_c4r4_b1_h16_l1k", "C4R4", 1, 16, 1024, 1024, seed=20260),
    1: Workload("v2lite_c4r4_b32_h16_l8k", "C4R4", 32, 16, 8192, 8192, seed=20261),
    2: Workload("longctx_c2r4_b64_h16_l16k_32k", "C2R4", 64, 16, 16384, 32768, seed=20262),
    3: Workload("v2_c4r4_b16_h128_l32k", "C4R4", 16, 128, 32768, 32768,
                outlier_factor=16.0, seed=20263),
    4: Workload("pressure_c4r4_b8_h128_l96k_128k", "C4R4", 8, 128, 98304, 131072,
                append_steps=8, seed=20264),
    # the V2-Lite shape in the fp32-RoPE-metadata format [QuantMLA App. C.4/C.5]
    5: Workload("v2lite_c4r4f_b32_h16_l8k", "C4R4F", 32, 16, 8192, 8192, seed=20265),
    # the V2-Lite shape with 8 new tokens per sequence, each asking a query
    # (a speculative-decoding verify step or a chunked-prefill tail)
    6: Workload("v2lite_c4r4_b32_h16_l8k_q8", "C4R4", 32, 16, 8192, 8192, seed=20266,
                queries=8),
    # a chunked-prefill step on the V2 shape: 256 new tokens per sequence,
    # each asking a query over its causal prefix of a 16K context
    7: Workload("v2_c4r4_b4_h128_l16k_chunk256", "C4R4", 4, 128, 16384, 16384, seed=20267,
                queries=256),
}

SOFTMAX_SCALE = 1.0 / math.sqrt(192.0)
QUERY_SD = 1.0 / math.sqrt(192.0)
ROPE_BASE = 10000.0


def to_bf16_bits(x):
    """float array -> uint16 bf16 bit patterns via torch's RNE conversion."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def rope_rotate(x, pos):
    """Rotate [n, 64] vectors to positions pos[n] (interleaved pairs, base 10000)."""
    p = np.arange(D_R // 2, dtype=np.float64)
    theta = ROPE_BASE ** (-2.0 * p / D_R)
    ang = np.asarray(pos, dtype=np.float64)[:, None] * theta[None, :]
    cs, sn = np.cos(ang), np.sin(ang)
    xe, xo = x[:, 0::2], x[:, 1::2]
    out = np.empty_like(x)
    out[:, 0::2] = xe * cs - xo * sn
    out[:, 1::2] = xe * sn + xo * cs
    return out


@dataclasses.dataclass
class Draw:
    """One drawn workload.  All bf16 tensors are uint16 bit patterns."""
    wl: Workload
    lens: np.ndarray            # int32 [B]   tokens cached before any append step
    block_table: np.ndarray     # int32 [B, max_blocks]
    num_pages: int
    c: list                     # per sequence uint16 [L_b + steps, 512]
    kr: list                    # per sequence uint16 [L_b + steps, 64]
    q_lat: np.ndarray           # uint16 [B, queries * H, 512] (query-major rows)
    q_rope: np.ndarray          # uint16 [B, queries * H, 64]
    scale: float = SOFTMAX_SCALE

    @property
    def B(self):
        return self.wl.batch

    @property
    def H(self):
        return self.wl.heads

    def slots(self, b, positions):
        positions = np.asarray(positions, dtype=np.int64)
        return self.block_table[b, positions // PAGE].astype(np.int64) * PAGE + positions % PAGE


def draw(wl, seed=None, lens=None, extra_tokens=None, shuffle_pages=True, spare_pages=0):
    """Draw a workload.

    Order of draws: lengths, page permutation, channel scales, outlier
    channels, then per sequence (c, k_R), then q_lat, q_rope.
    ``extra_tokens`` (default: wl.append_steps) rows are drawn past each
    sequence's length for later append steps; their pages are reserved.
    """
    rng = np.random.Generator(np.random.PCG64(wl.seed if seed is None else seed))
    B, H = wl.batch, wl.heads
    extra = wl.append_steps if extra_tokens is None else extra_tokens
    if lens is None:
        if wl.ragged:
            lens = rng.integers(wl.len_lo, wl.len_hi, size=B, endpoint=True)
        else:
            lens = np.full(B, wl.len_lo)
    lens = np.asarray(lens, dtype=np.int64)
    nblk = [-(-(int(L) + extra) // PAGE) for L in lens]
    max_blocks = max(max(nblk), 1)
    total = int(sum(nblk)) + spare_pages
    perm = rng.permutation(total) if shuffle_pages else np.arange(total)
    bt = np.full((B, max_blocks), -1, dtype=np.int32)
    k = 0
    for b in range(B):
        bt[b, :nblk[b]] = perm[k:k + nblk[b]]
        k += nblk[b]
    a = np.exp(0.5 * rng.standard_normal(D_C))
    outl = rng.choice(D_C, size=wl.n_outliers, replace=False)
    a[outl] *= wl.outlier_factor
    cs, krs = [], []
    for b in range(B):
        n = int(lens[b]) + extra
        c = rng.standard_normal((n, D_C)) * a[None, :]
        kr = rope_rotate(rng.standard_normal((n, D_R)), np.arange(n))
        cs.append(to_bf16_bits(c))
        krs.append(to_bf16_bits(kr))
    # query rows: queries x heads per sequence, query-major
    R = wl.queries * H
    q_lat = to_bf16_bits(rng.normal(0.0, QUERY_SD, size=(B, R, D_C)))
    q_rope = to_bf16_bits(rng.normal(0.0, QUERY_SD, size=(B, R, D_R)))
    return Draw(wl=wl, lens=lens.astype(np.int32), block_table=bt, num_pages=total,
                c=cs, kr=krs, q_lat=q_lat, q_rope=q_rope)


def small(fmt="C4R4", batch=2, heads=16, lens=(200, 77), seed=1, outlier_factor=8.0,
          extra_tokens=0, spare_pages=0, shuffle_pages=True, queries=1):
    """A small ad-hoc workload for tests (explicit lengths)."""
    wl = Workload("small", fmt, batch, heads, 0, 0, outlier_factor=outlier_factor, seed=seed,
                  queries=queries)
    return draw(wl, lens=np.asarray(lens), extra_tokens=extra_tokens,
                spare_pages=spare_pages, shuffle_pages=shuffle_pages)
