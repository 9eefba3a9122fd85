"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Bars: packed page bytes and protection rows bit-exact; reconstructed bf16
rows bit-exact; attention output within 2e-3 relative L2 for every
(sequence, head) row -- and every (sequence, query, head) row with several
queries -- and log-sum-exp within 1e-3 absolute (fp32 accumulation of bf16
MFMA products with bf16 hi + lo attention weights).  Different split plans of
one call agree within 1e-5 per row and 1e-5 in log-sum-exp.
"""

import numpy as np
import pytest

from bit_mla_kv_quant_amd import synth
from oracle import attention, layout, quant

from gpu_helpers import GpuCache, oracle_decode, oracle_decode_mq, oracle_page, t_bf16, t_i32

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

TOL_OUT = 2e-3
TOL_LSE = 1e-3
TOL_SPLIT = 1e-5


def rel_l2_rows(a, b):
    """rel-L2 of each row (last axis: the 512 latent dims) of a against b."""
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    return np.linalg.norm(a - b, axis=-1) / np.maximum(np.linalg.norm(b, axis=-1), 1e-30)


def say(*a):
    print("[case]", *a, flush=True)


def check_decode(d, cache, out, lse, lens, which=None, fmt=None):
    """Every (sequence, head) row within TOL_OUT rel-L2 of the oracle and its
    lse within TOL_LSE; returns the worst row."""
    worst = 0.0
    for b in (range(d.B) if which is None else which):
        L = int(lens[b])
        ro, rl = oracle_decode(d, b, L, fmt)
        if L == 0:
            assert np.all(out[b] == 0) and np.all(np.isneginf(lse[b])), b
            continue
        e = rel_l2_rows(out[b], ro)
        worst = max(worst, float(e.max()))
        assert np.all(e <= TOL_OUT), (b, L, int(e.argmax()), float(e.max()))
        assert np.max(np.abs(lse[b] - rl)) <= TOL_LSE, (b, L, np.max(np.abs(lse[b] - rl)))
    return worst


# --------------------------------------------------------------- writer ---
@pytest.mark.parametrize("fmt", ["C4R4", "C2R4", "C4R4F"])
def test_append_pages_and_prot_bit_exact(fmt):
    d = synth.small(fmt=fmt, batch=3, heads=16, lens=(300, 77, 133), seed=3, spare_pages=2)
    say("append", fmt, d.lens.tolist())
    c = GpuCache(d)
    c.fill()
    torch.cuda.synchronize()
    pages = c.pages.cpu().numpy()
    for pid in range(d.num_pages):
        np.testing.assert_array_equal(pages[pid], oracle_page(d, pid, d.lens), err_msg=f"page {pid}")
    prot = c.prot.cpu().numpy().view(np.uint16)
    for b in range(d.B):
        L = int(d.lens[b])
        idx = np.nonzero(attention.protected_mask(L))[0]
        rows = layout.prot_row(idx)
        want = np.concatenate([d.c[b][idx], d.kr[b][idx]], axis=1)
        np.testing.assert_array_equal(prot[b, rows], want)
        unused = np.setdiff1d(np.arange(132), rows)
        assert not prot[b, unused].any()


@pytest.mark.parametrize("fmt", ["C4R4", "C2R4", "C4R4F"])
def test_dequant_dump_bit_exact(fmt):
    from bit_mla_kv_quant_amd import ops
    d = synth.small(fmt=fmt, batch=2, heads=16, lens=(256, 100), seed=4, outlier_factor=16.0)
    say("dequant_dump", fmt)
    c = GpuCache(d)
    c.fill()
    for pid in range(d.num_pages):
        got = ops.mla_lb_dequant_dump(fmt, c.pages, pid).cpu().numpy().view(np.uint16)
        page = oracle_page(d, pid, d.lens)
        want = quant.dequantize_tokens(layout.read_page(page, fmt))
        np.testing.assert_array_equal(got, want, err_msg=f"page {pid}")


@pytest.mark.parametrize("fmt", ["C4R4", "C2R4", "C4R4F"])
def test_dequant_edge_values(fmt):
    """Constant groups, tiny (subnormal-scale) ranges and huge ranges survive
    the GPU writer and reconstruction bit for bit."""
    from bit_mla_kv_quant_amd import ops
    d = synth.small(fmt=fmt, batch=1, heads=16, lens=(64,), seed=5)
    rng = np.random.default_rng(5)
    c = quant.bf16_to_f32(d.c[0]).copy()
    c[0, :] = 1.25                                   # constant groups
    c[1, :64] = 0.0
    c[2, :] = rng.standard_normal(512) * 1e-38       # subnormal ranges
    c[3, :] = rng.standard_normal(512) * 1e30        # huge values
    c[4, :64] = np.float32(2.0) ** -130
    d.c[0] = quant.f32_to_bf16(c.astype(np.float32))
    kr = quant.bf16_to_f32(d.kr[0]).copy()
    kr[5, :] = -3.0
    kr[6, :] = rng.standard_normal(64) * 1e-38       # subnormal RoPE range
    kr[7, :] = rng.standard_normal(64) * 1e30        # huge RoPE values
    d.kr[0] = quant.f32_to_bf16(kr.astype(np.float32))
    say("dequant_edge", fmt)
    g = GpuCache(d)
    g.fill()
    torch.cuda.synchronize()
    np.testing.assert_array_equal(g.pages.cpu().numpy()[d.block_table[0, 0]],
                                  oracle_page(d, d.block_table[0, 0], d.lens))
    got = ops.mla_lb_dequant_dump(fmt, g.pages, int(d.block_table[0, 0])).cpu().numpy().view(np.uint16)
    want = quant.dequantize_tokens(quant.quantize_tokens(d.c[0], d.kr[0], fmt))
    np.testing.assert_array_equal(got, want)


@pytest.mark.parametrize("fmt", ["C4R4", "C4R4F"])
@pytest.mark.parametrize("H", [16, 128])
def test_decode_huge_scale_groups(fmt, H):
    """Packed tokens whose content or RoPE group has a scale beyond the fp8
    conversion's range (s * 2^9 overflows fp32) take the per-code conversion
    in both decode kernels; the attention still matches the oracle (such a
    token takes nearly all the weight of heads whose score it dominates)."""
    d = synth.small(fmt=fmt, batch=2, heads=H, lens=(700, 1300), seed=61)
    rng = np.random.default_rng(61)
    c = quant.bf16_to_f32(d.c[0]).copy()
    c[300, 64:128] = rng.uniform(-1.0, 1.0, 64) * 1e37      # content group 1 of a packed token
    d.c[0] = quant.f32_to_bf16(c.astype(np.float32))
    kr = quant.bf16_to_f32(d.kr[1]).copy()
    kr[900, :] = rng.uniform(-1.0, 1.0, 64) * 1e37          # RoPE group of a packed token
    d.kr[1] = quant.f32_to_bf16(kr.astype(np.float32))
    say("huge_scale", fmt, H)
    g = GpuCache(d)
    g.fill()
    for ns in (0, 1):
        out, lse = g.decode(num_splits=ns)
        assert np.all(np.isfinite(out)) and np.all(np.isfinite(lse))
        for b in range(d.B):
            L = int(d.lens[b])
            ro, rl = oracle_decode(d, b, L)
            assert np.all(rel_l2_rows(out[b], ro) <= TOL_OUT), (b, rel_l2_rows(out[b], ro).max())
            # scores of ~1e35 are fp32 sums of 576 products that cancel: their
            # error is bounded by gamma_576 * sum |q_j x_j| (gamma_576 < 1e-4),
            # so the lse bar grows with that magnitude
            rows = attention.effective_rows(d.c[b][:L], d.kr[b][:L], fmt)
            q = quant.bf16_to_f32(np.concatenate([d.q_lat[b], d.q_rope[b]], axis=1)).astype(np.float64)
            mag = d.scale * (np.abs(q) @ np.abs(rows).T).max(axis=1)
            assert np.all(np.abs(lse[b] - rl) <= TOL_LSE + 1e-4 * mag), b


# --------------------------------------------------------------- decode ---
EDGE_LENS = (0, 1, 3, 4, 5, 63, 64, 65, 127, 128, 129, 131, 132, 133, 200, 1000)


@pytest.mark.parametrize("fmt", ["C4R4", "C2R4", "C4R4F"])
@pytest.mark.parametrize("H", [16, 32, 64, 80, 96, 112, 128])
def test_decode_edge_lengths(fmt, H):
    """Every edge length (empty, sinks only, page and recent-window
    boundaries) at head counts routed to the 16-row kernel (16-80) and to the
    128-row kernel (96, 112 padded to a 128-row block; 128), over 1, 3 and
    the automatic number of splits."""
    d = synth.small(fmt=fmt, batch=len(EDGE_LENS), heads=H, lens=EDGE_LENS, seed=H)
    say("decode_edge", fmt, H)
    c = GpuCache(d, seq_slots=np.random.default_rng(H).permutation(d.B))
    c.fill()
    for ns in (0, 1, 3):
        out, lse = c.decode(num_splits=ns)
        w = check_decode(d, c, out, lse, d.lens)
        say("  num_splits", ns, "worst rel-L2", f"{w:.2e}")


@pytest.mark.parametrize("fmt", ["C4R4", "C2R4", "C4R4F"])
def test_split_invariance_and_determinism(fmt):
    d = synth.small(fmt=fmt, batch=4, heads=16, lens=(2000, 1500, 640, 4096), seed=9)
    say("split_invariance", fmt)
    c = GpuCache(d)
    c.fill()
    # Every partition meets the oracle bar.  Partitions are not bitwise equal:
    # the weights enter the MFMAs as bf16 hi + lo pairs relative to each
    # split's reference maximum (about 2^-17 relative per weight), and the
    # split sums are added in another order, so plans agree to about 1e-6.
    ref_out, ref_lse = c.decode(num_splits=1)
    check_decode(d, c, ref_out, ref_lse, d.lens)
    for ns in (2, 7, 0, 64):
        out, lse = c.decode(num_splits=ns)
        w = check_decode(d, c, out, lse, d.lens)
        worst_split = 0.0
        for b in range(d.B):
            e = rel_l2_rows(out[b], ref_out[b])
            worst_split = max(worst_split, float(e.max()))
            assert np.all(e <= TOL_SPLIT), (ns, b, int(e.argmax()), float(e.max()))
        say("  num_splits", ns, "worst rel-L2 vs oracle", f"{w:.2e}",
            "vs one split", f"{worst_split:.2e}")
        assert np.max(np.abs(lse - ref_lse)) <= TOL_SPLIT
    # a fixed plan is deterministic
    for ns in (1, 0):
        o1, l1 = c.decode(num_splits=ns)
        o2, l2 = c.decode(num_splits=ns)
        assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


@pytest.mark.parametrize("fmt", ["C4R4", "C2R4"])
def test_split_invariance_128_rows(fmt):
    """The 128-row kernel under several split plans, including one split of
    141 pages (the block-table window refilled twice inside the page loop)
    and a sequence shorter than the recent window."""
    d = synth.small(fmt=fmt, batch=3, heads=128, lens=(9000, 3000, 130), seed=19)
    say("split_invariance 128 rows", fmt)
    c = GpuCache(d)
    c.fill()
    ref_out, ref_lse = c.decode(num_splits=1)
    check_decode(d, c, ref_out, ref_lse, d.lens)
    for ns in (3, 0, 70):
        out, lse = c.decode(num_splits=ns)
        w = check_decode(d, c, out, lse, d.lens)
        worst = max(float(rel_l2_rows(out[b], ref_out[b]).max()) for b in range(d.B))
        say("  num_splits", ns, "worst rel-L2 vs oracle", f"{w:.2e}", "vs one split", f"{worst:.2e}")
        assert worst <= TOL_SPLIT, (ns, worst)
        assert np.max(np.abs(lse - ref_lse)) <= TOL_SPLIT


def test_sharp_attention():
    """Queries scaled x8: peaked softmax still within tolerance."""
    d = synth.small(fmt="C4R4", batch=2, heads=16, lens=(3000, 777), seed=12)
    d.q_lat = quant.f32_to_bf16(quant.bf16_to_f32(d.q_lat) * 8)
    d.q_rope = quant.f32_to_bf16(quant.bf16_to_f32(d.q_rope) * 8)
    say("sharp")
    c = GpuCache(d)
    c.fill()
    out, lse = c.decode()
    check_decode(d, c, out, lse, d.lens)


@pytest.mark.parametrize("H", [16, 128])
def test_score_jumps(H):
    """Tokens whose score for one head lies far above everything before them
    (2^100 and 2^190 in weight, in the packed and the protected region): the
    running reference maximum must move without losing the earlier tokens."""
    d = synth.small(fmt="C4R4", batch=2, heads=H, lens=(1500, 900), seed=31)
    l2e = 1.4426950408889634

    def plant(b, pos, head, log2_score):
        q = quant.bf16_to_f32(d.q_lat[b, head]).astype(np.float64)
        alpha = log2_score / (np.linalg.norm(q) ** 2 * d.scale * l2e)
        d.c[b][pos] = quant.f32_to_bf16((alpha * q).astype(np.float32))
        d.kr[b][pos] = 0

    plant(0, 300, 0, 100.0)      # packed, far beyond the first chunk's maximum
    plant(0, 1200, 0, 190.0)     # packed, far beyond again
    plant(1, 890, H - 1, 120.0)  # protected recent-window row
    say("score_jumps", H)
    c = GpuCache(d)
    c.fill()
    for ns in (1, 0, 5):
        out, lse = c.decode(num_splits=ns)
        w = check_decode(d, c, out, lse, d.lens)
        say("  num_splits", ns, "worst rel-L2", f"{w:.2e}")


@pytest.mark.parametrize("fmt", ["C4R4", "C2R4", "C4R4F"])
@pytest.mark.parametrize("H", [16, 128])
def test_token_aging(fmt, H):
    """Append one token per step from L=1 to 300 and decode each step: a
    token's packed bytes never change after insertion, tokens leaving the
    recent window switch to their packed copy (the protection buffer's ring
    wraps past 132 rows), and every step matches, on both kernels."""
    steps = 300
    d = synth.small(fmt=fmt, batch=1, heads=H, lens=(0,), seed=21, extra_tokens=steps)
    say("token_aging", fmt, H)
    c = GpuCache(d)
    prev = None
    for L in range(1, steps + 1):
        c.append([0], [np.array([L - 1])], [L])
        out, lse = c.decode(lens=[L])
        ro, rl = oracle_decode(d, 0, L)
        assert np.all(rel_l2_rows(out[0], ro) <= TOL_OUT), L
        assert np.max(np.abs(lse[0] - rl)) <= TOL_LSE, L
        if L % 50 == 0:
            pages = c.pages.cpu().numpy()
            if prev is not None:
                # all slots written before the previous snapshot are unchanged
                for pos in range(prev[1]):
                    pid, off = d.block_table[0, pos // 64], pos % 64
                    for region in _slot_regions(fmt, off):
                        assert np.array_equal(pages[pid][region], prev[0][pid][region]), pos
            prev = (pages, L)


# ---------------------------------------------------- fused writer + decode ---
@pytest.mark.parametrize("fmt", ["C4R4", "C2R4", "C4R4F"])
@pytest.mark.parametrize("H", [16, 64, 96, 128])
def test_fused_step_equals_append_then_decode(fmt, H):
    """mla_decode_lowbit_append writes the same page bytes and protection
    rows as kv_quant_append of each sequence's newest token, and returns the
    same out / lse bit for bit as mla_decode_lowbit after it; both match the
    oracle.  Lengths cover the first token, sink edges, page edges, the
    recent-window edge, several splits and an empty sequence."""
    lens = np.array([1, 4, 5, 64, 65, 132, 133, 300, 1000, 0])
    d = synth.small(fmt=fmt, batch=len(lens), heads=H, lens=lens, seed=41)
    say("fused_step", fmt, H, lens.tolist())
    base = GpuCache(d, seq_slots=np.random.default_rng(H).permutation(d.B))
    # every sequence holds its first L-1 tokens
    base.append(list(range(d.B)), [np.arange(max(L - 1, 0)) for L in lens],
                [max(L - 1, 0) for L in lens])
    torch.cuda.synchronize()
    for ns in (0, 1, 3):
        sep, fus = base.clone(), base.clone()
        sep.append([b for b in range(d.B) if lens[b] > 0],
                   [np.array([L - 1]) for L in lens if L > 0], [L for L in lens if L > 0])
        o1, l1 = sep.decode(lens=lens, num_splits=ns)
        o2, l2 = fus.fused_step(lens, num_splits=ns)
        np.testing.assert_array_equal(fus.pages.cpu().numpy(), sep.pages.cpu().numpy())
        np.testing.assert_array_equal(fus.prot.cpu().numpy(), sep.prot.cpu().numpy())
        np.testing.assert_array_equal(o2, o1)
        np.testing.assert_array_equal(l2, l1)
        w = check_decode(d, fus, o2, l2, lens)
        say("  num_splits", ns, "worst rel-L2", f"{w:.2e}")
    pages = fus.pages.cpu().numpy()
    for pid in range(d.num_pages):
        np.testing.assert_array_equal(pages[pid], oracle_page(d, pid, lens), err_msg=f"page {pid}")


@pytest.mark.parametrize("H", [16, 128])
def test_fused_step_skips_lengths_beyond_bound(H):
    """A fused call whose seq_lens[b] is max_seq_len + 1 stores nothing for
    that sequence (the clamped last token is already cached): its page bytes
    and protection rows are unchanged, and the whole call equals
    kv_quant_append of the in-bound sequence's token followed by
    mla_decode_lowbit with the same lengths, bit for bit."""
    d = synth.small(fmt="C4R4", batch=2, heads=H, lens=(300, 700), seed=73, extra_tokens=300)
    say("fused beyond bound", H)
    base = GpuCache(d)
    base.fill()
    torch.cuda.synchronize()
    lens = np.array([301, 701])
    for ns in (0, 1):
        sep, fus = base.clone(), base.clone()
        sep.append([0], [np.array([300])], [301])
        o1, l1 = sep.decode(lens=lens, num_splits=ns, max_seq_len=700)
        o2, l2 = fus.fused_step(lens, num_splits=ns, max_seq_len=700)
        np.testing.assert_array_equal(fus.pages.cpu().numpy(), sep.pages.cpu().numpy())
        np.testing.assert_array_equal(fus.prot.cpu().numpy(), sep.prot.cpu().numpy())
        np.testing.assert_array_equal(fus.prot.cpu().numpy()[1], base.prot.cpu().numpy()[1])
        np.testing.assert_array_equal(o2, o1)
        np.testing.assert_array_equal(l2, l1)
        check_decode(d, fus, o2, l2, [301, 700])


@pytest.mark.parametrize("fmt", ["C4R4", "C2R4"])
def test_fused_token_aging(fmt):
    """One fused step per token from L=1 to 260: every step matches the
    oracle, and the pages end byte-identical to the oracle's."""
    steps = 260
    d = synth.small(fmt=fmt, batch=2, heads=16, lens=(0, 0), seed=23, extra_tokens=steps)
    say("fused_token_aging", fmt)
    c = GpuCache(d)
    for L in range(1, steps + 1):
        out, lse = c.fused_step([L, L])
        check_decode(d, c, out, lse, [L, L])
    pages = c.pages.cpu().numpy()
    for pid in range(d.num_pages):
        np.testing.assert_array_equal(pages[pid], oracle_page(d, pid, [steps, steps]))


# ------------------------------------------------ several queries per sequence ---
def check_decode_mq(d, out, lse, lens, which=None, fmt=None):
    worst = 0.0
    for b in (range(d.B) if which is None else which):
        L = int(lens[b])
        ro, rl = oracle_decode_mq(d, b, L, fmt)
        for j in range(d.wl.queries):
            if L - d.wl.queries + 1 + j <= 0:      # empty causal prefix
                assert np.all(out[b, j] == 0) and np.all(np.isneginf(lse[b, j])), (b, j)
                continue
            e = rel_l2_rows(out[b, j], ro[j])
            worst = max(worst, float(e.max()))
            assert np.all(e <= TOL_OUT), (b, L, j, int(e.argmax()), float(e.max()))
            assert np.max(np.abs(lse[b, j] - rl[j])) <= TOL_LSE, (b, L, j)
    return worst


@pytest.mark.parametrize("seed", [2027, 2030, 2041, 2077])
def test_randomized_sweep(seed):
    """Sixteen random calls per fixed seed: format, heads (16-row and 128-row
    kernels), queries per sequence, ragged lengths from 0 to 6000 (sink, page
    and window edges among them), split count, shuffled sequence slots,
    outlier strength and query scale.  Every row against the oracle."""
    rng = np.random.default_rng(seed)
    edge = [0, 1, 4, 5, 64, 132, 133, 197]
    for case in range(16):
        fmt = str(rng.choice(["C4R4", "C2R4", "C4R4F"]))
        H = int(rng.choice([16, 32, 48, 64, 96, 128]))
        nq = int(rng.choice([1, 1, 2, 3]))
        B = int(rng.integers(1, 7))
        lens = np.where(rng.random(B) < 0.3, rng.choice(edge, B), rng.integers(1, 6001, B))
        ns = int(rng.choice([0, 0, 1, int(rng.integers(2, 10))]))
        qscale = float(rng.choice([1.0, 3.0]))
        # one spare page: a batch of empty sequences still has a page pool
        d = synth.small(fmt=fmt, batch=B, heads=H, lens=lens, queries=nq,
                        seed=3000 + 100 * (seed - 2027) + case,
                        outlier_factor=float(rng.choice([1.0, 8.0, 16.0])), spare_pages=1)
        if qscale != 1.0:
            d.q_lat = quant.f32_to_bf16(quant.bf16_to_f32(d.q_lat) * qscale)
            d.q_rope = quant.f32_to_bf16(quant.bf16_to_f32(d.q_rope) * qscale)
        say("sweep", case, fmt, "H", H, "nq", nq, "splits", ns, "q x", qscale, lens.tolist())
        c = GpuCache(d, seq_slots=rng.permutation(B))
        c.fill()
        if nq == 1:
            out, lse = c.decode(num_splits=ns)
            w = check_decode(d, c, out, lse, lens)
        else:
            out, lse = c.decode_mq(num_splits=ns)
            w = check_decode_mq(d, out, lse, lens)
        say("  worst rel-L2", f"{w:.2e}")


@pytest.mark.parametrize("fmt", ["C4R4", "C2R4", "C4R4F"])
@pytest.mark.parametrize("nq,H", [(1, 16), (2, 16), (3, 32), (4, 16), (2, 48), (3, 48), (8, 16), (2, 128),
                                  (11, 16), (5, 48)])
def test_multi_query_decode(fmt, nq, H):
    """nq queries per sequence, each over its causal prefix, against the
    oracle; lengths below nq (empty prefixes), at sink / page / window edges
    and over several splits.  Up to 80 rows and 144 rows take the 16-row
    kernel; 96 and 128 rows take the 128-row one, 2 x 48 = 96 rows padded to
    128 with a query boundary inside the block; 176 and 240 rows take two
    128-row blocks with the second padded, and at 5 x 48 the third query's
    heads straddle the two blocks; nq = 1 must equal mla_decode_lowbit."""
    lens = np.array([1, 3, 8, 9, 64, 65, 133, 140, 300, 1000])
    d = synth.small(fmt=fmt, batch=len(lens), heads=H, lens=lens, seed=51 + nq, queries=nq)
    say("multi_query", fmt, nq, H, lens.tolist())
    c = GpuCache(d, seq_slots=np.random.default_rng(nq).permutation(d.B))
    c.fill()
    for ns in (0, 1, 3):
        out, lse = c.decode_mq(num_splits=ns)
        w = check_decode_mq(d, out, lse, lens)
        say("  num_splits", ns, "worst rel-L2", f"{w:.2e}")
        if nq == 1:
            o1, l1 = c.decode(num_splits=ns)
            np.testing.assert_array_equal(out[:, 0], o1)
            np.testing.assert_array_equal(lse[:, 0], l1)


@pytest.mark.parametrize("nq,H", [(8, 128), (64, 16), (256, 16), (512, 128)])
def test_multi_query_prefill_chunks(nq, H):
    """Chunked prefill at real chunk sizes: nq new tokens per sequence, each
    asking a query over its causal prefix, up to the largest call
    (512 x 128 = 65536 query rows per sequence, MLA_LB_MAX_ROWS); lengths
    shorter than the chunk (empty prefixes), around the window edge and
    longer; every row against the oracle, single-split and split."""
    lens = np.array([70, 133, 600]) if nq * H <= 1024 else np.array([300, nq + 133, 2000])
    d = synth.small(fmt="C4R4", batch=len(lens), heads=H, lens=lens, seed=82 + nq, queries=nq)
    say("prefill chunk", nq, H, lens.tolist())
    c = GpuCache(d)
    c.fill()
    for ns in (0, 1):
        out, lse = c.decode_mq(num_splits=ns)
        w = check_decode_mq(d, out, lse, lens)
        say("  num_splits", ns, "worst rel-L2", f"{w:.2e}")
        del out, lse


@pytest.mark.parametrize("H", [16, 128])
def test_many_sequences(H):
    """1024 sequences of 0-199 tokens in one call (grid of 1024 sequences,
    shuffled cache slots): 48 sampled sequences, the empty one and those at
    the window edges among them, against the oracle."""
    rng = np.random.default_rng(83)
    lens = rng.integers(1, 200, size=1024)
    lens[:5] = [0, 1, 4, 132, 133]
    d = synth.small(fmt="C4R4", batch=len(lens), heads=H, lens=lens, seed=83 + H)
    say("many sequences", H, len(lens))
    c = GpuCache(d, seq_slots=rng.permutation(d.B))
    c.fill()
    which = sorted(set(range(5)) | set(rng.choice(len(lens), 43, replace=False).tolist()))
    for ns in (0, 1):
        out, lse = c.decode(num_splits=ns)
        w = check_decode(d, c, out, lse, lens, which=which)
        say("  num_splits", ns, "worst rel-L2", f"{w:.2e}")


@pytest.mark.parametrize("nq", [2, 8])
def test_multi_query_score_jumps(nq):
    """Score jumps with several queries: a token far above everything before
    it for one query row, planted where some rows' causal prefixes end before
    it (the last token) or include it (a packed token); the running reference
    of each row moves independently."""
    H = 16
    d = synth.small(fmt="C4R4", batch=2, heads=H, lens=(1500, 900), seed=33, queries=nq)
    l2e = 1.4426950408889634

    def plant(b, pos, row, log2_score):
        q = quant.bf16_to_f32(d.q_lat[b, row]).astype(np.float64)
        alpha = log2_score / (np.linalg.norm(q) ** 2 * d.scale * l2e)
        d.c[b][pos] = quant.f32_to_bf16((alpha * q).astype(np.float32))
        d.kr[b][pos] = 0

    plant(0, 400, 0, 100.0)                 # packed; query 0, head 0
    plant(0, 1499, (nq - 1) * H + 3, 150.0)  # the last token: only the last query sees it
    plant(1, 850, H + 5, 120.0)              # protected window row; query 1, head 5
    say("multi_query_score_jumps", nq)
    c = GpuCache(d)
    c.fill()
    for ns in (1, 0, 5):
        out, lse = c.decode_mq(num_splits=ns)
        w = check_decode_mq(d, out, lse, d.lens)
        say("  num_splits", ns, "worst rel-L2", f"{w:.2e}")


def test_config6_multi_query_v2lite():
    wl = synth.WORKLOADS[6]
    say("config 6", wl.name, "drawing")
    d = synth.draw(wl)
    c = GpuCache(d)
    c.fill()
    out, lse = c.decode_mq()
    w = check_decode_mq(d, out, lse, d.lens, which=[0, 31])
    say("config 6 worst rel-L2 on sampled sequences", f"{w:.2e}")


def _slot_regions(fmt, off):
    nblk = 2 if fmt == "C2R4" else 4
    mr = 8 if fmt == "C4R4F" else 4                  # RoPE (scale, zero) bytes
    base_r = 64 * 64 * nblk
    out = [slice((b * 64 + off) * 64, (b * 64 + off) * 64 + 64) for b in range(nblk)]
    out.append(slice(base_r + off * 32, base_r + off * 32 + 32))
    out.append(slice(base_r + 2048 + off * 32, base_r + 2048 + off * 32 + 32))
    out.append(slice(base_r + 4096 + off * mr, base_r + 4096 + off * mr + mr))
    return out


# ------------------------------------------------------ full-size configs ---
def _full_config(cfg, sample_b):
    wl = synth.WORKLOADS[cfg]
    say("config", cfg, wl.name, "drawing")
    d = synth.draw(wl)
    c = GpuCache(d)
    say("config", cfg, "filling", int(d.lens.sum()), "tokens")
    c.fill()
    say("config", cfg, "decoding")
    out, lse = c.decode()
    w = check_decode(d, c, out, lse, d.lens, which=sample_b)
    say("config", cfg, "worst rel-L2 on sampled sequences", f"{w:.2e}")
    # sampled pages bit-exact
    pages = c.pages.cpu().numpy()
    rng = np.random.default_rng(cfg)
    for pid in rng.choice(d.num_pages, size=4, replace=False):
        np.testing.assert_array_equal(pages[pid], oracle_page(d, pid, d.lens))
    return d, c


def test_config0_tiny():
    _full_config(0, sample_b=[0])


def test_config1_v2lite():
    _full_config(1, sample_b=[0, 17, 31])


def test_config2_c2r4_long():
    _full_config(2, sample_b=[0, 33, 63])


def test_config3_v2_h128():
    _full_config(3, sample_b=[0, 15])


def test_config2_fused_step():
    """The long-context C2R4 workload as the bench runs it: every sequence
    holds its first L-1 tokens, and one fused call stores token L-1 and
    decodes; sampled sequences against the oracle, the written pages
    byte-identical to the oracle's."""
    wl = synth.WORKLOADS[2]
    say("config 2 fused", wl.name, "drawing")
    d = synth.draw(wl)
    c = GpuCache(d)
    lens = d.lens.astype(np.int64)
    c.append(list(range(d.B)), [np.arange(L - 1) for L in lens], [L - 1 for L in lens])
    out, lse = c.fused_step(lens)
    w = check_decode(d, c, out, lse, lens, which=[0, 31, 63])
    say("config 2 fused worst rel-L2 on sampled sequences", f"{w:.2e}")
    pages = c.pages.cpu().numpy()
    for b in (0, 63):
        pid = d.block_table[b, (lens[b] - 1) // 64]
        np.testing.assert_array_equal(pages[pid], oracle_page(d, pid, lens))


def test_config5_v2lite_fp32_rope_metadata():
    _full_config(5, sample_b=[0, 31])


def test_config4_pressure_with_append_steps():
    d, c = _full_config(4, sample_b=[0])
    lens = d.lens.astype(np.int64).copy()
    for step in range(d.wl.append_steps):
        lens += 1
        if step % 2 == 0:                          # writer, then decode
            c.append(list(range(d.B)), [np.array([L - 1]) for L in lens], list(lens))
            out, lse = c.decode(lens=lens)
        else:                                      # the fused step
            out, lse = c.fused_step(lens)
        if step in (0, 1, d.wl.append_steps - 1):
            w = check_decode(d, c, out, lse, lens, which=[0, d.B - 1])
            say("config 4 step", step, "worst rel-L2", f"{w:.2e}")
    pages = c.pages.cpu().numpy()
    for b in (0, d.B - 1):
        for pid in np.unique(d.block_table[b, (lens[b] - d.wl.append_steps) // 64:(lens[b] - 1) // 64 + 1]):
            np.testing.assert_array_equal(pages[pid], oracle_page(d, pid, lens))


# ------------------------------------------- offline-calibrated cache scales ---
def test_calibrated_scales_through_kernels():
    """Statistics-only channel scales (library host helpers) applied to a
    cache with x16 outlier channels and RoPE pairs, as a model with the
    scales folded into its projections would produce it; the kernels run
    unchanged.  The decode of the scaled cache matches the oracle on the
    same inputs, and after compensation it is closer to full-precision
    attention than the decode of the unscaled cache."""
    from bit_mla_kv_quant_amd import ops
    from oracle import transforms
    from test_oracle_transforms import _outlier_draw
    d = _outlier_draw(seed=7, L=700, heads=16)
    s_c = ops.mla_lb_smooth_scales(ops.mla_lb_channel_stat(d.c[0]), 0.5).astype(np.float64)
    s_r = ops.mla_lb_smooth_scales(ops.mla_lb_channel_stat(d.kr[0]), 0.75, True).astype(np.float64)
    say("calibrated scales")
    plain = GpuCache(d)
    plain.fill()
    o_rtn, _ = plain.decode()

    def bf16(x):
        return quant.f32_to_bf16(np.asarray(x, np.float32))
    t = synth.small(fmt="C4R4", batch=3, heads=16, lens=tuple(d.lens), seed=7)
    t.c = [bf16(quant.bf16_to_f32(x) * s_c) for x in d.c]
    t.kr = [bf16(quant.bf16_to_f32(x) * s_r) for x in d.kr]
    t.q_lat = bf16(quant.bf16_to_f32(d.q_lat) / s_c)
    t.q_rope = bf16(quant.bf16_to_f32(d.q_rope) / s_r)
    t.block_table, t.num_pages = d.block_table, d.num_pages
    scaled = GpuCache(t)
    scaled.fill()
    o_sc, l_sc = scaled.decode()
    check_decode(t, scaled, o_sc, l_sc, t.lens)          # parity on the scaled inputs
    for b in (1, 2):                                      # held-out sequences
        ref, _ = transforms.exact_decode(d.c[b], d.kr[b], d.q_lat[b], d.q_rope[b], d.scale)
        e_rtn = transforms.nmse(o_rtn[b], ref)
        e_sc = transforms.nmse(o_sc[b] / s_c, ref)
        say(f"  seq {b}: NMSE plain {e_rtn:.2e}, scaled {e_sc:.2e}")
        assert e_sc < e_rtn / 3, (e_rtn, e_sc)


@pytest.mark.parametrize("H", [16, 128])
def test_hadamard_rotated_cache_through_kernels(H):
    """The content-path rotation [QuantMLA §3.1, App. C.1] in its fixed
    normalized-Hadamard form [QuantMLA App. D.2], applied with the library's
    host helper as a model with the rotation folded into its projections
    would produce the cache: latent rows and content queries times H, the
    RoPE path unchanged.  The kernels run unchanged: the decode of the
    rotated cache matches the oracle on the same inputs, and mapped back
    (o' H) it is closer to full-precision attention than the decode of the
    unrotated cache on x16 outlier channels."""
    from bit_mla_kv_quant_amd import ops
    from oracle import transforms
    from test_oracle_transforms import _outlier_draw
    d = _outlier_draw(seed=7, L=700, heads=H)
    say("hadamard rotation", H)
    plain = GpuCache(d)
    plain.fill()
    o_rtn, _ = plain.decode()

    def rot_bf16(bits):
        flat = quant.bf16_to_f32(bits).reshape(-1, 512)
        return quant.f32_to_bf16(ops.mla_lb_hadamard_rows(flat)).reshape(np.shape(bits))
    t = synth.small(fmt="C4R4", batch=3, heads=H, lens=tuple(d.lens), seed=7)
    t.c = [rot_bf16(x) for x in d.c]
    t.kr = d.kr
    t.q_lat = rot_bf16(d.q_lat)
    t.q_rope = d.q_rope
    t.block_table, t.num_pages = d.block_table, d.num_pages
    # the helper's rotation is the oracle's (inputs of both sides agree)
    h = transforms.hadamard(512)
    want_c, want_q = transforms.rotate_inputs(d.c[1], d.q_lat[1], h)
    assert np.mean(t.c[1] != want_c) < 1e-3 and np.mean(t.q_lat[1] != want_q) < 1e-3
    rot = GpuCache(t)
    rot.fill()
    o_rot, l_rot = rot.decode()
    check_decode(t, rot, o_rot, l_rot, t.lens)           # parity on the rotated inputs
    for b in (1, 2):
        ref, _ = transforms.exact_decode(d.c[b], d.kr[b], d.q_lat[b], d.q_rope[b], d.scale)
        back = ops.mla_lb_hadamard_rows(o_rot[b].astype(np.float32)).astype(np.float64)
        e_rtn, e_rot = transforms.nmse(o_rtn[b], ref), transforms.nmse(back, ref)
        say(f"  seq {b}: NMSE plain {e_rtn:.2e}, rotated {e_rot:.2e}")
        assert e_rot < e_rtn / 3, (e_rtn, e_rot)


# ------------------------------------------------------------ HIP graphs ---
@pytest.mark.parametrize("H", [16, 128])
def test_graph_replay_matches_eager(H):
    """The split decode (workspace and combine inside the graph) and the fused
    step captured in HIP graphs, the launch mode the benchmark times: six
    replays each, with eager calls on the same workspace, buffer fills and
    host synchronisations between them, every replay bit-identical to the
    eager call (outputs, and for the fused step the page bytes and
    protection rows)."""
    from bit_mla_kv_quant_amd import ops
    lens = np.array([700, 1000, 133, 5])
    d = synth.small(fmt="C4R4", batch=len(lens), heads=H, lens=lens, seed=91)
    say("graph replay", H)
    c = GpuCache(d)
    c.fill()
    ql, qr, tl = t_bf16(d.q_lat), t_bf16(d.q_rope), t_i32(lens)
    lat = t_bf16(np.stack([d.c[b][L - 1] for b, L in enumerate(lens)]))
    kr = t_bf16(np.stack([d.kr[b][L - 1] for b, L in enumerate(lens)]))
    msl, ns = int(lens.max()), 3
    ws = torch.empty(ops.mla_decode_lowbit_workspace("C4R4", d.B, H, msl, ns),
                     dtype=torch.uint8, device=c.pages.device)
    out = torch.empty((d.B, H, 512), dtype=torch.float32, device=c.pages.device)
    lse = torch.empty((d.B, H), dtype=torch.float32, device=c.pages.device)
    stream = torch.cuda.Stream()

    def decode():
        ops.mla_decode_lowbit("C4R4", ql, qr, c.pages, c.prot, c.seq_slot, c.block_table, tl,
                              msl, d.scale, ns, workspace=ws, out=out, lse=lse, stream=stream)

    def fused():
        ops.mla_decode_lowbit_append("C4R4", lat, kr, ql, qr, c.pages, c.prot, c.seq_slot,
                                     c.block_table, tl, msl, d.scale, ns, workspace=ws,
                                     out=out, lse=lse, stream=stream)

    for step in (decode, fused):
        with torch.cuda.stream(stream):
            step()
        stream.synchronize()
        ref_o, ref_l = out.cpu().clone(), lse.cpu().clone()
        ref_p, ref_r = c.pages.cpu().clone(), c.prot.cpu().clone()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            step()
        for rep in range(6):
            with torch.cuda.stream(stream):
                out.fill_(float("nan"))
                lse.fill_(float("nan"))
                if rep % 2:                        # an eager call on the same workspace
                    ops.mla_decode_lowbit("C4R4", ql, qr, c.pages, c.prot, c.seq_slot,
                                          c.block_table, tl, msl, d.scale, 2, workspace=ws,
                                          out=out, lse=lse, stream=stream)
            stream.synchronize()
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(out.cpu(), ref_o) and torch.equal(lse.cpu(), ref_l), (step, rep)
            assert torch.equal(c.pages.cpu(), ref_p) and torch.equal(c.prot.cpu(), ref_r), (step, rep)
        say("  ", step.__name__, "6 replays bit-identical")
    check_decode(d, c, ref_o.numpy().astype(np.float64), ref_l.numpy().astype(np.float64), lens)


# ------------------------------------------------------------ host guards ---
@pytest.mark.parametrize("H", [16, 128])
def test_seq_lens_clamped_to_max_seq_len(H):
    """seq_lens beyond max_seq_len are clamped on the device: a sequence whose
    cache holds 700 tokens, passed as 1000 with max_seq_len 700, decodes
    exactly its 700 tokens."""
    d = synth.small(fmt="C4R4", batch=2, heads=H, lens=(300, 700), seed=71, extra_tokens=300)
    say("clamp", H)
    c = GpuCache(d)
    c.fill()
    out, lse = c.decode(lens=[300, 1000], max_seq_len=700)
    check_decode(d, c, out, lse, [300, 700])


@pytest.mark.parametrize("H", [16, 128])
def test_unusable_block_table_entries_are_skipped(H):
    """Block-table entries outside [0, num_pages) are never dereferenced:
    the call completes, its outputs are finite, and the other sequences'
    results are bit-identical to the run with a valid table."""
    from bit_mla_kv_quant_amd import ops
    d = synth.small(fmt="C4R4", batch=3, heads=H, lens=(900, 640, 1200), seed=72)
    say("unusable pages", H)
    c = GpuCache(d)
    c.fill()
    ref_out, ref_lse = c.decode()
    bt = d.block_table.copy()
    bt[1, 3] = -1
    bt[1, 7] = d.num_pages + 5
    for ns in (0, 1):
        out, lse = ops.mla_decode_lowbit(
            "C4R4", t_bf16(d.q_lat), t_bf16(d.q_rope), c.pages, c.prot, c.seq_slot,
            t_i32(bt), t_i32(d.lens), int(d.lens.max()), d.scale, num_splits=ns)
        torch.cuda.synchronize()
        out = out.cpu().numpy().astype(np.float64)
        lse = lse.cpu().numpy().astype(np.float64)
        assert np.all(np.isfinite(out[1])) and np.all(np.isfinite(lse[1]))
        if ns == 0:
            np.testing.assert_array_equal(out[[0, 2]], ref_out[[0, 2]])
            np.testing.assert_array_equal(lse[[0, 2]], ref_lse[[0, 2]])
