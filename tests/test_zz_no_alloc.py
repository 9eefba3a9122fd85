"""mla_decode_lowbit_noalloc (split partials in the library's per-GPU
scratch, no workspace, no allocation by the call) through the C ABI against
mla_decode_lowbit with a caller workspace: bit-identical on the same plan, on
consecutive calls whose second input is smaller (the scratch keeps the first
call's partials; nothing in it may need clearing), and within the oracle's
bar; the automatic plan stays inside the scratch; explicit plans beyond it
are refused before any launch."""

import numpy as np
import pytest

from bit_mla_kv_quant_amd import synth

from gpu_helpers import GpuCache, oracle_decode, t_bf16, t_i32

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

PER_SPLIT_ROW = (512 + 4) * 4          # fp32 partial output + (max, sums) per row


def _calls(c, d, lens, ns):
    ops = c.ops
    args = (c.fmt, t_bf16(d.q_lat), t_bf16(d.q_rope), c.pages, c.prot, c.seq_slot,
            c.block_table, t_i32(lens), int(np.max(lens)), d.scale)
    o_ws, l_ws = ops.mla_decode_lowbit(*args, num_splits=ns)
    o_na, l_na = ops.mla_decode_lowbit_noalloc(*args, num_splits=ns)
    torch.cuda.synchronize()
    return (o_ws.cpu().numpy(), l_ws.cpu().numpy(), o_na.cpu().numpy(), l_na.cpu().numpy())


def _oracle_rows(d, lens, out, lse, which):
    for b in which:
        L = int(lens[b])
        ro, rl = oracle_decode(d, b, L)
        if L == 0:
            assert np.all(out[b] == 0) and np.all(np.isneginf(lse[b]))
            continue
        e = np.linalg.norm(out[b] - ro, axis=-1) / np.linalg.norm(ro, axis=-1)
        assert np.all(e <= 2e-3), (b, float(e.max()))
        assert np.max(np.abs(lse[b] - rl)) <= 1e-3


@pytest.mark.parametrize("H", [16, 128])
def test_noalloc_matches_workspace_entry_on_consecutive_calls(H):
    big = synth.small(fmt="C4R4", batch=6, heads=H, lens=(3000, 1500, 700, 133, 64, 0), seed=101)
    small = synth.small(fmt="C4R4", batch=2, heads=H, lens=(900, 65), seed=102)
    print("[case] noalloc consecutive", H, flush=True)
    caches = []
    for d in (big, small):
        c = GpuCache(d)
        c.fill()
        caches.append((c, d))
    for ns in (0, 3, 1):
        for c, d in caches:                       # the larger call, then the smaller one
            lens = d.lens
            o_ws, l_ws, o_na, l_na = _calls(c, d, lens, ns)
            np.testing.assert_array_equal(o_na, o_ws)
            np.testing.assert_array_equal(l_na, l_ws)
            _oracle_rows(d, lens, o_na.astype(np.float64), l_na.astype(np.float64),
                         range(d.B))


def test_noalloc_automatic_plan_fits_the_scratch():
    """64 sequences x 128 heads of 2500 tokens: the workspace entry's
    automatic plan needs more partials than the scratch holds, so the no-alloc
    call takes the largest plan that fits -- bit-identical to the workspace
    entry given that split count -- and an explicit plan beyond the scratch
    is refused."""
    from bit_mla_kv_quant_amd import ops
    B, H, L = 64, 128, 2500
    d = synth.small(fmt="C4R4", batch=B, heads=H, lens=(L,) * B, seed=103)
    print("[case] noalloc capped plan", flush=True)
    c = GpuCache(d)
    c.fill()
    per_split = B * H * PER_SPLIT_ROW
    fit = ops.NOALLOC_SCRATCH_BYTES // per_split
    auto_ws = ops.mla_decode_lowbit_workspace("C4R4", B, H, L, 0)
    auto_ns = auto_ws // per_split
    assert fit >= 2
    want_ns = min(auto_ns, fit) if auto_ns > 1 else 1
    lens = d.lens
    args = ("C4R4", t_bf16(d.q_lat), t_bf16(d.q_rope), c.pages, c.prot, c.seq_slot,
            c.block_table, t_i32(lens), L, d.scale)
    o_na, l_na = ops.mla_decode_lowbit_noalloc(*args, num_splits=0)
    o_ws, l_ws = ops.mla_decode_lowbit(*args, num_splits=int(want_ns))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(o_na.cpu().numpy(), o_ws.cpu().numpy())
    np.testing.assert_array_equal(l_na.cpu().numpy(), l_ws.cpu().numpy())
    _oracle_rows(d, lens, o_na.cpu().numpy().astype(np.float64),
                 l_na.cpu().numpy().astype(np.float64), (0, B - 1))
    with pytest.raises(ops.MlaLowbitError, match="EWORKSPACE"):
        ops.mla_decode_lowbit_noalloc(*args, num_splits=int(fit + 1))
