"""Host-side logic of bench.py (no GPU): the per-token sizes and kernel
routing it reports agree with the library, its protected-set count and FLOP
count agree with the oracle's definitions, and a request for more than one
GPU is refused before anything touches a device."""

import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from oracle import attention  # noqa: E402


@pytest.fixture(scope="module")
def ops():
    from bit_mla_kv_quant_amd import ops as o
    return o


def test_token_bytes_match_library_pages(ops):
    # a page is 64 token slots, nothing else
    for fmt, tb in bench.TOKEN_BYTES.items():
        assert ops.mla_lb_page_bytes(fmt) == 64 * tb, fmt
    assert ops.mla_lb_prot_bytes_per_seq() == bench.PROT_ROWS * bench.ROW_BYTES


def test_protected_count_matches_oracle_set():
    for L in list(range(0, 300)) + [1000, 8192, 131072]:
        assert bench.n_protected(L) == int(attention.protected_mask(L).sum()), L


def test_algorithmic_bytes_all_protected_and_packed():
    # L <= 132: every token is a bf16 row; long L: 132 bf16 rows + packed rest
    H = 16
    fixed = lambda L: H * 576 * 2 + H * 513 * 4 + -(-L // 64) * 4
    for L in (1, 64, 132):
        assert bench.algorithmic_bytes("C4R4", [L], H) == L * 1152 + fixed(L)
    for fmt in ("C4R4", "C2R4", "C4R4F"):
        L = 8192
        assert bench.algorithmic_bytes(fmt, [L], H) == (
            132 * 1152 + (L - 132) * bench.TOKEN_BYTES[fmt] + fixed(L))


def test_algorithmic_flops_count_causal_pairs():
    # brute force over (query, token) pairs of small sequences
    rng = np.random.default_rng(3)
    for nq in (1, 2, 5):
        lens = rng.integers(0, 40, size=6).tolist()
        pairs = 0
        for L in lens:
            for j in range(nq):
                for i in range(L):
                    pairs += i <= L - nq + j          # query j is token L - nq + j
        assert bench.algorithmic_flops(lens, 16, nq) == pairs * 16 * 2 * (576 + 512)


def test_rows128_mirrors_library_plan(ops):
    """The library's split plan reveals which kernel it routes to: automatic
    splits fill 256 CUs with B * (rows/16) groups on the 16-row kernel and
    B * ceil(rows/128) on the 128-row one (long enough sequences that no
    minimum-split cap binds)."""
    L = 2048 * 64 * 2
    seen = {True: 0, False: 0}
    for rows in range(16, 1025, 16):
        nq, H = (rows // 16, 16) if rows > 128 else (1, rows)
        ws = ops.mla_decode_lowbit_mq_workspace("C4R4", 1, nq, H, L, 0)
        ns = ws // (rows * 516 * 4)
        ns16, ns128 = -(-256 // (rows // 16)), -(-256 // -(-rows // 128))
        if ns16 == ns128:
            continue
        assert ns in (ns16, ns128), rows
        assert (ns == ns128) == bench.rows128(rows), rows
        seen[ns == ns128] += 1
    assert seen[True] > 0 and seen[False] > 0


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr


def test_cpu_baseline_reports_both_thread_counts_and_phases():
    """The CPU leg times the oracle twice -- BLAS on every core of the
    affinity set, then on one thread -- with unpack + dequantize and fp64
    attention reported apart, and records the host it ran on."""
    from bit_mla_kv_quant_amd import synth
    d = synth.draw(synth.WORKLOADS[0])
    r = bench.cpu_baseline(d, "C4R4", budget_s=0.2, budget_1t_s=0.2)
    for k in ("value", "unit", "cores", "kind", "sample"):
        assert k in r
    assert r["kind"] == "oracle" and r["unit"] == "KV-tokens/s"
    assert r["one_thread"]["blas_threads"] == 1
    assert r["cores"] == r["all_cores"]["blas_threads"] >= 1
    for leg in (r["all_cores"], r["one_thread"]):
        assert leg["dequant_s"] > 0 and leg["attention_s"] > 0 and leg["tokens"] >= 1024
        assert leg["kv_tokens_per_s"] == pytest.approx(
            leg["tokens"] / (leg["dequant_s"] + leg["attention_s"]), rel=1e-2)
    assert r["host"]["affinity_cores"] == len(os.sched_getaffinity(0))
    assert r["host"]["cpu_model"]
