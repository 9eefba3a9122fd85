"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, and rejects bad arguments on the host before any HIP call."""

import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mla_lowbit.h")


@pytest.fixture(scope="module")
def ops():
    from bit_mla_kv_quant_amd import ops as o
    return o


def header_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*([a-z_0-9]+)\s*\(", src, re.M)))


def test_header_declares_expected_calls(ops):
    fns = header_functions()
    assert set(fns) == set(ops.EXPORTED), fns


def test_library_exports_every_declared_symbol(ops):
    out = subprocess.run(["nm", "-D", "--defined-only", ops.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    syms = {l.split()[-1] for l in out.splitlines() if l.strip()}
    for fn in header_functions():
        assert fn in syms, fn
        assert getattr(ops.raw(), fn)


def test_pure_host_queries(ops):
    assert ops.mla_lb_version() >= 1
    assert ops.mla_lb_page_bytes("C4R4") == 20736
    assert ops.mla_lb_page_bytes("C2R4") == 12544
    assert ops.mla_lb_page_bytes("C4R4F") == 20992
    assert ops.mla_lb_page_bytes(3) == 0
    assert ops.mla_lb_page_bytes(7) == 0
    assert ops.mla_lb_prot_bytes_per_seq() == 152064
    for c in (0, -1, -2, -3, -4, -5, -99):
        assert isinstance(ops.mla_lb_strerror(c), str) and ops.mla_lb_strerror(c)


FAKE = ctypes.c_void_p(0x1000)   # never dereferenced: every call below fails validation


def _append(lib, f=0, T=4, null=None, num_pages=1, nslots=1):
    args = [FAKE] * 6
    if null is not None:
        args[null] = None
    return lib.kv_quant_append(f, *args, T, FAKE, num_pages, FAKE, nslots, None)


def test_append_validation(ops):
    lib = ops.raw()
    assert _append(lib, f=5) == -3
    assert _append(lib, T=-1) == -2
    assert lib.kv_quant_append(0, None, None, None, None, None, None, 0, None, 0, None, 0, None) == 0
    for k in range(6):
        assert _append(lib, null=k) == -1
    assert _append(lib, num_pages=0) == -2
    assert _append(lib, nslots=0) == -2


def _decode(lib, f=0, B=2, H=16, max_blocks=4, msl=200, scale=0.07, ns=0, ws=None, ws_bytes=0,
            null=None, num_pages=8, nslots=2):
    ptrs = {"q_lat": FAKE, "q_rope": FAKE, "pages": FAKE, "prot": FAKE, "seq_slot": FAKE,
            "block_table": FAKE, "seq_lens": FAKE, "out": FAKE, "lse": FAKE}
    if null:
        ptrs[null] = None
    return lib.mla_decode_lowbit(f, ptrs["q_lat"], ptrs["q_rope"], ptrs["pages"], num_pages,
                                 ptrs["prot"], nslots, ptrs["seq_slot"], ptrs["block_table"],
                                 max_blocks, ptrs["seq_lens"], msl, B, H, scale, ns, ws,
                                 ws_bytes, ptrs["out"], ptrs["lse"], None)


def test_decode_validation(ops):
    lib = ops.raw()
    assert _decode(lib, f=3) == -3
    for k in ("q_lat", "q_rope", "pages", "prot", "seq_slot", "block_table", "seq_lens", "out", "lse"):
        assert _decode(lib, null=k) == -1, k
    assert _decode(lib, scale=0.0) == -1
    assert _decode(lib, scale=float("inf")) == -1
    assert _decode(lib, scale=float("nan")) == -1
    for H in (0, 8, 24, 144, 256):
        assert _decode(lib, H=H) == -2, H
    assert _decode(lib, B=0) == -2
    assert _decode(lib, msl=257, max_blocks=4) == -2        # seq longer than the block table
    assert _decode(lib, msl=-1) == -2
    assert _decode(lib, ns=-1) == -2
    assert _decode(lib, num_pages=0) == -2
    assert _decode(lib, nslots=0) == -2
    # a split plan needs a workspace: none / too small -> EWORKSPACE
    need = ops.mla_decode_lowbit_workspace("C4R4", 2, 16, 200, 2)
    assert need == 2 * 2 * 16 * 516 * 4
    assert _decode(lib, ns=2, ws=None) == -4
    assert _decode(lib, ns=2, ws=FAKE, ws_bytes=need - 1) == -4


def test_fused_step_validation(ops):
    lib = ops.raw()

    def call(f=0, latent=FAKE, k_rope=FAKE, H=16, scale=0.07, ns=0, ws=None, ws_bytes=0,
             q_lat=FAKE):
        return lib.mla_decode_lowbit_append(f, latent, k_rope, q_lat, FAKE, FAKE, 8, FAKE, 2,
                                            FAKE, FAKE, 4, FAKE, 200, 2, H, scale, ns, ws,
                                            ws_bytes, FAKE, FAKE, None)
    assert call(f=3) == -3
    assert call(f=3, latent=None) == -3
    assert call(latent=None) == -1
    assert call(k_rope=None) == -1
    assert call(q_lat=None) == -1
    assert call(scale=-1.0) == -1
    assert call(H=24) == -2
    need = ops.mla_decode_lowbit_workspace("C4R4", 2, 16, 200, 2)
    assert call(ns=2) == -4
    assert call(ns=2, ws=FAKE, ws_bytes=need - 1) == -4


def test_multi_query_validation(ops):
    lib = ops.raw()

    def call(f=0, nq=4, H=16, scale=0.07, ns=0, ws=None, ws_bytes=0, q_lat=FAKE):
        return lib.mla_decode_lowbit_mq(f, q_lat, FAKE, FAKE, 8, FAKE, 2, FAKE, FAKE, 4, FAKE,
                                        200, 2, nq, H, scale, ns, ws, ws_bytes, FAKE, FAKE, None)
    assert call(f=3) == -3
    assert call(q_lat=None) == -1
    assert call(scale=0.0) == -1
    for nq in (0, -1, 513):                # 513 x 128 rows > MLA_LB_MAX_ROWS (65536)
        assert call(nq=nq, H=128) == -2, nq
    assert call(nq=4097, H=16) == -2
    assert ops.mla_decode_lowbit_mq_workspace("C4R4", 2, 512, 128, 200, 0) >= 0   # 65536 rows
    assert call(H=24) == -2
    need = ops.mla_decode_lowbit_mq_workspace("C4R4", 2, 4, 16, 200, 2)
    assert need == 2 * 2 * 64 * 516 * 4
    assert need == ops.mla_decode_lowbit_workspace("C4R4", 2, 64, 200, 2)
    assert call(ns=2) == -4
    assert call(ns=2, ws=FAKE, ws_bytes=need - 1) == -4
    with pytest.raises(ops.MlaLowbitError):
        ops.mla_decode_lowbit_mq_workspace("C4R4", 1, 0, 16, 100, 0)
    assert ops.mla_decode_lowbit_mq_workspace("C4R4", 1, 8, 128, 100000, 0) > 0


def test_dequant_dump_validation(ops):
    lib = ops.raw()
    assert lib.mla_lb_dequant_dump(3, FAKE, 4, 0, FAKE, None) == -3
    assert lib.mla_lb_dequant_dump(0, None, 4, 0, FAKE, None) == -1
    assert lib.mla_lb_dequant_dump(0, FAKE, 4, 4, FAKE, None) == -2
    assert lib.mla_lb_dequant_dump(0, FAKE, 4, -1, FAKE, None) == -2


def test_workspace_plan(ops):
    # single page or num_splits=1: one pass, no workspace
    assert ops.mla_decode_lowbit_workspace("C4R4", 4, 16, 64, 0) == 0
    assert ops.mla_decode_lowbit_workspace("C4R4", 4, 16, 100000, 1) == 0
    # automatic plans always fit the max-length sequence in <= 2*256 workgroups' worth of splits
    for (B, H, L) in [(1, 16, 1024), (32, 16, 8192), (64, 16, 32768), (16, 128, 32768), (8, 128, 131080)]:
        n = ops.mla_decode_lowbit_workspace("C4R4", B, H, L, 0)
        assert n % (B * H * 516 * 4) == 0
    with pytest.raises(ops.MlaLowbitError):
        ops.mla_decode_lowbit_workspace("C4R4", 1, 20, 100, 0)
    # large plans are sized exactly up to 2^60 bytes and refused beyond (at
    # 65535 sequences, 2^25 one-page splits and 65536 rows the product would
    # pass 2^64)
    big = 2**31 - 1
    n = ops.mla_decode_lowbit_mq_workspace("C4R4", 65535, 8, 128, big, 2**14)
    assert n == 65535 * 2**14 * 1024 * 516 * 4 and n < 2**60
    for nq, ns in ((8, big), (64, big), (512, big), (512, 2**17)):
        with pytest.raises(ops.MlaLowbitError, match="ESHAPE"):
            ops.mla_decode_lowbit_mq_workspace("C4R4", 65535, nq, 128, big, ns)
    n = ops.mla_decode_lowbit_mq_workspace("C4R4", 4, 512, 128, 131072, 16)
    assert n == 4 * 16 * 65536 * 516 * 4
    for call in (lambda: ops.mla_decode_lowbit_workspace("C4R4", 65536, 16, 1000, 0),
                 lambda: ops.mla_decode_lowbit_mq_workspace("C4R4", 65536, 2, 16, 1000, 0)):
        with pytest.raises(ops.MlaLowbitError):      # B beyond the grid limit
            call()


def test_calibration_helpers_match_oracle(ops):
    """Host calibration helpers (no GPU) against the oracle's fp64 values."""
    import numpy as np
    from bit_mla_kv_quant_amd import synth
    from oracle import transforms, quant
    d = synth.small(fmt="C4R4", batch=1, heads=16, lens=(777,), seed=4, outlier_factor=16.0)
    for x in (d.c[0], d.kr[0]):
        got = ops.mla_lb_channel_stat(x, 99.9)
        want = transforms.channel_stat(quant.bf16_to_f32(x))
        np.testing.assert_array_equal(got, want.astype(np.float32))
        for alpha in (0.0, 0.125, 0.5, 1.0):
            for pairs in ((False, True) if x.shape[1] == 64 else (False,)):
                s = ops.mla_lb_smooth_scales(got, alpha, pairs)
                ws = transforms.smooth_scales(got.astype(np.float64), alpha, pairs)
                np.testing.assert_allclose(s, ws, rtol=2 ** -23)
    lib = ops.raw()
    assert lib.mla_lb_smooth_scales(None, 4, 0.5, 0, FAKE) == -1
    assert lib.mla_lb_smooth_scales(FAKE, 3, 0.5, 1, FAKE) == -2
    assert lib.mla_lb_smooth_scales(FAKE, 4, -0.5, 0, FAKE) == -2
    assert lib.mla_lb_channel_stat(FAKE, 0, 4, 99.9, FAKE) == -2
    assert lib.mla_lb_channel_stat(FAKE, 4, 4, 101.0, FAKE) == -2
    assert lib.mla_lb_channel_stat(None, 4, 4, 99.9, FAKE) == -1


def test_header_is_plain_c_and_links(ops, tmp_path):
    """A C99 caller (gcc -pedantic) compiles against include/mla_lowbit.h,
    links libmla_lowbit.so and gets the host queries' answers."""
    import shutil
    if shutil.which("gcc") is None:
        pytest.skip("no gcc")
    src = tmp_path / "caller.c"
    src.write_text(r'''
#include <string.h>
#include "mla_lowbit.h"
int main(void) {
  float stat[4] = {4.0f, 1.0f, 0.25f, 16.0f}, s[4];
  size_t ws = 0;
  if (mla_lb_page_bytes(MLA_LB_C4R4) != 20736 || mla_lb_page_bytes(MLA_LB_C2R4) != 12544) return 1;
  if (mla_lb_prot_bytes_per_seq() != 152064) return 2;
  if (strlen(mla_lb_strerror(MLA_LB_EWORKSPACE)) == 0) return 3;
  if (mla_decode_lowbit_workspace(MLA_LB_C4R4, 2, 16, 200, 2, &ws) != MLA_LB_OK) return 4;
  if (ws != (size_t)2 * 2 * 16 * 516 * 4) return 5;
  if (mla_lb_smooth_scales(stat, 4, 1.0f, 1, s) != MLA_LB_OK) return 6;
  if (s[0] != 0.25f || s[1] != 0.25f || s[2] != 0.0625f || s[3] != 0.0625f) return 7;
  if (mla_decode_lowbit(MLA_LB_C4R4, 0, 0, 0, 1, 0, 1, 0, 0, 1, 0, 64, 1, 16, 0.1f, 0, 0, 0,
                        0, 0, 0) != MLA_LB_EINVAL) return 8;
  return 0;
}
''')
    exe = tmp_path / "caller"
    libdir = os.path.dirname(ops.LIB_PATH)
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror",
                    "-I", os.path.join(ROOT, "include"), str(src), "-L", libdir, "-lmla_lowbit",
                    f"-Wl,-rpath,{libdir}", "-o", str(exe)], check=True)
    assert subprocess.run([str(exe)]).returncode == 0


# ------------------------------------------- binding-side shape validation ---
def _decode_tensors(fmt="C4R4", B=2, H=16, nq=None, num_pages=4, max_blocks=3):
    import torch
    from bit_mla_kv_quant_amd import ops as o
    lead = (B, H) if nq is None else (B, nq, H)
    return dict(
        q_lat=torch.zeros(lead + (512,), dtype=torch.int16),
        q_rope=torch.zeros(lead + (64,), dtype=torch.int16),
        pages=torch.zeros((num_pages, o.mla_lb_page_bytes(fmt)), dtype=torch.uint8),
        prot=torch.zeros((B, 132, 576), dtype=torch.int16),
        seq_slot=torch.zeros(B, dtype=torch.int32),
        block_table=torch.zeros((B, max_blocks), dtype=torch.int32),
        seq_lens=torch.zeros(B, dtype=torch.int32),
        out=torch.zeros(lead + (512,), dtype=torch.float32),
        lse=torch.zeros(lead, dtype=torch.float32))


def _call_decode(ops, fmt, t, nq=False):
    fn = ops.mla_decode_lowbit_mq if nq else ops.mla_decode_lowbit
    return fn(fmt, t["q_lat"], t["q_rope"], t["pages"], t["prot"], t["seq_slot"],
              t["block_table"], t["seq_lens"], 100, 0.07, out=t["out"], lse=t["lse"])


@pytest.mark.parametrize("bad, msg", [
    ("pages_width", "pages"),        # a C4R4F call on a pool sized for C4R4
    ("prot_rows", "prot"),
    ("short_block_table", "block_table"),
    ("short_seq_lens", "seq_lens"),
    ("q_rope", "q_rope"),
    ("out", "out"),
    ("lse", "lse"),
])
def test_binding_rejects_mismatched_shapes(ops, bad, msg):
    """The binding checks every tensor's full shape against the format and
    (B, H) before the C call: the C layer only sees pointers, and a short
    tensor would be read or written past its end on the device."""
    import torch
    fmt = "C4R4F" if bad == "pages_width" else "C4R4"
    t = _decode_tensors("C4R4" if bad == "pages_width" else fmt)
    if bad == "prot_rows":
        t["prot"] = torch.zeros((2, 131, 576), dtype=torch.int16)
    elif bad == "short_block_table":
        t["block_table"] = torch.zeros((1, 3), dtype=torch.int32)
    elif bad == "short_seq_lens":
        t["seq_lens"] = torch.zeros(1, dtype=torch.int32)
    elif bad == "q_rope":
        t["q_rope"] = torch.zeros((2, 16, 32), dtype=torch.int16)
    elif bad == "out":
        t["out"] = torch.zeros((2, 8, 512), dtype=torch.float32)
    elif bad == "lse":
        t["lse"] = torch.zeros((2,), dtype=torch.float32)
    with pytest.raises(ValueError, match=msg):
        _call_decode(ops, fmt, t)


def test_binding_rejects_bad_shapes_on_every_entry_point(ops):
    import torch
    t = _decode_tensors(nq=4)
    t["q_rope"] = torch.zeros((2, 4, 16, 63), dtype=torch.int16)
    with pytest.raises(ValueError, match="q_rope"):
        _call_decode(ops, "C4R4", t, nq=True)
    t = _decode_tensors()
    lat, kr = torch.zeros((2, 512), dtype=torch.int16), torch.zeros((1, 64), dtype=torch.int16)
    with pytest.raises(ValueError, match="k_rope"):
        ops.mla_decode_lowbit_append("C4R4", lat, kr, t["q_lat"], t["q_rope"], t["pages"],
                                     t["prot"], t["seq_slot"], t["block_table"], t["seq_lens"],
                                     100, 0.07)
    T = 3
    args = [torch.zeros((T, 512), dtype=torch.int16), torch.zeros((T, 64), dtype=torch.int16),
            torch.zeros(T, dtype=torch.int64), torch.zeros(T, dtype=torch.int32),
            torch.zeros(T - 1, dtype=torch.int32), torch.zeros(T, dtype=torch.int32)]
    with pytest.raises(ValueError, match="pos"):
        ops.kv_quant_append("C2R4", *args, t["pages"], t["prot"])   # also a C4R4-sized pool
    with pytest.raises(ValueError, match="pages"):
        ops.mla_lb_dequant_dump("C2R4", t["pages"], 0)


def test_binding_requires_gpu_tensors(ops):
    """Correct shapes on the host are refused before the C call: every tensor
    must sit on one GPU."""
    t = _decode_tensors()
    with pytest.raises(ValueError, match="GPU tensor"):
        _call_decode(ops, "C4R4", t)


def test_host_layer_under_address_and_ub_sanitizers(tmp_path):
    """abi.cpp and noalloc.hip (validation, split plan, workspace sizing, the
    no-alloc variant's plan limit, calibration helpers)
    built for the host with AddressSanitizer and UndefinedBehaviorSanitizer,
    the kernel launchers replaced by stubs, and driven through every host
    path by tests/native/abi_host_check.cpp; any memory error, leak or
    undefined behaviour aborts the run.  Device code is built without
    sanitizers (each -fsanitize= applies to the host pass only)."""
    exe = tmp_path / "abi_host_check"
    cmd = ["/opt/rocm/bin/hipcc", "-x", "hip", "--offload-arch=gfx950", "-std=c++17", "-O1", "-g",
           "-fno-omit-frame-pointer",
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all",
           os.path.join(ROOT, "bit_mla_kv_quant_amd", "csrc", "abi.cpp"),
           os.path.join(ROOT, "bit_mla_kv_quant_amd", "csrc", "noalloc.hip"),
           os.path.join(ROOT, "tests", "native", "abi_host_check.cpp"), "-o", str(exe)]
    if not os.path.exists(cmd[0]):
        pytest.skip("hipcc not available")
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, (r.stdout[-2000:], r.stderr[-4000:])
    assert "abi host checks passed" in r.stdout


def test_hadamard_helper_matches_oracle(ops):
    """mla_lb_hadamard_rows against the oracle's Sylvester matrix product
    (fp64 reference, the helper rounds once to fp32); bad orders refused."""
    import numpy as np
    from oracle import transforms
    rng = np.random.default_rng(3)
    for n in (1, 2, 64, 512):
        x = (rng.standard_normal((5, n)) * 10).astype(np.float32)
        want = x.astype(np.float64) @ transforms.hadamard(n)
        got = ops.mla_lb_hadamard_rows(x)
        np.testing.assert_allclose(got, want, rtol=2e-7, atol=1e-6 * np.abs(want).max())
    with pytest.raises(ops.MlaLowbitError):
        ops.mla_lb_hadamard_rows(np.zeros((2, 48), np.float32))
