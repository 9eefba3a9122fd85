"""ctypes binding of libmla_lowbit.so (argument marshalling only).

Every entry point of ``include/mla_lowbit.h`` has a function of the same name
here.  Tensors are torch tensors on the GPU; bf16 data may be passed as
``torch.bfloat16`` or as ``torch.int16`` bit patterns.  All compute runs in the
HIP kernels of the library; if the library is not built, importing this module
raises -- there is no fallback.
"""

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# the in-tree build; MLA_LOWBIT_LIB names another build of the same library
LIB_PATH = os.environ.get("MLA_LOWBIT_LIB") or os.path.join(_HERE, "libmla_lowbit.so")

FORMATS = {"C4R4": 0, "C2R4": 1, "C4R4F": 2}

ERRORS = {0: "MLA_LB_OK", -1: "MLA_LB_EINVAL", -2: "MLA_LB_ESHAPE", -3: "MLA_LB_EFORMAT",
          -4: "MLA_LB_EWORKSPACE", -5: "MLA_LB_EHIP"}


class MlaLowbitError(RuntimeError):
    def __init__(self, fn, code):
        self.code = code
        msg = _lib.mla_lb_strerror(code).decode()
        super().__init__(f"{fn} failed: {ERRORS.get(code, code)} ({msg})")


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is not built; run `python -m bit_mla_kv_quant_amd.build` "
            "(hipcc, gfx950).  There is no CPU fallback.")
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, I64, SZ, F = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t,
                          ctypes.c_float)
    sig = {
        "mla_lb_version": (ctypes.c_int, []),
        "mla_lb_strerror": (ctypes.c_char_p, [ctypes.c_int]),
        "mla_lb_page_bytes": (SZ, [ctypes.c_int]),
        "mla_lb_prot_bytes_per_seq": (SZ, []),
        "kv_quant_append": (ctypes.c_int, [ctypes.c_int, P, P, P, P, P, P, I32, P, I64, P, I32, P]),
        "mla_decode_lowbit_workspace": (ctypes.c_int, [ctypes.c_int, I32, I32, I32, I32,
                                                       ctypes.POINTER(SZ)]),
        "mla_decode_lowbit": (ctypes.c_int, [ctypes.c_int, P, P, P, I64, P, I32, P, P, I32, P,
                                             I32, I32, I32, F, I32, P, SZ, P, P, P]),
        "mla_decode_lowbit_append": (ctypes.c_int, [ctypes.c_int, P, P, P, P, P, I64, P, I32, P,
                                                    P, I32, P, I32, I32, I32, F, I32, P, SZ, P,
                                                    P, P]),
        "mla_decode_lowbit_noalloc": (ctypes.c_int, [ctypes.c_int, P, P, P, I64, P, I32, P, P,
                                                     I32, P, I32, I32, I32, F, I32, P, P, P]),
        "mla_decode_lowbit_mq_workspace": (ctypes.c_int, [ctypes.c_int, I32, I32, I32, I32, I32,
                                                          ctypes.POINTER(SZ)]),
        "mla_decode_lowbit_mq": (ctypes.c_int, [ctypes.c_int, P, P, P, I64, P, I32, P, P, I32, P,
                                                I32, I32, I32, I32, F, I32, P, SZ, P, P, P]),
        "mla_lb_channel_stat": (ctypes.c_int, [P, I64, I32, ctypes.c_double, P]),
        "mla_lb_smooth_scales": (ctypes.c_int, [P, I32, F, I32, P]),
        "mla_lb_hadamard_rows": (ctypes.c_int, [P, I64, I32, P]),
        "mla_lb_dequant_dump": (ctypes.c_int, [ctypes.c_int, P, I64, I64, P, P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


_lib = _load()

# Names the header declares (checked by the ABI tests).
EXPORTED = ("mla_lb_version", "mla_lb_strerror", "mla_lb_page_bytes",
            "mla_lb_prot_bytes_per_seq", "kv_quant_append", "mla_decode_lowbit_workspace",
            "mla_decode_lowbit", "mla_decode_lowbit_append", "mla_decode_lowbit_noalloc",
            "mla_decode_lowbit_mq_workspace",
            "mla_decode_lowbit_mq", "mla_lb_channel_stat", "mla_lb_smooth_scales",
            "mla_lb_hadamard_rows", "mla_lb_dequant_dump")


def raw():
    """The ctypes handle (for tests that drive the C ABI directly)."""
    return _lib


def _fmt(f):
    return FORMATS[f] if isinstance(f, str) else int(f)


def _ptr(t, dtypes, name):
    if t is None:
        return None
    if t.dtype not in dtypes:
        raise TypeError(f"{name}: dtype {t.dtype} not in {dtypes}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


_BF16 = (torch.bfloat16, torch.int16)


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _check(fn, code):
    if code != 0:
        raise MlaLowbitError(fn, code)


# ---- argument checks before the C call.  The C layer sees only pointers and
# the sizes passed with them, so a tensor smaller than its declared shape
# would be read or written past its end on the device; every tensor's full
# shape is therefore checked here against the format and (B, nq, H), and all
# tensors must sit on one GPU.
def _shape(t, want, name):
    """want: tuple of ints (exact) or None (any size) per dimension."""
    if t is None:
        raise ValueError(f"{name}: missing")
    got = tuple(t.shape)
    if len(got) != len(want) or any(w is not None and g != w for g, w in zip(got, want)):
        shown = tuple("*" if w is None else w for w in want)
        raise ValueError(f"{name}: shape {got}, expected {shown}")


def _rows_at_least(t, n, name):
    if t is None:
        raise ValueError(f"{name}: missing")
    if t.dim() < 1 or t.shape[0] < n:
        raise ValueError(f"{name}: needs at least {n} rows, has shape {tuple(t.shape)}")


def _same_gpu(fn, *named):
    dev = None
    for name, t in named:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError(f"{fn}: {name} must be a GPU tensor (device {t.device})")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError(f"{fn}: {name} is on {t.device}, other tensors on {dev}")


def _cache_shapes(fmt, pages, prot):
    pb = _lib.mla_lb_page_bytes(_fmt(fmt))
    if pb == 0:
        raise ValueError(f"unknown cache format {fmt!r}")
    _shape(pages, (None, pb), "pages")
    _shape(prot, (None, 132, 576), "prot")


def _decode_shapes(fmt, q_lat, q_rope, pages, prot, seq_slot, block_table, seq_lens, out, lse,
                   lead):
    """lead: the leading query dims, (B, H) or (B, nq, H)."""
    B = lead[0]
    _shape(q_lat, lead + (512,), "q_lat")
    _shape(q_rope, lead + (64,), "q_rope")
    _cache_shapes(fmt, pages, prot)
    _rows_at_least(seq_slot, B, "seq_slot")
    _shape(seq_slot, (None,), "seq_slot")
    _shape(block_table, (None, None), "block_table")
    _rows_at_least(block_table, B, "block_table")
    _rows_at_least(seq_lens, B, "seq_lens")
    _shape(seq_lens, (None,), "seq_lens")
    if out is not None:
        _shape(out, lead + (512,), "out")
    if lse is not None:
        _shape(lse, lead, "lse")


def mla_lb_version():
    return _lib.mla_lb_version()


def mla_lb_page_bytes(fmt):
    return _lib.mla_lb_page_bytes(_fmt(fmt))


def mla_lb_prot_bytes_per_seq():
    return _lib.mla_lb_prot_bytes_per_seq()


def mla_lb_strerror(code):
    return _lib.mla_lb_strerror(code).decode()


def kv_quant_append(fmt, latent, k_rope, slot_mapping, seq_slot, pos, new_len, pages, prot,
                    stream=None):
    """Quantize and insert T tokens.  latent [T,512], k_rope [T,64] bf16;
    slot_mapping int64 [T]; seq_slot, pos, new_len int32 [T];
    pages uint8 [num_pages, page_bytes]; prot bf16 [num_seq_slots, 132, 576]."""
    T = latent.shape[0]
    _shape(latent, (T, 512), "latent")
    _shape(k_rope, (T, 64), "k_rope")
    for name, t in (("slot_mapping", slot_mapping), ("seq_slot", seq_slot), ("pos", pos),
                    ("new_len", new_len)):
        _shape(t, (T,), name)
    _cache_shapes(fmt, pages, prot)
    _same_gpu("kv_quant_append", ("latent", latent), ("k_rope", k_rope),
              ("slot_mapping", slot_mapping), ("seq_slot", seq_slot), ("pos", pos),
              ("new_len", new_len), ("pages", pages), ("prot", prot))
    code = _lib.kv_quant_append(
        _fmt(fmt), _ptr(latent, _BF16, "latent"), _ptr(k_rope, _BF16, "k_rope"),
        _ptr(slot_mapping, (torch.int64,), "slot_mapping"),
        _ptr(seq_slot, (torch.int32,), "seq_slot"), _ptr(pos, (torch.int32,), "pos"),
        _ptr(new_len, (torch.int32,), "new_len"), T,
        _ptr(pages, (torch.uint8,), "pages"), pages.shape[0],
        _ptr(prot, _BF16, "prot"), prot.shape[0], _stream(stream))
    _check("kv_quant_append", code)


def mla_decode_lowbit_workspace(fmt, B, H, max_seq_len, num_splits=0):
    n = ctypes.c_size_t(0)
    _check("mla_decode_lowbit_workspace",
           _lib.mla_decode_lowbit_workspace(_fmt(fmt), B, H, max_seq_len, num_splits,
                                            ctypes.byref(n)))
    return n.value


def mla_decode_lowbit(fmt, q_lat, q_rope, pages, prot, seq_slot, block_table, seq_lens,
                      max_seq_len, softmax_scale, num_splits=0, workspace=None, out=None,
                      lse=None, stream=None):
    """Decode attention; returns (out fp32 [B,H,512], lse fp32 [B,H])."""
    if q_lat.dim() != 3:
        raise ValueError(f"q_lat: shape {tuple(q_lat.shape)}, expected (B, H, 512)")
    B, H = q_lat.shape[0], q_lat.shape[1]
    _decode_shapes(fmt, q_lat, q_rope, pages, prot, seq_slot, block_table, seq_lens, out, lse,
                   (B, H))
    _same_gpu("mla_decode_lowbit", ("q_lat", q_lat), ("q_rope", q_rope), ("pages", pages),
              ("prot", prot), ("seq_slot", seq_slot), ("block_table", block_table),
              ("seq_lens", seq_lens), ("workspace", workspace), ("out", out), ("lse", lse))
    dev = q_lat.device
    if out is None:
        out = torch.empty((B, H, 512), dtype=torch.float32, device=dev)
    if lse is None:
        lse = torch.empty((B, H), dtype=torch.float32, device=dev)
    need = mla_decode_lowbit_workspace(fmt, B, H, max_seq_len, num_splits)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    code = _lib.mla_decode_lowbit(
        _fmt(fmt), _ptr(q_lat, _BF16, "q_lat"), _ptr(q_rope, _BF16, "q_rope"),
        _ptr(pages, (torch.uint8,), "pages"), pages.shape[0], _ptr(prot, _BF16, "prot"),
        prot.shape[0], _ptr(seq_slot, (torch.int32,), "seq_slot"),
        _ptr(block_table, (torch.int32,), "block_table"), block_table.shape[1],
        _ptr(seq_lens, (torch.int32,), "seq_lens"), int(max_seq_len), B, H,
        float(softmax_scale), int(num_splits),
        None if workspace is None else ctypes.c_void_p(workspace.data_ptr()), ws_bytes,
        _ptr(out, (torch.float32,), "out"), _ptr(lse, (torch.float32,), "lse"), _stream(stream))
    _check("mla_decode_lowbit", code)
    return out, lse


NOALLOC_SCRATCH_BYTES = 64 << 20


def mla_decode_lowbit_noalloc(fmt, q_lat, q_rope, pages, prot, seq_slot, block_table, seq_lens,
                              max_seq_len, softmax_scale, num_splits=0, out=None, lse=None,
                              stream=None):
    """mla_decode_lowbit with the split partials in the library's per-GPU
    scratch (no workspace, no allocation by the call); out / lse are
    allocated here only when not passed.  Returns (out, lse)."""
    if q_lat.dim() != 3:
        raise ValueError(f"q_lat: shape {tuple(q_lat.shape)}, expected (B, H, 512)")
    B, H = q_lat.shape[0], q_lat.shape[1]
    _decode_shapes(fmt, q_lat, q_rope, pages, prot, seq_slot, block_table, seq_lens, out, lse,
                   (B, H))
    _same_gpu("mla_decode_lowbit_noalloc", ("q_lat", q_lat), ("q_rope", q_rope),
              ("pages", pages), ("prot", prot), ("seq_slot", seq_slot),
              ("block_table", block_table), ("seq_lens", seq_lens), ("out", out), ("lse", lse))
    dev = q_lat.device
    if out is None:
        out = torch.empty((B, H, 512), dtype=torch.float32, device=dev)
    if lse is None:
        lse = torch.empty((B, H), dtype=torch.float32, device=dev)
    code = _lib.mla_decode_lowbit_noalloc(
        _fmt(fmt), _ptr(q_lat, _BF16, "q_lat"), _ptr(q_rope, _BF16, "q_rope"),
        _ptr(pages, (torch.uint8,), "pages"), pages.shape[0], _ptr(prot, _BF16, "prot"),
        prot.shape[0], _ptr(seq_slot, (torch.int32,), "seq_slot"),
        _ptr(block_table, (torch.int32,), "block_table"), block_table.shape[1],
        _ptr(seq_lens, (torch.int32,), "seq_lens"), int(max_seq_len), B, H,
        float(softmax_scale), int(num_splits),
        _ptr(out, (torch.float32,), "out"), _ptr(lse, (torch.float32,), "lse"), _stream(stream))
    _check("mla_decode_lowbit_noalloc", code)
    return out, lse


def mla_decode_lowbit_append(fmt, latent, k_rope, q_lat, q_rope, pages, prot, seq_slot,
                             block_table, seq_lens, max_seq_len, softmax_scale, num_splits=0,
                             workspace=None, out=None, lse=None, stream=None):
    """One decode step with the cache writer fused in: stores the newest token
    (latent [B,512], k_rope [B,64] bf16 at position seq_lens[b]-1) into pages
    and prot, then decodes; returns (out fp32 [B,H,512], lse fp32 [B,H])."""
    if q_lat.dim() != 3:
        raise ValueError(f"q_lat: shape {tuple(q_lat.shape)}, expected (B, H, 512)")
    B, H = q_lat.shape[0], q_lat.shape[1]
    _shape(latent, (B, 512), "latent")       # one new token per sequence
    _shape(k_rope, (B, 64), "k_rope")
    _decode_shapes(fmt, q_lat, q_rope, pages, prot, seq_slot, block_table, seq_lens, out, lse,
                   (B, H))
    _same_gpu("mla_decode_lowbit_append", ("latent", latent), ("k_rope", k_rope),
              ("q_lat", q_lat), ("q_rope", q_rope), ("pages", pages), ("prot", prot),
              ("seq_slot", seq_slot), ("block_table", block_table), ("seq_lens", seq_lens),
              ("workspace", workspace), ("out", out), ("lse", lse))
    dev = q_lat.device
    if out is None:
        out = torch.empty((B, H, 512), dtype=torch.float32, device=dev)
    if lse is None:
        lse = torch.empty((B, H), dtype=torch.float32, device=dev)
    need = mla_decode_lowbit_workspace(fmt, B, H, max_seq_len, num_splits)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    code = _lib.mla_decode_lowbit_append(
        _fmt(fmt), _ptr(latent, _BF16, "latent"), _ptr(k_rope, _BF16, "k_rope"),
        _ptr(q_lat, _BF16, "q_lat"), _ptr(q_rope, _BF16, "q_rope"),
        _ptr(pages, (torch.uint8,), "pages"), pages.shape[0], _ptr(prot, _BF16, "prot"),
        prot.shape[0], _ptr(seq_slot, (torch.int32,), "seq_slot"),
        _ptr(block_table, (torch.int32,), "block_table"), block_table.shape[1],
        _ptr(seq_lens, (torch.int32,), "seq_lens"), int(max_seq_len), B, H,
        float(softmax_scale), int(num_splits),
        None if workspace is None else ctypes.c_void_p(workspace.data_ptr()), ws_bytes,
        _ptr(out, (torch.float32,), "out"), _ptr(lse, (torch.float32,), "lse"), _stream(stream))
    _check("mla_decode_lowbit_append", code)
    return out, lse


def mla_decode_lowbit_mq_workspace(fmt, B, nq, H, max_seq_len, num_splits=0):
    n = ctypes.c_size_t(0)
    _check("mla_decode_lowbit_mq_workspace",
           _lib.mla_decode_lowbit_mq_workspace(_fmt(fmt), B, nq, H, max_seq_len, num_splits,
                                               ctypes.byref(n)))
    return n.value


def mla_decode_lowbit_mq(fmt, q_lat, q_rope, pages, prot, seq_slot, block_table, seq_lens,
                         max_seq_len, softmax_scale, num_splits=0, workspace=None, out=None,
                         lse=None, stream=None):
    """Attention of the last nq tokens of each sequence over their causal
    prefixes.  q_lat [B,nq,H,512], q_rope [B,nq,H,64] bf16; returns
    (out fp32 [B,nq,H,512], lse fp32 [B,nq,H])."""
    if q_lat.dim() != 4:
        raise ValueError(f"q_lat: shape {tuple(q_lat.shape)}, expected (B, nq, H, 512)")
    B, nq, H = q_lat.shape[0], q_lat.shape[1], q_lat.shape[2]
    _decode_shapes(fmt, q_lat, q_rope, pages, prot, seq_slot, block_table, seq_lens, out, lse,
                   (B, nq, H))
    _same_gpu("mla_decode_lowbit_mq", ("q_lat", q_lat), ("q_rope", q_rope), ("pages", pages),
              ("prot", prot), ("seq_slot", seq_slot), ("block_table", block_table),
              ("seq_lens", seq_lens), ("workspace", workspace), ("out", out), ("lse", lse))
    dev = q_lat.device
    if out is None:
        out = torch.empty((B, nq, H, 512), dtype=torch.float32, device=dev)
    if lse is None:
        lse = torch.empty((B, nq, H), dtype=torch.float32, device=dev)
    need = mla_decode_lowbit_mq_workspace(fmt, B, nq, H, max_seq_len, num_splits)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    code = _lib.mla_decode_lowbit_mq(
        _fmt(fmt), _ptr(q_lat, _BF16, "q_lat"), _ptr(q_rope, _BF16, "q_rope"),
        _ptr(pages, (torch.uint8,), "pages"), pages.shape[0], _ptr(prot, _BF16, "prot"),
        prot.shape[0], _ptr(seq_slot, (torch.int32,), "seq_slot"),
        _ptr(block_table, (torch.int32,), "block_table"), block_table.shape[1],
        _ptr(seq_lens, (torch.int32,), "seq_lens"), int(max_seq_len), B, nq, H,
        float(softmax_scale), int(num_splits),
        None if workspace is None else ctypes.c_void_p(workspace.data_ptr()), ws_bytes,
        _ptr(out, (torch.float32,), "out"), _ptr(lse, (torch.float32,), "lse"), _stream(stream))
    _check("mla_decode_lowbit_mq", code)
    return out, lse


def mla_lb_channel_stat(x_bits, pct=99.9):
    """Host helper: per-channel pct-th percentile of |x| for bf16 bits
    x_bits (numpy uint16/int16 [rows, n]); returns float32 [n]."""
    import numpy as np
    x = np.ascontiguousarray(x_bits).view(np.uint16)
    rows, n = x.shape
    out = np.empty(n, np.float32)
    _check("mla_lb_channel_stat",
           _lib.mla_lb_channel_stat(x.ctypes.data, rows, n, float(pct), out.ctypes.data))
    return out


def mla_lb_smooth_scales(stat, alpha, pair_tied=False):
    """Host helper: s_j = max(a_j, 1e-8)^-alpha (pairs tied on request)."""
    import numpy as np
    a = np.ascontiguousarray(stat, dtype=np.float32)
    out = np.empty(a.shape[0], np.float32)
    _check("mla_lb_smooth_scales",
           _lib.mla_lb_smooth_scales(a.ctypes.data, a.shape[0], float(alpha), int(bool(pair_tied)),
                                     out.ctypes.data))
    return out


def mla_lb_hadamard_rows(x):
    """Host helper: x (numpy float32 [rows, n], n a power of two) times the
    normalized Hadamard matrix H_n; returns float32 [rows, n]."""
    import numpy as np
    a = np.ascontiguousarray(x, dtype=np.float32)
    if a.ndim != 2:
        raise ValueError(f"x: shape {a.shape}, expected (rows, n)")
    out = np.empty_like(a)
    _check("mla_lb_hadamard_rows",
           _lib.mla_lb_hadamard_rows(a.ctypes.data, a.shape[0], a.shape[1], out.ctypes.data))
    return out


def mla_lb_dequant_dump(fmt, pages, page_id, out=None, stream=None):
    """bf16 bits [64, 576] (int16) reconstructed by the decode kernel for one page."""
    pb = _lib.mla_lb_page_bytes(_fmt(fmt))
    if pb == 0:
        raise ValueError(f"unknown cache format {fmt!r}")
    _shape(pages, (None, pb), "pages")
    if out is not None:
        _shape(out, (64, 576), "out")
    _same_gpu("mla_lb_dequant_dump", ("pages", pages), ("out", out))
    if out is None:
        out = torch.empty((64, 576), dtype=torch.int16, device=pages.device)
    _check("mla_lb_dequant_dump",
           _lib.mla_lb_dequant_dump(_fmt(fmt), _ptr(pages, (torch.uint8,), "pages"),
                                    pages.shape[0], int(page_id), _ptr(out, _BF16, "out"),
                                    _stream(stream)))
    return out
