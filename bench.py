"""Benchmark of the low-bit MLA decode hot path on one MI355X.

    python bench.py [--steps K] [--warmup W] [--config N] [--step fused|separate] [--no-cpu] [--no-graph]

One step = one decode step of a whole batch through the C ABI: the writer
for each sequence's current token (quantize, pack, slot-mapped insert, BF16
window refresh), then decode over every cached token (paged low-bit + BF16
protected rows, one global softmax, split-KV merge).  By default both run in
one launch (mla_decode_lowbit_append); --step separate times kv_quant_append
followed by mla_decode_lowbit.
The default workload is the largest single-GPU one, the 128K cache-pressure
C4R4 cache: batch 8, 128 heads sharing one latent (DeepSeek-V2 shape), 96K to
128K tokens per sequence, 64-token pages with a shuffled block table, the
writer of every sequence's newest token interleaved with each decode step.

Inputs are synthetic and seeded (bit_mla_kv_quant_amd.synth), uploaded before
timing.  To keep the 256 MB last-level cache from serving the KV history, the
bench cycles R full replicas of every input (pages, protection buffers,
queries, tables) whose total exceeds 1 GiB; step i uses replica i mod R.
Each replica's step is captured once in a HIP graph and replayed.

Printed: ONE JSON line with the KV-tokens/s of the whole step, plus
  roofline      the decode call's algorithmic bytes / its average duration
                (HIP events around back-to-back decode-only replays on the
                stream they run on), against the 8 TB/s HBM peak;
  cpu_baseline  the CPU oracle decoding a bounded sample of the same workload
                on the host cores.
"""

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "low-bit MLA decode KV-tokens/s + achieved HBM TB/s vs MI355X peak"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, published
PAGE = 64
PROT_ROWS = 132
ROW_BYTES = 576 * 2            # one bf16 cache row [c | k_R]
TOKEN_BYTES = {"C4R4": 324, "C2R4": 196, "C4R4F": 328}   # packed codes + (scale, zero) per token
KERNEL_SOURCES = ("bit_mla_kv_quant_amd/csrc/decode.hip", "bit_mla_kv_quant_amd/csrc/decode_h16.hip",
                  "bit_mla_kv_quant_amd/csrc/decode_h128.hip", "bit_mla_kv_quant_amd/csrc/dequant.h",
                  "bit_mla_kv_quant_amd/csrc/common.h", "bit_mla_kv_quant_amd/csrc/quantize.h",
                  "bit_mla_kv_quant_amd/csrc/internal.h", "bit_mla_kv_quant_amd/build.py")


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def rows128(rows):
    """The library's choice of decode kernel for `rows` query rows per
    sequence: the 128-row kernel when 5 * ceil(rows / 128) < ceil(rows / 16)."""
    return 5 * -(-rows // 128) < -(-rows // 16)


def n_protected(L):
    return min(L, 4) + max(0, min(128, L - 4)) if L > 0 else 0


def algorithmic_bytes(fmt, lens, H, nq=1):
    """Bytes the decode call must move: packed history of unprotected tokens,
    bf16 rows of protected ones, queries, outputs, block-table entries
    (nq queries of H heads per sequence)."""
    kv = sum((L - n_protected(L)) * TOKEN_BYTES[fmt] + n_protected(L) * ROW_BYTES for L in lens)
    B = len(lens)
    q = B * nq * H * 576 * 2
    out = B * nq * H * 513 * 4
    bt = sum(-(-L // PAGE) * 4 for L in lens)
    return kv + q + out + bt


def algorithmic_flops(lens, H, nq=1):
    """Score and aggregation FLOPs: query j of a length-L sequence sees
    L - nq + 1 + j tokens."""
    seen = sum(max(0, L - nq + 1 + j) for L in lens for j in range(nq))
    return seen * H * 2 * (576 + 512)


def kernel_source_hash():
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def stored_traffic(workload):
    """HBM bytes per decode launch from the committed rocprofv3 counter
    summary, or None if absent or taken on other kernel sources."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json.txt")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    return rec.get("hbm_bytes_per_launch")


def cache_accounting(ops, fmt, lens):
    """Persistent cache bytes of the batch in the library's layout against a
    BF16 paged cache: per sequence, its pages (plus an 8-byte reverse page
    map each) and one protection buffer, against 64 x 1152 bytes per page."""
    pb, prot = ops.mla_lb_page_bytes(fmt), ops.mla_lb_prot_bytes_per_seq()
    packed = sum(-(-L // PAGE) * (pb + 8) + prot for L in lens)
    bf16 = sum(-(-L // PAGE) * PAGE * ROW_BYTES for L in lens)
    return {"packed": packed, "bf16": bf16, "ratio": round(bf16 / packed, 4)}


# --------------------------------------------------------------- workload ---
def upload(ops, torch, d, fmt, dev):
    """Page pool + protection buffers filled through kv_quant_append with the
    first L_b - nq tokens of every sequence (the last nq are the step's new
    tokens, nq = queries per sequence)."""
    B = d.B
    nq = d.wl.queries
    pb = ops.mla_lb_page_bytes(fmt)
    pages = torch.zeros((d.num_pages, pb), dtype=torch.uint8, device=dev)
    prot = torch.zeros((B, PROT_ROWS, 576), dtype=torch.int16, device=dev)

    def i16(x):
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to(dev)

    seq_slot = torch.arange(B, dtype=torch.int32, device=dev)
    for b in range(B):
        L = int(d.lens[b]) - nq
        if L <= 0:
            continue
        P = np.arange(L, dtype=np.int64)
        ops.kv_quant_append(
            fmt, i16(d.c[b][:L]), i16(d.kr[b][:L]),
            torch.from_numpy(d.slots(b, P)).to(dev),
            torch.full((L,), b, dtype=torch.int32, device=dev),
            torch.from_numpy(P.astype(np.int32)).to(dev),
            torch.full((L,), L, dtype=torch.int32, device=dev), pages, prot)
    # the step's own tokens per sequence: positions L_b - nq .. L_b - 1,
    # sequence length L_b (sequence-major, nq per sequence)
    newpos = [np.arange(int(d.lens[b]) - nq, int(d.lens[b]), dtype=np.int64) for b in range(B)]
    step = {
        "latent": i16(np.concatenate([d.c[b][newpos[b]] for b in range(B)])),
        "k_rope": i16(np.concatenate([d.kr[b][newpos[b]] for b in range(B)])),
        "slot": torch.from_numpy(np.concatenate([d.slots(b, newpos[b]) for b in range(B)])).to(dev),
        "seq_slot": torch.from_numpy(np.repeat(np.arange(B, dtype=np.int32), nq)).to(dev),
        "pos": torch.from_numpy(np.concatenate(newpos).astype(np.int32)).to(dev),
        "new_len": torch.from_numpy(np.repeat(d.lens.astype(np.int32), nq)).to(dev),
    }
    torch.cuda.synchronize()
    return {
        "pages": pages, "prot": prot, "seq_slot": seq_slot,
        "block_table": torch.from_numpy(d.block_table).to(dev),
        "seq_lens": torch.from_numpy(d.lens.astype(np.int32)).to(dev),
        "q_lat": i16(d.q_lat).view(B, nq, d.H, 512) if nq > 1 else i16(d.q_lat),
        "q_rope": i16(d.q_rope).view(B, nq, d.H, 64) if nq > 1 else i16(d.q_rope),
        "step": step,
    }


def clone_replica(torch, r):
    out = {}
    for k, v in r.items():
        out[k] = {kk: vv.clone() for kk, vv in v.items()} if isinstance(v, dict) else v.clone()
    return out


def footprint(r):
    n = 0
    for v in r.values():
        vals = v.values() if isinstance(v, dict) else [v]
        n += sum(t.numel() * t.element_size() for t in vals)
    return n


# ------------------------------------------------------------ cpu leg ------
def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def _oracle_leg(d, fmt, budget_s, threads):
    """The CPU oracle (as it stands) decoding whole sequences of the workload,
    cycling through the batch, with BLAS limited to `threads`, until about
    budget_s seconds of work are done (at least one sequence).  The two
    phases are timed apart: unpack + dequantize (the fp32 quantizer and
    reconstruction of every token, oracle.attention.effective_rows) and fp64
    attention (oracle.attention.attend / the causal form for several
    queries)."""
    import threadpoolctl
    from oracle import attention, quant
    t_deq = t_att = 0.0
    tokens = nseq = 0
    nq = d.wl.queries
    with threadpoolctl.threadpool_limits(limits=threads, user_api="blas"):
        used = max([i.get("num_threads", 1) for i in threadpoolctl.threadpool_info()
                    if i.get("user_api") == "blas"] or [1])
        while True:
            b = nseq % d.B
            L = int(d.lens[b])
            t0 = time.perf_counter()
            rows = attention.effective_rows(d.c[b][:L], d.kr[b][:L], fmt)
            t1 = time.perf_counter()
            ql = quant.bf16_to_f32(d.q_lat[b]).astype(np.float64)
            qr = quant.bf16_to_f32(d.q_rope[b]).astype(np.float64)
            if nq > 1:
                ql, qr = ql.reshape(nq, d.H, 512), qr.reshape(nq, d.H, 64)
                for j in range(nq):
                    n = L - nq + 1 + j
                    if n > 0:
                        attention.attend(ql[j], qr[j], rows[:n], d.scale)
            else:
                attention.attend(ql, qr, rows, d.scale)
            t2 = time.perf_counter()
            t_deq += t1 - t0
            t_att += t2 - t1
            tokens += L
            nseq += 1
            if t_deq + t_att >= budget_s:
                break
    return {"tokens": tokens, "sequences": nseq, "dequant_s": round(t_deq, 3),
            "attention_s": round(t_att, 3), "blas_threads": int(used),
            "kv_tokens_per_s": round(tokens / (t_deq + t_att), 1),
            "dequant_kv_tokens_per_s": round(tokens / t_deq, 1),
            "attention_kv_tokens_per_s": round(tokens / t_att, 1)}


def cpu_baseline(d, fmt, budget_s=12.0, budget_1t_s=8.0):
    """The oracle timed on the host: once with BLAS on every core of this
    process's affinity set, once on one thread; phases reported apart."""
    import threadpoolctl
    aff = sorted(os.sched_getaffinity(0))
    ncores = len(aff)
    allc = _oracle_leg(d, fmt, budget_s, ncores)
    one = _oracle_leg(d, fmt, budget_1t_s, 1)
    blas = [i for i in threadpoolctl.threadpool_info() if i.get("user_api") == "blas"]
    blas_name = (f"{blas[0].get('internal_api')} {blas[0].get('version')}" if blas else "none")
    return {"value": allc["kv_tokens_per_s"], "unit": "KV-tokens/s", "cores": allc["blas_threads"],
            "kind": "oracle",
            "sample": (f"{allc['sequences']} whole-sequence decodes cycling over the {d.B} "
                       f"sequences of the same workload ({allc['tokens']} KV tokens, "
                       f"{d.wl.queries} x {d.H} query rows): fp32 quantize + dequantize of every "
                       f"token {allc['dequant_s']} s, fp64 attention {allc['attention_s']} s, "
                       f"BLAS on {allc['blas_threads']} threads"),
            "all_cores": allc, "one_thread": one,
            "host": {"cpu_model": _cpu_model(), "nproc": os.cpu_count(),
                     "affinity_cores": ncores, "affinity": f"{aff[0]}-{aff[-1]}" if aff else "",
                     "blas": blas_name}}


# ------------------------------------------------------------------ main ---
def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    # The timed region carries a fixed cost of about 0.6 ms (the first launch
    # and the closing synchronisations): 3000 steps keep it near 0.04% of the
    # default workload's step loop (about 1.5 s) and 0.5% of the shortest
    # (the 8K V2-Lite one, 0.13 s).
    ap.add_argument("--steps", type=int, default=3000)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--config", type=int, default=4,
                    help="synthetic workload id (0-7); default 4, the largest: 128K cache "
                         "pressure, B8 H128, append interleaved")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle leg")
    ap.add_argument("--no-graph", action="store_true", help="launch eagerly instead of graphs")
    ap.add_argument("--splits", type=int, default=0,
                    help="splits per max-length sequence (0: the library's automatic plan)")
    ap.add_argument("--step", choices=("fused", "separate"), default="fused",
                    help="fused: mla_decode_lowbit_append (writer inside the decode launch); "
                         "separate: kv_quant_append then mla_decode_lowbit")
    ap.add_argument("--min-rotation-gib", type=float, default=1.0)
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="also run one device copy of this size (HBM counter calibration)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}); "
              "the decode path has no multi-GPU leg in this library.", file=sys.stderr)
        sys.exit(2)

    import torch
    from bit_mla_kv_quant_amd import ops, synth   # raises if libmla_lowbit.so is missing

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    wl = synth.WORKLOADS[args.config]
    fmt = wl.fmt
    log("workload", wl.name, "drawing")
    d = synth.draw(wl, extra_tokens=0)
    lens = [int(x) for x in d.lens]
    B, H = d.B, d.H
    nq = wl.queries
    max_len = max(lens)
    if nq > 1 and args.step == "fused":
        args.step = "separate"        # the fused writer serves one new token per sequence

    log("uploading + filling cache through kv_quant_append")
    base = upload(ops, torch, d, fmt, dev)
    fp = footprint(base)
    R = max(1, math.ceil(args.min_rotation_gib * (1 << 30) / fp))
    reps = [base] + [clone_replica(torch, base) for _ in range(R - 1)]
    torch.cuda.synchronize()
    log(f"replicas {R} x {fp / 2**20:.1f} MiB")

    ws_bytes = ops.mla_decode_lowbit_mq_workspace(fmt, B, nq, H, max_len, args.splits)
    oshape = (B, nq, H) if nq > 1 else (B, H)
    for r in reps:
        r["ws"] = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
        r["out"] = torch.empty(oshape + (512,), dtype=torch.float32, device=dev)
        r["lse"] = torch.empty(oshape, dtype=torch.float32, device=dev)

    stream = torch.cuda.Stream()   # default priority

    def do_append(r):
        s = r["step"]
        ops.kv_quant_append(fmt, s["latent"], s["k_rope"], s["slot"], s["seq_slot"], s["pos"],
                            s["new_len"], r["pages"], r["prot"], stream=stream)

    def do_decode(r):
        fn = ops.mla_decode_lowbit_mq if nq > 1 else ops.mla_decode_lowbit
        fn(fmt, r["q_lat"], r["q_rope"], r["pages"], r["prot"], r["seq_slot"],
           r["block_table"], r["seq_lens"], max_len, d.scale, args.splits,
           workspace=r["ws"] if ws_bytes else None, out=r["out"], lse=r["lse"], stream=stream)

    def do_fused(r):
        s = r["step"]
        ops.mla_decode_lowbit_append(fmt, s["latent"], s["k_rope"], r["q_lat"], r["q_rope"],
                                     r["pages"], r["prot"], r["seq_slot"], r["block_table"],
                                     r["seq_lens"], max_len, d.scale, args.splits,
                                     workspace=r["ws"] if ws_bytes else None, out=r["out"],
                                     lse=r["lse"], stream=stream)

    def do_step(r):
        if args.step == "fused":
            do_fused(r)
        else:
            do_append(r)
            do_decode(r)

    use_graph = not args.no_graph
    steps_fn, dec_fn = [], []
    if use_graph:
        with torch.cuda.stream(stream):
            for r in reps:          # one eager pass first (warms the library)
                do_step(r)
        stream.synchronize()
        for r in reps:
            g1, g2 = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
            with torch.cuda.graph(g1, stream=stream):
                do_step(r)
            with torch.cuda.graph(g2, stream=stream):
                do_decode(r)
            steps_fn.append(g1.replay)
            dec_fn.append(g2.replay)
        graphs_keepalive = steps_fn, dec_fn  # noqa: F841
    else:
        steps_fn = [(lambda r=r: do_step(r)) for r in reps]
        dec_fn = [(lambda r=r: do_decode(r)) for r in reps]

    if args.copy_probe_mib:
        n = args.copy_probe_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            dst.copy_(src)
        stream.synchronize()
        log(f"copy probe: {n} bytes read + {n} bytes written")
        del src, dst

    # ---- warmup
    with torch.cuda.stream(stream):
        for i in range(args.warmup):
            steps_fn[i % R]()
    stream.synchronize()

    # ---- timed region: exactly K steps
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    with torch.cuda.stream(stream):
        for i in range(args.steps):
            steps_fn[i % R]()
    stream.synchronize()
    torch.cuda.synchronize()
    t_steps = time.perf_counter() - t0
    ms_per_step = 1e3 * t_steps / args.steps
    kv_tokens = sum(lens)
    value = kv_tokens / (t_steps / args.steps)

    # ---- decode-only launches, HIP events on the stream they run on
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        for i in range(min(args.warmup, R)):
            dec_fn[i % R]()
        ev0.record(stream)
        for i in range(args.steps):
            dec_fn[i % R]()
        ev1.record(stream)
    ev1.synchronize()
    dec_ms = ev0.elapsed_time(ev1) / args.steps
    ab = algorithmic_bytes(fmt, lens, H, nq)
    fl = algorithmic_flops(lens, H, nq)
    achieved_gbs = ab / (dec_ms * 1e-3) / 1e9
    achieved_tflops = fl / (dec_ms * 1e-3) / 1e12
    # which roof binds: bytes at 8 TB/s vs flops at 2.5 PF
    mfma_bound = fl / (BF16_PEAK_TFLOPS * 1e12) > ab / (HBM_PEAK_GBS * 1e9)
    if mfma_bound:
        roof = {"bound": "mfma", "achieved": round(achieved_tflops, 2), "peak": BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved_tflops / BF16_PEAK_TFLOPS, 4)}
    else:
        roof = {"bound": "hbm", "achieved": round(achieved_gbs, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved_gbs / HBM_PEAK_GBS, 4)}
    roof["traffic"] = stored_traffic(wl.name)
    entry = "mla_decode_lowbit_mq" if nq > 1 else "mla_decode_lowbit"
    roof["kernel"] = (f"{entry} (decode128_kernel + combine_kernel)" if rows128(nq * H)
                      else f"{entry} (decode16w_kernel + combine_kernel)")
    roof["algorithmic_bytes_per_launch"] = ab
    roof["algorithmic_flops_per_launch"] = fl
    roof["launch_ms"] = round(dec_ms, 5)
    roof["hbm_frac"] = round(achieved_gbs / HBM_PEAK_GBS, 4)

    # ---- append-only timing (context)
    with torch.cuda.stream(stream):
        ev0.record(stream)
        for i in range(args.steps):
            do_append(reps[i % R])
        ev1.record(stream)
    ev1.synchronize()
    app_ms = ev0.elapsed_time(ev1) / args.steps

    res = {
        "metric": METRIC, "value": round(value, 1), "unit": "KV-tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "format": fmt, "batch": B, "heads": H, "queries": nq,
                   "context": [min(lens), max(lens)], "page_tokens": PAGE,
                   "d_c": 512, "d_r": 64, "sink": 4, "recent": 128, "replicas": R,
                   "hip_graph": use_graph, "parallelism": "split-kv on 1 GPU",
                   "step": ("mla_decode_lowbit_append (writer of the B new tokens fused "
                            "into the decode launch)" if args.step == "fused" else
                            f"kv_quant_append({nq if nq > 1 else ''}B tokens) + {entry}")},
        "roofline": roof,
        "decode_kv_tokens_per_s": round(kv_tokens / (dec_ms * 1e-3), 1),
        "append_ms": round(app_ms, 5),
        "packed_bytes_per_token": TOKEN_BYTES[fmt], "bf16_bytes_per_token": ROW_BYTES,
        "cache_bytes": cache_accounting(ops, fmt, lens),
    }
    if not args.no_cpu:
        log("cpu oracle leg")
        res["cpu_baseline"] = cpu_baseline(d, fmt)
    else:
        res["cpu_baseline"] = None
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
