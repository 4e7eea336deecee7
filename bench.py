"""Benchmark of the binary-hash KV retrieval decode step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 2] [--hash i]
                    [--replicas R] [--no-cpu] [--prefill] [--exact] [--evict]
                    [--sign] [--no-window] [--unfused | --qheads | --varlen]

Default workload: retrieval at 512K tokens -- 8 KV heads x 524,288 cached 128-bit codes
(uniform random bits plus 1% planted near neighbours of the query code), top-1024 per
head, then exact attention over the 1024 selected bf16 K/V rows of each head.  One step
is hk_hamming_scan + hk_select_attend (together hk_retrieve_attend).  Other workloads
(--workload 0/1/3/4) run the whole step after the keys were encoded as one
hk_decode_step call: the query hash, the Hamming scan and select+attend (top-k list and
sink + local window, merged); the parts are also timed one by one.  With --unfused the
separate calls run instead (hk_retrieve_topk, hk_sparse_decode, ...).

Inputs are resident in HBM before timing.  R replicas of the per-step inputs (codes,
query codes, queries) rotate so that the bytes a step reads are not left in the 256 MB
Infinity Cache or the L2 by the previous steps.

Prints ONE JSON line.  `value` is microseconds per decode step (lower is better).
`roofline` describes the dominant kernel (the Hamming scan): algorithmic bytes per
launch over its average duration, timed with HIP events on the launch stream around
back-to-back launches.  `kernels["select+attend"]` gives the gather the same way (K/V row
bytes over the back-to-back duration of select + attend + merge).  `cpu_baseline` times
the CPU oracle on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "retrieve+sparse-attn µs/decode step @512K tok; achieved HBM GB/s vs peak"
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
KERNEL_SOURCES = ["include/hk.h", "hash_top_kv_amd/csrc/hk_internal.h",
                  "hash_top_kv_amd/csrc/select_core.h", "hash_top_kv_amd/csrc/attend_core.h",
                  "hash_top_kv_amd/csrc/retrieve.hip", "hash_top_kv_amd/csrc/attend.hip",
                  "hash_top_kv_amd/csrc/fused.hip", "hash_top_kv_amd/csrc/encode.hip",
                  "hash_top_kv_amd/csrc/evict.hip", "hash_top_kv_amd/csrc/exact.hip",
                  "hash_top_kv_amd/csrc/probe.hip", "hash_top_kv_amd/csrc/api.hip",
                  "include/hk_probe.h", "hash_top_kv_amd/csrc/encode_core.h",
                  "hash_top_kv_amd/csrc/tiny.hip"]


def _code_only(text: str) -> str:
    """C/C++ source without comments or layout: edits to comments keep the digest."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def source_digest(files=KERNEL_SOURCES) -> str:
    """Digest of what the kernels are built from: the sources (comments aside) and the
    build script with its compiler flags."""
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, f), encoding="utf-8") as fh:
            h.update(_code_only(fh.read()).encode())
    with open(os.path.join(ROOT, "hash_top_kv_amd", "build.py"), "rb") as fh:
        h.update(fh.read())
    return h.hexdigest()[:16]


def stream_read_rate(torch, hkp, mib=1024, reps=20):
    """Measured read rate beside the 8 TB/s spec peak: hk_read_probe (16-byte
    non-temporal loads, 2048 workgroups) over a 1 GiB buffer, launched back to back."""
    x = torch.ones((mib << 20) // 4, dtype=torch.int32, device="cuda")
    sink = hkp.read_probe(x)
    for _ in range(3):
        hkp.read_probe(x, sink)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        hkp.read_probe(x, sink)
    b.record()
    torch.cuda.synchronize()
    gbs = x.numel() * 4 * reps / (a.elapsed_time(b) * 1e6)
    del x, sink
    torch.cuda.empty_cache()
    return {"gbs": round(gbs, 1), "frac_of_peak": round(gbs / HBM_PEAK_GBS, 4),
            "how": "hk_read_probe: 1 GiB, 16-byte non-temporal loads, 20 launches back to back"}


def same_size_read_rate(torch, hkp, nbytes, reps=200):
    """hk_read_probe over exactly nbytes (the scan's algorithmic bytes), launched back to
    back over buffers rotated through 1 GiB so that no launch finds its data in a cache:
    what a pure read of that size reaches, launch ramp and drain included."""
    n = nbytes - nbytes % 16
    if n <= 0:
        return None
    R = min(64, max(1, -(-(1 << 30) // n)))
    bufs = [torch.ones(n // 4, dtype=torch.int32, device="cuda") for _ in range(R)]
    sink = hkp.read_probe(bufs[0])
    for i in range(2 * R):
        hkp.read_probe(bufs[i % R], sink)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for i in range(reps):
        hkp.read_probe(bufs[i % R], sink)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / reps
    del bufs, sink
    torch.cuda.empty_cache()
    return {"bytes": n, "us_per_launch": round(ms * 1e3, 3), "gbs": round(n / ms / 1e6, 1),
            "how": f"hk_read_probe: {n} bytes, {R} rotating buffers, {reps} launches back to back"}


def graph_us(torch, fns, reps):
    """Average time of one call of fns[i] when all of fns are captured, in order, in one
    HIP graph and the graph is replayed reps times (no host launch cost)."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for fn in fns:
            fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for fn in fns:
            fn()
    for _ in range(2):
        g.replay()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        g.replay()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / (reps * len(fns)) * 1e3


def same_rows_gather(torch, hkp, ctx, sel_fn, n_lists=8, reps=20):
    """hk_gather_probe over exactly the K/V rows that select+attend gathers (the row lists
    of n_lists consecutive steps, in the rotation of the step's own timing), at the best
    of a few workgroup sizes: a pure read of those rows, with nothing of the selection or
    the attention.  Both it and select+attend are timed as HIP-graph replays, so that the
    host's launch cost is in neither."""
    lists = [ctx["gather_rows"](i) for i in range(n_lists)]
    K, V = ctx["K"], ctx["V"]
    n = lists[0].numel()
    if n == 0:
        return None, None
    best = None
    for rpb in (256, 512, 1024, 2048):
        sink = hkp.gather_probe(K, V, lists[0], rpb)
        us = graph_us(torch, [lambda i=i, rpb=rpb, sink=sink: hkp.gather_probe(
            K, V, lists[i % n_lists], rpb, sink) for i in range(2 * n_lists)], reps)
        if best is None or us < best[0]:
            best = (us, rpb)
    sel_us = graph_us(torch, [lambda i=i: sel_fn(i) for i in range(n_lists)], 2 * reps)
    nbytes = n * 512
    rotated = nbytes * n_lists
    return ({"rows_256B": n, "bytes": nbytes, "us_per_launch": round(best[0], 3),
             "gbs": round(nbytes / best[0] / 1e3, 1), "rows_per_workgroup": best[1],
             # the K/V rows of the rotated lists fit in the 256 MB last-level cache: the
             # rate is then a cache-resident rate, not an HBM one
             "rotated_bytes": rotated, "cache_resident": rotated <= (256 << 20),
             "how": f"hk_gather_probe: the K and V rows of {n_lists} steps' selections and "
                    "windows, HIP-graph replay, best of 256/512/1024/2048 rows per workgroup"},
            sel_us)


def profile_tag(args, info) -> str:
    """Workload tag of the committed profile summaries: w<n>, plus the hash for the
    workload that runs two (w4_lsh64, w4_mlp128) and for sign codes (w3_sign128), and
    _nowin without the window, so that a variant never reads another command's figures."""
    tag = f"w{args.workload}"
    if args.workload == 4 or args.sign:
        tag += "_" + info.get("hash", "").replace("-", "")
    if args.no_window:
        tag += "_nowin"
    return tag


def read_trace(tag: str, kernel: str):
    """The committed rocprofv3 kernel-trace summary of this workload's step: the average
    durations of `kernel` (over its back-to-back dispatches and over all of them), if the
    kernel sources have not changed since it was taken (else None)."""
    path = os.path.join(ROOT, "profiles", f"decode_step_{tag}_kernel_trace.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if ":" in line and not line.startswith("#") and "|" not in line:
            k, v = line.split(":", 1)
            vals[k.strip()] = v.strip()
    if vals.get("source_digest") != source_digest():
        return None
    try:
        out = {"summary": os.path.relpath(path, ROOT),
               "back_to_back_avg_us": float(vals[f"{kernel}_back_to_back_avg_us"]),
               "all_dispatches_avg_us": float(vals[f"{kernel}_all_avg_us"])}
    except (KeyError, ValueError):
        return None
    for key in (f"{kernel}_back_to_back_median_gap_us", "read_probe_same_size_avg_us",
                f"{kernel}_tight_avg_us", f"{kernel}_tight_dispatches"):
        if key in vals:
            out[key.replace(f"{kernel}_", "")] = float(vals[key])
    return out


def read_traffic(name: str):
    """HBM bytes per launch of a kernel from a committed counter summary, if the kernel
    sources have not changed since it was taken (else None)."""
    path = os.path.join(ROOT, "profiles", f"{name}_counters.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            vals[k.strip()] = v.strip()
    if vals.get("source_digest") != source_digest():
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_info():
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count()
    model = ""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return cores, model


class Timer:
    """Pairs of HIP events on the current (launch) stream."""

    def __init__(self, torch, n):
        self.torch = torch
        self.ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(n)]
        self.i = 0

    def start(self):
        self.ev[self.i][0].record()

    def stop(self):
        self.ev[self.i][1].record()
        self.i += 1

    def mean_ms(self):
        return float(np.mean([a.elapsed_time(b) for a, b in self.ev[:self.i]]))


def build_retrieval_case(args, torch, hk, synth):
    """Workload 2: given codes; a step is hk_hamming_scan + hk_select_attend (the fused
    hk_retrieve_attend), or with --unfused hk_hamming_scan + hk_topk_select +
    hk_sparse_decode."""
    wl = synth.WORKLOADS[2]
    R = args.replicas
    kv = synth.make_kv(wl)
    K = synth.to_device(kv["K"], wl.dtype)
    V = synth.to_device(kv["V"], wl.dtype)
    reps = []
    for r in range(R):
        g = synth.make_given_codes(wl, replica=r)
        reps.append({"codes": synth.to_device(g["codes"], wl.dtype),
                     "qcodes": synth.to_device(g["qcodes"], wl.dtype),
                     "Q": synth.to_device(synth.make_q(wl, replica=r), wl.dtype),
                     "planted": (g["planted_pos"], g["planted_delta"]) if r == 0 else None})
    B, Hkv, N, k = wl.B, wl.Hkv, wl.N, wl.k
    idx = torch.empty((B, Hkv, k), dtype=torch.int32, device="cuda")
    count = torch.empty((B, Hkv), dtype=torch.int32, device="cuda")
    o = torch.empty((B, wl.Hq, 128), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, wl.Hq), dtype=torch.float32, device="cuda")
    # One workspace per replica: the select+attend timed back to back then rotates over
    # the R replicas' selections instead of replaying one.
    if args.unfused:
        wss = [hk.workspace(hk.retrieve_topk_workspace(128, B, Hkv, N, 0, 0, k)) for _ in range(R)]
        wsd = hk.workspace(hk.sparse_decode_workspace(B, wl.Hq, Hkv, k))
    else:
        wss = [hk.workspace(hk.retrieve_attend_workspace(128, B, wl.Hq, Hkv, N, 0, 0, k))
               for _ in range(R)]

    def scan(i):
        rp = reps[i % R]
        hk.hamming_scan(rp["codes"], rp["qcodes"], 128, N, 0, 0, k, wss[i % R])

    def rest(i):
        rp = reps[i % R]
        if args.unfused:
            hk.topk_select(128, B, Hkv, N, 0, 0, k, idx, count, wss[i % R])
            hk.sparse_decode(rp["Q"], K, V, idx, k, count=count, o=o, lse=lse, ws=wsd)
        else:
            hk.select_attend(128, rp["Q"], K, V, N, 0, 0, k, idx, count, o, lse, wss[i % R])

    def check():
        scan(0)
        rest(0)
        torch.cuda.synchronize()
        pos, dl = reps[0]["planted"]
        got = idx.cpu().numpy()
        for h in range(Hkv):
            order = np.lexsort((pos[0, h], dl[0, h]))
            want = np.sort(pos[0, h][order[:k]])
            assert np.array_equal(got[0, h], want), f"head {h}: top-k differs from the planted set"

    def gather_rows(i):
        """The K/V rows step i gathers, as rows of the [B*Hkv*N] table (no window)."""
        scan(i)
        rest(i)
        base = torch.arange(B * Hkv, device="cuda", dtype=torch.int64).view(B, Hkv, 1) * N
        return (idx[..., :k].to(torch.int64) + base).flatten().to(torch.int32)

    scan_bytes = B * Hkv * N * 16
    gather_bytes = B * Hkv * k * 2 * 128 * 2 + B * wl.Hq * 128 * 2
    info = {"workload": wl.name, "B": B, "Hq": wl.Hq, "Hkv": Hkv, "N": N, "k": k,
            "code_bits": 128, "kv_dtype": "bf16", "replicas": R,
            "rotating_code_bytes": R * scan_bytes,
            "step": ("hk_hamming_scan + hk_topk_select + hk_sparse_decode" if args.unfused
                     else "hk_hamming_scan + hk_select_attend (= hk_retrieve_attend)")}
    parts = [("hamming_scan", scan, scan_bytes), ("select+attend", rest, gather_bytes)]
    return parts, check, info, {"wl": wl, "reps": reps, "kv": kv, "K": K, "V": V,
                                "gather_rows": None if args.unfused else gather_rows}


def build_full_case(args, torch, hk, synth):
    """Workloads 0, 1, 3, 4: hk_encode_query + hk_hamming_scan + hk_select_attend (the
    whole step after the keys were encoded), or with --unfused the separate calls."""
    from hash_top_kv_amd.step import DecodeStep, QHeadStep, VarlenDecodeStep
    wl = synth.WORKLOADS[args.workload]
    if args.no_window:
        wl = synth.scaled(wl, n_sink=0, n_local=0, name=wl.name + ", no window")
    spec = synth.HashSpec("sign", 128) if args.sign else wl.hashes[args.hash]
    R = args.replicas
    kv = synth.make_kv(wl)
    K = synth.to_device(kv["K"], wl.dtype)
    V = synth.to_device(kv["V"], wl.dtype)
    del kv
    hnp = synth.make_hash(wl, spec, args.hash)
    h = hk.Hash(spec.kind, spec.bits, dtype=K.dtype, **synth.hash_to_device(hnp))
    codes = torch.empty((wl.B, wl.Hkv, wl.N, spec.words), dtype=torch.int32, device="cuda")
    hk.encode_keys(h, K, codes)
    torch.cuda.synchronize()
    # Copies of the code cache so that consecutive steps read codes from HBM, not from
    # the 256 MB Infinity Cache (only needed while the codes are small).
    C = wl.N - wl.n_sink - wl.n_local
    scan_bytes = wl.B * wl.Hkv * C * spec.bits // 8
    ncopies = 1 if scan_bytes * 1 >= (512 << 20) else max(1, min(R, -(-(512 << 20) // scan_bytes)))
    code_sets = [codes] + [codes.clone() for _ in range(ncopies - 1)]
    steps = [DecodeStep(K, V, cs, spec.bits, wl.N, wl.n_sink, wl.n_local, wl.k, wl.Hq, h)
             for cs in code_sets]
    qsteps = ([QHeadStep(K, V, cs, spec.bits, wl.N, wl.n_sink, wl.n_local, wl.k, wl.Hq, h)
               for cs in code_sets] if args.qheads else [])
    # Variable lengths: sequence b holds N - floor(b N / 2B) tokens (from N down to about
    # N/2), the budget stays the workload's k.
    lengths = [wl.N - (b * wl.N) // (2 * wl.B) for b in range(wl.B)]
    ctx_len = torch.tensor(lengths, dtype=torch.int32, device="cuda")
    vsteps = ([VarlenDecodeStep(K, V, cs, spec.bits, ctx_len, wl.N, wl.n_sink, wl.n_local, wl.k,
                                wl.Hq, h) for cs in code_sets] if args.varlen else [])
    Qs = [synth.to_device(synth.make_q(wl, replica=r), wl.dtype) for r in range(R)]

    def st(i):
        return steps[i % len(steps)]

    def enc(i):
        st(i).encode(Qs[i % R])

    def scan(i):
        st(i).scan(st(i).qcodes)

    def whole_step(i):
        st(i)(Qs[i % R])

    def rest(i):
        st(i).select_attend(Qs[i % R])

    def unfused(i):
        st(i).unfused(Qs[i % R])

    def qst(i):
        return qsteps[i % len(qsteps)]

    def var_step(i):
        vsteps[i % len(vsteps)](Qs[i % R])

    def q_enc(i):
        qst(i).encode(Qs[i % R])

    def q_ret(i):
        qst(i).retrieve(qst(i).qcodes)

    def q_att(i):
        qst(i).attend(Qs[i % R])

    def check():
        st(0)(Qs[0])
        torch.cuda.synchronize()
        assert bool((st(0).count == st(0).keff).all())
        if qsteps:
            qst(0)(Qs[0])
            torch.cuda.synchronize()
            assert bool((qst(0).count == qst(0).keff).all())

    def gather_rows(i):
        """The K/V rows step i gathers (each head's selection, then its window), as
        256-byte rows of the [B*Hkv*N] table (two per token for fp32)."""
        enc(i)
        scan(i)
        rest(i)
        s = st(i)
        base = torch.arange(wl.B * wl.Hkv, device="cuda", dtype=torch.int64).view(wl.B, wl.Hkv, 1) * wl.N
        win = s.win.to(torch.int64).view(1, 1, -1).expand(wl.B, wl.Hkv, -1)
        tok = torch.cat([s.idx[..., :s.keff].to(torch.int64), win], dim=2) + base
        if wl.dtype == "f32":
            tok = torch.stack([2 * tok, 2 * tok + 1], dim=-1)
        return tok.flatten().to(torch.int32)

    esz = 4 if wl.dtype == "f32" else 2
    s0 = steps[0]
    gather_bytes = wl.B * wl.Hkv * (s0.keff + s0.n_win) * 2 * 128 * esz
    info = {"workload": wl.name, "B": wl.B, "Hq": wl.Hq, "Hkv": wl.Hkv, "N": wl.N, "k": wl.k,
            "n_sink": wl.n_sink, "n_local": wl.n_local, "hash": f"{spec.kind}-{spec.bits}",
            "kv_dtype": wl.dtype, "replicas": R, "code_copies": ncopies,
            "step": ("hk_encode_query + hk_retrieve_topk + 2 x hk_sparse_decode + hk_lse_merge"
                     if args.unfused else
                     "hk_encode_query (per query head) + hk_retrieve_topk_qheads + "
                     "hk_sparse_decode_qheads + hk_sparse_decode (window) + hk_lse_merge"
                     if args.qheads else
                     "hk_encode_query + hk_retrieve_attend_varlen (lengths " +
                     ",".join(map(str, lengths)) + ")"
                     if args.varlen else
                     "hk_decode_step (one call: query hash, retrieval, attention)"
                     if args.workload in (0, 1) else
                     "hk_decode_step (one call: hk_encode_query + hk_hamming_scan + "
                     "hk_select_attend; sign codes hash the query inside the scan)")}
    if args.unfused:
        parts = [("decode_step", unfused, None)]
    elif args.varlen:
        parts = [("encode_query+retrieve_attend_varlen", var_step, None)]
    elif args.qheads:
        parts = [("encode_query", q_enc, None),
                 ("retrieve_topk_qheads", q_ret, scan_bytes),
                 ("attend_qheads+window+merge", q_att,
                  wl.B * wl.Hq * (s0.keff + s0.n_win) * 2 * 128 * esz)]
    elif args.workload in (0, 1):
        # latency-bound: hk_decode_step (c0's single head runs in one workgroup; c1's scan
        # hashes the query itself)
        parts = [("decode_step", whole_step, None)]
    else:
        parts = [("encode_query", enc, None), ("hamming_scan", scan, scan_bytes),
                 ("select+attend", rest, gather_bytes)]
    plain = not (args.unfused or args.varlen or args.qheads)
    # Workloads 3 and 4 time their parts separately but run the step as the one call
    # (hk_decode_step) that DecodeStep makes.
    return parts, check, info, {"wl": wl, "K": K, "V": V, "h": h, "codes": codes, "spec": spec,
                                "code_sets": code_sets, "Qs": Qs, "steps": steps, "qsteps": qsteps,
                                "gather_rows": gather_rows if plain else None,
                                "step": whole_step if plain and args.workload not in (0, 1) else None}


def qhead_overlap(torch, hk, ctx):
    """How much the G per-query-head selections of a KV head overlap: the IoU of every
    pair of query heads in a group (the traffic a deduplicated union would save)."""
    wl, qs = ctx["wl"], ctx["qsteps"][0]
    qs(ctx["Qs"][0])
    G = wl.Hq // wl.Hkv
    pairs = [(b, g * G + i, g * G + j) for b in range(wl.B) for g in range(wl.Hkv)
             for i in range(G) for j in range(i + 1, G)]
    if not pairs:
        return None
    bi = torch.tensor([p[0] for p in pairs], device="cuda")
    ha = torch.tensor([p[1] for p in pairs], device="cuda")
    hb = torch.tensor([p[2] for p in pairs], device="cuda")
    a, b = qs.idx[bi, ha].contiguous(), qs.idx[bi, hb].contiguous()
    ca, cb = qs.count[bi, ha].contiguous(), qs.count[bi, hb].contiguous()
    inter = hk.topk_intersect(a, ca, b, cb)
    torch.cuda.synchronize()
    i, x, y = (t.cpu().numpy().astype(np.float64) for t in (inter, ca, cb))
    iou = i / np.maximum(x + y - i, 1)
    return {"pairs": len(pairs), "iou_mean": round(float(iou.mean()), 4),
            "iou_max": round(float(iou.max()), 4)}


def time_prefill(torch, hk, ctx, steps):
    """MFMA key encode of the whole cache (prefill), bf16: flops per launch / duration."""
    wl, K, h, codes, spec = ctx["wl"], ctx["K"], ctx["h"], ctx["codes"], ctx["spec"]
    for _ in range(10):            # the clocks settle over the first milliseconds of work
        hk.encode_keys(h, K, codes)
    t = Timer(torch, steps)
    for _ in range(steps):
        t.start()
        hk.encode_keys(h, K, codes)
        t.stop()
    torch.cuda.synchronize()
    ms = t.mean_ms()
    M = wl.B * wl.Hkv * wl.N
    bytes_ = M * 128 * 2 + M * spec.bits // 8
    if spec.kind == "sign":                    # no product: bound by HBM
        return {"kernel": "encode_keys_sign", "rows": M, "us": ms * 1e3,
                "hbm_gbs": bytes_ / ms / 1e6, "frac_of_peak": bytes_ / ms / 1e6 / HBM_PEAK_GBS}
    flops = 2 * M * (128 * 256 + 256 * spec.bits) if spec.kind == "mlp" else 2 * M * 128 * spec.bits
    return {"kernel": f"encode_keys_mfma ({spec.kind}-{spec.bits})", "rows": M, "us": ms * 1e3,
            "tflops": flops / ms / 1e9, "mfma_frac": flops / ms / 1e9 / MFMA_BF16_PEAK_TFLOPS,
            "hbm_gbs": bytes_ / ms / 1e6}


def time_evict(torch, hk, synth, ctx, steps):
    """HashEvict's eviction step on the same cache (it runs after the decode-step timing:
    every step overwrites one slot per head).  Parts: the query hash + hk_evict_select
    (victim per head), the new key's hash + hk_evict_replace, and attention over every
    cached token; hk_evict_select alone, back to back over the code copies, for its HBM
    rate (b/8 bytes per candidate)."""
    from hash_top_kv_amd.step import EvictStep
    wl, K, V, h, spec = ctx["wl"], ctx["K"], ctx["V"], ctx["h"], ctx["spec"]
    sets, Qs = ctx["code_sets"], ctx["Qs"]
    es = [EvictStep(K, V, cs, spec.bits, wl.N, wl.n_sink, wl.n_local, wl.Hq, h) for cs in sets]
    new = synth.make_kv(synth.scaled(wl, N=1, wid=90))
    k_new = synth.to_device(np.ascontiguousarray(new["K"][:, :, 0]), wl.dtype)
    v_new = synth.to_device(np.ascontiguousarray(new["V"][:, :, 0]), wl.dtype)
    # check: every head has a victim among its candidates (parity is the tests' job)
    es[0].select(Qs[0])
    torch.cuda.synchronize()
    vic = es[0].victim.cpu().numpy()
    assert ((vic >= wl.n_sink) & (vic < wl.N - wl.n_local)).all()
    C = wl.N - wl.n_sink - wl.n_local
    scan_bytes = wl.B * wl.Hkv * C * spec.bits // 8
    esz = 4 if wl.dtype == "f32" else 2
    attend_bytes = wl.B * wl.Hkv * wl.N * 2 * 128 * esz
    R = len(Qs)

    def timed(fn, n):
        for i in range(4):
            fn(i)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for i in range(n):
            fn(i)
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / n * 1e3

    def sel_only(i):
        e = es[i % len(es)]
        hk.evict_select(e.codes, e.qcodes, spec.bits, wl.N, wl.n_sink, wl.n_local, e.victim, e.ws_e)

    us_sel = timed(sel_only, max(steps, 50))
    us_select = timed(lambda i: es[i % len(es)].select(Qs[i % R]), steps)
    us_replace = timed(lambda i: es[i % len(es)].replace(k_new, v_new), steps)
    us_attend = timed(lambda i: es[0].attend(Qs[i % R]), min(steps, 20))
    return {"step": "hk_encode_query + hk_evict_select, hk_encode_query + hk_evict_replace, "
                    "hk_sparse_decode over all tokens",
            "hash": f"{spec.kind}-{spec.bits}",
            "us_query_hash_and_select": round(us_select, 3),
            "us_key_hash_and_replace": round(us_replace, 3),
            "us_attend_all_tokens": round(us_attend, 3),
            "attend_gbs": round(attend_bytes / us_attend / 1e3, 1),
            "evict_select": {"us_per_launch": round(us_sel, 3), "alg_bytes": scan_bytes,
                             "gbs": round(scan_bytes / us_sel / 1e3, 1),
                             "frac_of_peak": round(scan_bytes / us_sel / 1e3 / HBM_PEAK_GBS, 4)}}


def time_exact(torch, hk, ctx, steps):
    """Exact top-k by logit (the "oracle top-k") on the same cache and query: its time and
    HBM rate (every candidate's K row read once), and the retrieval IoU of the hash top-k
    against it, per (batch, KV head)."""
    wl, K = ctx["wl"], ctx["K"]
    st, Q = ctx["steps"][0], ctx["Qs"][0]
    st(Q)
    idx_e, cnt_e = hk.exact_topk(Q, K, wl.N, wl.n_sink, wl.n_local, wl.k)
    ws = hk.workspace(hk.exact_topk_workspace(wl.B, wl.Hkv, wl.N, wl.n_sink, wl.n_local, wl.k))
    inter = hk.topk_intersect(st.idx, st.count, idx_e, cnt_e)
    torch.cuda.synchronize()
    i, a, b = (x.cpu().numpy().reshape(-1).astype(np.float64) for x in (inter, st.count, cnt_e))
    union = a + b - i
    iou = np.where(union > 0, i / np.maximum(union, 1), 1.0)
    n = max(5, min(steps, 50))
    for _ in range(3):
        hk.exact_topk(Q, K, wl.N, wl.n_sink, wl.n_local, wl.k, idx_e, cnt_e, ws)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(n):
        hk.exact_topk(Q, K, wl.N, wl.n_sink, wl.n_local, wl.k, idx_e, cnt_e, ws)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) / n * 1e3
    esz = 4 if wl.dtype == "f32" else 2
    nbytes = wl.B * wl.Hkv * (wl.N - wl.n_sink - wl.n_local) * 128 * esz
    return {"call": "hk_exact_topk", "us": round(us, 3), "alg_bytes": nbytes,
            "gbs": round(nbytes / us / 1e3, 1), "frac_of_peak": round(nbytes / us / 1e3 / HBM_PEAK_GBS, 4),
            "hash": ctx["spec"].kind + "-" + str(ctx["spec"].bits),
            "iou_hash_vs_exact": {"mean": round(float(iou.mean()), 4), "min": round(float(iou.min()), 4),
                                  "max": round(float(iou.max()), 4), "heads": int(iou.size)}}


def _oracle_head_worker(job, barrier, results):
    """One CPU worker: builds one (batch, KV head)'s inputs, waits for every worker to be
    ready, then times the oracle's decode step of that head repeatedly for `seconds`: the
    group's query hash, Hamming distances over every cached code, the stable-argsort
    top-k, the widening of the selected and window rows from their stored form,
    attention of the G query heads over both sets and the log-sum-exp merge.  Puts
    (median seconds, repetitions) on `results`."""
    import oracle
    import synth
    wid, hidx, sign, no_window, b, g, seconds = job
    wl = synth.WORKLOADS[wid]
    if no_window:
        wl = synth.scaled(wl, n_sink=0, n_local=0)
    G = wl.Hq // wl.Hkv
    kv = synth.make_kv(wl, heads=[(b, g)])
    Ks, Vs = kv["K"][b, g].copy(), kv["V"][b, g].copy()      # stored form
    del kv
    q = oracle.widen(synth.make_q(wl)[b, g * G:(g + 1) * G], wl.dtype)
    qcode = hp = None
    if sign or wl.hashes:
        spec = synth.HashSpec("sign", 128) if sign else wl.hashes[hidx]
        hp = oracle.prepare_hash(synth.make_hash(wl, spec, hidx))
        codes = np.concatenate([oracle.encode(oracle.widen(Ks[r:r + 32768], wl.dtype), hp)[0]
                                for r in range(0, wl.N, 32768)])   # the cache's codes
    else:                                                           # codes given directly
        gc = synth.make_given_codes(wl, heads=[(b, g)])
        codes, qcode = gc["codes"][b, g].copy(), gc["qcodes"][b, g]
    scale = 1.0 / math.sqrt(wl.d)
    win = oracle.window_indices(wl.N, wl.n_sink, wl.n_local)

    def step():
        qc = qcode if hp is None else oracle.encode_query(q[None], hp, 1)[0][0, 0]
        idx = oracle.select_topk(codes, qc, wl.N, wl.n_sink, wl.n_local, wl.k)
        K1, V1 = oracle.widen(Ks[idx], wl.dtype), oracle.widen(Vs[idx], wl.dtype)
        K2, V2 = oracle.widen(Ks[win], wl.dtype), oracle.widen(Vs[win], wl.dtype)
        for h in range(G):
            o1, l1 = oracle.attend(q[h], K1, V1, scale)
            o2, l2 = oracle.attend(q[h], K2, V2, scale)
            oracle.lse_merge(np.stack([o1, o2]), np.array([l1, l2]))

    step()
    barrier.wait()
    times = []
    t_end = time.perf_counter() + seconds
    while time.perf_counter() < t_end or not times:
        t0 = time.perf_counter()
        step()
        times.append(time.perf_counter() - t0)
    results.put((float(np.median(times)), len(times)))


def cpu_baseline_run(args):
    """The CPU oracle on every host core (a process of its own, started with one BLAS
    thread per worker, that never touches the GPU): P = min(cores, heads) workers each
    time one (batch, KV head)'s oracle decode step, all at once; a whole step over all
    B*Hkv heads on P cores takes ceil(B*Hkv / P) rounds of the median head time."""
    import multiprocessing as mp
    import synth
    cores, model = cpu_info()
    wl = synth.WORKLOADS[args.workload]
    heads = [(b, g) for b in range(wl.B) for g in range(wl.Hkv)]
    P = max(1, min(cores, len(heads)))
    ctx = mp.get_context("fork")
    barrier, results = ctx.Barrier(P), ctx.Queue()
    procs = [ctx.Process(target=_oracle_head_worker,
                         args=((args.workload, args.hash, args.sign, args.no_window, b, g,
                                args.cpu_seconds), barrier, results))
             for b, g in heads[:P]]
    for p in procs:
        p.start()
    res = [results.get() for _ in procs]
    for p in procs:
        p.join()
    per_head = float(np.median([r[0] for r in res]))
    rounds = -(-len(heads) // P)
    us = per_head * rounds * 1e6
    return {"value": round(us, 1), "unit": "us/step", "cores": P, "kind": "oracle",
            "sample": f"{P} of the {len(heads)} (batch, KV head) decode steps, one per core, "
                      f"timed together for {args.cpu_seconds:g} s ({sum(r[1] for r in res)} "
                      f"repetitions): median {per_head * 1e3:.2f} ms per head; a step is "
                      f"{rounds} round(s) of {P} heads. NumPy float64, one BLAS thread per "
                      f"process; host has {cores} usable cores ({model})"}


def cpu_baseline(args):
    """Runs cpu_baseline_run in a child process (this one has initialised the GPU)."""
    import subprocess
    env = dict(os.environ, OMP_NUM_THREADS="1", OPENBLAS_NUM_THREADS="1", MKL_NUM_THREADS="1")
    cmd = [sys.executable, os.path.abspath(__file__), "--cpu-baseline-only",
           "--workload", str(args.workload), "--hash", str(args.hash),
           "--cpu-seconds", str(args.cpu_seconds)]
    if args.sign:
        cmd.append("--sign")
    if args.no_window:
        cmd.append("--no-window")
    r = subprocess.run(cmd, capture_output=True, text=True, env=env, timeout=600)
    if r.returncode != 0:
        raise RuntimeError(f"CPU baseline failed:\n{r.stderr[-2000:]}")
    return json.loads(r.stdout.strip().splitlines()[-1])


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", type=int, default=2)
    ap.add_argument("--hash", type=int, default=0, help="index of the workload's hash (workload 4: 0 = LSH-64, 1 = MLP-128)")
    ap.add_argument("--replicas", type=int, default=8)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--prefill", action="store_true", help="also time the key encode of the whole cache")
    ap.add_argument("--prefill-only", action="store_true",
                    help="only time the key encode of the whole cache (workloads 0, 1, 3, 4)")
    ap.add_argument("--no-kernel-timing", action="store_true")
    ap.add_argument("--no-graph", action="store_true",
                    help="skip the HIP-graph replay of the step")
    ap.add_argument("--no-window", action="store_true",
                    help="no sink or local window (s = w = 0): retrieval alone, the variant "
                         "without a static window")
    ap.add_argument("--sign", action="store_true",
                    help="use sign codes of the keys themselves (128 bits) instead of the "
                         "workload's hash")
    ap.add_argument("--varlen", action="store_true",
                    help="time the step for sequences of different lengths (N down to N/2)")
    ap.add_argument("--qheads", action="store_true",
                    help="time the per-query-head selection variant of the step instead")
    ap.add_argument("--exact", action="store_true",
                    help="also time the exact top-k by logit and report the hash top-k's IoU with it")
    ap.add_argument("--evict", action="store_true",
                    help="also time HashEvict's eviction step on the same cache (last)")
    ap.add_argument("--unfused", action="store_true",
                    help="run the step through the separate calls instead of the fused one")
    ap.add_argument("--cpu-baseline-only", action="store_true",
                    help="only time the CPU oracle on the workload (no GPU) and print its JSON")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MB",
                    help="only run a plain device copy of MB megabytes 10 times (calibrates "
                         "the HBM byte counters) and exit")
    args = ap.parse_args()

    if args.cpu_baseline_only:
        print(json.dumps(cpu_baseline_run(args)), flush=True)
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (the step would "
              "shard by (batch, KV head), with no exchange inside a step)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import hash_top_kv_amd as hk
    from hash_top_kv_amd import probe as hkp
    import synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    torch.cuda.set_device(0)
    if args.copy_probe:
        n = args.copy_probe << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dsts = [torch.empty(n, dtype=torch.uint8, device="cuda") for _ in range(2)]
        for i in range(10):
            dsts[i % 2].copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": n, "launches": 10}))
        return
    build = build_retrieval_case if args.workload == 2 else build_full_case
    parts, check, info, ctx = build(args, torch, hk, synth)
    if args.prefill_only:
        if args.workload == 2:
            print("workload 2 has no key encode (its codes are given)", file=sys.stderr)
            sys.exit(2)
        pre = time_prefill(torch, hk, ctx, max(args.steps, 1))
        print(json.dumps({"metric": "key encode (prefill) of the whole cache", "config": info,
                          "prefill": pre}), flush=True)
        return
    check()

    one_call = ctx.get("step")

    def step(i):
        if one_call is not None:
            one_call(i)
            return
        for _, fn, _ in parts:
            fn(i)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # Timed region: exactly K steps, synchronised on both sides.
    t0 = time.perf_counter()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(args.steps):
        step(i)
    e1.record()
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3
    ms_step = e0.elapsed_time(e1) / args.steps

    # The same steps replayed from a HIP graph: one graph holds one step per input
    # replica (the replicas rotate as in the eager loop), captured after the eager
    # timing on a side stream of default priority.
    graph = None
    if not args.no_graph:
        R = len(ctx.get("Qs", ctx.get("reps", [None])))
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for i in range(R):
                step(i)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(R):
                step(i)
        for _ in range(3):
            g.replay()
        torch.cuda.synchronize()
        reps = max(1, args.steps // R)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            g.replay()
        b.record()
        torch.cuda.synchronize()
        graph = {"us_per_step": round(a.elapsed_time(b) / (reps * R) * 1e3, 3),
                 "steps": reps * R, "steps_per_graph": R}
        check()

    kern = {}
    pct = None
    if not args.no_kernel_timing:
        # The whole step between its own event pair, for the spread of step times; then
        # each part of the step with an event pair around it inside the step loop (the
        # pairs add their own overhead, so these figures are upper bounds).
        whole = Timer(torch, args.steps)
        for i in range(args.steps):
            whole.start()
            step(i)
            whole.stop()
        torch.cuda.synchronize()
        d = np.array([a.elapsed_time(b) for a, b in whole.ev[:whole.i]]) * 1e3
        pct = {"p10": round(float(np.percentile(d, 10)), 3), "p50": round(float(np.median(d)), 3),
               "p90": round(float(np.percentile(d, 90)), 3),
               "note": "one event pair around each step (the pair adds its own overhead)"}
        timers = [Timer(torch, args.steps) for _ in parts]
        for i in range(args.steps):
            for (name, fn, _), t in zip(parts, timers):
                t.start()
                fn(i)
                t.stop()
        torch.cuda.synchronize()
        for (name, fn, nbytes), t in zip(parts, timers):
            ms = t.mean_ms()
            ent = {"us_in_step": round(ms * 1e3, 3)}
            if nbytes:
                ent["alg_bytes"] = nbytes
                ent["gbs_in_step"] = round(nbytes / ms / 1e6, 1)
            kern[name] = ent
        # The Hamming scan alone, launched back to back over rotating code replicas
        # between one event pair: its average launch duration.
        scan = [p for p in parts if p[0] == "hamming_scan"]
        if scan:
            _, fn, nbytes = scan[0]
            n = max(args.steps, 50)
            for i in range(8):
                fn(i)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            for i in range(n):
                fn(i)
            b.record()
            torch.cuda.synchronize()
            ms = a.elapsed_time(b) / n
            # The same launches captured back to back in a HIP graph and replayed: no host
            # launch cost, and in a profiler's trace each of these dispatches starts as
            # the previous one ends, the condition of the event timing above.
            us_graph = graph_us(torch, [lambda i=i: fn(i) for i in range(8)], 25)
            kern["hamming_scan"].update({"us_per_launch": round(ms * 1e3, 3),
                                         "gbs": round(nbytes / ms / 1e6, 1),
                                         "frac_of_peak": round(nbytes / ms / 1e6 / HBM_PEAK_GBS, 4),
                                         "us_per_launch_graph": round(us_graph, 3)})
        # Select + attend + merge alone, back to back the same way: each workspace still
        # holds its last scan's distances and histograms, so every launch is a complete
        # selection and gather.  Its K/V row bytes per launch / duration = the gather rate
        # (threshold, compaction and merge included).
        sel = [p for p in parts if p[0] == "select+attend"]
        if sel and sel[0][2]:
            _, fn, nbytes = sel[0]
            n = max(args.steps, 50)
            for i in range(8):
                fn(i)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            for i in range(n):
                fn(i)
            b.record()
            torch.cuda.synchronize()
            ms = a.elapsed_time(b) / n
            kern["select+attend"].update({"us_per_launch": round(ms * 1e3, 3),
                                          "gbs": round(nbytes / ms / 1e6, 1),
                                          "frac_of_peak": round(nbytes / ms / 1e6 / HBM_PEAK_GBS, 4)})
            if ctx.get("gather_rows"):
                same, sel_us = same_rows_gather(torch, hkp, ctx, fn)
                if same:
                    kern["select+attend"]["us_per_launch_graph"] = round(sel_us, 3)
                    kern["select+attend"]["same_rows_gather"] = same
                    kern["select+attend"]["frac_of_same_rows_gather"] = round(
                        same["us_per_launch"] / sel_us, 4)

    roofline = None
    sc = kern.get("hamming_scan", {})
    stream = None if args.no_kernel_timing else stream_read_rate(torch, hkp)
    if "gbs" in sc:
        a = sc["gbs"]
        tag = profile_tag(args, info)
        roofline = {"kernel": "hamming_scan", "bound": "hbm", "achieved": a, "peak": HBM_PEAK_GBS,
                    "unit": "GB/s", "frac": round(a / HBM_PEAK_GBS, 4),
                    "traffic": read_traffic(f"hamming_scan_{tag}"),
                    "alg_bytes_per_launch": sc["alg_bytes"], "us_per_launch": sc["us_per_launch"],
                    "us_per_launch_graph": sc.get("us_per_launch_graph")}
        # The same kernel in the committed rocprofv3 trace of this command.  The profiler
        # leaves gaps between most dispatches, and a dispatch that starts on an idle GPU
        # pays the launch ramp that back-to-back launches overlap with the previous
        # kernel's drain; the dispatches that start as the previous one ends (graph
        # replays) are the condition of the event timing, and their average is the one
        # compared with it.
        tr = read_trace(tag, "hamming_scan")
        if tr:
            for key in ("back_to_back_avg_us", "all_dispatches_avg_us", "tight_avg_us"):
                if key in tr:
                    tr["frac_" + key[:-7]] = round(sc["alg_bytes"] / tr[key] / 1e3 / HBM_PEAK_GBS, 4)
            if "tight_avg_us" in tr:
                tr["events_over_trace_tight"] = round(sc["us_per_launch"] / tr["tight_avg_us"], 4)
        roofline["trace"] = tr
        if stream:
            roofline["frac_of_measured_read"] = round(a / stream["gbs"], 4)
            same = same_size_read_rate(torch, hkp, sc["alg_bytes"])
            if same:
                stream["same_size_as_scan"] = same
                roofline["frac_of_same_size_read"] = round(a / same["gbs"], 4)
                # What starting on an idle GPU costs: the trace's dispatches after a gap
                # against the event timing, for the scan and for the plain read of the
                # same bytes (a kernel that is nothing but the read).
                if tr and "read_probe_same_size_avg_us" in tr:
                    tr["isolated_minus_events_us"] = {
                        "hamming_scan": round(tr["back_to_back_avg_us"] - sc["us_per_launch"], 3),
                        "same_size_read": round(tr["read_probe_same_size_avg_us"] - same["us_per_launch"], 3)}
    out = {"metric": METRIC, "value": round(ms_step * 1e3, 3), "unit": "us/step", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 6),
           "higher_is_better": False, "scaling": "weak", "vs_baseline": None,
           "dtype": "u32+" + ("f32" if info.get("kv_dtype") == "f32" else "bf16"),
           "data": "synthetic",
           "config": info, "roofline": roofline, "kernels": kern,
           "step_us_spread": pct, "hip_graph": graph, "stream_read": stream,
           "wall_ms_timed_region": round(wall_ms, 3)}
    if args.prefill and args.workload != 2:
        out["prefill"] = time_prefill(torch, hk, ctx, 10)
    if args.qheads and args.workload != 2:
        out["qhead_overlap"] = qhead_overlap(torch, hk, ctx)
    if args.exact and args.workload != 2:
        out["exact_topk"] = time_exact(torch, hk, ctx, args.steps)
    if args.evict and args.workload != 2:
        out["evict"] = time_evict(torch, hk, synth, ctx, min(args.steps, 200))
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(args)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
