#!/usr/bin/env python3
"""Benchmark of the CSA/HCA attention core on one MI355X.

Headline workload: the 1M-context CSA decode, Pro-like -- 16 sequences,
1,048,576 cached tokens each (262,144 compressed entries, m = 4), fp8 (e4m3)
indexer keys with per-row scales (64 heads x 128), top-k 1024, bf16 MQA over
512-wide entries for 128 query heads, 128-token window, sink.  One step = the
whole hot path for one new token per sequence: compress (window row, newest
entry, newest indexer key), indexer score, top-k, sparse MQA.  Inputs are
synthetic (seeded N(0,1), U(0,1) head weights) and resident in HBM before
timing starts.

Timing: each input replica's step is captured once as a HIP graph; the timed
steps replay the graphs round-robin over replicas whose working set exceeds
twice the 256 MB Infinity Cache, so no step finds the previous step's data
there.  The K timed steps run back to back between two events (the headline
ms_per_step); a second pass brackets every step with timing-only events for
the median and the 10th / 90th percentiles, and times the indexer launch
inside each step (the roofline's kernel).

Prints ONE JSON line.  Also reported, each against its roofline: the same 1M
decode with MXFP4 indexer keys (the FP4 query-key path) and the recall of its
selection against the fp8 one, the Flash-like CSA decode (8 sequences x 16,384
entries, k = 512), the HCA dense decode (4 sequences x 8,192 entries), the
HCA and 1M CSA decodes with mixed KV rows (e4m3 codes under a row scale plus
bf16 rotated dims, 580 bytes per row instead of 1,024), the cache append, the
prefill indexer (16,384 queries x 32,768 entries, bf16), each call of the
chunked-prefill step and the grouped output projection (prefill and decode
rows); and the fp64 oracle timed on a bounded sample of the decode workload on
the host cores.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFS = 2500.0    # dense bf16 matrix peak
MALL_BYTES = 256 << 20         # Infinity Cache


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-secondary", action="store_true",
                    help="skip the Flash-like decode, HCA decode and prefill-step measurements")
    ap.add_argument("--no-graph", action="store_true", help="launch eagerly instead of replaying graphs")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="repeat the oracle's sample until this much CPU time has passed")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 512 MiB device copy (3x) to calibrate HBM byte counters")
    return ap.parse_args()


# ---------------------------------------------------------------------------
# timing helpers
# ---------------------------------------------------------------------------
class TimingEvent:
    """A HIP event made for timing only (hipEventDisableSystemFence): recording it
    skips the system-scope cache writeback and invalidation that a default event
    performs, which costs several microseconds of idle GPU per record on MI355X.
    Elapsed times are read after a full device synchronisation."""
    _hip = None

    def __init__(self):
        import torch
        if TimingEvent._hip is None:
            TimingEvent._hip = ctypes.CDLL("libamdhip64.so")
        self._torch = torch
        self.h = ctypes.c_void_p()
        st = TimingEvent._hip.hipEventCreateWithFlags(ctypes.byref(self.h), ctypes.c_uint(0x20000000))
        if st != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed ({st})")

    def record(self):
        stream = ctypes.c_void_p(self._torch.cuda.current_stream().cuda_stream)
        if TimingEvent._hip.hipEventRecord(self.h, stream) != 0:
            raise RuntimeError("hipEventRecord failed")

    def elapsed_time(self, end) -> float:
        ms = ctypes.c_float()
        if TimingEvent._hip.hipEventElapsedTime(ctypes.byref(ms), self.h, end.h) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def __del__(self):
        if self.h and TimingEvent._hip is not None:
            TimingEvent._hip.hipEventDestroy(self.h)


def capture(fns, use_graph: bool):
    """One HIP graph per function (each a replica's step or part of it); returns
    the replay callables and None, or the eager functions and the reason the
    capture was not used."""
    import torch
    if not use_graph:
        return list(fns), "disabled"
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    try:
        with torch.cuda.stream(s):
            for fn in fns:          # warm on the capture stream first
                fn()
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        graphs = []
        for fn in fns:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=s):
                fn()
            graphs.append(g)
        torch.cuda.synchronize()
        capture.keep.extend(graphs)
        return [g.replay for g in graphs], None
    except Exception as e:  # noqa: BLE001 -- reported in the JSON line
        torch.cuda.synchronize()
        return list(fns), f"{type(e).__name__}: {e}"


capture.keep = []


def _pct(xs, q):
    xs = sorted(xs)
    if not xs:
        return None
    pos = q * (len(xs) - 1)
    lo = int(pos)
    hi = min(lo + 1, len(xs) - 1)
    return xs[lo] + (xs[hi] - xs[lo]) * (pos - lo)


def time_rotating(steps, K: int, warmup: int):
    """K steps replayed round-robin over the replicas, back to back between two
    events; returns the average ms per step."""
    import torch
    R = len(steps)
    for s in range(warmup):
        steps[s % R]()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for s in range(K):
        steps[s % R]()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / K


def time_each(parts, K: int, inner: int | None = None):
    """K steps, each a sequence of replica parts with a timing-only event before
    every part and after the last; returns per-step ms and, for part `inner`,
    per-launch ms."""
    import torch
    R = len(parts)
    n = len(parts[0])
    ev = [[TimingEvent() for _ in range(n + 1)] for _ in range(K)]
    torch.cuda.synchronize()
    for s in range(K):
        for p in range(n):
            ev[s][p].record()
            parts[s % R][p]()
        ev[s][n].record()
    torch.cuda.synchronize()
    per_step = [ev[s][0].elapsed_time(ev[s + 1][0]) for s in range(K - 1)]
    per_inner = [ev[s][inner].elapsed_time(ev[s][inner + 1]) for s in range(K)] if inner is not None else []
    return per_step, per_inner


def dist(xs):
    return {"median": round(_pct(xs, 0.5), 5), "p10": round(_pct(xs, 0.1), 5),
            "p90": round(_pct(xs, 0.9), 5), "mean": round(sum(xs) / len(xs), 5), "n": len(xs)}


def _roof(achieved: float, bound: str, **extra) -> dict:
    peak, unit = (HBM_PEAK_GBS, "GB/s") if bound == "hbm" else (MFMA_BF16_PEAK_TFS, "TFLOP/s")
    d = {"bound": bound, "achieved": round(achieved, 2), "peak": peak, "unit": unit,
         "frac": round(achieved / peak, 4)}
    d.update(extra)
    return d


def replicas_for(bytes_per_replica: float, at_least: int = 2) -> int:
    """Replicas whose combined working set is at least twice the Infinity Cache."""
    need = int((2 * MALL_BYTES + bytes_per_replica - 1) // max(bytes_per_replica, 1))
    return max(at_least, need)


def traffic_from_profiles(kernel_tag: str, src_file: str):
    """HBM bytes per launch measured with rocprofv3 --pmc (FETCH_SIZE + WRITE_SIZE,
    copy-kernel calibrated), valid only while the kernel source is unchanged."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"{kernel_tag}.pmc.md")
    if not os.path.exists(path):
        return None
    txt = open(path).read()
    m_b = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)", txt)
    m_h = re.search(r"source_sha256:\s*([0-9a-f]{64})", txt)
    if not (m_b and m_h):
        return None
    cur = hashlib.sha256(open(src_file, "rb").read()).hexdigest()
    return float(m_b.group(1)) if cur == m_h.group(1) else None


# ---------------------------------------------------------------------------
# algorithmic work of the decode steps (bytes every step must move once; the
# fp32 scores between the indexer and the top-k are an intermediate and are
# not counted)
# ---------------------------------------------------------------------------
def kv_row_bytes(wl) -> int:
    """Bytes of one stored entry or window row: d values of the storage type, or
    a mixed row (d - rope_dim e4m3 codes, rope_dim bf16 values, an fp32 scale)."""
    if wl.kv_dtype == "mixed":
        return (wl.d - wl.rope_dim) + 2 * wl.rope_dim + 4
    return wl.d * {"bf16": 2, "f32": 4}[wl.kv_dtype]


def csa_decode_bytes(wl) -> dict:
    esz = {"mxfp4": 0.5, "e4m3": 1, "bf16": 2, "f32": 4}
    kv = esz[wl.dtype]
    B, N, dI, H, k, d = wl.B, wl.N_cap, wl.d_I, wl.H_I, wl.k, wl.d
    keys = int(B * N * dI * esz[wl.k_dtype])
    scales = {"e4m3": B * N * 4, "mxfp4": B * N * (dI // 32)}.get(wl.k_dtype, 0)
    q_index = B * (H * dI * 2 + H * 4)
    gather = B * k * kv_row_bytes(wl)
    window = B * wl.n_win * kv_row_bytes(wl)
    q = out = B * wl.n_h * d * kv
    idx = B * k * 4
    # the step's compressions: the new token's window row (one bf16 candidate
    # row), the newest KV entry and indexer key (2m candidates of C and Z
    # each); the three rows written
    new_in = B * 2 * (d + 4 * wl.m * d + 4 * wl.m * dI)
    new_out = B * (2 * kv_row_bytes(wl) + int(dI * esz[wl.k_dtype]) + {"e4m3": 4, "mxfp4": dI // 32}.get(wl.k_dtype, 0))
    compress = new_in + new_out
    step = keys + scales + gather + window + q + out + q_index + idx + compress
    return {"step": step, "index_kernel": keys + scales + q_index, "front_kernel": keys + scales + q_index + compress,
            "keys": keys, "scales": scales, "gather": gather, "window": window, "q": q, "out": out,
            "q_index_w_idx": q_index + idx, "compress": compress}


def hca_decode_bytes(wl) -> dict:
    n_vis = min(wl.N_cap, (wl.q_pos0 + 1) // wl.m)
    entries = wl.B * n_vis * kv_row_bytes(wl)
    tail = wl.B * 2 * wl.m * wl.d * 2          # C and Z of the recompressed block
    window = wl.B * wl.n_win * kv_row_bytes(wl)
    qo = 2 * wl.B * wl.n_h * wl.d * 2
    return {"step": entries + tail + window + qo, "attention": entries + window + qo}


# ---------------------------------------------------------------------------
# workloads
# ---------------------------------------------------------------------------
def csa_decode(wl, K: int, warmup: int, use_graph: bool, keep_raw_first: bool = False):
    """A CSA decode workload: R replicas, whole-step graphs (pass 1) and the
    step's three parts launched directly between timing-only events (pass 2:
    per-step distribution and the indexer's launch time; an event pair around
    a graph launch would also count the graph's own launch latency)."""
    import torch

    from long_context_attention_02_amd.pipeline import CSADecode
    ab = csa_decode_bytes(wl)
    per_replica = ab["step"]
    R = replicas_for(per_replica)
    runs = [CSADecode(wl, "cuda", keep_raw=(keep_raw_first and r == 0)) for r in range(R)]
    torch.cuda.synchronize()
    steps, err = capture([r.step for r in runs], use_graph)
    ms_step = time_rotating(steps, K, warmup)
    # the front (the step's compressions and the indexer: one launch where the
    # library covers it) timed on its own; with two launches, the indexer's
    fused = bool(runs[0].fused_front)
    if fused:
        parts = [[r.front, (lambda r=r: (r.select(), r.attend()))] for r in runs]
    else:
        parts = [[r.compress_new, r.index, (lambda r=r: (r.select(), r.attend()))] for r in runs]
    for s in range(warmup):
        for f in parts[s % R]:
            f()
    per_step, per_index = time_each(parts, K, inner=0 if fused else 1)
    res = {"workload": wl.name, "replicas": R, "graph": err or "hip graph replay",
           "ms_per_step": ms_step, "step_ms_with_events": dist(per_step), "fused_front": fused,
           "index_ms": dist(per_index), "bytes": ab}
    if fused:
        # the indexer launch alone (csa_index_score on the same rows), for comparison
        # with the fused launch that also runs the step's compressions
        _, alone = time_each([[r.index] for r in runs], K, inner=0)
        res["index_alone_ms"] = dist(alone)
    return res, runs


def hca_decode(K: int, warmup: int, use_graph: bool, wl=None):
    """Dense MQA (HCA) decode: 4 sequences over 8,192 entries of 128 tokens each (1M
    context) plus window and sink; the step also recompresses the newest block.
    Entries and window rows in bf16, or as mixed rows (wl = HCA_DECODE_MIXED)."""
    import torch

    from long_context_attention_02_amd.pipeline import HCADecode
    from synth.workloads import HCA_DECODE
    wl = wl or HCA_DECODE

    ab = hca_decode_bytes(wl)
    R = replicas_for(ab["step"])
    runs = [HCADecode(wl, "cuda", keep_raw=False) for _ in range(R)]
    steps, err = capture([r.step for r in runs], use_graph)
    ms_step = time_rotating(steps, K, warmup)
    pre = [r.compress_new for r in runs]
    att = [r.attend for r in runs]
    per_step, per_attn = time_each([[pre[r], att[r]] for r in range(R)], K, inner=1)
    pre_ms = [a - b for a, b in zip(per_step, per_attn)]
    n_vis = min(wl.N_cap, (wl.q_pos0 + 1) // wl.m)
    flops = 4.0 * wl.B * wl.n_h * (n_vis + wl.n_win) * wl.d
    attn_ms = _pct(per_attn, 0.5)
    out = {"workload": wl.name, "replicas": R, "graph": err or "hip graph replay",
           "ms_per_step": round(ms_step, 5), "tokens/s": round(wl.B / (ms_step * 1e-3), 1),
           "step_ms_with_events": dist(per_step), "compress_ms": dist(pre_ms),
           "hca_dense_mqa_ms": dist(per_attn), "algorithmic_bytes": ab,
           "roofline": _roof(ab["step"] / (ms_step * 1e-3) / 1e9, "hbm", scope="whole step"),
           "attention_roofline": _roof(ab["attention"] / (attn_ms * 1e-3) / 1e9, "hbm",
                                       kernel="hca_dense_mqa (attention + combine)"),
           "attention_TFLOP/s": round(flops / (attn_ms * 1e-3) / 1e12, 2)}
    del runs, steps, pre, att
    capture.keep.clear()
    torch.cuda.empty_cache()
    return out


def prefill_indexer(steps: int, warmup: int):
    """csa_index_score on the chunked-prefill shapes: 16,384 queries over 32,768 entries."""
    import torch

    import long_context_attention_02_amd as csa
    from synth import Gen
    from synth.workloads import CSA_PREFILL_PRO as wl, T_KI, T_QI, T_WI

    g = Gen(wl.wid, "cuda")
    qI = g.normal(T_QI, (1, wl.Tq, wl.H_I, wl.d_I), "bf16")
    wI = g.uniform(T_WI, (1, wl.Tq, wl.H_I))
    K = g.normal(T_KI, (1, wl.N_cap, wl.d_I), "bf16")
    pos = (wl.q_pos0 + torch.arange(wl.Tq, dtype=torch.int32, device="cuda")).view(1, -1).contiguous()
    I = torch.empty((1, wl.Tq, wl.N_cap), dtype=torch.float32, device="cuda")
    for _ in range(warmup):
        csa.csa_index_score(qI, wI, K, pos, I, m=wl.m)
    torch.cuda.synchronize()
    # every launch timed on its own (timing-only events); the median is reported
    ev = [(TimingEvent(), TimingEvent()) for _ in range(steps)]
    for a, b in ev:
        a.record()
        csa.csa_index_score(qI, wI, K, pos, I, m=wl.m)
        b.record()
    torch.cuda.synchronize()
    per = [a.elapsed_time(b) for a, b in ev]
    ms = _pct(per, 0.5)
    pairs = sum(min(wl.N_cap, (wl.q_pos0 + t + 1) // wl.m) for t in range(wl.Tq))
    flops = 2.0 * pairs * wl.H_I * wl.d_I
    tfs = flops / (ms * 1e-3) / 1e12
    del qI, wI, K, I
    torch.cuda.empty_cache()
    return {"workload": wl.name, "ms": dist(per), "TFLOP/s": round(tfs, 2), "causal_flops": flops,
            "roofline": _roof(tfs, "mfma")}


def _timed(fn, steps: int, warmup: int) -> list:
    """Per-call ms of fn() over `steps` calls, timing-only events on the current stream."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    ev = [(TimingEvent(), TimingEvent()) for _ in range(steps)]
    for a, b in ev:
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in ev]


def prefill_rows(steps: int, warmup: int):
    """The chunked-prefill step (16,384 queries over 32,768 entries, k = 1024) call by
    call: compression of the chunk, indexer, top-k and sparse MQA."""
    import torch

    from long_context_attention_02_amd.pipeline import CSAPrefill
    from synth.workloads import CSA_PREFILL_PRO as wl

    run = CSAPrefill(wl, "cuda", keep_raw=False)
    per = {"compress": _timed(run.compress_new, steps, warmup), "index": _timed(run.index, steps, warmup),
           "topk": _timed(run.select, steps, warmup), "sparse_mqa": _timed(run.attend, steps, warmup)}
    ms = {k: _pct(v, 0.5) for k, v in per.items()}
    n_new = run.s_new1 - run.s_new0
    n_vis = [min(wl.N_cap, (wl.q_pos0 + t + 1) // wl.m) for t in range(wl.Tq)]
    # compress: window rows (read + write), candidates of the new KV entries and indexer keys
    # (C and Z of sets a and b, 2 * 2m rows each), entries written
    comp_bytes = (2 * wl.B * wl.Tq * wl.d * 2 + wl.B * n_new * (4 * wl.m * (wl.d + wl.d_I) * 2
                                                                + (wl.d + wl.d_I) * 2))
    topk_bytes = 4 * wl.B * sum(n_vis) + 4 * wl.B * wl.Tq * wl.k
    attn_flops = 4.0 * wl.B * wl.Tq * wl.n_h * (wl.k + wl.n_win) * wl.d
    index_flops = 2.0 * wl.B * sum(n_vis) * wl.H_I * wl.d_I
    out = {"workload": wl.name, "ms": {k: round(v, 4) for k, v in ms.items()}, "calls": steps,
           "compress": {"algorithmic_bytes": comp_bytes,
                        "roofline": _roof(comp_bytes / (ms["compress"] * 1e-3) / 1e9, "hbm")},
           "index": {"flops": index_flops,
                     "roofline": _roof(index_flops / (ms["index"] * 1e-3) / 1e12, "mfma")},
           "topk": {"algorithmic_bytes": topk_bytes,
                    "roofline": _roof(topk_bytes / (ms["topk"] * 1e-3) / 1e9, "hbm")},
           "sparse_mqa": {"flops": attn_flops,
                          "roofline": _roof(attn_flops / (ms["sparse_mqa"] * 1e-3) / 1e12, "mfma")}}
    del run
    torch.cuda.empty_cache()
    return out


def grouped_out_proj(steps: int, warmup: int):
    """The grouped output projection of the Pro-like attention outputs: 128 heads x 512
    in 16 groups, each projected to 1,024, then the 16,384-wide concatenation to 7,168.
    At 16,384 rows (a prefill chunk) against the bf16 MFMA peak; at 16 rows (a decode
    step) against HBM, since the 369 MB of weights dominate (two weight replicas
    alternate, so the Infinity Cache cannot hold them)."""
    import torch

    import long_context_attention_02_amd as csa
    from synth import Gen

    n_h, c, G, d_g, d = 128, 512, 16, 1024, 7168
    W = n_h * c // G
    g = Gen(7, "cuda")
    weights = [((g.normal(2 + 10 * r, (G, d_g, W), "f32", per_slot=False) / W ** 0.5).to(torch.bfloat16),
                (g.normal(3 + 10 * r, (d, G * d_g), "f32", per_slot=False) / (G * d_g) ** 0.5).to(torch.bfloat16))
               for r in range(2)]
    wbytes = (G * d_g * W + d * G * d_g) * 2
    out = {"shape": {"heads": n_h, "head_dim": c, "groups": G, "d_g": d_g, "d": d}}
    for T, label in ((16384, "prefill_16384_rows"), (16, "decode_16_rows")):
        o = g.normal(1, (T, n_h, c), "bf16", per_slot=False)
        y = torch.empty((T, G * d_g), dtype=torch.bfloat16, device="cuda")
        res = torch.empty((T, d), dtype=torch.bfloat16, device="cuda")
        ws = torch.empty(max(csa.csa_out_proj_workspace_size(T, n_h, c, G, d_g, d), 1), dtype=torch.uint8,
                         device="cuda")
        calls = [(lambda W1=W1, W2=W2: csa.csa_grouped_out_proj(o, W1, W2, y, res, workspace=ws))
                 for W1, W2 in weights]
        it = iter(range(10 ** 9))
        per = _timed(lambda: calls[next(it) % 2](), steps, warmup)
        ms = _pct(per, 0.5)
        flops = 2.0 * T * (n_h * c * d_g + G * d_g * d)
        nbytes = wbytes + (T * n_h * c + 2 * T * G * d_g + T * d) * 2
        entry = {"ms": dist(per), "flops": flops, "bytes": nbytes,
                 "TFLOP/s": round(flops / (ms * 1e-3) / 1e12, 2), "GB/s": round(nbytes / (ms * 1e-3) / 1e9, 1)}
        entry["roofline"] = (_roof(flops / (ms * 1e-3) / 1e12, "mfma") if T > 64
                             else _roof(nbytes / (ms * 1e-3) / 1e9, "hbm"))
        out[label] = entry
        del o, y, res, ws
        torch.cuda.empty_cache()
    del weights
    torch.cuda.empty_cache()
    return out


def cache_append(steps: int, warmup: int):
    """csa_cache_append at the Pro shapes (c = 512, indexer 128 fp8, m = 4, m' = 128,
    window 128): a decode step appending one token to 16 sequences at a position
    where a CSA and an HCA block complete (the step's most work), and a 16,384-token
    prefill chunk of one sequence."""
    import torch

    import long_context_attention_02_amd as csa
    from synth import Gen

    c, dI, m, mh, W_cap = 512, 128, 4, 128, 128
    R = csa.cache_ring_slots(m, mh)
    names = ("Ca", "Za", "Cb", "Zb", "ICa", "IZa", "ICb", "IZb", "Ch", "Zh", "Wraw")
    g = Gen(9, "cuda")
    out = {}
    for B, n_new, T0, label in ((16, 1, 1048575, "decode_16x1_token"), (1, 16384, 114688, "prefill_1x16384")):
        new = {k: g.normal(i + 1, (B, n_new, dI if k.startswith("I") else c), "bf16", per_slot=False)
               for i, k in enumerate(names)}
        N_csa, N_hca = (T0 + n_new) // m + 1, (T0 + n_new) // mh + 1
        st = dict(tail=torch.zeros((B, R, 6 * c + 4 * dI), dtype=torch.bfloat16, device="cuda"),
                  E_csa=torch.zeros((B, N_csa, c), dtype=torch.bfloat16, device="cuda"),
                  K_idx=torch.zeros((B, N_csa, dI), dtype=torch.float8_e4m3fn, device="cuda"),
                  K_scale=torch.ones((B, N_csa), dtype=torch.float32, device="cuda"),
                  E_hca=torch.zeros((B, N_hca, c), dtype=torch.bfloat16, device="cuda"),
                  W=torch.zeros((B, W_cap, c), dtype=torch.bfloat16, device="cuda"))
        T0t = torch.full((B,), T0, dtype=torch.int32, device="cuda")
        gamma = torch.ones(c, dtype=torch.float32, device="cuda")

        def call():
            csa.csa_cache_append(T0t, new, st["tail"], st["E_csa"], st["K_idx"], st["E_hca"], st["W"], m=m,
                                 m_hca=mh, K_scale=st["K_scale"], gamma=gamma, rope_dim=64)
        per = _timed(call, steps, warmup)
        ms = _pct(per, 0.5)
        n_csa = (T0 + n_new) // m - T0 // m
        n_hca = (T0 + n_new) // mh - T0 // mh
        nbytes = B * (n_new * (7 * c + 4 * dI) * 2            # new rows read
                      + min(n_new, W_cap) * c * 2               # window rows written
                      + n_csa * (c * 2 + dI + 4)                # entries and keys written
                      + n_hca * c * 2                           # HCA entries written
                      + min(n_new, R) * (6 * c + 4 * dI) * 2)   # tail ring written
        out[label] = {"ms": dist(per), "csa_entries": n_csa, "hca_entries": n_hca, "bytes": nbytes,
                      "roofline": _roof(nbytes / (ms * 1e-3) / 1e9, "hbm")}
        del new, st
        torch.cuda.empty_cache()
    return out


def cpu_baseline(run, seconds: float):
    """The fp64 oracle on all sequences of the same decode step, repeated until
    `seconds` of host time have passed (at least once)."""
    from threadpoolctl import threadpool_info

    from oracle import steps
    from tests._pipeline_ref import csa_decode_params

    wl = run.wl
    inputs = [csa_decode_params(run, b) for b in range(wl.B)]   # decoding the bytes is not timed
    n = 0
    t0 = time.perf_counter()
    while True:
        for p, rows in inputs:
            steps.csa_decode_sequence(p, rows)
            n += 1
        dt = time.perf_counter() - t0
        if dt >= seconds:
            break
    threads = max([d.get("num_threads", 1) for d in threadpool_info()] + [1])
    return {"value": round(n / dt, 4), "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{n} sequence-steps ({n // wl.B} passes over all {wl.B} sequences of one step), "
                      f"full step each (fp64 numpy; BLAS threads {threads}, host nproc {os.cpu_count()})",
            "seconds": round(dt, 3)}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (the CSA/HCA core "
              "runs on a single MI355X here)", file=sys.stderr)
        sys.exit(2)
    import torch

    from synth.workloads import (CSA_DECODE_1M as wl, CSA_DECODE_1M_MIXED, CSA_DECODE_1M_MX4, CSA_DECODE_FLASH,
                                 HCA_DECODE_MIXED)

    torch.cuda.set_device(0)
    use_graph = not args.no_graph
    K = args.steps
    head, runs = csa_decode(wl, K, args.warmup, use_graph, keep_raw_first=not args.no_cpu_baseline)
    ms_step = head["ms_per_step"]
    ab = head["bytes"]
    tokens_s = wl.B / (ms_step * 1e-3)
    idx_ms = head["index_ms"]["mean"]
    fused = head["fused_front"]
    kern_bytes = ab["front_kernel"] if fused else ab["index_kernel"]
    kern_name = ("index_decode_front (csa_decode_front: the step's compressions beside the indexer)" if fused
                 else "index_mfma_decode (csa_index_score)")
    idx_gbs = kern_bytes / (idx_ms * 1e-3) / 1e9
    step_gbs = ab["step"] / (ms_step * 1e-3) / 1e9
    src = os.path.join(ROOT, "long_context_attention_02_amd", "csrc", "index_score.hip")
    traffic = traffic_from_profiles("index_decode_front_1M_fp8" if fused else "index_score_decode_1M_fp8", src)

    result = {
        "metric": "CSA decode tokens/s + HBM GB/s at 1M ctx; indexer prefill TFLOP/s (%peak)",
        "value": round(tokens_s, 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "batch": wl.B, "context_tokens": wl.ctx,
                   "compressed_entries": wl.N_cap, "m": wl.m, "top_k": wl.k, "indexer": "64x128 e4m3",
                   "query_heads": wl.n_h, "entry_dim": wl.d, "window": wl.n_win},
        "timing": {"replicas": head["replicas"], "launch": head["graph"],
                   "step_ms_with_events": head["step_ms_with_events"]},
        "roofline": {"bound": "hbm", "kernel": kern_name,
                     "achieved": round(idx_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(idx_gbs / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "algorithmic_bytes": kern_bytes,
                     "avg_launch_ms": round(idx_ms, 5), "launch_ms": head["index_ms"],
                     "indexer_alone": None if "index_alone_ms" not in head else {
                         "kernel": "index_mfma_decode (csa_index_score, the same rows)",
                         "launch_ms": head["index_alone_ms"],
                         "frac": round(ab["index_kernel"] / (head["index_alone_ms"]["mean"] * 1e-3) / 1e9
                                       / HBM_PEAK_GBS, 4)}},
        "step_roofline": {"bound": "hbm", "scope": "whole decode step (compress, index, top-k, attention)",
                          "achieved": round(step_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                          "frac": round(step_gbs / HBM_PEAK_GBS, 4), "algorithmic_bytes": ab["step"],
                          "bytes": ab},
    }
    if args.copy_calibration:
        src_t = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
        dst_t = torch.empty_like(src_t)
        for _ in range(3):
            dst_t.copy_(src_t)
        torch.cuda.synchronize()
        result["copy_calibration_bytes_each_way"] = 512 << 20
        del src_t, dst_t
    keep = runs[0] if not args.no_cpu_baseline else None
    fp8_idx = runs[0].idx[:, 0].cpu()
    del runs
    capture.keep.clear()
    torch.cuda.empty_cache()
    if not args.no_secondary:
        # the same step with MXFP4 indexer keys (the FP4 query-key path); its
        # selection against the fp8 selection of the same underlying keys
        mx, mx_runs = csa_decode(CSA_DECODE_1M_MX4, K, args.warmup, use_graph)
        mx_idx = mx_runs[0].idx[:, 0].cpu()
        del mx_runs
        capture.keep.clear()
        torch.cuda.empty_cache()
        recall = [len(set(fp8_idx[b].tolist()) & set(mx_idx[b].tolist())) / wl.k for b in range(wl.B)]
        mms = mx["ms_per_step"]
        mab = mx["bytes"]
        mx_idx_ms = mx["index_ms"]["mean"]
        result["csa_decode_mxfp4"] = {
            "workload": mx["workload"], "replicas": mx["replicas"], "graph": mx["graph"],
            "ms_per_step": round(mms, 5), "tokens/s": round(wl.B / (mms * 1e-3), 1),
            "step_ms_with_events": mx["step_ms_with_events"], "fused_front": mx["fused_front"],
            "index_ms": mx["index_ms"], "algorithmic_bytes": mab,
            "roofline": _roof(mab["front_kernel" if mx["fused_front"] else "index_kernel"] / (mx_idx_ms * 1e-3) / 1e9,
                              "hbm", kernel=("index_mx4_front (csa_decode_front, MXFP4 keys: the step's "
                                             "compressions beside the indexer)") if mx["fused_front"]
                              else "index_mx4_decode (csa_index_score, MXFP4 keys)",
                              traffic=traffic_from_profiles("index_mx4_front_1M", src) if mx["fused_front"] else None,
                              algorithmic_bytes=mab["front_kernel" if mx["fused_front"] else "index_kernel"]),
            "step_roofline": _roof(mab["step"] / (mms * 1e-3) / 1e9, "hbm", scope="whole step"),
            "recall_at_k_vs_fp8_selection": {"mean": round(sum(recall) / len(recall), 5),
                                             "min": round(min(recall), 5), "k": wl.k,
                                             "note": "synthetic N(0,1) keys and queries; the pages' "
                                                     "recall figure is for trained weights"}}
        fl, fl_runs = csa_decode(CSA_DECODE_FLASH, K, args.warmup, use_graph)
        del fl_runs
        capture.keep.clear()
        torch.cuda.empty_cache()
        fms = fl["ms_per_step"]
        result["csa_decode_flash"] = {
            "workload": fl["workload"], "replicas": fl["replicas"], "graph": fl["graph"],
            "ms_per_step": round(fms, 5), "tokens/s": round(CSA_DECODE_FLASH.B / (fms * 1e-3), 1),
            "step_ms_with_events": fl["step_ms_with_events"], "fused_front": fl["fused_front"],
            "index_ms": fl["index_ms"],
            "algorithmic_bytes": fl["bytes"]["step"],
            "roofline": _roof(fl["bytes"]["step"] / (fms * 1e-3) / 1e9, "hbm", scope="whole step")}
        result["hca_decode"] = hca_decode(K, args.warmup, use_graph)
        # mixed KV rows (fp8 codes + bf16 rotated dims): the dense attention of the
        # HCA step and the CSA 1M step
        result["hca_decode_mixed_kv"] = hca_decode(K, args.warmup, use_graph, wl=HCA_DECODE_MIXED)
        mk, mk_runs = csa_decode(CSA_DECODE_1M_MIXED, K, args.warmup, use_graph)
        del mk_runs
        capture.keep.clear()
        torch.cuda.empty_cache()
        result["csa_decode_mixed_kv"] = {
            "workload": mk["workload"], "replicas": mk["replicas"], "graph": mk["graph"],
            "ms_per_step": round(mk["ms_per_step"], 5),
            "tokens/s": round(CSA_DECODE_1M_MIXED.B / (mk["ms_per_step"] * 1e-3), 1),
            "step_ms_with_events": mk["step_ms_with_events"], "fused_front": mk["fused_front"],
            "index_ms": mk["index_ms"], "algorithmic_bytes": mk["bytes"],
            "roofline": _roof(mk["bytes"]["step"] / (mk["ms_per_step"] * 1e-3) / 1e9, "hbm", scope="whole step")}
        result["grouped_out_proj"] = grouped_out_proj(steps=20, warmup=3)
        result["cache_append"] = cache_append(steps=50, warmup=5)
    if not args.no_prefill:
        if keep is not None:
            keep.I = None
        torch.cuda.empty_cache()
        result["prefill_indexer"] = prefill_indexer(steps=11, warmup=5)
        if not args.no_secondary:
            result["prefill_step"] = prefill_rows(steps=3, warmup=1)
    if keep is not None:
        result["cpu_baseline"] = cpu_baseline(keep, args.cpu_seconds)
    print(json.dumps(result))


if __name__ == "__main__":
    main()
