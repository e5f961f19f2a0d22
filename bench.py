#!/usr/bin/env python3
"""Benchmark of the CSA/HCA attention core on one MI355X.

Workload: 1M-context CSA decode, Pro-like -- 16 sequences, 1,048,576 cached
tokens each (262,144 compressed entries, m = 4), fp8 (e4m3) indexer keys with
per-row scales (64 heads x 128), top-k 1024, bf16 MQA over 512-wide entries for
128 query heads, 128-token window, sink.  One step = the whole hot path for
one new token per sequence: compress (window row, newest entry, newest indexer
key), indexer score, top-k, sparse MQA.  Inputs are synthetic (seeded N(0,1),
U(0,1) head weights) and resident in HBM before timing starts.

Prints ONE JSON line.  Also reported: the prefill indexer (16,384 queries x
32,768 entries, 64 heads x 128, bf16) in TFLOP/s; the HCA dense decode (4
sequences x 8,192 entries) and each call of the chunked-prefill step, each
against its roofline; and the fp64 oracle timed on a bounded sample of the
decode workload on the host cores.
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


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-secondary", action="store_true",
                    help="skip the HCA decode and prefill-step measurements")
    ap.add_argument("--cpu-sample", type=int, default=16, help="sequences the oracle runs")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 512 MiB device copy (3x) to calibrate HBM byte counters")
    return ap.parse_args()


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


def cpu_baseline(run, n_seq: int):
    """The fp64 oracle on n_seq sequences of the same workload (host cores)."""
    from threadpoolctl import threadpool_info

    from oracle import steps
    from tests._pipeline_ref import csa_decode_params

    wl = run.wl
    n_seq = max(1, min(n_seq, wl.B))
    inputs = [csa_decode_params(run, b) for b in range(n_seq)]   # decoding the bytes is not timed
    t0 = time.perf_counter()
    for p, rows in inputs:
        steps.csa_decode_sequence(p, rows)
    dt = time.perf_counter() - t0
    threads = max([d.get("num_threads", 1) for d in threadpool_info()] + [1])
    return {"value": round(n_seq / dt, 4), "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{n_seq} of {wl.B} sequences, full step each (fp64 numpy; BLAS threads "
                      f"{threads}, host nproc {os.cpu_count()})",
            "seconds": round(dt, 3)}


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
    # every launch timed on its own (timing-only events); the median is reported,
    # the mean beside it (single launches vary by a few percent with the clock)
    ev = [(TimingEvent(), TimingEvent()) for _ in range(steps)]
    for a, b in ev:
        a.record()
        csa.csa_index_score(qI, wI, K, pos, I, m=wl.m)
        b.record()
    torch.cuda.synchronize()
    per = sorted(a.elapsed_time(b) for a, b in ev)
    ms = per[len(per) // 2] if len(per) % 2 else 0.5 * (per[len(per) // 2 - 1] + per[len(per) // 2])
    ms_mean = sum(per) / len(per)
    pairs = sum(min(wl.N_cap, (wl.q_pos0 + t + 1) // wl.m) for t in range(wl.Tq))
    flops = 2.0 * pairs * wl.H_I * wl.d_I
    tfs = flops / (ms * 1e-3) / 1e12
    del qI, wI, K, I
    return {"workload": wl.name, "ms": round(ms, 4), "ms_mean": round(ms_mean, 4),
            "ms_min": round(per[0], 4), "launches": steps, "TFLOP/s": round(tfs, 2),
            "causal_flops": flops,
            "roofline": {"bound": "mfma", "achieved": round(tfs, 2), "peak": MFMA_BF16_PEAK_TFS,
                         "unit": "TFLOP/s", "frac": round(tfs / MFMA_BF16_PEAK_TFS, 4)}}


def _timed(fn, steps: int, warmup: int) -> float:
    """Average ms of fn() over `steps` calls, HIP events on the current stream."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(steps):
        fn()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / steps


def _roof(achieved: float, bound: str) -> dict:
    peak, unit = (HBM_PEAK_GBS, "GB/s") if bound == "hbm" else (MFMA_BF16_PEAK_TFS, "TFLOP/s")
    return {"bound": bound, "achieved": round(achieved, 2), "peak": peak, "unit": unit,
            "frac": round(achieved / peak, 4)}


def hca_decode(steps: int, warmup: int):
    """Dense MQA (HCA) decode: 4 sequences over 8,192 entries of 128 tokens each (1M
    context) plus window and sink; the step also recompresses the newest block."""
    import torch

    from long_context_attention_02_amd.pipeline import HCADecode
    from synth.workloads import HCA_DECODE as wl

    run = HCADecode(wl, "cuda", keep_raw=False)
    step_ms = _timed(run.step, steps, warmup)
    attn_ms = _timed(run.attend, steps, warmup)
    n_vis = min(wl.N_cap, (wl.q_pos0 + 1) // wl.m)
    rows = wl.B * (n_vis + wl.n_win)
    attn_bytes = rows * wl.d * 2 + 2 * wl.B * wl.n_h * wl.d * 2          # rows read; q and out
    attn_flops = 4.0 * wl.B * wl.n_h * (n_vis + wl.n_win) * wl.d
    del run
    torch.cuda.empty_cache()
    return {"workload": wl.name, "step_ms": round(step_ms, 5), "tokens/s": round(wl.B / (step_ms * 1e-3), 1),
            "hca_dense_mqa_ms": round(attn_ms, 5), "algorithmic_bytes": attn_bytes,
            "flops": attn_flops, "TFLOP/s": round(attn_flops / (attn_ms * 1e-3) / 1e12, 2),
            "roofline": _roof(attn_bytes / (attn_ms * 1e-3) / 1e9, "hbm")}


def prefill_rows(steps: int, warmup: int):
    """The chunked-prefill step (16,384 queries over 32,768 entries, k = 1024) call by
    call: compression of the chunk, indexer, top-k and sparse MQA."""
    import torch

    from long_context_attention_02_amd.pipeline import CSAPrefill
    from synth.workloads import CSA_PREFILL_PRO as wl

    run = CSAPrefill(wl, "cuda", keep_raw=False)
    ms = {"compress": _timed(run.compress_new, steps, warmup), "index": _timed(run.index, steps, warmup),
          "topk": _timed(run.select, steps, warmup), "sparse_mqa": _timed(run.attend, steps, warmup)}
    n_new = run.s_new1 - run.s_new0
    n_vis = [min(wl.N_cap, (wl.q_pos0 + t + 1) // wl.m) for t in range(wl.Tq)]
    # compress: window rows (read + write), candidates of the new KV entries and indexer keys
    # (C and Z of sets a and b, 2 * 2m rows each), entries written
    comp_bytes = (2 * wl.B * wl.Tq * wl.d * 2 + wl.B * n_new * (4 * wl.m * (wl.d + wl.d_I) * 2
                                                                + (wl.d + wl.d_I) * 2))
    topk_bytes = 4 * wl.B * sum(n_vis) + 4 * wl.B * wl.Tq * wl.k
    attn_flops = 4.0 * wl.B * wl.Tq * wl.n_h * (wl.k + wl.n_win) * wl.d
    index_flops = 2.0 * wl.B * sum(n_vis) * wl.H_I * wl.d_I
    out = {"workload": wl.name, "ms": {k: round(v, 4) for k, v in ms.items()},
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


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (the CSA/HCA core "
              "runs on a single MI355X here)", file=sys.stderr)
        sys.exit(2)
    import torch

    from long_context_attention_02_amd.pipeline import CSADecode
    from synth.workloads import CSA_DECODE_1M as wl

    torch.cuda.set_device(0)
    run = CSADecode(wl, "cuda", keep_raw=not args.no_cpu_baseline)
    torch.cuda.synchronize()
    for _ in range(args.warmup):
        run.step()
    torch.cuda.synchronize()

    K = args.steps
    # the indexer's own launch times, from timing-only events on the step's stream
    ev_idx = [(TimingEvent(), TimingEvent()) for _ in range(K)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record()
    for s in range(K):
        run.step(index_events=ev_idx[s])
    t_end.record()
    torch.cuda.synchronize()
    ms_step = t_start.elapsed_time(t_end) / K
    idx_ms = sum(a.elapsed_time(b) for a, b in ev_idx) / K

    ab = run.algorithmic_bytes()
    tokens_s = wl.B / (ms_step * 1e-3)
    idx_gbs = ab["index_kernel"] / (idx_ms * 1e-3) / 1e9
    step_gbs = ab["step"] / (ms_step * 1e-3) / 1e9
    src = os.path.join(ROOT, "long_context_attention_02_amd", "csrc", "index_score.hip")
    traffic = traffic_from_profiles("index_score_decode_1M_fp8", src)

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
        "step_hbm_GBps": round(step_gbs, 1),
        "step_algorithmic_bytes": ab["step"],
        "roofline": {"bound": "hbm", "kernel": "index_mfma_decode (csa_index_score)",
                     "achieved": round(idx_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(idx_gbs / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "algorithmic_bytes": ab["index_kernel"],
                     "avg_launch_ms": round(idx_ms, 5)},
    }
    if args.copy_calibration:
        src_t = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
        dst_t = torch.empty_like(src_t)
        for _ in range(3):
            dst_t.copy_(src_t)
        torch.cuda.synchronize()
        result["copy_calibration_bytes_each_way"] = 512 << 20
        del src_t, dst_t
    if not args.no_prefill:
        del run.I
        torch.cuda.empty_cache()
        result["prefill_indexer"] = prefill_indexer(steps=11, warmup=5)
    if not args.no_secondary:
        if hasattr(run, "I"):
            del run.I
        torch.cuda.empty_cache()
        result["hca_decode"] = hca_decode(steps=20, warmup=5)
        result["prefill_step"] = prefill_rows(steps=3, warmup=1)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(run, args.cpu_sample)
    print(json.dumps(result))


if __name__ == "__main__":
    main()
