"""Benchmark of the SageAttention 8-bit attention forward on one MI355X.

One step = the whole hot path on the text-LLM workload (B=1, H=8, N=4096,
d=128, fp16 P.V, quantisation blocks 128 x 64) run twice, non-causal and
causal: smooth K + INT8 Q/K (sage_quantize), then the fused attention kernel
(sage_attn_quantized).  Inputs are synthetic (seeded, fp16, already resident
in HBM before the timed region starts).

value = attention TOPS of the step = (4 B H N^2 d + 4 B H N^2 d / 2) / t,
with t from K steps that carry no events of their own (an event pair between
two kernels costs several microseconds on the stream).
roofline = the dominant kernel (the non-causal fused attention) against the
MI355X dense INT8 MFMA peak; its duration is measured live on the stream it
runs on: K launches back to back between one HIP event pair (average per
launch; per-launch event pairs, which add a few microseconds each, give the
median and min in `timing`).  cpu_baseline = the CPU oracle on the same step,
its (head, mask) units spread over one single-threaded worker process per
host core.
timing = median and min of the per-launch HIP event times (fused kernel,
non-causal and causal), the sage_quantize pre-pass against the HBM peak
(algorithmic bytes: fp16 Q and K read once, int8 written, scales, mean), and
sage_attn end to end (its own workspace).  inputs_sha256 = provenance of
the synthetic fp16 Q, K, V.
extra = the larger workloads, inputs drawn with each workload's own recipe
(synth.generate): kernel-only TOPS of the fused kernel, sage_attn end to end
(pre-pass included) plain, with Q smoothed and with 4-bit (MXFP4) Q and K,
and the pre-pass alone at N=32K; median and min over 50 timed calls each.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
       python bench.py --profile CASE [--steps K] [--warmup W]   (one extra case only)
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

INT8_PEAK_TOPS = 5000.0          # MI355X dense INT8 MFMA, published
FP16_PEAK_TFLOPS = 2500.0
HBM_PEAK_BPS = 8.0e12            # MI355X HBM3E, published
METRIC = "attention TOPS (4·B·H·N²·d/t) at d=128, N=4K–32K; % of INT8 MFMA peak"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_fwd_text_noncausal_traffic.json")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true")
    ap.add_argument("--copy-calib", action="store_true",
                    help="first run a plain copy kernel of 256 MiB in / 256 MiB out (HBM counter calibration)")
    ap.add_argument("--profile", metavar="CASE",
                    help="run only this extra case (--warmup, then --steps timed calls) and print its timing: "
                         "the command the rocprofv3 summaries are taken with")
    return ap.parse_args()


def kernel_source_digest() -> str:
    h = hashlib.sha256()
    for f in ("attn_fwd.hip", "sage_internal.h"):
        h.update(open(os.path.join(ROOT, "quantized_attention_transformer_amd", "csrc", f), "rb").read())
    return h.hexdigest()[:16]


def traffic_or_null():
    """HBM bytes per launch of the dominant kernel from the committed rocprofv3
    counter runs, or None when the kernel source changed since they were taken."""
    try:
        t = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_digest") != kernel_source_digest():
        return None
    return t.get("hbm_bytes_per_launch")


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(attention shards by (sequence, head) with no communication between GPUs).",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from quantized_attention_transformer_amd import sage, synth
    import ctypes

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    L = sage.lib()
    if args.copy_calib:
        src = torch.ones(64 << 20, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.mul(src, 1.0, out=dst)         # reads 256 MiB, writes 256 MiB
        torch.cuda.synchronize()
        del src, dst
    if args.profile:
        profile_case(sage, torch, dev, args.profile, args.steps, args.warmup)
        return

    wl = synth.TEXT
    inp = synth.generate(wl)
    B, N, H, d = inp.q.shape
    q, k, v = (torch.from_numpy(x).to(dev) for x in (inp.q, inp.k, inp.v))
    prob = sage.make_problem(q, "bnhd", blk_q=wl.blk_q, blk_k=wl.blk_k)
    # int8 Q/K in head-major layout (the layout sage_attn uses for its workspace)
    q8 = torch.empty((B, H, N, d), dtype=torch.int8, device=dev)
    k8 = torch.empty((B, H, N, d), dtype=torch.int8, device=dev)
    sq = torch.empty((B, H, -(-N // wl.blk_q)), dtype=torch.float32, device=dev)
    sk = torch.empty((B, H, -(-N // wl.blk_k)), dtype=torch.float32, device=dev)
    km = torch.empty((B, H, d), dtype=torch.float32, device=dev)
    ws = torch.empty(max(16, sage.quantize_workspace_bytes(prob)), dtype=torch.uint8, device=dev)
    out = torch.empty_like(q)
    s_in, s8, so = sage.strides_of(q, "bnhd"), sage.strides_of(q8, "bhnd"), sage.strides_of(out, "bnhd")
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)
    P = ctypes.byref(prob)

    def quantize():
        rc = L.sage_quantize(P, q.data_ptr(), s_in, k.data_ptr(), s_in, 0.0, q8.data_ptr(), s8, k8.data_ptr(), s8,
                             sq.data_ptr(), sk.data_ptr(), km.data_ptr(), ws.data_ptr(), ws.numel(), sp)
        assert rc == 0, L.sage_last_error()

    def attention(causal):
        rc = L.sage_attn_quantized(P, q8.data_ptr(), s8, k8.data_ptr(), s8, sq.data_ptr(), sk.data_ptr(),
                                   v.data_ptr(), s_in, None, out.data_ptr(), so, int(causal), 0, sp)
        assert rc == 0, L.sage_last_error()

    def evpair():
        return torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    ev = {c: [evpair() for _ in range(args.steps)] for c in (False, True)}
    evq = {c: [evpair() for _ in range(args.steps)] for c in (False, True)}

    def step(i=None, events=None):
        # The steps of the timed region carry no events of their own (an event
        # pair between two kernels costs several microseconds on the stream);
        # two further passes of the same steps put HIP events around the fused
        # kernel (events="attn") and around the pre-pass (events="quant").
        for causal in (False, True):
            if events == "quant":
                evq[causal][i][0].record(stream)
            quantize()
            if events == "quant":
                evq[causal][i][1].record(stream)
            if events == "attn":
                ev[causal][i][0].record(stream)
            attention(causal)
            if events == "attn":
                ev[causal][i][1].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for i in range(args.steps):
        step(i)
    t1.record(stream)
    torch.cuda.synchronize()
    total_ms = t0.elapsed_time(t1)
    # per-launch durations: K launches of one kernel back to back between one
    # event pair on the launch stream (average), then per-launch event pairs
    # (median, min; each pair adds a few microseconds of its own)
    def back_to_back(fn):
        a, b = evpair()
        a.record(stream)
        for _ in range(args.steps):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / args.steps
    avg_nc = back_to_back(lambda: attention(False))
    avg_c = back_to_back(lambda: attention(True))
    avg_q = back_to_back(quantize)
    for events in ("attn", "quant"):
        for i in range(args.steps):
            step(i, events)
        torch.cuda.synchronize()
    ms_step = total_ms / args.steps
    ops_nc = sage.attention_ops([N] * B, H, d, False)
    ops_c = sage.attention_ops([N] * B, H, d, True)
    value = (ops_nc + ops_c) / (ms_step * 1e-3) / 1e12
    t_attn = {c: np.array([a.elapsed_time(b) for a, b in ev[c]]) for c in (False, True)}
    t_quant = np.concatenate([[a.elapsed_time(b) for a, b in evq[c]] for c in (False, True)])
    kern_nc, kern_c = avg_nc, avg_c
    achieved = ops_nc / (kern_nc * 1e-3) / 1e12
    nbq, nbk = -(-N // wl.blk_q), -(-N // wl.blk_k)
    # algorithmic bytes of sage_quantize: fp16 Q and K read once, int8 written, plus scales and the mean
    quant_bytes = 3 * 2 * B * N * H * d + 4 * B * H * (nbq + nbk) + 4 * B * H * d
    q_med = float(np.median(t_quant))
    q_avg = avg_q

    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "i8+f16",
        "data": "synthetic",
        "config": {"workload": "text-LLM attention B1 H8 N4096 d128 fp16 P.V, blocks 128x64; one step = "
                               "sage_quantize + fused attention, non-causal then causal",
                   "batch": B, "heads": H, "seq_len": N, "head_dim": d, "blk_q": wl.blk_q, "blk_k": wl.blk_k,
                   "parallelism": "single GPU"},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": INT8_PEAK_TOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / INT8_PEAK_TOPS, 4), "traffic": traffic_or_null(),
                     "kernel": "fused attention, non-causal (k_attn<128,...,CAUSAL=false>)",
                     "kernel_ms": round(kern_nc, 5), "causal_kernel_ms": round(kern_c, 5),
                     "mixed_ceiling_frac": round(2 / 3, 4)},
    }

    result["timing"] = {
        "attn_kernel_ms": {("causal" if c else "noncausal"): {"back_to_back_avg": round(avg_c if c else avg_nc, 5),
                                                              "event_median": round(float(np.median(t_attn[c])), 5),
                                                              "event_min": round(float(t_attn[c].min()), 5)}
                           for c in (False, True)},
        "prepass": {"call": "sage_quantize (2 launches: Q quantisation + K column sums, then K quantisation)",
                    "ms_back_to_back_avg": round(q_avg, 5),
                    "ms_event_median": round(q_med, 5), "ms_event_min": round(float(t_quant.min()), 5),
                    "algorithmic_bytes": quant_bytes, "GB/s": round(quant_bytes / (q_avg * 1e-3) / 1e9, 1),
                    "frac_hbm_peak": round(quant_bytes / (q_avg * 1e-3) / HBM_PEAK_BPS, 4)},
        "sage_attn_end_to_end": end_to_end(sage, torch, q, k, v, wl, ops_nc, ops_c),
    }
    result["inputs_sha256"] = {n: hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()
                               for n, a in (("q", inp.q), ("k", inp.k), ("v", inp.v))}

    if not args.no_extra:
        result["extra"] = extra_workloads(sage, torch, dev)

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(inp, wl, ops_nc + ops_c)

    print(json.dumps(result), flush=True)


def end_to_end(sage, torch, q, k, v, wl, ops_nc, ops_c, warmup=10, runs=50):
    """sage_attn (quantisation + attention in one call, its own workspace) on
    the step's inputs: median and min over single-call HIP event timings."""
    import numpy as np
    out = torch.empty_like(q)
    ws = torch.empty(max(16, sage.workspace_bytes(sage.make_problem(q, "bnhd", blk_q=wl.blk_q, blk_k=wl.blk_k))),
                     dtype=torch.uint8, device=q.device)
    res = {}
    for causal, ops in ((False, ops_nc), (True, ops_c)):
        def run():
            sage.attn(q, k, v, causal=causal, blk_q=wl.blk_q, blk_k=wl.blk_k, out=out, workspace=ws)
        for _ in range(warmup):
            run()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(runs)]
        for a, b in evs:
            a.record()
            run()
            b.record()
        torch.cuda.synchronize()
        t = np.array([a.elapsed_time(b) for a, b in evs])
        med = float(np.median(t))
        res["causal" if causal else "noncausal"] = {"ms_median": round(med, 5), "ms_min": round(float(t.min()), 5),
                                                    "TOPS": round(ops / (med * 1e-3) / 1e12, 1)}
    return res


# Extra workloads: (name, workload, causal, pv_mode, kind).  kind "kernel" times
# the fused kernel alone (sage_attn_quantized on pre-quantised inputs), "e2e"
# sage_attn (pre-pass + fused kernel), "sq" / "fp4" sage_attn with Q smoothed /
# with 4-bit (MXFP4) Q and K, "prepass" sage_quantize alone, "gqa" the fused
# kernel with 8 K/V heads for the 32 query heads.
EXTRA_CASES = [
    ("long causal B1 H32 N32768 d128", "LONG", True, 0, "kernel"),
    ("fp8-PV B4 H16 N8192 d128", "FP8", False, 1, "kernel"),
    ("fp8-PV smooth-V B4 H16 N8192 d128", "FP8", False, 2, "kernel"),
    ("fp16-PV B4 H16 N8192 d128", "FP8", False, 0, "kernel"),
    ("video B2 H24 N16384 d64", "VIDEO", False, 0, "kernel"),
    ("varlen causal H32 d128", "VARLEN", True, 0, "kernel"),
    ("gqa causal B1 H32 kv8 N8192 d128", "LONG", True, 0, "gqa"),
    ("sage_attn fp16-PV B4 H16 N8192 d128", "FP8", False, 0, "e2e"),
    ("sage_attn FP8-PV B4 H16 N8192 d128", "FP8", False, 1, "e2e"),
    ("sage_attn smooth-Q fp16-PV B4 H16 N8192 d128", "FP8", False, 0, "sq"),
    ("sage_attn 4-bit QK (MXFP4) fp16-PV B4 H16 N8192 d128", "FP8", False, 0, "fp4"),
    ("sage_attn 4-bit QK (MXFP4) FP8-PV B4 H16 N8192 d128", "FP8", False, 1, "fp4"),
    ("sage_quantize long B1 H32 N32768 d128", "LONG", False, 0, "prepass"),
    ("sage_quantize text B1 H8 N4096 d128", "TEXT", False, 0, "prepass"),
]


class _Inputs:
    """Device copies of one workload's seeded inputs (synth.generate, the
    workload's own recipe), drawn once and shared by the cases that use it."""

    def __init__(self, torch, dev):
        self.torch, self.dev, self.cache = torch, dev, {}

    def get(self, wl_name, gqa=False):
        from quantized_attention_transformer_amd import synth
        key = (wl_name, gqa)
        if key not in self.cache:
            self.cache.clear()
            self.torch.cuda.empty_cache()
            wl = getattr(synth, wl_name)
            inp = synth.generate(wl, seqlen=8192) if gqa else synth.generate(wl)
            t = [self.torch.from_numpy(x).to(self.dev) for x in (inp.q, inp.k, inp.v)]
            if gqa:                           # 8 K/V heads for the 32 query heads
                t[1], t[2] = t[1][:, :, :8].contiguous(), t[2][:, :, :8].contiguous()
            cu = None if inp.cu_seqlens is None else self.torch.from_numpy(inp.cu_seqlens).to(self.dev)
            self.cache[key] = (wl, t, cu, inp.seqlens.tolist())
            del inp
        return self.cache[key]


def prepare_case(sage, torch, inputs, name, wl_name, causal, mode, kind):
    """Returns (run, ops, bytes): a closure that enqueues one call of the case,
    its attention operation count (0 for the pre-pass) and, for the pre-pass,
    its algorithmic HBM bytes."""
    wl, (q, k, v), cu, seqlens = inputs.get(wl_name, gqa=(kind == "gqa"))
    kw = {} if cu is None else dict(cu_seqlens=cu, max_seqlen=max(seqlens))
    H, d = q.shape[-2], q.shape[-1]
    if kind == "prepass":
        # sage_quantize through the C ABI on preallocated outputs (int8 Q and K
        # in the head-major layout sage_attn's workspace uses)
        import ctypes
        L = sage.lib()
        prob = sage.make_problem(q, blk_q=wl.blk_q, blk_k=wl.blk_k, k=k, **kw)
        B, N, Hq, d = q.shape if q.dim() == 4 else (1, q.shape[0], q.shape[1], q.shape[2])
        q8 = torch.empty((B, Hq, N, d), dtype=torch.int8, device=q.device)
        k8 = torch.empty((B, k.shape[-2], N, d), dtype=torch.int8, device=q.device)
        sq = torch.empty((len(seqlens), Hq, -(-max(seqlens) // wl.blk_q)), dtype=torch.float32, device=q.device)
        sk = torch.empty((len(seqlens), k.shape[-2], -(-max(seqlens) // wl.blk_k)), dtype=torch.float32,
                         device=q.device)
        km = torch.empty((len(seqlens), k.shape[-2], d), dtype=torch.float32, device=q.device)
        ws = torch.empty(max(16, sage.quantize_workspace_bytes(prob)), dtype=torch.uint8, device=q.device)
        s_in, s8 = sage.strides_of(q, "bnhd"), sage.strides_of(q8, "bhnd")
        s8k = sage.strides_of(k8, "bhnd")
        sp = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        P = ctypes.byref(prob)

        def run():
            rc = L.sage_quantize(P, q.data_ptr(), s_in, k.data_ptr(), sage.strides_of(k, "bnhd"), 0.0, q8.data_ptr(),
                                 s8, k8.data_ptr(), s8k, sq.data_ptr(), sk.data_ptr(), km.data_ptr(), ws.data_ptr(),
                                 ws.numel(), sp)
            assert rc == 0, L.sage_last_error()
        ntok = sum(seqlens)
        nbq = sum(-(-L // wl.blk_q) for L in seqlens)
        nbk = sum(-(-L // wl.blk_k) for L in seqlens)
        nbytes = 3 * 2 * ntok * H * d + 4 * H * (nbq + nbk) + 4 * len(seqlens) * H * d
        return run, 0.0, nbytes
    out = torch.empty_like(q)
    if kind in ("e2e", "sq", "fp4"):
        prob = sage.make_problem(q, blk_q=wl.blk_q, blk_k=wl.blk_k, k=k, **kw)
        prob.smooth_q = int(kind == "sq")
        prob.qk_fp4 = int(kind == "fp4")
        ws = torch.empty(sage.workspace_bytes(prob, mode), dtype=torch.uint8, device=q.device)

        def run():
            sage.attn(q, k, v, causal=causal, pv_mode=mode, blk_q=wl.blk_q, blk_k=wl.blk_k, out=out,
                      workspace=ws, smooth_q=(kind == "sq"), qk_fp4=(kind == "fp4"), **kw)
    else:
        qd = sage.quantize(q, k, blk_q=wl.blk_q, blk_k=wl.blk_k, **kw)
        vv, sv = (sage.quantize_v_fp8(v, smooth=(mode == 2), **kw) if mode >= 1 else (v, None))

        def run():
            sage.attn_quantized(qd["q8"], qd["k8"], qd["q_scale"], qd["k_scale"], vv, v_scale=sv, causal=causal,
                                pv_mode=mode, blk_q=wl.blk_q, blk_k=wl.blk_k, out=out, **kw)
    return run, sage.attention_ops(seqlens, H, d, causal), 0


def time_case(torch, run, warmup=10, runs=50):
    """Per-call HIP event times (ms) of `runs` calls after `warmup` untimed ones."""
    import numpy as np
    for _ in range(warmup):
        run()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(runs)]
    for a, b in evs:
        a.record()
        run()
        b.record()
    torch.cuda.synchronize()
    return np.array([a.elapsed_time(b) for a, b in evs])


def case_result(t, ops, nbytes):
    import numpy as np
    med, mn = float(np.median(t)), float(t.min())
    r = {"runs": int(len(t)), "ms_median": round(med, 5), "ms_min": round(mn, 5)}
    if ops:
        r.update(TOPS=round(ops / (med * 1e-3) / 1e12, 1), TOPS_best=round(ops / (mn * 1e-3) / 1e12, 1),
                 frac_int8_peak=round(ops / (med * 1e-3) / 1e12 / INT8_PEAK_TOPS, 4))
    if nbytes:
        r.update(algorithmic_bytes=int(nbytes), GBps=round(nbytes / (med * 1e-3) / 1e9, 1),
                 frac_hbm_peak=round(nbytes / (med * 1e-3) / HBM_PEAK_BPS, 4))
    return r


def extra_workloads(sage, torch, dev, runs=50):
    """The larger workloads (inputs drawn with each workload's own recipe):
    kernel-only TOPS of the fused attention, sage_attn end to end, and the
    pre-pass at N=32K; median and min over `runs` timed calls each."""
    inputs = _Inputs(torch, dev)
    res = {}
    for name, wl_name, causal, mode, kind in EXTRA_CASES:
        run, ops, nbytes = prepare_case(sage, torch, inputs, name, wl_name, causal, mode, kind)
        res[name] = case_result(time_case(torch, run, runs=runs), ops, nbytes)
        print(f"extra: {name}: {res[name]}", file=sys.stderr, flush=True)
        del run
    inputs.cache.clear()
    torch.cuda.empty_cache()
    return res


def profile_case(sage, torch, dev, name, steps, warmup):
    """Only one extra case, `steps` timed calls (for rocprofv3 runs)."""
    match = [c for c in EXTRA_CASES if c[0] == name]
    if not match:
        raise SystemExit(f"unknown case {name!r}; cases: " + "; ".join(c[0] for c in EXTRA_CASES))
    run, ops, nbytes = prepare_case(sage, torch, _Inputs(torch, dev), *match[0])
    r = case_result(time_case(torch, run, warmup=warmup, runs=steps), ops, nbytes)
    print(json.dumps({"case": name, **r}), flush=True)


def _oracle_unit(a):
    """One (head, mask) unit of the oracle, single-threaded (a worker process)."""
    q, k, v, seqlens, causal, blk_q, blk_k = a
    from oracle import sage_oracle as O
    try:
        from threadpoolctl import threadpool_limits
        ctx = threadpool_limits(limits=1)
    except ImportError:                      # pragma: no cover
        ctx = None
    try:
        O.sage_attn(q, k, v, seqlens, None, causal, blk_q, blk_k)
    finally:
        if ctx is not None:
            ctx.__exit__(None, None, None)


def cpu_baseline(inp, wl, ops, min_seconds=1.5):
    """The CPU oracle (as it stands) on the same step: quantisation and fp64
    attention, non-causal then causal, full workload.  Every (head, mask) pair
    is an independent unit (the mean, the scales and the softmax rows are per
    head), so the units run in parallel worker processes, one per host core
    the process may use, each single-threaded (its BLAS included)."""
    import concurrent.futures as cf
    import multiprocessing as mp
    affinity = len(os.sched_getaffinity(0))
    H = inp.q.shape[2]
    units = [(inp.q[:, :, h:h + 1], inp.k[:, :, h:h + 1], inp.v[:, :, h:h + 1], inp.seqlens, causal,
              wl.blk_q, wl.blk_k) for causal in (False, True) for h in range(H)]
    workers = min(affinity, len(units))
    with cf.ProcessPoolExecutor(max_workers=workers, mp_context=mp.get_context("spawn")) as ex:
        list(ex.map(_oracle_unit, units[:workers]))      # start the workers (imports) before timing
        t = time.perf_counter()
        reps = 0
        while True:                                       # whole steps, at least min_seconds of wall time
            list(ex.map(_oracle_unit, units))
            reps += 1
            dt = time.perf_counter() - t
            if dt >= min_seconds:
                break
    return {"value": round(reps * ops / dt / 1e12, 5), "unit": "TOPS", "cores": workers, "kind": "oracle",
            "host_affinity_cores": affinity, "host_nproc": os.cpu_count(),
            "sample": f"the full step (B1 H8 N4096 d128, quantise + attention, non-causal and causal) {reps} times "
                      f"in {dt:.2f} s: {len(units)} (head, mask) units per step over {workers} single-threaded "
                      f"worker processes (numpy, BLAS limited to one thread each)"}


if __name__ == "__main__":
    main()
