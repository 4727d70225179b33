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
MI355X dense INT8 MFMA peak; its duration is measured live with HIP events
around it, on the stream it runs on, in a second pass of the same K steps
(the pre-pass in a third).  cpu_baseline = the CPU oracle on the same step.
timing = median and min of the per-launch HIP event times (fused kernel,
non-causal and causal), the sage_quantize pre-pass against the HBM peak
(algorithmic bytes: fp16 Q and K read once, int8 written, scales, mean), and
sage_attn end to end (its own workspace).  inputs_sha256 = provenance of
the synthetic fp16 Q, K, V.
extra = kernel-only TOPS of the fused kernel on the larger workloads, and
sage_attn end to end (pre-pass included) plain, with Q smoothed, and with 4-bit
(MXFP4) Q and K on one.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
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
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(attention shards by (sequence, head) with no communication; see the design notes).",
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

    if args.copy_calib:
        src = torch.ones(64 << 20, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.mul(src, 1.0, out=dst)         # reads 256 MiB, writes 256 MiB
        torch.cuda.synchronize()
        del src, dst
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
    kern_nc = float(t_attn[False].mean())
    kern_c = float(t_attn[True].mean())
    achieved = ops_nc / (kern_nc * 1e-3) / 1e12
    nbq, nbk = -(-N // wl.blk_q), -(-N // wl.blk_k)
    # algorithmic bytes of sage_quantize: fp16 Q and K read once, int8 written, plus scales and the mean
    quant_bytes = 3 * 2 * B * N * H * d + 4 * B * H * (nbq + nbk) + 4 * B * H * d
    q_med = float(np.median(t_quant))

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
        "attn_kernel_ms": {("causal" if c else "noncausal"): {"median": round(float(np.median(t_attn[c])), 5),
                                                              "min": round(float(t_attn[c].min()), 5)}
                           for c in (False, True)},
        "prepass": {"call": "sage_quantize (2 launches: Q quantisation + K column sums, then K quantisation)",
                    "ms_median": round(q_med, 5), "ms_min": round(float(t_quant.min()), 5),
                    "algorithmic_bytes": quant_bytes, "GB/s": round(quant_bytes / (q_med * 1e-3) / 1e9, 1),
                    "frac_hbm_peak": round(quant_bytes / (q_med * 1e-3) / HBM_PEAK_BPS, 4)},
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


def extra_workloads(sage, torch, dev):
    """Kernel-only TOPS of the fused attention on the larger workloads
    (inputs drawn on the GPU with the workloads' distributions)."""
    from quantized_attention_transformer_amd import synth
    res = {}
    g = torch.Generator(device=dev)
    cases = [("long causal B1 H32 N32768 d128", synth.LONG, True, 0, None),
             ("fp8-PV B4 H16 N8192 d128", synth.FP8, False, 1, None),
             ("fp8-PV smooth-V B4 H16 N8192 d128", synth.FP8, False, 2, None),
             ("fp16-PV B4 H16 N8192 d128", synth.FP8, False, 0, None),
             ("video B2 H24 N16384 d64", synth.VIDEO, False, 0, None),
             ("varlen causal H32 d128", synth.VARLEN, True, 0, "varlen"),
             ("gqa causal B1 H32 kv8 N8192 d128", synth.LONG, True, 0, "gqa"),
             # whole forward pass (sage_attn: pre-pass + fused kernel), plain and with Q smoothed
             ("sage_attn fp16-PV B4 H16 N8192 d128", synth.FP8, False, 0, "e2e"),
             ("sage_attn smooth-Q fp16-PV B4 H16 N8192 d128", synth.FP8, False, 0, "sq"),
             ("sage_attn 4-bit QK (MXFP4) fp16-PV B4 H16 N8192 d128", synth.FP8, False, 0, "fp4"),
             ("sage_attn 4-bit QK (MXFP4) FP8-PV B4 H16 N8192 d128", synth.FP8, False, 1, "fp4")]
    for name, wl, causal, mode, kind in cases:
        g.manual_seed(wl.seed)
        if kind == "varlen":
            import numpy as np
            lens = synth.draw_varlen_lengths(np.random.default_rng(wl.seed), wl.varlen_nseq, wl.varlen_min,
                                             wl.varlen_max, wl.varlen_total_max)
            T = int(lens.sum())
            shape = (T, wl.heads, wl.head_dim)
            cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]).astype(np.int32), device=dev)
            kw = dict(cu_seqlens=cu, max_seqlen=int(lens.max()))
            seqlens = lens.tolist()
        elif kind == "gqa":
            shape = (1, 8192, wl.heads, wl.head_dim)
            kw = {}
            seqlens = [8192]
        else:
            shape = (wl.batch, wl.seqlen, wl.heads, wl.head_dim)
            kw = {}
            seqlens = [wl.seqlen] * wl.batch
        q = torch.randn(shape, generator=g, device=dev, dtype=torch.float32).half()
        bias = torch.randn((wl.heads, wl.head_dim), generator=g, device=dev) * wl.bias_std
        k = (torch.randn(shape, generator=g, device=dev, dtype=torch.float32) + bias).half()
        v = torch.randn(shape, generator=g, device=dev, dtype=torch.float32).half()
        if kind == "gqa":                         # 8 K/V heads for the 32 query heads
            k, v = k[:, :, :8].contiguous(), v[:, :, :8].contiguous()
        qd = sage.quantize(q, k, blk_q=wl.blk_q, blk_k=wl.blk_k, **kw)
        vv, sv = (sage.quantize_v_fp8(v, smooth=(mode == 2), **kw) if mode >= 1 else (v, None))
        out = torch.empty_like(q)
        ws = None
        if kind in ("e2e", "sq", "fp4"):
            prob = sage.make_problem(q, blk_q=wl.blk_q, blk_k=wl.blk_k, k=k)
            prob.smooth_q = int(kind == "sq")
            prob.qk_fp4 = int(kind == "fp4")
            ws = torch.empty(sage.workspace_bytes(prob, mode), dtype=torch.uint8, device=dev)

        def run():
            if ws is not None:
                sage.attn(q, k, v, causal=causal, pv_mode=mode, blk_q=wl.blk_q, blk_k=wl.blk_k, out=out,
                          workspace=ws, smooth_q=(kind == "sq"), qk_fp4=(kind == "fp4"))
                return
            sage.attn_quantized(qd["q8"], qd["k8"], qd["q_scale"], qd["k_scale"], vv, v_scale=sv, causal=causal,
                                pv_mode=mode, blk_q=wl.blk_q, blk_k=wl.blk_k, out=out, **kw)
        for _ in range(2):
            run()
        torch.cuda.synchronize()
        n = 5
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(n):
            run()
        b.record()
        torch.cuda.synchronize()
        ms = a.elapsed_time(b) / n
        ops = sage.attention_ops(seqlens, wl.heads, wl.head_dim, causal)
        tops = ops / (ms * 1e-3) / 1e12
        res[name] = {"kernel_ms": round(ms, 4), "TOPS": round(tops, 1), "frac_int8_peak": round(tops / INT8_PEAK_TOPS, 4)}
        del q, k, v, qd, vv, out, ws
        torch.cuda.empty_cache()
    return res


def cpu_baseline(inp, wl, ops):
    """The CPU oracle (as it stands) on the same step: quantisation and fp64
    attention, non-causal then causal, full workload."""
    from oracle import sage_oracle as O
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
    except ImportError:                      # pragma: no cover
        threadpool_limits, threadpool_info = None, None
    cores = min(16, len(os.sched_getaffinity(0)))
    ctx = threadpool_limits(limits=cores) if threadpool_limits else None
    try:
        t = time.perf_counter()
        for causal in (False, True):
            O.sage_attn(inp.q, inp.k, inp.v, inp.seqlens, None, causal, wl.blk_q, wl.blk_k)
        dt = time.perf_counter() - t
        used = cores
        if threadpool_info:
            used = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    finally:
        if ctx is not None:
            ctx.__exit__(None, None, None)
    return {"value": round(ops / dt / 1e12, 5), "unit": "TOPS", "cores": used, "kind": "oracle",
            "sample": f"the full step (B1 H8 N4096 d128, quantise + attention, non-causal and causal) in "
                      f"{dt:.1f} s; matrix products on {used} BLAS threads, elementwise work single-threaded"}


if __name__ == "__main__":
    main()
