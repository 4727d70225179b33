"""sage_attn against the CPU oracle on seeded random configurations.

The method ("SageAttention：低比特量化Attention，实现推理加速", section 技术方案;
"4比特量化三倍加速不掉点！清华即插即用的SageAttention迎来升级", section 技术方案)
runs through every option here: dense or packed (varlen, with empty and
one-token sequences) batches; head dimension 64, 96 or 128; grouped-query
heads; causal or not; fp16, FP8 or smoothed-V FP8 P.V; smooth Q; 4-bit Q.K^T;
Q blocks of 1-256 rows and K blocks of 16-256 rows.  The configurations are
drawn once, from a fixed seed, so every run checks the same ones.  Tolerances
as in the other parity tests: fp16 P.V cos >= 0.99995 and max |dO| <= 4e-3,
FP8 cos >= 0.9995.
"""
import dataclasses

import numpy as np
import pytest

from oracle import sage_oracle as O
from quantized_attention_transformer_amd import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def draw_configs(seed=2026, n=32):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        d = int(rng.choice([64, 96, 128]))
        varlen = bool(rng.random() < 0.35)
        H = int(rng.choice([1, 2, 3, 4, 6]))
        hk = int(rng.choice([x for x in range(1, H + 1) if H % x == 0]))
        causal = bool(rng.random() < 0.5)
        mode = int(rng.choice([0, 1, 2]))
        fp4 = bool(d != 64 and rng.random() < 0.2)
        sq = bool(rng.random() < 0.25)
        blk_k = int(rng.choice([64, 128, 256] if (sq or fp4) else [16, 32, 64, 128, 256]))
        blk_q = 128 if fp4 else int(rng.choice([1, 16, 32, 64, 128, 256]))
        if varlen:
            lens = [int(x) for x in rng.choice([0, 1, 2, 17, 64, 65, 127, 128, 129, 300, 511], size=int(rng.integers(1, 5)))]
            if sum(lens) == 0:
                lens[0] = 33
            shape = dict(seqlens=lens)
        else:
            shape = dict(seqlen=int(rng.integers(1, 600)), batch=int(rng.integers(1, 3)))
        out.append(dict(d=d, varlen=varlen, H=H, hk=hk, causal=causal, mode=mode, fp4=fp4, sq=sq, blk_q=blk_q,
                        blk_k=blk_k, shape=shape))
    return out


def cfg_id(c):
    s = c["shape"]
    where = ("varlen" + "-".join(map(str, s["seqlens"]))) if c["varlen"] else f"B{s['batch']}N{s['seqlen']}"
    return (f"d{c['d']}-{where}-H{c['H']}kv{c['hk']}-{'causal' if c['causal'] else 'full'}-pv{c['mode']}"
            f"-blk{c['blk_q']}x{c['blk_k']}{'-sq' if c['sq'] else ''}{'-fp4' if c['fp4'] else ''}")


CONFIGS = draw_configs()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from quantized_attention_transformer_amd import sage
    sage.lib()


def dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def cos(a, b):
    a = np.asarray(a, np.float64).ravel()
    b = np.asarray(b, np.float64).ravel()
    return float(a @ b / (np.linalg.norm(a) * np.linalg.norm(b)))


@pytest.mark.parametrize("c", CONFIGS, ids=[cfg_id(c) for c in CONFIGS])
def test_random_config_against_oracle(c):
    from quantized_attention_transformer_amd import sage
    wl = dataclasses.replace(synth.VARLEN if c["varlen"] else synth.TEXT, head_dim=c["d"])
    inp = synth.generate(wl, heads=c["H"], **c["shape"])
    if c["hk"] != c["H"]:
        z = dict(inp.__dict__)
        z["k"] = np.ascontiguousarray(inp.k[..., :c["hk"], :])
        z["v"] = np.ascontiguousarray(inp.v[..., :c["hk"], :])
        inp = synth.Inputs(**z)
    print(f"[{cfg_id(c)}] q{inp.q.shape} k{inp.k.shape}", flush=True)
    kw = {} if inp.cu_seqlens is None else dict(cu_seqlens=dev(inp.cu_seqlens), max_seqlen=inp.max_seqlen)
    o = sage.attn(dev(inp.q), dev(inp.k), dev(inp.v), causal=c["causal"], pv_mode=c["mode"], blk_q=c["blk_q"],
                  blk_k=c["blk_k"], smooth_q=c["sq"], qk_fp4=c["fp4"], **kw)
    torch.cuda.synchronize()
    o = o.cpu().numpy()
    ref, _ = O.sage_attn(inp.q, inp.k, inp.v, inp.seqlens, inp.cu_seqlens, c["causal"], c["blk_q"], c["blk_k"],
                         pv_fp8=c["mode"] >= 1, smooth_v=c["mode"] == 2, smooth_q=c["sq"], qk_fp4=c["fp4"])
    n = None if inp.cu_seqlens is None else int(inp.cu_seqlens[-1])
    o, ref = o[:n], ref[:n]
    cs, e = cos(o, ref), float(np.abs(o - ref).max())
    print(f"[{cfg_id(c)}] cos={cs:.7f} maxabs={e:.3e}", flush=True)
    assert np.isfinite(o).all()
    if c["mode"]:
        assert cs >= 0.9995
    else:
        assert cs >= 0.99995 and e <= 4e-3
