"""GPU parity of grouped-query attention (K and V with fewer heads than Q) and
of the scaled-dot-product-attention drop-in, through the C ABI, against the
CPU oracle.  The drop-in interface is the one the SageAttention pages
replace in one line ("SageAttention：低比特量化Attention，实现推理加速", section
即插即用; "4比特量化三倍加速不掉点！清华即插即用的SageAttention迎来升级", section
即插即用举例); its grouped-query form lets query head h read K/V head
h / (H / H_kv).

Bit-exact: K quantisation per K head; GQA output = the output with each K/V
head repeated (same kernel arithmetic).  Tolerance as in the other parity
tests: fp16 P.V cos >= 0.99995 and max |dO| <= 4e-3, FP8 cos >= 0.9995.
"""
import numpy as np
import pytest

from oracle import sage_oracle as O
from quantized_attention_transformer_amd import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

COS_FP16, MAXABS_FP16, COS_FP8 = 0.99995, 4e-3, 0.9995


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from quantized_attention_transformer_amd import sage
    sage.lib()


def S():
    from quantized_attention_transformer_amd import sage
    return sage


def dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def cos(a, b):
    a = np.asarray(a, np.float64).ravel()
    b = np.asarray(b, np.float64).ravel()
    return float(a @ b / (np.linalg.norm(a) * np.linalg.norm(b)))


def gqa_inputs(wl, hk, **kw):
    """The workload's Q with K and V cut to their first hk heads."""
    inp = synth.generate(wl, **kw)
    z = dict(inp.__dict__)
    z["k"] = np.ascontiguousarray(inp.k[..., :hk, :])
    z["v"] = np.ascontiguousarray(inp.v[..., :hk, :])
    return synth.Inputs(**z)


def gpu_kwargs(inp):
    if inp.cu_seqlens is None:
        return {}
    return dict(cu_seqlens=dev(inp.cu_seqlens), max_seqlen=inp.max_seqlen)


CASES = [
    # (name, workload, overrides, kv heads, causal, pv mode)
    ("B2N333H6kv2d128", synth.TEXT, dict(seqlen=333, batch=2, heads=6), 2, False, 0),
    ("B2N333H6kv2d128-causal-fp8", synth.TEXT, dict(seqlen=333, batch=2, heads=6), 2, True, 1),
    ("B1N600H4kv1d64-mqa-causal", synth.VIDEO, dict(seqlen=600, batch=1, heads=4), 1, True, 0),
    ("varlen-H8kv2-causal", synth.VARLEN, dict(seqlens=[37, 0, 130, 300], heads=8), 2, True, 0),
    ("B1N400H8kv4d128-smooth-v", synth.TEXT, dict(seqlen=400, batch=1, heads=8), 4, False, 2),
]


@pytest.mark.parametrize("name,wl,kw,hk,causal,mode", CASES, ids=[c[0] for c in CASES])
def test_gqa_against_oracle(name, wl, kw, hk, causal, mode):
    inp = gqa_inputs(wl, hk, **kw)
    q, k, v = dev(inp.q), dev(inp.k), dev(inp.v)
    # the pre-pass per K head, bit-exact
    g = S().quantize(q, k, blk_q=wl.blk_q, blk_k=wl.blk_k, **gpu_kwargs(inp))
    ref_q = O.quantize_qk(inp.q, inp.k, inp.seqlens, inp.cu_seqlens, wl.blk_q, wl.blk_k)
    n = None if inp.cu_seqlens is None else int(inp.cu_seqlens[-1])
    assert np.array_equal(host(g["k8"])[:n], ref_q["k8"][:n])
    assert np.array_equal(host(g["q8"])[:n], ref_q["q8"][:n])
    np.testing.assert_array_equal(host(g["k_mean"]), ref_q["km"])
    o = host(S().attn(q, k, v, causal=causal, pv_mode=mode, blk_q=wl.blk_q, blk_k=wl.blk_k, **gpu_kwargs(inp)))
    ref, _ = O.sage_attn(inp.q, inp.k, inp.v, inp.seqlens, inp.cu_seqlens, causal, wl.blk_q, wl.blk_k,
                         pv_fp8=mode >= 1, smooth_v=mode == 2)
    o, ref = o[:n], ref[:n]
    c, e = cos(o, ref), float(np.abs(o - ref).max())
    print(f"[{name}] cos={c:.7f} maxabs={e:.3e}", flush=True)
    assert np.isfinite(o).all()
    if mode:
        assert c >= COS_FP8
    else:
        assert c >= COS_FP16 and e <= MAXABS_FP16


@pytest.mark.parametrize("hk", [1, 2])
def test_gqa_equals_repeated_kv_heads(hk):
    inp = gqa_inputs(synth.TEXT, hk, seqlen=500, batch=2, heads=4)
    q, k, v = dev(inp.q), dev(inp.k), dev(inp.v)
    kr, vr = (t.repeat_interleave(4 // hk, dim=2).contiguous() for t in (k, v))
    for causal in (False, True):
        for mode in (0, 1):
            a = S().attn(q, k, v, causal=causal, pv_mode=mode)
            b = S().attn(q, kr, vr, causal=causal, pv_mode=mode)
            assert torch.equal(a, b), (causal, mode)


def test_sdpa_drop_in():
    inp = gqa_inputs(synth.TEXT, 2, seqlen=300, batch=2, heads=4)
    # torch's layout: [B, H, N, d]
    q, k, v = (dev(x).permute(0, 2, 1, 3).contiguous() for x in (inp.q, inp.k, inp.v))
    for causal in (False, True):
        o = S().scaled_dot_product_attention(q, k, v, is_causal=causal, enable_gqa=True)
        assert o.shape == q.shape
        ref, _ = O.sage_attn(inp.q, inp.k, inp.v, inp.seqlens, None, causal, 128, 64)
        oh = host(o).transpose(0, 2, 1, 3)
        assert cos(oh, ref) >= COS_FP16 and np.abs(oh - ref).max() <= MAXABS_FP16
    # an explicit scale is the softmax scale
    o2 = S().scaled_dot_product_attention(q, k, v, scale=0.05, enable_gqa=True)
    ref2, _ = O.sage_attn(inp.q, inp.k, inp.v, inp.seqlens, None, False, 128, 64, sm_scale=0.05)
    oh2 = host(o2).transpose(0, 2, 1, 3)
    assert cos(oh2, ref2) >= COS_FP16
