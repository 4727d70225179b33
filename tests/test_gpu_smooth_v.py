"""GPU parity of the smoothed-V FP8 P.V path (pv_mode SAGE_PV_FP8_SMOOTH_V)
against the CPU oracle: "4比特量化三倍加速不掉点！清华即插即用的SageAttention迎来升级",
the optional V smoothing after section 技术方案 (subtract mean(V) per channel
before the E4M3 quantisation, add it back to the output).

Bit-exact: the means, scales and E4M3 codes of the smoothed V.  Tolerance:
FP8 path cos >= 0.9995 against the oracle's fp64 output, taken on O minus
each channel's mean (the offset alone would make any result look close).  V
carries per-channel offsets of std 4 over N(0, 1) values: large for E4M3's 3
mantissa bits, small enough that the fp16 rounding of O stays far below the
part compared.
"""
import numpy as np
import pytest

from oracle import sage_oracle as O
from quantized_attention_transformer_amd import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

COS_FP8 = 0.9995


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


def with_offsets(inp, std=4.0, seed=5):
    """The workload's V plus a per-(head, channel) offset ~ N(0, std^2), in fp16."""
    rng = np.random.default_rng(seed)
    H, d = inp.v.shape[-2], inp.v.shape[-1]
    off = rng.standard_normal((H, d)) * std
    v = (inp.v.astype(np.float64) + off).astype(np.float16)
    z = dict(inp.__dict__)
    z["v"] = v
    return synth.Inputs(**z)


def gpu_kwargs(inp):
    if inp.cu_seqlens is None:
        return {}
    return dict(cu_seqlens=dev(inp.cu_seqlens), max_seqlen=inp.max_seqlen)


QUANT = [
    ("fp8-full", synth.FP8, {}),
    ("varlen-small", synth.VARLEN, dict(seqlens=[700, 0, 1, 1500], heads=4)),
    ("tiny-d64", synth.TINY, {}),
]


@pytest.mark.parametrize("name,wl,kw", QUANT, ids=[c[0] for c in QUANT])
def test_quantize_v_fp8_smooth_bitexact(name, wl, kw):
    inp = with_offsets(synth.generate(wl, **kw))
    print(f"[{name}] v{inp.v.shape} seqlens={list(inp.seqlens)}", flush=True)
    v8, svm = S().quantize_v_fp8(dev(inp.v), smooth=True, **gpu_kwargs(inp))
    rv8, rsv, rvm = O.quant_v_fp8(inp.v, inp.seqlens, inp.cu_seqlens, smooth=True)
    svm = host(svm)
    np.testing.assert_array_equal(svm[1], rvm)
    np.testing.assert_array_equal(svm[0], rsv)
    g8 = host(v8)
    if inp.cu_seqlens is None:
        np.testing.assert_array_equal(g8, rv8)
    else:
        np.testing.assert_array_equal(g8[:inp.cu_seqlens[-1]], rv8[:inp.cu_seqlens[-1]])


SMALL = [
    ("B2N333H3d128", synth.TEXT, dict(seqlen=333, batch=2, heads=3), False, 128, 64),
    ("B2N333H3d128-causal", synth.TEXT, dict(seqlen=333, batch=2, heads=3), True, 128, 64),
    ("B1N200H2d64-causal-blk32x16", synth.VIDEO, dict(seqlen=200, batch=1, heads=2), True, 32, 16),
    ("varlen-ragged-causal", synth.VARLEN, dict(seqlens=[37, 0, 130, 64, 1, 600], heads=3), True, 128, 64),
]


@pytest.mark.parametrize("name,wl,kw,causal,bq,bk", SMALL, ids=[c[0] for c in SMALL])
def test_attn_smooth_v_small_full_compare(name, wl, kw, causal, bq, bk):
    inp = with_offsets(synth.generate(wl, **kw))
    o = host(S().attn(dev(inp.q), dev(inp.k), dev(inp.v), causal=causal, pv_mode=S().SAGE_PV_FP8_SMOOTH_V,
                      blk_q=bq, blk_k=bk, **gpu_kwargs(inp)))
    ref, _ = O.sage_attn(inp.q, inp.k, inp.v, inp.seqlens, inp.cu_seqlens, causal, bq, bk, pv_fp8=True,
                         smooth_v=True)
    plain = host(S().attn(dev(inp.q), dev(inp.k), dev(inp.v), causal=causal, pv_mode=S().SAGE_PV_FP8,
                          blk_q=bq, blk_k=bk, **gpu_kwargs(inp)))
    if inp.cu_seqlens is not None:
        o, ref, plain = o[:inp.cu_seqlens[-1]], ref[:inp.cu_seqlens[-1]], plain[:inp.cu_seqlens[-1]]
    mean = np.nanmean(ref, axis=tuple(range(ref.ndim - 2)), keepdims=True)
    c = cos(o - mean, ref - mean)
    c_plain = cos(plain - mean, ref - mean)
    print(f"[{name}/fp8-smooth-v] cos beyond the mean={c:.7f} (plain FP8 {c_plain:.5f}) "
          f"maxabs={np.abs(o - ref).max():.3e}", flush=True)
    assert np.isfinite(o).all() and c >= COS_FP8
    assert c_plain < c - 1e-3


def test_attn_smooth_v_full_size_sampled_rows():
    # the FP8 workload at full size with its own V distribution (at N = 8192 the
    # attention is diffuse and O beyond the mean is ~0.02, below what fp16 output
    # resolves next to an offset; the offsets are covered by the small cases and by
    # the bit-exact full-size quantisation above)
    wl = synth.FP8
    inp = synth.generate(wl)
    o = host(S().attn(dev(inp.q), dev(inp.k), dev(inp.v), causal=False, pv_mode=S().SAGE_PV_FP8_SMOOTH_V,
                      blk_q=wl.blk_q, blk_k=wl.blk_k))
    rng = np.random.default_rng(3)
    rows = {s: np.unique(np.concatenate([np.arange(128), np.arange(wl.seqlen - 128, wl.seqlen),
                                         rng.integers(0, wl.seqlen, 64)])) for s in range(wl.batch)}
    ref, _ = O.sage_attn(inp.q, inp.k, inp.v, inp.seqlens, None, False, wl.blk_q, wl.blk_k, pv_fp8=True,
                         smooth_v=True, rows_by_seq=rows)
    mask = ~np.isnan(ref)
    c = cos(o[mask], ref[mask])
    print(f"[fp8-full/smooth-v] cos={c:.7f} maxabs={np.abs(o[mask] - ref[mask]).max():.3e} n={mask.sum()}",
          flush=True)
    assert np.isfinite(o).all() and c >= COS_FP8


def test_attn_smooth_v_constant_values_give_them_exactly():
    inp = synth.generate(synth.TEXT, seqlen=300, batch=1, heads=2)
    row = inp.v[:, :1]
    v = np.broadcast_to(row, inp.v.shape).copy()
    v8, svm = S().quantize_v_fp8(dev(v), smooth=True)
    assert not host(v8).any() and not host(svm)[0].any()
    for causal in (False, True):
        o = host(S().attn(dev(inp.q), dev(inp.k), dev(v), causal=causal, pv_mode=S().SAGE_PV_FP8_SMOOTH_V))
        np.testing.assert_array_equal(o, v)


def test_attn_quantized_smooth_v_entry_matches_attn():
    inp = with_offsets(synth.generate(synth.TEXT, seqlen=700, batch=2, heads=2))
    q, k, v = dev(inp.q), dev(inp.k), dev(inp.v)
    g = S().quantize(q, k, blk_q=128, blk_k=64)
    v8, svm = S().quantize_v_fp8(v, smooth=True)
    for causal in (False, True):
        o1 = S().attn_quantized(g["q8"], g["k8"], g["q_scale"], g["k_scale"], v8, v_scale=svm, causal=causal,
                                pv_mode=S().SAGE_PV_FP8_SMOOTH_V)
        o2 = S().attn(q, k, v, causal=causal, pv_mode=S().SAGE_PV_FP8_SMOOTH_V)
        assert torch.equal(o1, o2)
