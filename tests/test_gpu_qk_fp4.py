"""GPU parity of the 4-bit Q.K^T variant ("4比特量化三倍加速不掉点！清华即插即用的SageAttention迎来升级",
section 技术方案: the INT4 kernel, here in gfx950's 4-bit matrix format, OCP MXFP4)
through the C ABI, against the CPU oracle.

Bit-exact: the E2M1 codes and E8M0 scales of Q' (or Q_s) and of the smoothed K,
and K's mean.  Attention output against the oracle, whose S is exact from the
same codes: fp16 P.V cos >= 0.99995 and max |dO| <= 4e-3, FP8 cos >= 0.9995,
as in the other parity tests (the MFMA's fp32 sums of exact products differ
from the oracle's S by fp32 rounding only).  The accuracy of 4-bit Q and K
against exact attention is a property of the method (cos ~0.986 on N(0, 1)
inputs); it is checked only relative to smoothing Q.
"""
import dataclasses

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


def gpu_kwargs(inp):
    if inp.cu_seqlens is None:
        return {}
    return dict(cu_seqlens=dev(inp.cu_seqlens), max_seqlen=inp.max_seqlen)


def vary(inp, q_std=0.0, hk=None, zero_block=False, seed=11):
    """The workload with optional per-(head, channel) Q offsets, K/V cut to hk heads,
    and Q channels 32..63 zeroed (an all-zero MXFP4 block in every row)."""
    rng = np.random.default_rng(seed)
    H, d = inp.q.shape[-2], inp.q.shape[-1]
    z = dict(inp.__dict__)
    q = inp.q.astype(np.float64) + (rng.standard_normal((H, d)) * q_std if q_std else 0.0)
    if zero_block:
        q[..., 32:64] = 0.0
    z["q"] = q.astype(np.float16)
    if hk:
        z["k"] = np.ascontiguousarray(inp.k[..., :hk, :])
        z["v"] = np.ascontiguousarray(inp.v[..., :hk, :])
    return synth.Inputs(**z)


def unpack(b):
    """uint8 [..., d/2] -> E2M1 codes [..., d] (channel 2c in the low nibble of byte c)."""
    out = np.empty(b.shape[:-1] + (2 * b.shape[-1],), np.uint8)
    out[..., 0::2] = b & 0xF
    out[..., 1::2] = b >> 4
    return out


def scales_by_seq(sc, inp):
    """Device scales [B, N, H, nb] or [T, H, nb] as the oracle's [nseq, H, maxL, nb]."""
    nb = sc.shape[-1]
    out = np.zeros((inp.nseq, sc.shape[-2], inp.max_seqlen, nb), np.uint8)
    for s in range(inp.nseq):
        L = int(inp.seqlens[s])
        blk = sc[s, :L] if inp.cu_seqlens is None else sc[inp.cu_seqlens[s]:inp.cu_seqlens[s + 1]]
        out[s, :, :L] = blk.transpose(1, 0, 2)
    return out


TEXT96 = dataclasses.replace(synth.TEXT, name="text d96", head_dim=96)

QUANT = [
    # (name, workload, overrides, q offset std, kv heads, smooth Q, zero block)
    ("text-full", synth.TEXT, {}, 0.0, 0, False, False),
    ("text-full-smooth-q", synth.TEXT, {}, 4.0, 0, True, False),
    ("varlen-ragged", synth.VARLEN, dict(seqlens=[37, 0, 130, 64, 1, 600], heads=3), 0.0, 0, False, True),
    ("tiny-d64", synth.TINY, {}, 0.0, 0, False, False),
    ("gqa-h8-kv2-smooth-q", synth.TEXT, dict(seqlen=400, heads=8), 3.0, 2, True, False),
    ("video-d64-outlier-channels", synth.VIDEO, dict(seqlen=700, batch=1, heads=2), 0.0, 0, False, False),
]


@pytest.mark.parametrize("name,wl,kw,qstd,hk,sq,zb", QUANT, ids=[c[0] for c in QUANT])
def test_quantize_mxfp4_bitexact(name, wl, kw, qstd, hk, sq, zb):
    inp = vary(synth.generate(wl, **kw), q_std=qstd, hk=hk, zero_block=zb)
    print(f"[{name}] q{inp.q.shape} k{inp.k.shape}", flush=True)
    g = S().quantize_mxfp4(dev(inp.q), dev(inp.k), smooth_q=sq, **gpu_kwargs(inp))
    ref = O.quantize_qk_fp4(inp.q, inp.k, inp.seqlens, inp.cu_seqlens, smooth_q=sq)
    n = None if inp.cu_seqlens is None else int(inp.cu_seqlens[-1])
    np.testing.assert_array_equal(host(g["k_mean"]), ref["km"])
    if sq:
        np.testing.assert_array_equal(host(g["q_mean"]), ref["qm"])
    assert np.array_equal(unpack(host(g["q4"]))[:n], ref["q4"][:n])
    assert np.array_equal(unpack(host(g["k4"]))[:n], ref["k4"][:n])
    np.testing.assert_array_equal(scales_by_seq(host(g["q_scale"]), inp), ref["qsc"])
    np.testing.assert_array_equal(scales_by_seq(host(g["k_scale"]), inp), ref["ksc"])
    if zb:
        assert not scales_by_seq(host(g["q_scale"]), inp)[:, :, :, 1].any()


ATTN = [
    # (name, workload, overrides, causal, pv mode, q offset std, kv heads, smooth Q)
    ("B2N333H3", synth.TEXT, dict(seqlen=333, batch=2, heads=3), False, 0, 0.0, 0, False),
    ("B2N333H3-causal", synth.TEXT, dict(seqlen=333, batch=2, heads=3), True, 0, 0.0, 0, False),
    ("B2N333H3-fp8", synth.TEXT, dict(seqlen=333, batch=2, heads=3), False, 1, 0.0, 0, False),
    ("B1N500H2-causal-smooth-v", synth.TEXT, dict(seqlen=500, batch=1, heads=2), True, 2, 0.0, 0, False),
    ("varlen-ragged-causal", synth.VARLEN, dict(seqlens=[37, 0, 130, 64, 1, 600], heads=3), True, 0, 0.0, 0, False),
    ("B1N400H8kv2-gqa-causal-fp8", synth.TEXT, dict(seqlen=400, batch=1, heads=8), True, 1, 0.0, 2, False),
    ("B1N500H2-smooth-q", synth.TEXT, dict(seqlen=500, batch=1, heads=2), False, 0, 4.0, 0, True),
    ("B1N500H2-causal-smooth-q-fp8", synth.TEXT, dict(seqlen=500, batch=1, heads=2), True, 1, 4.0, 0, True),
    ("B1N300H2-d96", TEXT96, dict(seqlen=300, batch=1, heads=2), True, 0, 0.0, 0, False),
]


@pytest.mark.parametrize("name,wl,kw,causal,mode,qstd,hk,sq", ATTN, ids=[c[0] for c in ATTN])
def test_attn_qk_fp4_against_oracle(name, wl, kw, causal, mode, qstd, hk, sq):
    inp = vary(synth.generate(wl, **kw), q_std=qstd, hk=hk)
    print(f"[{name}] q{inp.q.shape} k{inp.k.shape} seqlens={list(inp.seqlens)}", flush=True)
    o = host(S().attn(dev(inp.q), dev(inp.k), dev(inp.v), causal=causal, pv_mode=mode, qk_fp4=True, smooth_q=sq,
                      **gpu_kwargs(inp)))
    ref, _ = O.sage_attn(inp.q, inp.k, inp.v, inp.seqlens, inp.cu_seqlens, causal, 128, 64, pv_fp8=mode >= 1,
                         smooth_v=mode == 2, smooth_q=sq, qk_fp4=True)
    n = None if inp.cu_seqlens is None else int(inp.cu_seqlens[-1])
    o, ref = o[:n], ref[:n]
    c, e = cos(o, ref), float(np.abs(o - ref).max())
    print(f"[{name}] cos={c:.7f} maxabs={e:.3e}", flush=True)
    assert np.isfinite(o).all()
    if mode:
        assert c >= COS_FP8
    else:
        assert c >= COS_FP16 and e <= MAXABS_FP16


def test_attn_qk_fp4_full_size_sampled_rows():
    wl = synth.TEXT
    inp = synth.generate(wl)
    for causal in (False, True):
        o = host(S().attn(dev(inp.q), dev(inp.k), dev(inp.v), causal=causal, qk_fp4=True))
        rng = np.random.default_rng(5)
        rows = {0: np.unique(np.concatenate([np.arange(128), np.arange(wl.seqlen - 128, wl.seqlen),
                                             rng.integers(0, wl.seqlen, 64)]))}
        ref, _ = O.sage_attn(inp.q, inp.k, inp.v, inp.seqlens, None, causal, 128, 64, rows_by_seq=rows, qk_fp4=True)
        mask = ~np.isnan(ref)
        c, e = cos(o[mask], ref[mask]), float(np.abs(o[mask] - ref[mask]).max())
        print(f"[text full causal={causal} qk-fp4] cos={c:.7f} maxabs={e:.3e}", flush=True)
        assert np.isfinite(o).all() and c >= COS_FP16 and e <= MAXABS_FP16


def test_attn_qk_fp4_smooth_q_closer_to_exact_attention():
    inp = vary(synth.generate(synth.TEXT, seqlen=512, batch=1, heads=4), q_std=4.0)
    q, k, v = dev(inp.q), dev(inp.k), dev(inp.v)
    ex = O.exact_attention(inp.q, inp.k, inp.v, inp.seqlens, None, False)
    plain = host(S().attn(q, k, v, qk_fp4=True))
    smooth = host(S().attn(q, k, v, qk_fp4=True, smooth_q=True))
    int8 = host(S().attn(q, k, v))
    rms = lambda o: float(np.sqrt(np.mean((o - ex) ** 2)))  # noqa: E731
    print(f"[qk-fp4 accuracy] rms vs exact: fp4 {rms(plain):.3e}, fp4 + smooth Q {rms(smooth):.3e}, "
          f"int8 {rms(int8):.3e}", flush=True)
    assert rms(smooth) < 0.5 * rms(plain)


def test_qk_fp4_entry_rules():
    q = torch.zeros((1, 64, 2, 64), dtype=torch.float16, device="cuda")
    with pytest.raises(RuntimeError):
        S().attn(q, q, q, qk_fp4=True)          # head_dim 64: the 4-bit kernel runs 128 channels
