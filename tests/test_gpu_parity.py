"""GPU parity: the HIP library (through its C ABI) against the CPU oracle.

Bit-exact: INT8 Q/K codes, their scales, mean(K), the E4M3 V and its scales
(every workload at full size) and the INT32 score tiles (debug entry point).
Tolerance (against the oracle's fp64 output): fp16 P.V path cos >= 0.99995
and max |O - O_ref| <= 4e-3; FP8 P.V path cos >= 0.9995.
Small cases span several tiles with ragged tails and are compared in full;
full-size workloads are compared on sampled query rows.
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


def gpu_kwargs(inp):
    if inp.cu_seqlens is None:
        return {}
    return dict(cu_seqlens=dev(inp.cu_seqlens), max_seqlen=inp.max_seqlen)


def valid_scale_mask(seqlens, nb, blk):
    m = np.zeros((len(seqlens), nb), bool)
    for s, L in enumerate(seqlens):
        m[s, :-(-int(L) // blk)] = True
    return m


def check_close(tag, o_gpu, o_ref, cos_min, max_abs=None):
    mask = ~np.isnan(o_ref)
    a, b = o_gpu[mask].astype(np.float64), o_ref[mask]
    c, e = cos(a, b), float(np.abs(a - b).max())
    print(f"[{tag}] cos={c:.7f} maxabs={e:.3e} n={a.size}", flush=True)
    assert np.isfinite(a).all()
    assert c >= cos_min
    if max_abs is not None:
        assert e <= max_abs


# ---------------------------------------------------------------- E4M3 convert

def test_e4m3_convert_matches_oracle_on_every_code_and_tie():
    vals = [O.e4m3_value(c) for c in range(127)]
    xs = vals + [(vals[i] + vals[i + 1]) / 2 for i in range(126)]
    xs += [np.nextafter(np.float16(x), np.float16(500)) for x in xs[127:]]
    xs += [np.nextafter(np.float16(x), np.float16(0)) for x in xs[127:253]]
    xs = np.array(xs, np.float64)
    xs = np.concatenate([xs, -xs])
    L, d = 512, 64
    v = np.zeros((1, L, 1, d), np.float16)
    v[0, 0, 0, :] = 448.0                      # absmax 448 -> scale exactly 1
    flat = v[0, 1:, 0, :].reshape(-1)
    flat[:len(xs)] = xs.astype(np.float16)
    v[0, 1:, 0, :] = flat.reshape(L - 1, d)
    v8, sv = S().quantize_v_fp8(dev(v))
    assert (host(sv) == 1.0).all()
    want, _, _ = O.quant_v_fp8(v, [L], None)
    np.testing.assert_array_equal(host(v8), want)


# ---------------------------------------------------------------- pre-pass, bit-exact

QUANT_CASES = [synth.TINY, synth.TEXT, synth.VIDEO, synth.VARLEN, synth.LONG, synth.FP8]


PER_TOKEN_CASES = [("text-full-blk1", synth.TEXT, {}), ("varlen-ragged-blk1", synth.VARLEN,
                                                          dict(seqlens=[37, 0, 130, 64, 1, 300], heads=3)),
                   ("tiny-d64-blk1", synth.TINY, {})]


@pytest.mark.parametrize("wl", QUANT_CASES, ids=lambda w: w.name)
def test_quantize_bitexact_full_size(wl):
    check_quantize(wl.name, synth.generate(wl), wl.blk_q, wl.blk_k)


@pytest.mark.parametrize("name,wl,kw", PER_TOKEN_CASES, ids=[c[0] for c in PER_TOKEN_CASES])
def test_quantize_per_token_q_bitexact(name, wl, kw):
    # blk_q = 1: one Q scale per token
    check_quantize(name, synth.generate(wl, **kw), 1, wl.blk_k)


def check_quantize(name, inp, blk_q, blk_k):
    print(f"[{name}] shapes q{inp.q.shape} seqlens={list(inp.seqlens)} blocks {blk_q}/{blk_k}", flush=True)
    g = S().quantize(dev(inp.q), dev(inp.k), blk_q=blk_q, blk_k=blk_k, **gpu_kwargs(inp))
    ref = O.quantize_qk(inp.q, inp.k, inp.seqlens, inp.cu_seqlens, blk_q, blk_k)
    np.testing.assert_array_equal(host(g["k_mean"]), ref["km"])
    mq = valid_scale_mask(inp.seqlens, ref["sq"].shape[2], blk_q)
    mk = valid_scale_mask(inp.seqlens, ref["sk"].shape[2], blk_k)
    np.testing.assert_array_equal(host(g["q_scale"])[mq[:, None, :].repeat(inp.q.shape[-2], 1)],
                                  ref["sq"][mq[:, None, :].repeat(inp.q.shape[-2], 1)])
    np.testing.assert_array_equal(host(g["k_scale"])[mk[:, None, :].repeat(inp.q.shape[-2], 1)],
                                  ref["sk"][mk[:, None, :].repeat(inp.q.shape[-2], 1)])
    q8, k8 = host(g["q8"]), host(g["k8"])
    assert np.array_equal(q8, ref["q8"]), f"q8 mismatches: {(q8 != ref['q8']).sum()}"
    assert np.array_equal(k8, ref["k8"]), f"k8 mismatches: {(k8 != ref['k8']).sum()}"


@pytest.mark.parametrize("wl,kw", [(synth.FP8, {}), (synth.VARLEN, dict(seqlens=[700, 0, 1, 1500], heads=4))],
                         ids=["fp8-full", "varlen-small"])
def test_quantize_v_fp8_bitexact(wl, kw):
    inp = synth.generate(wl, **kw)
    v8, sv = S().quantize_v_fp8(dev(inp.v), **gpu_kwargs(inp))
    rv8, rsv, _ = O.quant_v_fp8(inp.v, inp.seqlens, inp.cu_seqlens)
    np.testing.assert_array_equal(host(sv), rsv)
    g8 = host(v8)
    if inp.cu_seqlens is None:
        np.testing.assert_array_equal(g8, rv8)
    else:
        np.testing.assert_array_equal(g8[:inp.cu_seqlens[-1]], rv8[:inp.cu_seqlens[-1]])


def test_quantize_nondefault_blocks_and_layout():
    wl = synth.TEXT
    inp = synth.generate(wl, seqlen=1000, batch=2, heads=3)
    q = dev(inp.q).permute(0, 2, 1, 3).contiguous()       # [B, H, N, d]
    k = dev(inp.k).permute(0, 2, 1, 3).contiguous()
    g = S().quantize(q, k, layout="bhnd", blk_q=48, blk_k=16, sm_scale=0.3)
    ref = O.quantize_qk(inp.q, inp.k, inp.seqlens, None, 48, 16, sm_scale=0.3)
    np.testing.assert_array_equal(host(g["q8"]).transpose(0, 2, 1, 3), ref["q8"])
    np.testing.assert_array_equal(host(g["k8"]).transpose(0, 2, 1, 3), ref["k8"])
    np.testing.assert_array_equal(host(g["q_scale"]), ref["sq"])
    np.testing.assert_array_equal(host(g["k_scale"]), ref["sk"])


# ---------------------------------------------------------------- integer scores, bit-exact

# The dump comes from the fused kernel itself (a dump instantiation): N = 1000
# and 1024 give 16 key tiles, so both halves run steady-state (qk_pv) phase
# pairs as well as edge phases (qk_tile), through the 5-slot K ring.
@pytest.mark.parametrize("N,H,d", [(256, 2, 64), (1000, 2, 128), (1024, 1, 128), (132, 3, 64), (1000, 2, 64),
                                   (1024, 2, 64), (768, 2, 128)])
def test_debug_qk_i32_bitexact(N, H, d):
    wl = synth.TEXT if d == 128 else synth.TINY
    inp = synth.generate(wl, seqlen=N, batch=1, heads=H)
    ref = O.quantize_qk(inp.q, inp.k, inp.seqlens, None, 64, 64)
    s = host(S().debug_qk_i32(dev(ref["q8"]), dev(ref["k8"])))
    for h in range(H):
        want = O.scores_int(ref["q8"][0, :, h], ref["k8"][0, :, h])
        assert np.array_equal(s[0, h], want), f"head {h}: {(s[0, h] != want).sum()} mismatches"


@pytest.mark.parametrize("d", [64, 128])
def test_debug_qk_i32_extreme_codes_and_gqa(d):
    """Codes of magnitude 127 everywhere (|S| up to 127^2 d, the edge of the
    accumulator seed's range), two batches, and K with half the heads."""
    rng = np.random.default_rng(d)
    B, N, H, Hk = 2, 1024, 4, 2
    q8 = (rng.choice([-127, 127], size=(B, N, H, d)) * (rng.random((B, N, H, d)) < 0.97)).astype(np.int8)
    k8 = rng.choice([-127, 127], size=(B, N, Hk, d)).astype(np.int8)
    k8[:, :64] = 127                           # keys of the first tile agree with some rows exactly
    q8[:, :8] = 127
    s = host(S().debug_qk_i32(dev(q8), dev(k8)))
    for b in range(B):
        for h in range(H):
            want = O.scores_int(q8[b, :, h], k8[b, :, h // (H // Hk)])
            assert np.array_equal(s[b, h], want), f"batch {b} head {h}: {(s[b, h] != want).sum()} mismatches"
    assert np.abs(s).max() == 127 * 127 * d


# ---------------------------------------------------------------- attention

def run_attn(inp, causal, pv_fp8=False, blk_q=None, blk_k=None, layout="bnhd", sm_scale=None):
    wl = inp.wl
    mode = 1 if pv_fp8 else 0
    q, k, v = dev(inp.q), dev(inp.k), dev(inp.v)
    if layout == "bhnd":
        q, k, v = (t.permute(0, 2, 1, 3).contiguous() for t in (q, k, v))
    o = S().attn(q, k, v, causal=causal, pv_mode=mode, blk_q=blk_q or wl.blk_q, blk_k=blk_k or wl.blk_k,
                 layout=layout, sm_scale=sm_scale, **gpu_kwargs(inp))
    o = host(o)
    if layout == "bhnd":
        o = o.transpose(0, 2, 1, 3)
    return o


SMALL = [
    # (name, workload, overrides, causal, blk_q, blk_k)
    ("tiny-full", synth.TINY, {}, False, None, None),
    ("B2N333H3d128", synth.TEXT, dict(seqlen=333, batch=2, heads=3), False, 128, 64),
    ("B2N333H3d128-causal", synth.TEXT, dict(seqlen=333, batch=2, heads=3), True, 128, 64),
    ("B1N200H2d64-blk32x16", synth.VIDEO, dict(seqlen=200, batch=1, heads=2), False, 32, 16),
    ("B1N200H2d64-causal-blk32x16", synth.VIDEO, dict(seqlen=200, batch=1, heads=2), True, 32, 16),
    ("varlen-ragged", synth.VARLEN, dict(seqlens=[37, 0, 130, 64, 1, 300], heads=3), False, 128, 64),
    ("varlen-ragged-causal", synth.VARLEN, dict(seqlens=[37, 0, 130, 64, 1, 300], heads=3), True, 128, 64),
    ("B1N577H2d128-blk256x256-causal", synth.LONG, dict(seqlen=577, batch=1, heads=2), True, 256, 256),
    ("B2N333H3d128-blk1x64", synth.TEXT, dict(seqlen=333, batch=2, heads=3), False, 1, 64),
    ("varlen-ragged-causal-blk1x16", synth.VARLEN, dict(seqlens=[37, 0, 130, 64, 1, 300], heads=3), True, 1, 16),
]


@pytest.mark.parametrize("name,wl,kw,causal,bq,bk", SMALL, ids=[c[0] for c in SMALL])
@pytest.mark.parametrize("fp8", [False, True], ids=["fp16pv", "fp8pv"])
def test_attn_small_full_compare(name, wl, kw, causal, bq, bk, fp8):
    inp = synth.generate(wl, **kw)
    bq, bk = bq or wl.blk_q, bk or wl.blk_k
    o = run_attn(inp, causal, fp8, bq, bk)
    ref, _ = O.sage_attn(inp.q, inp.k, inp.v, inp.seqlens, inp.cu_seqlens, causal, bq, bk, pv_fp8=fp8)
    if inp.cu_seqlens is not None:          # rows past the last sequence are not part of the output
        o, ref = o[:inp.cu_seqlens[-1]], ref[:inp.cu_seqlens[-1]]
    if fp8:
        check_close(name + "/fp8", o, ref, COS_FP8)
    else:
        check_close(name, o, ref, COS_FP16, MAXABS_FP16)


def sample_rows(L, n_rand, seed, tile=128):
    """The first and last query tile, a whole tile in the middle of the
    sequence (mid-sequence causal tiles: many full key tiles, then the
    diagonal), and n_rand random rows."""
    rng = np.random.default_rng(seed)
    mid = (L // 2) // tile * tile
    rows = set(range(min(L, tile))) | set(range(max(0, L - tile), L)) | set(range(mid, min(L, mid + tile)))
    rows |= set(rng.integers(0, L, size=n_rand).tolist())
    return np.array(sorted(rows))


FULL = [
    ("text", synth.TEXT, False, False, None),
    ("text-causal", synth.TEXT_CAUSAL, True, False, None),
    ("video", synth.VIDEO, False, False, 64),
    ("varlen", synth.VARLEN, True, False, 64),
    ("long-causal", synth.LONG, True, False, 64),
    ("fp8", synth.FP8, False, True, 64),
]


@pytest.mark.parametrize("name,wl,causal,fp8,nrand", FULL, ids=[c[0] for c in FULL])
def test_attn_full_size(name, wl, causal, fp8, nrand):
    inp = synth.generate(wl)
    print(f"[{name}] q{inp.q.shape} seqlens={list(inp.seqlens)}", flush=True)
    o = run_attn(inp, causal, fp8)
    rows = None
    if nrand is not None:
        rows = {s: sample_rows(int(L), nrand, 7 + s) for s, L in enumerate(inp.seqlens) if L > 0}
    ref, _ = O.sage_attn(inp.q, inp.k, inp.v, inp.seqlens, inp.cu_seqlens, causal, wl.blk_q, wl.blk_k,
                         pv_fp8=fp8, rows_by_seq=rows)
    if fp8:
        check_close(name, o, ref, COS_FP8)
    else:
        check_close(name, o, ref, COS_FP16, MAXABS_FP16)


def test_attn_closed_forms():
    wl = synth.TEXT
    inp = synth.generate(wl, seqlen=300, batch=1, heads=2)
    o = run_attn(inp, True)
    # causal row 0 attends only to key 0: O[0] = V[0] exactly
    np.testing.assert_array_equal(o[0, 0], inp.v[0, 0])
    # Q = 0: every code and score is 0, O is the running mean of V
    z = dict(inp.__dict__)
    z["q"] = np.zeros_like(inp.q)
    zi = synth.Inputs(**z)
    for causal in (False, True):
        o = run_attn(zi, causal)
        vf = inp.v[0].astype(np.float64)
        want = (np.cumsum(vf, 0) / np.arange(1, 301)[:, None, None]) if causal else np.broadcast_to(vf.mean(0), vf.shape)
        assert np.abs(o[0] - want).max() <= 2e-3
    # identical keys: smoothed K is 0, scores 0, uniform attention
    k = dict(inp.__dict__)
    k["k"] = np.broadcast_to(inp.k[:, :1], inp.k.shape).copy()
    ki = synth.Inputs(**k)
    g = S().quantize(dev(ki.q), dev(ki.k), blk_q=128, blk_k=64)
    assert not host(g["k8"]).any() and not host(g["k_scale"]).any()
    o = run_attn(ki, False)
    assert np.abs(o[0] - inp.v[0].astype(np.float64).mean(0)).max() <= 2e-3


def test_attn_deterministic_layout_and_varlen_equals_dense():
    wl = synth.VARLEN
    inp = synth.generate(wl, seqlens=[200, 333, 64], heads=2)
    for causal in (False, True):
        for fp8 in (False, True):
            a = run_attn(inp, causal, fp8)
            b = run_attn(inp, causal, fp8)
            assert np.array_equal(a, b)
            for s, L in enumerate(inp.seqlens):
                lo, hi = inp.cu_seqlens[s], inp.cu_seqlens[s + 1]
                dense = synth.Inputs(wl, inp.q[None, lo:hi], inp.k[None, lo:hi], inp.v[None, lo:hi], None,
                                     np.array([L]))
                d = run_attn(dense, causal, fp8)
                assert np.array_equal(d[0], a[lo:hi]), (causal, fp8, s)
    dense = synth.generate(synth.TEXT, seqlen=200, batch=2, heads=3)
    for causal in (False, True):
        assert np.array_equal(run_attn(dense, causal), run_attn(dense, causal, layout="bhnd"))


def test_attn_quantized_entry_matches_attn():
    wl = synth.TEXT
    inp = synth.generate(wl, seqlen=700, batch=2, heads=2)
    q, k, v = dev(inp.q), dev(inp.k), dev(inp.v)
    for causal in (False, True):
        g = S().quantize(q, k, blk_q=128, blk_k=64)
        o1 = S().attn_quantized(g["q8"], g["k8"], g["q_scale"], g["k_scale"], v, causal=causal)
        o2 = S().attn(q, k, v, causal=causal)
        assert torch.equal(o1, o2)
        v8, sv = S().quantize_v_fp8(v)
        o1 = S().attn_quantized(g["q8"], g["k8"], g["q_scale"], g["k_scale"], v8, v_scale=sv, causal=causal,
                                pv_mode=1)
        o2 = S().attn(q, k, v, causal=causal, pv_mode=1)
        assert torch.equal(o1, o2)


def test_empty_inputs():
    q = torch.zeros((1, 0, 2, 64), dtype=torch.float16, device="cuda")
    o = S().attn(q, q, q, causal=True)
    assert o.shape == q.shape
    cu = torch.zeros(4, dtype=torch.int32, device="cuda")
    qv = torch.zeros((0, 2, 64), dtype=torch.float16, device="cuda")
    o = S().attn(qv, qv, qv, cu_seqlens=cu, max_seqlen=0)
    assert o.shape == qv.shape


@pytest.mark.parametrize("wl_name", ["TEXT", "VIDEO"])
def test_packed_qkv_views_and_strided_output(wl_name):
    """Q, K and V as views of one packed [B, N, 3, H, d] tensor (token stride
    3·H·d) and O written into a slice of a wider buffer (token stride (H+1)·d):
    bit-identical to contiguous tensors, causal and not, fp16 and FP8 P·V; the
    buffer's other head slot is left as it was.  The SDPA drop-in on the
    transposed [B, H, N, d] views of the packed tensor gives the same bits as on
    their contiguous copies."""
    wl = getattr(synth, wl_name)
    inp = synth.generate(wl, seqlen=333, batch=2, heads=4)
    q, k, v = dev(inp.q), dev(inp.k), dev(inp.v)
    qkv = torch.stack([q, k, v], dim=2)
    qv, kv, vv = qkv.unbind(2)
    assert qv.stride(1) == 3 * q.shape[2] * q.shape[3]
    B, N, H, D = q.shape
    for causal in (False, True):
        for pv in (S().SAGE_PV_FP16, S().SAGE_PV_FP8):
            ref = S().attn(q, k, v, causal=causal, pv_mode=pv, blk_q=wl.blk_q, blk_k=wl.blk_k)
            buf = torch.full((B, N, H + 1, D), 7.0, dtype=torch.float16, device="cuda")
            out = buf[:, :, :H]
            got = S().attn(qv, kv, vv, causal=causal, pv_mode=pv, blk_q=wl.blk_q, blk_k=wl.blk_k, out=out)
            torch.cuda.synchronize()
            assert got.data_ptr() == out.data_ptr()
            assert torch.equal(got, ref), (causal, pv)
            assert bool((buf[:, :, H] == 7.0).all())
    qh, kh, vh = (t.transpose(1, 2) for t in (qv, kv, vv))
    assert not qh.is_contiguous()
    for causal in (False, True):
        a = S().scaled_dot_product_attention(qh, kh, vh, is_causal=causal, blk_q=wl.blk_q, blk_k=wl.blk_k)
        b = S().scaled_dot_product_attention(qh.contiguous(), kh.contiguous(), vh.contiguous(), is_causal=causal,
                                             blk_q=wl.blk_q, blk_k=wl.blk_k)
        torch.cuda.synchronize()
        assert torch.equal(a, b), causal
