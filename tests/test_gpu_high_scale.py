"""GPU parity at large score scales: Q and K ~ N(0, sigma^2) with sigma up to
10 (and 20, 300 for the exact slow path), where q_scale * k_scale is large and
the softmax is peaked -- the regime an SDPA drop-in meets on real
activations.  The fused kernel's exponent x c - (1.5*2^23 c + m) must then
round only at the size of the result ("SageAttention：低比特量化Attention，
实现推理加速", 技术方案 item 3: the softmax and P.V keep 16-bit accuracy).

Bars against the oracle's fp64 output, as for every workload: fp16 P.V cos >=
0.99995 and max |O - O_ref| <= 4e-3; FP8 P.V cos >= 0.9995.  Every case is
compared in full (several 64-key tiles, a ragged tail, 128-row query tiles).
"""
import numpy as np
import pytest

from oracle import sage_oracle as O

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

COS_FP16, MAXABS_FP16, COS_FP8 = 0.99995, 4e-3, 0.9995


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from quantized_attention_transformer_amd import sage
    sage.lib()


def inputs(seed, sigma, d, L=777, H=2, q_offset=0.0):
    """Q, K ~ N(0, sigma^2) (K plus a per-channel bias of std 2, Q plus a
    per-channel offset of std q_offset), V ~ N(0, 1); fp16 [1, L, H, d]."""
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((1, L, H, d)) * sigma + rng.standard_normal((1, 1, H, d)) * q_offset
    k = rng.standard_normal((1, L, H, d)) * sigma + rng.standard_normal((1, 1, H, d)) * 2.0
    v = rng.standard_normal((1, L, H, d))
    return q.astype(np.float16), k.astype(np.float16), v.astype(np.float16)


def run_case(tag, seed, sigma, d, causal, pv_mode=0, smooth_q=False, q_offset=0.0):
    from quantized_attention_transformer_amd import sage
    q, k, v = inputs(seed, sigma, d, q_offset=q_offset)
    L = q.shape[1]
    out = sage.attn(*(torch.from_numpy(x).cuda() for x in (q, k, v)), causal=causal, pv_mode=pv_mode,
                    smooth_q=smooth_q)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    ref, qd = O.sage_attn(q, k, v, [L], None, causal, 128, 64, pv_fp8=pv_mode != 0, smooth_v=pv_mode == 2,
                          smooth_q=smooth_q)
    a, b = got.ravel(), ref.ravel()
    c = float(a @ b / np.linalg.norm(a) / np.linalg.norm(b))
    e = float(np.abs(a - b).max())
    cmax = float(qd["sq"].max() * qd["sk"].max() * O.LOG2E)
    print(f"[{tag}] sigma={sigma} d={d} causal={causal} pv={pv_mode} smooth_q={smooth_q}: "
          f"c<={cmax:.3g} cos={c:.8f} maxabs={e:.3e}", flush=True)
    assert np.isfinite(a).all()
    if pv_mode == 0:
        assert c >= COS_FP16 and e <= MAXABS_FP16, (c, e)
    else:
        assert c >= COS_FP8, c
    return cmax


@pytest.mark.parametrize("sigma", [6.0, 10.0])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_fp16_pv_high_scale(sigma, d, causal):
    run_case("fp16", 100 + int(sigma) + d, sigma, d, causal)


@pytest.mark.parametrize("sigma", [6.0, 10.0])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_smooth_q_high_scale(sigma, d, causal):
    run_case("smooth-q", 200 + int(sigma) + d, sigma, d, causal, smooth_q=True, q_offset=4.0 * sigma)


@pytest.mark.parametrize("sigma", [3.0, 6.0, 10.0, 20.0, 40.0])
@pytest.mark.parametrize("causal", [False, True])
def test_fp8_pv_high_scale(sigma, causal):
    """sigma >= 6 puts c = q_scale k_scale log2(e) past 2^-9, where the FP8
    path forms the exponent with the seed subtracted first (exactly); sigma 3
    stays on the rounded-bias form."""
    cmax = run_case("fp8", 300 + int(sigma), sigma, 128, causal, pv_mode=1)
    run_case("fp8-smooth-v", 310 + int(sigma), sigma, 128, causal, pv_mode=2)
    if sigma >= 6:
        assert cmax >= 2.0 ** -9


@pytest.mark.parametrize("d", [64, 128])
def test_exact_slow_path_when_c_reaches_one(d):
    """sigma = 300: q_scale * k_scale * log2(e) >= 1 and the fp16 path forms
    the exponent with the seed subtracted first -- still the fp16 bars.  (The
    FP8 path is not held to the oracle here: its scores reach ~4e7 in base-2
    units, where fp32 resolves them only to a few units, and the E4M3 rounding
    of the dominant weight, not cancelled by the unquantised denominator,
    follows the fractional part of the fp64 row maximum.)"""
    cmax = run_case("slow", 400 + d, 300.0, d, False)
    assert cmax >= 1.0
    run_case("slow-causal", 410 + d, 300.0, d, True)
