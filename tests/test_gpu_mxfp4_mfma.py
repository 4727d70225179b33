"""Probe of the 4-bit matrix instruction's MXFP4 form (v_mfma_scale_f32_32x32x64_f8f6f4
with E2M1 operands and per-lane E8M0 scales) through sage_debug_mxfp4_mfma, against
the oracle's E2M1 decoding.  This is the Q.K^T product of the 4-bit variant
("4比特量化三倍加速不掉点！清华即插即用的SageAttention迎来升级", section 技术方案: the
INT4 kernel; gfx950's 4-bit matrix format is OCP MXFP4).  Pinned here: the nibble
order of a lane's operand, which lane's scale applies to which 32 products, and
that the products and their sum come out exact when the sum is representable.
"""
import numpy as np
import pytest

from oracle import sage_oracle as O

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from quantized_attention_transformer_amd import sage
    sage.lib()


def run(a4, b4, sa, sb, c):
    from quantized_attention_transformer_amd import sage
    d = sage.debug_mxfp4_mfma(*(torch.from_numpy(np.ascontiguousarray(x)).cuda() for x in (a4, b4, sa, sb)),
                              torch.from_numpy(c.astype(np.float32)).cuda())
    torch.cuda.synchronize()
    return d.cpu().numpy().astype(np.float64)


def reference(a4, b4, sa, sb, c):
    a = O.e2m1_decode(a4) * np.exp2(np.repeat(sa.astype(np.float64) - 127, 32, axis=1))
    b = O.e2m1_decode(b4) * np.exp2(np.repeat(sb.astype(np.float64) - 127, 32, axis=0))
    return c.astype(np.float64) + a @ b


def test_single_products_land_at_their_row_column_and_k():
    # one nonzero product per k: A[m][k] = 1.5 (code 3) only in row m = k % 32, B[k][n] = 3
    # (code 5) only in column n = (3k) % 32, distinct scales per (row, k-block): a wrong
    # nibble order, lane half or scale lane would move or rescale it
    for k in range(64):
        a4 = np.zeros((32, 64), np.uint8)
        b4 = np.zeros((64, 32), np.uint8)
        m, n = k % 32, (3 * k) % 32
        a4[m, k] = 3
        b4[k, n] = 5
        sa = (120 + np.arange(64).reshape(32, 2) % 9).astype(np.uint8)
        sb = (125 + np.arange(64).reshape(2, 32) % 5).astype(np.uint8)
        c = np.zeros((32, 32))
        d = run(a4, b4, sa, sb, c)
        ref = reference(a4, b4, sa, sb, c)
        assert np.array_equal(d, ref), k
        assert d[m, n] != 0


def test_random_codes_and_scales():
    rng = np.random.default_rng(71)
    for it in range(4):
        a4 = rng.integers(0, 16, size=(32, 64)).astype(np.uint8)
        b4 = rng.integers(0, 16, size=(64, 32)).astype(np.uint8)
        sa = rng.integers(126, 129, size=(32, 2)).astype(np.uint8)
        sb = rng.integers(126, 129, size=(2, 32)).astype(np.uint8)
        c = rng.integers(-64, 64, size=(32, 32)).astype(np.float64) / 4
        d = run(a4, b4, sa, sb, c)
        ref = reference(a4, b4, sa, sb, c)
        # every product is a multiple of 2^-4 (0.5 * 0.5 * 2^-1 * 2^-1) below 6*6*2*2, the
        # whole sum far below 2^24 of that unit, and products span < 2^12: exact in fp32
        assert np.array_equal(d, ref), it


def test_zero_scale_code_and_negative_zero():
    a4 = np.full((32, 64), 0x8, np.uint8)   # -0
    b4 = np.full((64, 32), 7, np.uint8)     # 6
    sa = np.zeros((32, 2), np.uint8)        # 2^-127
    sb = np.full((2, 32), 127, np.uint8)
    c = np.ones((32, 32))
    assert np.array_equal(run(a4, b4, sa, sb, c), c)
