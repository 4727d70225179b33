"""Sequences longer than the fused kernel's per-tile k_scale table in LDS
(4096 key tiles of 64 keys): past that length a workgroup reads each tile's
k_scale with a scalar load instead.  One dense sequence of 263,144 tokens
(4112 key tiles, ragged last tile), one head, d = 64, against the oracle on
sampled query rows: the first and last 128, the rows around key tile 4096,
and random ones.  Causal rows before token 262,144 still use the table, the
ones after it do not; non-causal rows all read past it.  Tolerance as in the
other parity tests (fp16 P.V: cos >= 0.99995, max |dO| <= 4e-3; FP8 P.V:
cos >= 0.9995)."""
import numpy as np
import pytest

from oracle import sage_oracle as O
from quantized_attention_transformer_amd import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

COS_FP16, MAXABS_FP16, COS_FP8 = 0.99995, 4e-3, 0.9995
N = 4096 * 64 + 1000


@pytest.fixture(scope="module")
def inp():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return synth.generate(synth.VIDEO, seqlen=N, batch=1, heads=1)


def cos(a, b):
    a = np.asarray(a, np.float64).ravel()
    b = np.asarray(b, np.float64).ravel()
    return float(a @ b / (np.linalg.norm(a) * np.linalg.norm(b)))


@pytest.mark.parametrize("causal,fp8", [(False, False), (True, False), (False, True)],
                         ids=["fp16pv", "fp16pv-causal", "fp8pv"])
def test_sequence_past_the_k_scale_table(inp, causal, fp8):
    from quantized_attention_transformer_amd import sage
    rng = np.random.default_rng(5)
    rows = set(range(128)) | set(range(N - 128, N)) | set(range(4096 * 64 - 96, 4096 * 64 + 96))
    rows |= set(rng.integers(0, N, size=48).tolist())
    rows = np.array(sorted(rows))
    wl = inp.wl
    q, k, v = (torch.from_numpy(np.ascontiguousarray(x)).cuda() for x in (inp.q, inp.k, inp.v))
    o = sage.attn(q, k, v, causal=causal, pv_mode=1 if fp8 else 0, blk_q=wl.blk_q, blk_k=wl.blk_k)
    torch.cuda.synchronize()
    o = o.cpu().numpy()[:, rows]
    ref, _ = O.sage_attn(inp.q, inp.k, inp.v, inp.seqlens, None, causal, wl.blk_q, wl.blk_k, pv_fp8=fp8,
                         rows_by_seq={0: rows})
    ref = ref[:, rows]
    c, e = cos(o, ref), float(np.abs(o - ref).max())
    print(f"[N={N} causal={causal} fp8={fp8}] {len(rows)} rows: cos={c:.7f} maxabs={e:.3e}", flush=True)
    assert np.isfinite(o).all()
    if fp8:
        assert c >= COS_FP8
    else:
        assert c >= COS_FP16 and e <= MAXABS_FP16
