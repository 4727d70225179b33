"""sage_attn_noalloc (the entry point for callers that cannot allocate device
memory) against sage_attn with a caller workspace, through the C ABI: the
same kernels on the library's fixed scratch array, so the outputs are
bit-identical.  Two calls in a row, the second on a smaller problem (the
array keeps the first call's contents), across the P.V modes, causal and
packed inputs, smooth Q and 4-bit Q.K^T; a problem above the array's size is
refused with SAGE_ERR_WORKSPACE and leaves the output untouched."""
import ctypes

import numpy as np
import pytest

from quantized_attention_transformer_amd import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from quantized_attention_transformer_amd import sage
    sage.lib()


def S():
    from quantized_attention_transformer_amd import sage
    return sage


def tensors(inp):
    dev = lambda x: torch.from_numpy(np.ascontiguousarray(x)).cuda()  # noqa: E731
    kw = {} if inp.cu_seqlens is None else dict(cu_seqlens=dev(inp.cu_seqlens), max_seqlen=inp.max_seqlen)
    return dev(inp.q), dev(inp.k), dev(inp.v), kw


CASES = [
    ("text fp16", synth.TEXT, dict(seqlen=2048, heads=4), dict(pv_mode=0)),
    ("text causal FP8", synth.TEXT, dict(seqlen=1500, heads=2), dict(pv_mode=1, causal=True)),
    ("tiny d64 smooth-V", synth.TINY, dict(seqlen=700, heads=3), dict(pv_mode=2)),
    ("varlen causal", synth.VARLEN, dict(seqlens=[300, 0, 1, 1025, 64], heads=4), dict(pv_mode=0, causal=True)),
    ("smooth Q", synth.TEXT, dict(seqlen=900, heads=2), dict(pv_mode=0, smooth_q=True)),
    ("4-bit QK", synth.TEXT, dict(seqlen=640, heads=2), dict(pv_mode=1, qk_fp4=True)),
]


@pytest.mark.parametrize("big,small", [(0, 1), (1, 2), (2, 3), (3, 4), (4, 5), (5, 0)])
def test_noalloc_equals_sage_attn_two_calls(big, small):
    sage = S()
    for i in (big, small):
        tag, wl, shape, kw = CASES[i]
        inp = synth.generate(wl, **shape)
        q, k, v, vk = tensors(inp)
        ref = sage.attn(q, k, v, blk_q=wl.blk_q, blk_k=wl.blk_k, **vk, **kw)
        out = torch.full_like(q, float("nan"))
        sage.attn_noalloc(q, k, v, out, blk_q=wl.blk_q, blk_k=wl.blk_k, **vk, **kw)
        torch.cuda.synchronize()
        a, b = out.cpu().numpy(), ref.cpu().numpy()
        if inp.cu_seqlens is not None:       # rows of the packed layout only (all tokens are in some sequence)
            a, b = a[:inp.cu_seqlens[-1]], b[:inp.cu_seqlens[-1]]
        print(f"[{tag}] equal={np.array_equal(a, b, equal_nan=False)}", flush=True)
        assert np.isfinite(a).all()
        assert np.array_equal(a, b), tag


def test_noalloc_refuses_problems_above_the_scratch_size():
    sage = S()
    # B1 H16 N16384 d128: q8 + k8 alone are 64 MiB, beyond the 64 MiB array with the scales
    q = torch.zeros((1, 16384, 16, 128), dtype=torch.float16, device="cuda")
    prob = sage.make_problem(q)
    assert sage.workspace_bytes(prob) > sage.NOALLOC_SCRATCH_BYTES
    out = torch.full_like(q, 7.0)
    with pytest.raises(sage.SageError) as e:
        sage.attn_noalloc(q, q, q, out)
    assert e.value.status == -3 and "scratch" in str(e.value)
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())
