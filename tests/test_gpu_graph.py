"""sage_attn under HIP graph capture.

The library only enqueues kernels on the caller's stream: it allocates
nothing, makes no memset nodes and never synchronises. So a whole forward
call can be captured once and replayed, as serving loops do. Each graph here
(fp16, FP8 and smoothed-V FP8 P.V; causal and not; smooth Q; 4-bit Q.K^T) is
replayed several times, with eager calls of the library and host
synchronisations between the replays. Every replay must give the eager
result bit for bit.
"""
import numpy as np
import pytest

from quantized_attention_transformer_amd import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

CASES = [
    # (name, pv mode, causal, smooth Q, 4-bit Q.K^T)
    ("fp16", 0, False, False, False),
    ("fp16-causal", 0, True, False, False),
    ("fp8", 1, False, False, False),
    ("fp8-smooth-v-causal", 2, True, False, False),
    ("fp16-smooth-q", 0, False, True, False),
    ("fp16-qk-fp4-causal", 0, True, False, True),
]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from quantized_attention_transformer_amd import sage
    sage.lib()


@pytest.mark.parametrize("name,mode,causal,sq,fp4", CASES, ids=[c[0] for c in CASES])
def test_sage_attn_graph_replays_equal_eager(name, mode, causal, sq, fp4):
    from quantized_attention_transformer_amd import sage
    inp = synth.generate(synth.TEXT, seqlen=700, batch=2, heads=4)
    print(f"[{name}] q{inp.q.shape}", flush=True)
    q, k, v = (torch.from_numpy(np.ascontiguousarray(x)).cuda() for x in (inp.q, inp.k, inp.v))
    prob = sage.make_problem(q, "bnhd")
    prob.smooth_q, prob.qk_fp4 = int(sq), int(fp4)
    ws = torch.empty(max(16, sage.workspace_bytes(prob, mode)), dtype=torch.uint8, device="cuda")
    out = torch.empty_like(q)

    def call():
        sage.attn(q, k, v, causal=causal, pv_mode=mode, smooth_q=sq, qk_fp4=fp4, out=out, workspace=ws)

    call()
    torch.cuda.synchronize()
    ref = out.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):  # warm-up on a side stream, as capture requires
        call()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for rep in range(4):
        out.zero_()
        ws.fill_(0xFF)  # the replay must not depend on what the workspace held
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"replay {rep}"
        call()  # eager work between the replays
        torch.cuda.synchronize()
        assert torch.equal(out, ref)
