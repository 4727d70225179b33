"""C-ABI checks that need no GPU: the library loads, exports every function
include/sage.h declares, and rejects bad arguments before enqueuing work
(no HIP call is made on these paths)."""
import ctypes
import os
import re

import pytest

from quantized_attention_transformer_amd import sage

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sage.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sage_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("sage_quantize", "sage_attn", "sage_attn_quantized", "sage_quantize_v_fp8", "sage_debug_qk_i32",
              "sage_workspace_bytes", "sage_last_error"):
        assert n in names


def test_library_exports_every_declared_symbol():
    L = sage.lib()
    for n in declared_functions():
        assert hasattr(L, n), n
    assert set(declared_functions()) == set(sage.EXPORTED)


def _prob(**kw):
    d = dict(nseq=1, heads=2, max_seqlen=256, head_dim=64, total_tokens=0, cu_seqlens=None, blk_q=64, blk_k=64)
    d.update(kw)
    return sage.Problem(**d)


def _ws(p, mode=0):
    n = ctypes.c_size_t(0)
    rc = sage.lib().sage_workspace_bytes(ctypes.byref(p), mode, ctypes.byref(n))
    return rc, n.value


def test_workspace_bytes_layout():
    rc, n = _ws(_prob())
    assert rc == 0
    # int8 Q and K (2 x 32 KiB), scales, mean, fp64 K column-sum partials (one per 128
    # tokens: 2 heads x 2 chunks x 64 channels x 8 bytes); 256-byte aligned regions
    assert n == 2 * 32768 + 256 + 256 + 512 + 2048
    rc8, n8 = _ws(_prob(), 1)
    assert rc8 == 0 and n8 == n + 32768 + 512
    # quantize-only workspace: the column-sum partials
    m = ctypes.c_size_t(0)
    assert sage.lib().sage_quantize_workspace_bytes(ctypes.byref(_prob()), ctypes.byref(m)) == 0
    assert m.value == 2048
    # one Q scale per token: 2 heads x 256 scales
    rc1, n1 = _ws(_prob(blk_q=1))
    assert rc1 == 0 and n1 == n - 256 + 2048
    # smoothed V: per chunk of 512 tokens (1 here) and channel an fp64 sum and fp32
    # max and min (2 heads x 64 channels), and the scales followed by the means
    sv = ctypes.c_size_t(0)
    assert sage.lib().sage_quantize_v_fp8_smooth_workspace_bytes(ctypes.byref(_prob()), ctypes.byref(sv)) == 0
    assert sv.value == 1024 + 512 + 512
    rcs, ns = _ws(_prob(), 2)
    assert rcs == 0 and ns == n + 32768 + 2 * 512 + sv.value


@pytest.mark.parametrize("kw,status", [
    (dict(head_dim=80), -2),
    (dict(head_dim=0), -2),
    (dict(blk_q=24), -1),
    (dict(blk_k=1), -1),
    (dict(blk_q=2), -1),
    (dict(kv_heads=3), -1),
    (dict(kv_heads=-1), -1),
    (dict(smooth_q=2), -1),
    (dict(qk_fp4=2), -1),
    (dict(qk_fp4=1, head_dim=64), -2),
    (dict(smooth_q=1, blk_k=16), -2),
    (dict(blk_k=512), -1),
    (dict(blk_k=0), -1),
    (dict(heads=0), -1),
    (dict(nseq=-1), -1),
    (dict(max_seqlen=-5), -1),
])
def test_problem_validation(kw, status):
    rc, _ = _ws(_prob(**kw))
    assert rc == status
    assert sage.lib().sage_last_error().decode() != ""


def test_null_problem_and_bad_mode():
    n = ctypes.c_size_t(0)
    assert sage.lib().sage_workspace_bytes(None, 0, ctypes.byref(n)) == -1
    assert sage.lib().sage_workspace_bytes(ctypes.byref(_prob()), 7, ctypes.byref(n)) == -1
    assert sage.lib().sage_workspace_bytes(ctypes.byref(_prob()), 3, ctypes.byref(n)) == -1


def test_smooth_v_rejects_small_workspace_and_null_output():
    p = _prob()
    need = ctypes.c_size_t(0)
    assert sage.lib().sage_quantize_v_fp8_smooth_workspace_bytes(ctypes.byref(p), ctypes.byref(need)) == 0
    st = _strides()
    r = sage.lib().sage_quantize_v_fp8_smooth(ctypes.byref(p), FAKE, st, FAKE, st, FAKE, FAKE, need.value - 1, None)
    assert r == -3 and "workspace" in sage.lib().sage_last_error().decode()
    r = sage.lib().sage_quantize_v_fp8_smooth(ctypes.byref(p), FAKE, st, FAKE, st, None, FAKE, need.value, None)
    assert r == -1 and "v_scale_mean" in sage.lib().sage_last_error().decode()


def test_gqa_workspace_counts_kv_heads():
    # 4 query heads over 1 K/V head: int8 Q 4 heads, int8 K 1 head, Q scales 4 heads, K
    # scales, mean and column-sum partials 1 head
    p = _prob(heads=4, kv_heads=1)
    rc, n = _ws(p)
    assert rc == 0
    # q8 4x256x64, k8 1x256x64, q scales (16 floats), k scales (4), mean (64 floats) each in a
    # 256-byte region, 2 chunks x 64 fp64 column sums
    assert n == 4 * 16384 + 16384 + 256 + 256 + 256 + 1024


def test_head_dim_96_runs_on_the_128_channel_layout():
    # sage_attn owns its intermediates: at head_dim 96 they take the 128-channel layout
    for mode in (0, 1, 2):
        for kw in (dict(), dict(heads=4, kv_heads=2), dict(blk_q=1)):
            rc96, n96 = _ws(_prob(head_dim=96, **kw), mode)
            rc128, n128 = _ws(_prob(head_dim=128, **kw), mode)
            assert rc96 == 0 and rc128 == 0 and n96 == n128, (mode, kw)
    # entries whose int8/E4M3 outputs the caller lays out take 64 or 128 only
    m = ctypes.c_size_t(0)
    assert sage.lib().sage_quantize_workspace_bytes(ctypes.byref(_prob(head_dim=96)), ctypes.byref(m)) == -2
    assert "96" in sage.lib().sage_last_error().decode()
    assert sage.lib().sage_quantize_v_fp8_smooth_workspace_bytes(ctypes.byref(_prob(head_dim=96)),
                                                                 ctypes.byref(m)) == -2
    st = _strides()
    p = _prob(head_dim=96)
    assert sage.lib().sage_quantize_v_fp8(ctypes.byref(p), FAKE, st, FAKE, st, FAKE, None) == -2


def test_sdpa_wrapper_rejects_what_it_does_not_do():
    import torch
    q = torch.zeros((1, 4, 8, 64), dtype=torch.float16)
    kv = torch.zeros((1, 2, 8, 64), dtype=torch.float16)
    with pytest.raises(NotImplementedError):
        sage.scaled_dot_product_attention(q, q, q, attn_mask=torch.ones(8, 8, dtype=torch.bool))
    with pytest.raises(NotImplementedError):
        sage.scaled_dot_product_attention(q, q, q, dropout_p=0.1)
    with pytest.raises(ValueError):
        sage.scaled_dot_product_attention(q, kv, kv)            # fewer K/V heads without enable_gqa
    with pytest.raises(ValueError):
        sage.scaled_dot_product_attention(q, torch.zeros((1, 3, 8, 64), dtype=torch.float16),
                                          torch.zeros((1, 3, 8, 64), dtype=torch.float16), enable_gqa=True)


def test_debug_fp8_mfma_rejects_bad_scales():
    r = sage.lib().sage_debug_fp8_mfma(FAKE, FAKE, FAKE, 255, 127, FAKE, None)
    assert r == -1 and "E8M0" in sage.lib().sage_last_error().decode()
    r = sage.lib().sage_debug_fp8_mfma(None, FAKE, FAKE, 127, 127, FAKE, None)
    assert r == -1


FAKE = ctypes.c_void_p(0x10000)          # 16-byte aligned, never dereferenced: validation fails first


def _strides(s=256 * 2 * 64, h=64, n=128):
    return sage.Strides(s, h, n)


def test_attn_rejects_small_workspace():
    p = _prob()
    rc, need = _ws(p)
    st = _strides()
    r = sage.lib().sage_attn(ctypes.byref(p), FAKE, st, FAKE, st, FAKE, st, FAKE, st, 0, 0.0, 0, FAKE, need - 1,
                             None)
    assert r == -3
    assert "workspace" in sage.lib().sage_last_error().decode()


def test_attn_rejects_null_and_misaligned():
    p = _prob()
    rc, need = _ws(p)
    st = _strides()
    r = sage.lib().sage_attn(ctypes.byref(p), None, st, FAKE, st, FAKE, st, FAKE, st, 0, 0.0, 0, FAKE, need, None)
    assert r == -1 and "Q is NULL" in sage.lib().sage_last_error().decode()
    r = sage.lib().sage_attn(ctypes.byref(p), ctypes.c_void_p(0x10004), st, FAKE, st, FAKE, st, FAKE, st, 0, 0.0, 0,
                             FAKE, need, None)
    assert r == -1 and "aligned" in sage.lib().sage_last_error().decode()
    bad = _strides(n=100)                 # token stride not a multiple of 8 elements
    r = sage.lib().sage_attn(ctypes.byref(p), FAKE, bad, FAKE, st, FAKE, st, FAKE, st, 0, 0.0, 0, FAKE, need, None)
    assert r == -1 and "strides" in sage.lib().sage_last_error().decode()


def test_empty_problem_is_a_no_op():
    p = _prob(max_seqlen=0)
    st = _strides()
    # nothing to do: OK without touching any pointer or the GPU
    assert sage.lib().sage_attn(ctypes.byref(p), None, st, None, st, None, st, None, st, 1, 0.0, 0, None, 0,
                                None) == 0
    p = _prob(nseq=0)
    assert sage.lib().sage_quantize(ctypes.byref(p), None, st, None, st, 0.0, None, st, None, st, None, None, None,
                                    None, 0, None) == 0


def test_debug_entry_limits():
    p = _prob(max_seqlen=2048)
    st = _strides()
    assert sage.lib().sage_debug_qk_i32(ctypes.byref(p), FAKE, st, FAKE, st, FAKE, None) == -2
    cu = ctypes.c_void_p(0x20000)
    p = _prob(cu_seqlens=cu.value, total_tokens=10)
    assert sage.lib().sage_debug_qk_i32(ctypes.byref(p), FAKE, st, FAKE, st, FAKE, None) == -2


def test_binding_requires_max_seqlen_for_varlen():
    import torch
    q = torch.zeros((10, 2, 64), dtype=torch.float16)
    cu = torch.tensor([0, 10], dtype=torch.int32)
    with pytest.raises(ValueError):
        sage.make_problem(q, cu_seqlens=cu)


def test_smooth_q_workspace_and_entry_rules():
    rc, n = _ws(_prob())
    rcs, ns = _ws(_prob(smooth_q=1))
    # plus Q's column-sum partials (2 heads x 2 chunks x 64 channels x 8 bytes), mean(Q')
    # (2 x 64 floats) and the per-key compensation (2 heads x 256 tokens x 4 bytes)
    assert rc == 0 and rcs == 0 and ns == n + 2048 + 512 + 2048
    m = ctypes.c_size_t(0)
    assert sage.lib().sage_quantize_smooth_q_workspace_bytes(ctypes.byref(_prob(smooth_q=1)), ctypes.byref(m)) == 0
    assert m.value == 2048 + 2048
    st = _strides()
    # sage_quantize and sage_attn_quantized do not take smooth_q; sage_quantize_smooth_q needs it
    p = _prob(smooth_q=1)
    r = sage.lib().sage_quantize(ctypes.byref(p), FAKE, st, FAKE, st, 0.0, FAKE, st, FAKE, st, FAKE, FAKE, FAKE,
                                 FAKE, 1 << 20, None)
    assert r == -2 and "smooth_q" in sage.lib().sage_last_error().decode()
    r = sage.lib().sage_attn_quantized(ctypes.byref(p), FAKE, st, FAKE, st, FAKE, FAKE, FAKE, st, FAKE, FAKE, st,
                                       0, 0, None)
    assert r == -2
    p0 = _prob()
    r = sage.lib().sage_quantize_smooth_q(ctypes.byref(p0), FAKE, st, FAKE, st, 0.0, FAKE, st, FAKE, st, FAKE, FAKE,
                                          FAKE, FAKE, FAKE, FAKE, 1 << 20, None)
    assert r == -1
    r = sage.lib().sage_quantize_smooth_q(ctypes.byref(p), FAKE, st, FAKE, st, 0.0, FAKE, st, FAKE, st, FAKE, FAKE,
                                          FAKE, FAKE, None, FAKE, 1 << 20, None)
    assert r == -1 and "delta" in sage.lib().sage_last_error().decode()
    r = sage.lib().sage_quantize_smooth_q(ctypes.byref(p), FAKE, st, FAKE, st, 0.0, FAKE, st, FAKE, st, FAKE, FAKE,
                                          FAKE, FAKE, FAKE, FAKE, m.value - 1, None)
    assert r == -3


def test_qk_fp4_workspace_and_entry_rules():
    # 4-bit Q and K (head_dim 128): packed codes (d/2 bytes per row) and one E8M0 byte per
    # 32 channels in place of the INT8 rows and block scales
    p = _prob(head_dim=128, qk_fp4=1)
    rc, n = _ws(p)
    assert rc == 0
    # q4 2x256x64, k4 2x256x64, scales 2x256x4 each, k_mean 2x128 floats, K column-sum
    # partials 2 heads x 2 chunks x 128 channels x 8 bytes
    assert n == 32768 + 32768 + 2048 + 2048 + 1024 + 4096
    m = ctypes.c_size_t(0)
    assert sage.lib().sage_quantize_mxfp4_workspace_bytes(ctypes.byref(p), ctypes.byref(m)) == 0
    assert m.value == 4096
    assert sage.lib().sage_quantize_mxfp4_workspace_bytes(ctypes.byref(_prob(head_dim=128, qk_fp4=1, smooth_q=1)),
                                                        ctypes.byref(m)) == 0
    assert m.value == 8192
    st = _strides()
    r = sage.lib().sage_quantize(ctypes.byref(p), FAKE, st, FAKE, st, 0.0, FAKE, st, FAKE, st, FAKE, FAKE, FAKE,
                                 FAKE, 1 << 20, None)
    assert r == -2 and "qk_fp4" in sage.lib().sage_last_error().decode()
    r = sage.lib().sage_attn_quantized(ctypes.byref(p), FAKE, st, FAKE, st, FAKE, FAKE, FAKE, st, FAKE, FAKE, st,
                                       0, 0, None)
    assert r == -2
    # the quantiser itself takes head_dim 64 too; missing scale outputs are refused
    p64 = _prob(qk_fp4=1)
    r = sage.lib().sage_quantize_mxfp4(ctypes.byref(p64), FAKE, st, FAKE, st, 0.0, FAKE, st, None, st, FAKE, st,
                                       FAKE, st, FAKE, None, None, FAKE, 1 << 20, None)
    assert r == -1 and "q_sc" in sage.lib().sage_last_error().decode()
