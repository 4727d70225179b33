"""Packed-sequence offsets are clamped on the device: whatever cu_seqlens
holds, every sequence's token range lies inside [0, total_tokens) and no
length exceeds max_seqlen (the per-sequence scale rows, workspace and output
are sized from max_seqlen and total_tokens).  The library's own index
helpers (sage_internal.h, compiled for the host here) run on random
malformed offset arrays."""
import os
import shutil
import subprocess

import numpy as np
import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(os.path.dirname(HERE), "quantized_attention_transformer_amd", "csrc")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"


@pytest.fixture(scope="module")
def model(tmp_path_factory):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    exe = str(tmp_path_factory.mktemp("seqclamp") / "seq_clamp_model")
    r = subprocess.run([HIPCC, "-x", "hip", "--offload-arch=gfx950", "-O1", "-I" + CSRC,
                        os.path.join(HERE, "seq_clamp_model.cpp"), "-o", exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return exe


def run_model(exe, cases):
    text = "".join(f"{len(cu) - 1} {ms} {T}\n" + " ".join(str(int(c)) for c in cu) + "\n" for cu, ms, T in cases)
    out = subprocess.run([exe], input=text, capture_output=True, text=True, check=True).stdout.split()
    vals = np.array(out, dtype=np.int64).reshape(-1, 2)
    res, i = [], 0
    for cu, _, _ in cases:
        n = len(cu) - 1
        res.append(vals[i:i + n])
        i += n
    return res


def test_well_formed_offsets_unchanged(model):
    rng = np.random.default_rng(5)
    cases = []
    for _ in range(200):
        lens = rng.integers(0, 300, size=rng.integers(1, 12))
        cu = np.concatenate([[0], np.cumsum(lens)])
        cases.append((cu, int(lens.max()), int(cu[-1])))
    for (cu, _, _), got in zip(cases, run_model(model, cases)):
        assert (got[:, 0] == cu[:-1]).all() and (got[:, 1] == np.diff(cu)).all()


def test_malformed_offsets_stay_in_bounds(model):
    rng = np.random.default_rng(6)
    cases = []
    for _ in range(2000):
        n = int(rng.integers(1, 10))
        T = int(rng.integers(0, 500))
        ms = int(rng.integers(0, 200))
        kind = rng.integers(0, 4)
        if kind == 0:      # anything, including negative and huge offsets
            cu = rng.integers(-2**31, 2**31 - 1, size=n + 1)
        elif kind == 1:    # decreasing
            cu = np.sort(rng.integers(-50, 600, size=n + 1))[::-1]
        elif kind == 2:    # lengths beyond max_seqlen, offsets past total
            cu = np.concatenate([[0], np.cumsum(rng.integers(0, 400, size=n))])
        else:
            cu = rng.integers(-5, T + 5, size=n + 1)
        cases.append((cu, ms, T))
    for (cu, ms, T), got in zip(cases, run_model(model, cases)):
        start, length = got[:, 0], got[:, 1]
        assert (start >= 0).all() and (start <= T).all()
        assert (length >= 0).all() and (length <= ms).all()
        assert (start + length <= T).all()
