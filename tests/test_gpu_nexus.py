"""Nexus inner attention on the GPU (iha_nexus_inner) against the oracle's nexus_inner on the
same fp16 inputs, and against the orthogonal-rows closed form.  Bar: max|err| <= 2e-2 * RMS
of the oracle output (fp16 operands and probabilities, fp32 accumulation), as for the bf16
forward."""
import math
import sys

import numpy as np
import pytest
import torch

import oracle
import interleaved_head_layer_amd as iha
from interleaved_head_layer_amd import workloads as wl

pytestmark = pytest.mark.gpu
TOL = 2e-2
DEV = "cuda:0"
CODE = {"none": oracle.MASK_NONE, "causal": oracle.MASK_CAUSAL, "window": oracle.MASK_WINDOW}


def note(msg):
    print(f"[case] {msg}", file=sys.stderr, flush=True)


def check(gpu, ref, what):
    assert np.all(np.isfinite(gpu)), f"{what}: non-finite output"
    rms = float(np.sqrt(np.mean(ref ** 2)))
    err = float(np.max(np.abs(gpu - ref)))
    note(f"{what}: max|err| = {err:.3e}, RMS = {rms:.3e}, ratio = {err / rms:.3e}")
    assert err <= TOL * rms, f"{what}: max|err|/RMS = {err / rms:.3e} > {TOL}"


@pytest.mark.parametrize("B,L,H,d,mask,window,scale", [
    (2, 333, 2, 128, "none", 0, 1.0),       # ragged tiles; diagonal-dominated rows
    (2, 333, 2, 128, "causal", 0, 0.3),     # flatter rows
    (1, 1000, 3, 64, "causal", 0, 0.5),
    (1, 600, 2, 128, "window", 37, 0.3),
    (1, 77, 2, 128, "window", 1, 1.0),      # L not a multiple of 8; every row sees itself only
    (1, 1, 1, 64, "none", 0, 1.0),          # a single position
])
def test_nexus_inner_vs_oracle(B, L, H, d, mask, window, scale):
    note(f"nexus inner B={B} L={L} H={H} d={d} mask={mask} window={window} scale={scale}")
    q, _, _ = wl.make_stacked_qkv(B, L, H, d, seed=L + d, scale=scale)
    got = iha.iha_nexus_inner(torch.from_numpy(q).to(DEV).half(), mask, window)
    torch.cuda.synchronize()
    ref = oracle.nexus_inner(q, CODE[mask], window)
    check(got.cpu().numpy().astype(np.float64), ref, f"nexus d={d} L={L} {mask}")


@pytest.mark.parametrize("mask,window", [("none", 0), ("causal", 0), ("window", 5)])
def test_nexus_inner_orthogonal_rows_closed_form(mask, window):
    """Rows c * e_i: row i's output is c a / (a + v - 1) at channel i and c / (a + v - 1) at
    the other v - 1 visible channels, a = exp(c^2 / sqrt(d))."""
    n, d, c = 64, 128, 3.0
    Q = np.zeros((1, n, 1, d), np.float32)
    Q[0, :, 0, :n] = c * np.eye(n)
    got = iha.iha_nexus_inner(torch.from_numpy(Q).to(DEV).half(), mask, window)
    torch.cuda.synchronize()
    a = math.exp(c * c / math.sqrt(d))
    ref = np.zeros((n, d))
    for i in range(n):
        vis = range(n) if mask == "none" else range(i + 1) if mask == "causal" else range(max(0, i - window + 1), i + 1)
        den = a + len(vis) - 1
        for j in vis:
            ref[i, j] = c * (a if j == i else 1.0) / den
    check(got.cpu().numpy()[0, :, 0].astype(np.float64), ref, f"nexus closed form {mask}")


def test_nexus_inner_rejects_bad_arguments():
    q = torch.zeros((1, 64, 2, 96), dtype=torch.float16, device=DEV)
    with pytest.raises(iha.IHAError):
        iha.iha_nexus_inner(q, "causal")                  # d = 96 not compiled
    q = torch.zeros((1, 64, 2, 128), dtype=torch.float16, device=DEV)
    with pytest.raises(iha.IHAError):
        iha.iha_nexus_inner(q, "window", 0)               # empty allowed sets
