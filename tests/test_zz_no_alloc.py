"""iha_forward_static (the entry point that allocates nothing: its workspace is the library's
static per-device buffer) against iha_forward (caller workspace) on the same inputs: two calls
in a row, the second on a smaller problem, each equal bit for bit (same kernels, same
workspace layout); then the size limit and the check flag."""
import sys

import numpy as np
import pytest
import torch

import interleaved_head_layer_amd as iha
from interleaved_head_layer_amd import workloads as wl

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def note(msg):
    print(f"[case] {msg}", file=sys.stderr, flush=True)


def dev_inputs(w):
    x = wl.make_inputs(w)
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    t = lambda a, d=dt: torch.from_numpy(a).to(DEV).to(d).contiguous()
    return (t(x["X"]), t(x["WQ"]), t(x["WK"]), t(x["WV"]), t(x["aQ"], torch.float32),
            t(x["aK"], torch.float32), t(x["aV"], torch.float32), t(x["R"], torch.float32))


def test_static_workspace_matches_caller_workspace_twice():
    cases = [wl.custom(2, 640, 1024, 16, 2, "window", seed=31),   # fused path, 2 x 640 tokens
             wl.custom(1, 200, 256, 2, 3, "causal", seed=32)]     # smaller, unfused path, P = 3
    for w in cases:
        prob = iha.make_problem(w.B, w.N, w.D, w.H, w.P, w.mask, w.window)
        assert iha.iha_workspace_bytes(prob) <= iha.STATIC_WORKSPACE_BYTES
        note(f"static workspace: {w.describe()}")
        args = dev_inputs(w)
        ref = iha.iha_forward(*args, w.H, w.P, w.mask, w.window)
        out = torch.full((w.B, w.N, w.D), float("nan"), dtype=torch.float32, device=DEV)
        iha.iha_forward_static(*args, w.H, w.P, w.mask, out, window=w.window)
        torch.cuda.synchronize()
        a, b = ref.cpu().numpy(), out.cpu().numpy()
        assert np.all(np.isfinite(b))
        assert np.array_equal(a, b), f"max |diff| = {np.abs(a - b).max():.3e}"


def test_static_workspace_limit_and_check_flag():
    big = wl.custom(4, 4096, 2048, 16, 2, "window", seed=33)
    prob = iha.make_problem(big.B, big.N, big.D, big.H, big.P, big.mask, big.window)
    assert iha.iha_workspace_bytes(prob) > iha.STATIC_WORKSPACE_BYTES
    X = torch.zeros((big.B, big.N, big.D), dtype=torch.bfloat16, device=DEV)
    W = torch.zeros((big.D, big.D), dtype=torch.bfloat16, device=DEV)
    a = torch.zeros((big.H, big.H, big.P), dtype=torch.float32, device=DEV)
    R = torch.zeros((big.H, big.H * big.P), dtype=torch.float32, device=DEV)
    out = torch.zeros((big.B, big.N, big.D), dtype=torch.float32, device=DEV)
    note("static workspace: problem beyond the limit")
    with pytest.raises(iha.IHAError) as e:
        iha.iha_forward_static(X, W, W, W, a, a, a, R, big.H, big.P, "window", out)
    assert "WORKSPACE" in str(e.value)
    del X, out
    w = wl.custom(1, 64, 256, 2, 2, "causal", seed=34)
    args = list(dev_inputs(w))
    args[0] = args[0].clone()
    args[0][0, 5, 7] = float("nan")
    out = torch.empty((w.B, w.N, w.D), dtype=torch.float32, device=DEV)
    note("static workspace: NaN input with IHA_FLAG_CHECK")
    with pytest.raises(iha.IHAError) as e:
        iha.iha_forward_static(*args, w.H, w.P, w.mask, out, flags=iha.IHA_FLAG_CHECK)
    assert "NONFINITE" in str(e.value)
    args = dev_inputs(w)
    iha.iha_forward_static(*args, w.H, w.P, w.mask, out, flags=iha.IHA_FLAG_CHECK)
