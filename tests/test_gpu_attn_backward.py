"""Parity of the attention backward (iha_attention_backward) with the double-precision
gradients of oracle/backward.py, on generator-made fp16 stacked Q, K, V and dO.

Bar: max|err| <= 2e-2 * RMS of the oracle's gradient, per gradient tensor - the bf16
forward's bar.  The HIP path rounds Q * scale, the probabilities, dS and the recomputed
forward output to fp16 (relative 2^-11 each) and accumulates in fp32; that puts its error
near 1e-3 of the RMS, well inside the bar.
"""
import math
import sys

import numpy as np
import pytest
import torch

from interleaved_head_layer_amd import workloads as wl
import interleaved_head_layer_amd as iha
from oracle import backward as bw

pytestmark = pytest.mark.gpu

TOL = 2e-2
DEV = "cuda:0"
CODE = {"none": bw.MASK_NONE, "causal": bw.MASK_CAUSAL, "window": bw.MASK_WINDOW}


def note(msg):
    print(f"[case] {msg}", file=sys.stderr, flush=True)


def check(gpu, ref, what):
    assert np.all(np.isfinite(gpu)), f"{what}: non-finite gradient"
    rms = float(np.sqrt(np.mean(ref ** 2)))
    err = float(np.max(np.abs(gpu - ref)))
    if rms == 0.0:
        # A row whose only visible key is itself has probability 1 and no score gradient:
        # dQ and dK are exactly zero (window 1).  Inputs are O(1), so bound the error absolutely.
        note(f"{what}: exact gradient is zero, max|err| = {err:.3e}")
        assert err <= 1e-3, f"{what}: max|err| = {err:.3e} against an exact zero"
        return
    note(f"{what}: max|err| = {err:.3e}, RMS = {rms:.3e}, ratio = {err / rms:.3e}")
    assert err <= TOL * rms, f"{what}: max|err|/RMS = {err / rms:.3e} > {TOL}"


def gpu_grads(q, k, v, g, mask, window):
    t = lambda a: torch.from_numpy(a).to(DEV).half().contiguous()
    out = iha.iha_attention_backward(t(q), t(k), t(v), t(g), mask, window)
    torch.cuda.synchronize()
    return [o.cpu().numpy().astype(np.float64) for o in out]


CASES = [
    # B, L, H, d, mask, window
    (2, 333, 2, 64, "causal", 0),      # ragged query and key tiles
    (2, 333, 2, 128, "window", 37),
    (1, 200, 3, 128, "none", 0),
    (1, 77, 2, 64, "window", 1),       # every row sees only itself; L not a multiple of 8
    (1, 1, 1, 128, "causal", 0),       # a single row
    (1, 1024, 2, 128, "window", 256),  # several key and query tiles per workgroup
    (1, 600, 2, 128, "window", 100000),  # window beyond the sequence = causal
    (2, 256, 2, 64, "none", 0),
    # the d = 128 causal kernels over several tiles: two-deep prefetch, longest-first causal
    # tile order, skipped tiles, ragged tails
    (2, 333, 2, 128, "causal", 0),
    (1, 1000, 2, 128, "causal", 0),
    (1, 1000, 2, 64, "causal", 0),
    (1, 700, 2, 128, "none", 0),       # no mask, 11 key tiles through the prefetch path
]


@pytest.mark.parametrize("B,L,H,d,mask,window", CASES)
def test_attention_backward_vs_oracle(B, L, H, d, mask, window):
    note(f"attention backward B={B} L={L} H={H} d={d} mask={mask} window={window}")
    q, k, v = wl.make_stacked_qkv(B, L, H, d, seed=L + d, scale=1.0)
    g = wl.make_stacked_grad(B, L, H, d, seed=L + d)
    dQ, dK, dV = gpu_grads(q, k, v, g, mask, window)
    ref = bw.attention_grads(q, k, v, g, CODE[mask], min(window, L) if mask == "window" else 0)
    for name, got in (("dQ", dQ), ("dK", dK), ("dV", dV)):
        check(got, ref[name], f"{name} L={L} d={d} {mask}")


def test_attention_backward_bench_scale_window_sampled():
    """The per-head shape of the 4 x 4096-token, P = 2 window workload (L = 8192 stacked rows,
    16 heads, d = 128, window 1024).  A window mask depends only on q - k, so the rows
    [k - W + 1, k + W) hold every query that sees key k and every key those queries see: the
    oracle on that crop gives the exact dK[k], dV[k] and dQ of queries k .. k + W - 1."""
    B, L, H, d, W = 4, 8192, 16, 128, 1024
    note(f"attention backward sampled B={B} L={L} H={H} d={d} window={W}")
    q, k, v = wl.make_stacked_qkv(B, L, H, d, seed=2024, scale=1.0)
    g = wl.make_stacked_grad(B, L, H, d, seed=2024)
    dQ, dK, dV = gpu_grads(q, k, v, g, "window", W)
    rng = np.random.default_rng(11)
    samples = [(0, 0, 0), (3, 15, L - 1), (1, 7, 5000)] + [
        (int(rng.integers(B)), int(rng.integers(H)), int(rng.integers(L))) for _ in range(3)]
    for b, h, key in samples:
        lo, hi = max(0, key - W + 1), min(L, key + W)
        crop = lambda a: a[b:b + 1, lo:hi, h:h + 1]
        ref = bw.attention_grads(crop(q), crop(k), crop(v), crop(g), bw.MASK_WINDOW, W)
        r = key - lo
        check(dK[b, key, h], ref["dK"][0, r, 0], f"dK b={b} h={h} key={key}")
        check(dV[b, key, h], ref["dV"][0, r, 0], f"dV b={b} h={h} key={key}")
        check(dQ[b, key:hi, h], ref["dQ"][0, r:, 0], f"dQ b={b} h={h} rows {key}..{hi - 1}")


def test_attention_backward_rejects_bad_arguments():
    q = torch.zeros((1, 64, 2, 128), dtype=torch.float16, device=DEV)
    with pytest.raises(iha.IHAError):
        iha.iha_attention_backward(q, q, q, q, "window", 0)   # empty allowed sets
    q2 = torch.zeros((1, 64, 2, 96), dtype=torch.float16, device=DEV)
    with pytest.raises(iha.IHAError):
        iha.iha_attention_backward(q2, q2, q2, q2, "causal")  # d = 96 not compiled
