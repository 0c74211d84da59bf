"""Closed forms of the IHA page's strictness construction pushed through the GPU path (no oracle).

"Interleaved Head Attention" page, section 4.1 (the strictness construction behind Theorem 5):
with every token equal (X = 1 x^T), P = 2 and the second pseudo query and key negated
(alpha^Q = alpha^K = identity mixing with coefficients [1, -1]), a pseudo query of head h
scores s_h = q_h . k_h / sqrt(d) against every first pseudo key and -s_h against every second
one.  With V-bar = [V; V] every output row is exactly v_h; with V-bar = [V; -V] it is
tanh(s_h) v_h without a mask, and (n0 e^s - n1 e^-s) / (n0 e^s + n1 e^-s) v_h under a mask on
the interleaved position i = t*P + j, where n0 and n1 count the visible first and second
pseudo keys (textbook "Attention mechanism", section 5.3, eq. 5.11: softmax over the allowed
set).  R = [I 0] keeps the first pseudo block of each head.

The expected values are computed here in float64 from the bf16 inputs; the GPU keeps fp16
intermediates, so the bar is the bf16 path's 2e-2 of the RMS.  Lengths of 150-300 tokens span
several 128-row query tiles and 64-key tiles and the fp32 first rows; (D, H) = (1024, 16)
takes the mixing fused into the projection GEMM, (256, 2) the separate mixing kernels.
"""
import math
import sys

import numpy as np
import pytest
import torch

from interleaved_head_layer_amd import workloads as wl
import interleaved_head_layer_amd as iha

pytestmark = pytest.mark.gpu
TOL = 2e-2
DEV = "cuda:0"


def note(msg):
    print(f"[case] {msg}", file=sys.stderr, flush=True)


def eye_mix(H, P, coef):
    """alpha[m][h][j] = coef[j] if m == h else 0."""
    a = np.zeros((H, H, P), np.float32)
    for h in range(H):
        a[h, h, :] = coef
    return a


def first_block_R(H, P):
    """R[h][h*P + 0] = 1: output head h is pseudo block 0 of head h."""
    R = np.zeros((H, H * P), np.float32)
    for h in range(H):
        R[h, h * P] = 1.0
    return R


def setup(N, D, H, seed):
    rng = np.random.default_rng(seed)
    x = wl.round_to_bf16(rng.standard_normal(D).astype(np.float32))
    W = [wl.round_to_bf16((rng.standard_normal((D, D)) / math.sqrt(D)).astype(np.float32)) for _ in range(3)]
    d = D // H
    q, k, v = [(x.astype(np.float64) @ Wi.astype(np.float64)).reshape(H, d) for Wi in W]
    s = (q * k).sum(1) / math.sqrt(d)
    X = np.broadcast_to(x, (1, N, D)).copy()
    return X, W, s, v


def run(X, W, aQK, aV, R, H, P, mask, window):
    bf = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV).bfloat16()
    f32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV)
    out = iha.iha_forward(bf(X), bf(W[0]), bf(W[1]), bf(W[2]), f32(aQK), f32(aQK), f32(aV), f32(R), H, P, mask,
                          window)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64)[0]


def check(gpu, ref, what):
    assert np.all(np.isfinite(gpu)), what
    rms = float(np.sqrt(np.mean(ref ** 2)))
    err = float(np.max(np.abs(gpu - ref)))
    note(f"{what}: max|err| = {err:.3e}, RMS = {rms:.3e}, ratio = {err / rms:.3e}")
    assert err <= TOL * rms, f"{what}: {err / rms:.3e}"


@pytest.mark.parametrize("D,H", [(256, 2), (1024, 16)])
@pytest.mark.parametrize("vsign", [1.0, -1.0])
def test_strictness_no_mask(D, H, vsign):
    N, P = 150, 2
    X, W, s, v = setup(N, D, H, seed=71 + D)
    out = run(X, W, eye_mix(H, P, [1.0, -1.0]), eye_mix(H, P, [1.0, vsign]), first_block_R(H, P), H, P,
              "none", None)
    f = np.ones(H) if vsign > 0 else np.tanh(s)
    ref = np.broadcast_to((f[:, None] * v).reshape(-1), out.shape)
    check(out, ref, f"strictness D={D} H={H} V-bar=[V; {'+' if vsign > 0 else '-'}V], no mask")


@pytest.mark.parametrize("D,H", [(256, 2), (1024, 16)])
@pytest.mark.parametrize("mask,window", [("causal", None), ("window", 1), ("window", 4), ("window", 37)])
def test_strictness_interleaved_mask_counts(D, H, mask, window):
    N, P = 300, 2
    X, W, s, v = setup(N, D, H, seed=91 + D)
    out = run(X, W, eye_mix(H, P, [1.0, -1.0]), eye_mix(H, P, [1.0, -1.0]), first_block_R(H, P), H, P, mask,
              window)
    ref = np.zeros_like(out)
    for t in range(N):
        i = 2 * t  # pseudo query (t, 0)
        if mask == "causal":
            n0, n1 = t + 1, t
        else:
            n0 = sum(1 for u in range(N) if i - window < 2 * u <= i)
            n1 = sum(1 for u in range(N) if i - window < 2 * u + 1 <= i)
        f = (n0 * np.exp(s) - n1 * np.exp(-s)) / (n0 * np.exp(s) + n1 * np.exp(-s))
        ref[t] = (f[:, None] * v).reshape(-1)
    check(out, ref, f"strictness D={D} H={H} {mask} window={window} (counts on t*P + j)")
