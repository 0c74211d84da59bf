"""Parity of the layer backward (iha_backward: dX, dW_Q/K/V, dalpha_Q/K/V, dR) with the
double-precision reverse mode of oracle/backward.py, on seeded bf16 inputs.

Bar: max|err| <= 2e-2 * RMS of the oracle's gradient, per gradient tensor (the bf16
forward's bar).  The HIP path rounds the stacked Q~, K~, V~, dP-bar, the probabilities and
dS to fp16 (relative 2^-11) and dY to bf16 (2^-9) and accumulates in fp32: its error is a
few 1e-3 of the RMS.
"""
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
NAMES = ["X", "WQ", "WK", "WV", "aQ", "aK", "aV", "R"]


def note(msg):
    print(f"[case] {msg}", file=sys.stderr, flush=True)


def check(gpu, ref, what):
    assert np.all(np.isfinite(gpu)), f"{what}: non-finite gradient"
    rms = float(np.sqrt(np.mean(ref ** 2)))
    err = float(np.max(np.abs(gpu - ref)))
    if rms < 1e-12:
        # Every row sees only itself (window 1): the scores carry no gradient and dQ-bar,
        # dK-bar - hence dalpha_Q, dalpha_K, dW_Q, dW_K - are exactly zero.
        note(f"{what}: exact gradient is zero, max|err| = {err:.3e}")
        assert err <= 1e-3, f"{what}: max|err| = {err:.3e} against an exact zero"
        return
    note(f"{what}: max|err| = {err:.3e}, RMS = {rms:.3e}, ratio = {err / rms:.3e}")
    assert err <= TOL * rms, f"{what}: max|err|/RMS = {err / rms:.3e} > {TOL}"


def run_gpu(x, G, H, P, mask, window, flags=0):
    bf = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV).bfloat16()
    f32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV)
    out = iha.iha_backward(bf(x["X"]), bf(x["WQ"]), bf(x["WK"]), bf(x["WV"]), f32(x["aQ"]), f32(x["aK"]),
                           f32(x["aV"]), f32(x["R"]), f32(G), H, P, mask, window, flags=flags)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy().astype(np.float64) for k, v in out.items()}


CASES = [
    # B, N, D, H, P, mask, window (None: N // (2P))
    (1, 96, 128, 2, 2, "causal", None),     # B*N not a multiple of 64 (padded GEMM K)
    (2, 160, 256, 2, 3, "window", None),    # d = 128, P = 3
    (1, 64, 256, 4, 1, "none", None),       # P = 1: plain multi-head attention
    (1, 200, 1280, 10, 2, "causal", None),  # H*P = 20 (two reduction tiles); D not a multiple of 256
    (2, 128, 1024, 16, 4, "window", None),  # H*P = 64
    (1, 40, 2560, 20, 4, "causal", None),   # the wide layer's heads (20 x 128, P = 4)
    (1, 24, 2176, 34, 1, "causal", None),   # H > 32
    (1, 50, 128, 2, 2, "window", 1),        # every stacked row sees only itself
    (1, 1, 128, 2, 2, "causal", None),      # one token
]


@pytest.mark.parametrize("B,N,D,H,P,mask,window", CASES)
def test_layer_backward_matches_oracle(B, N, D, H, P, mask, window, progress):
    w = wl.custom(B, N, D, H, P, mask, seed=31 + N + D + P, window=window)
    progress(f"layer backward {w.describe()} window={w.window}")
    x = wl.make_inputs(w)
    G = wl.make_output_grad(w)
    ref = bw.forward_and_grads(x["X"], x["WQ"], x["WK"], x["WV"], x["aQ"], x["aK"], x["aV"], x["R"],
                               H, P, w.mask, w.window, G)
    got = run_gpu(x, G, H, P, mask, w.window)
    for k in NAMES:
        check(got[k], ref[k], k)


def test_layer_backward_repeatable(progress):
    """Two calls on the same inputs give identical bits (no atomics in the reductions)."""
    w = wl.custom(1, 128, 512, 8, 2, "causal", seed=5)
    progress(f"layer backward repeatability {w.describe()}")
    x = wl.make_inputs(w)
    G = wl.make_output_grad(w)
    a = run_gpu(x, G, 8, 2, "causal", w.window)
    b = run_gpu(x, G, 8, 2, "causal", w.window)
    for k in NAMES:
        assert np.array_equal(a[k], b[k]), k


def test_layer_backward_check_flag(progress):
    """IHA_FLAG_CHECK: clean inputs pass; a non-finite G and stacked values beyond the fp16
    range are reported."""
    w = wl.custom(1, 64, 256, 4, 2, "causal", seed=9)
    progress(f"layer backward check flag {w.describe()}")
    x = wl.make_inputs(w)
    G = wl.make_output_grad(w)
    run_gpu(x, G, 4, 2, "causal", w.window, flags=iha.IHA_FLAG_CHECK)
    Gbad = G.copy()
    Gbad[0, 3, 5] = np.nan
    with pytest.raises(iha.IHAError) as e:
        run_gpu(x, Gbad, 4, 2, "causal", w.window, flags=iha.IHA_FLAG_CHECK)
    assert e.value.status == 4  # IHA_ERR_NONFINITE
    xbig = dict(x)
    xbig["X"] = wl.round_to_bf16(x["X"] * np.float32(1e6))
    with pytest.raises(iha.IHAError) as e:
        run_gpu(xbig, G, 4, 2, "causal", w.window, flags=iha.IHA_FLAG_CHECK)
    assert e.value.status == 8  # IHA_ERR_RANGE


def test_layer_backward_rejects_f32(progress):
    progress("layer backward rejects fp32 inputs")
    prob = iha.make_problem(1, 64, 128, 2, 2, "causal", dtype=iha.IHA_F32)
    with pytest.raises(iha.IHAError) as e:
        iha.iha_backward_workspace_bytes(prob)
    assert e.value.status == 6  # IHA_ERR_UNSUPPORTED


# ------------------------------------------------------------------ full size
# At the full sizes the oracle cannot form whole-layer gradients (dR, dalpha and dW sum over
# every token; in causal mode every gradient depends on the whole sequence).  Two checks hold
# there instead:
#  * exact identities of the layer's structure, for L = sum(G * X~) with X~ from iha_forward:
#    X~ is linear in R, in alpha_V and in W_V, so <dR, R> = <dalpha_V, alpha_V> =
#    <dW_V, W_V> = L; the scores are unchanged by alpha_Q * c, alpha_K / c (and by W_Q * c,
#    W_K / c), and Q~ is linear in both W_Q and alpha_Q, so <dalpha_Q, alpha_Q> =
#    <dalpha_K, alpha_K> = <dW_Q, W_Q> = <dW_K, W_K>; every projection is linear in X, so
#    <dX, X> = sum over Q, K, V of <dW, W>.  A transposed, dropped or mis-scaled gradient
#    breaks one of them by order one.  Bar: 1e-3 of the sum of the terms' magnitudes.
#  * under the window mask a token's dX depends only on the tokens within one window on either
#    side (its stacked rows see keys back to W_s - 1 positions; the queries that see them lie
#    within W_s - 1 positions after, and their own keys start no earlier): the oracle's
#    backward on that sub-sequence gives those tokens' dX exactly.
FULL = ["iha_window_p2_b4_n4096", "iha_window_p4_b2_n8192_wide", "iha_causal_p4_b2_n8192_wide"]
ID_TOL = 1e-3


def _upload(x, G):
    bf = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV).bfloat16()
    f32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV)
    t = {k: bf(x[k]) for k in ("X", "WQ", "WK", "WV")}
    t.update({k: f32(x[k]) for k in ("aQ", "aK", "aV", "R")})
    t["G"] = f32(G)
    return t


@pytest.mark.parametrize("name", FULL)
def test_layer_backward_full_size_identities(name, progress):
    w = wl.WORKLOADS[name]
    progress(f"layer backward identities {w.describe()}")
    x = wl.make_inputs(w)
    G = wl.make_output_grad(w)
    t = _upload(x, G)
    args = [t[k] for k in ("X", "WQ", "WK", "WV", "aQ", "aK", "aV", "R")]
    out = iha.iha_forward(*args, w.H, w.P, ["none", "causal", "window"][w.mask], w.window)
    g = iha.iha_backward(*args, t["G"], w.H, w.P, ["none", "causal", "window"][w.mask], w.window)
    torch.cuda.synchronize()
    dot = lambda a, b: float((a.double() * b.double()).sum())
    mag = lambda a, b: float((a.double() * b.double()).abs().sum())
    L, Lmag = dot(t["G"], out), mag(t["G"], out)
    pairs = {"R": (g["R"], t["R"]), "aV": (g["aV"], t["aV"]), "WV": (g["WV"], t["WV"]),
             "aQ": (g["aQ"], t["aQ"]), "aK": (g["aK"], t["aK"]), "WQ": (g["WQ"], t["WQ"]),
             "WK": (g["WK"], t["WK"]), "X": (g["X"], t["X"])}
    v = {k: dot(a, b) for k, (a, b) in pairs.items()}
    m = {k: mag(a, b) for k, (a, b) in pairs.items()}
    v["L"], m["L"] = L, Lmag
    v["W"] = v["WQ"] + v["WK"] + v["WV"]
    m["W"] = m["WQ"] + m["WK"] + m["WV"]
    progress(" ".join(f"{k}={v[k]:.6g}" for k in v))
    for a, b in [("R", "L"), ("aV", "L"), ("WV", "L"), ("aQ", "aK"), ("WQ", "aQ"), ("WK", "aK"),
                 ("X", "W")]:
        scale = m[a] + m[b]
        rel = abs(v[a] - v[b]) / scale
        note(f"{name}: <d{a},{a}> = {v[a]:.6g} vs {b} = {v[b]:.6g}: |diff| / scale = {rel:.3e}")
        assert rel <= ID_TOL, (a, b, rel)


@pytest.mark.parametrize("name", ["iha_window_p2_b4_n4096", "iha_window_p4_b2_n8192_wide"])
def test_layer_backward_full_size_window_tokens(name, progress):
    w = wl.WORKLOADS[name]
    assert w.mask == wl.MASK_WINDOW
    x = wl.make_inputs(w)
    G = wl.make_output_grad(w)
    t = _upload(x, G)
    args = [t[k] for k in ("X", "WQ", "WK", "WV", "aQ", "aK", "aV", "R")]
    g = iha.iha_backward(*args, t["G"], w.H, w.P, "window", w.window)
    torch.cuda.synchronize()
    dX = g["X"].cpu().numpy().astype(np.float64)
    del g, t
    torch.cuda.empty_cache()
    margin = -(-w.window // w.P)   # whole tokens covering W_s stacked positions
    b = w.B - 1
    for t0 in (w.N // 2, margin + 3):
        t1 = t0 + 4
        s, e = t0 - margin, min(w.N, t1 + margin)
        assert s >= 0
        progress(f"{name}: oracle backward on tokens {s}..{e - 1} of sequence {b} for dX of {t0}..{t1 - 1}")
        ref = bw.forward_and_grads(x["X"][b:b + 1, s:e], x["WQ"], x["WK"], x["WV"], x["aQ"], x["aK"],
                                   x["aV"], x["R"], w.H, w.P, w.mask, w.window, G[b:b + 1, s:e])["X"]
        check(dX[b, t0:t1], ref[0, t0 - s:t1 - s], f"{name} dX tokens {t0}..{t1 - 1}")
