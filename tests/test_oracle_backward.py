"""Pins of the double-precision backward reference (oracle/backward.py), CPU only.

The analytic gradients of L = sum(G * X~) are checked element by element against central
finite differences of L (step 1e-6 in float64: truncation ~1e-12, rounding ~1e-10), for every
input tensor, under every mask mode and several P; a dropped term, a wrong sign or a
transposed index in any adjoint fails these.  The forward part is checked against the C++
oracle's forward.
"""
import numpy as np
import pytest

import oracle
from oracle import backward as bw

CASES = [
    # B, N, D, H, P, mask, window
    (1, 5, 8, 2, 2, bw.MASK_NONE, 0),
    (2, 4, 6, 3, 1, bw.MASK_CAUSAL, 0),
    (1, 6, 8, 2, 3, bw.MASK_CAUSAL, 0),
    (1, 7, 8, 2, 2, bw.MASK_WINDOW, 3),
    (2, 5, 12, 3, 2, bw.MASK_WINDOW, 4),
]


def _inputs(B, N, D, H, P, seed):
    rng = np.random.default_rng(seed)
    x = dict(X=rng.standard_normal((B, N, D)),
             WQ=rng.standard_normal((D, D)) / np.sqrt(D), WK=rng.standard_normal((D, D)) / np.sqrt(D),
             WV=rng.standard_normal((D, D)) / np.sqrt(D),
             aQ=rng.standard_normal((H, H, P)) / np.sqrt(H), aK=rng.standard_normal((H, H, P)) / np.sqrt(H),
             aV=rng.standard_normal((H, H, P)) / np.sqrt(H),
             R=rng.standard_normal((H, H * P)) / np.sqrt(H * P))
    G = rng.standard_normal((B, N, D))
    return x, G


def _loss(x, G, H, P, mask, window):
    out = bw.forward_and_grads(x["X"], x["WQ"], x["WK"], x["WV"], x["aQ"], x["aK"], x["aV"], x["R"],
                               H, P, mask, window, G)["out"]
    return float((G * out).sum())


@pytest.mark.parametrize("B,N,D,H,P,mask,window", CASES)
def test_forward_part_matches_the_oracle(B, N, D, H, P, mask, window):
    x, G = _inputs(B, N, D, H, P, seed=1)
    g = bw.forward_and_grads(x["X"], x["WQ"], x["WK"], x["WV"], x["aQ"], x["aK"], x["aV"], x["R"],
                             H, P, mask, window, G)
    ref = oracle.forward(x["X"], x["WQ"], x["WK"], x["WV"], x["aQ"], x["aK"], x["aV"], x["R"],
                         H, P, mask, window)
    np.testing.assert_allclose(g["out"], ref, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("B,N,D,H,P,mask,window", CASES)
def test_gradients_match_finite_differences(B, N, D, H, P, mask, window):
    x, G = _inputs(B, N, D, H, P, seed=2)
    g = bw.forward_and_grads(x["X"], x["WQ"], x["WK"], x["WV"], x["aQ"], x["aK"], x["aV"], x["R"],
                             H, P, mask, window, G)
    rng = np.random.default_rng(3)
    eps = 1e-6
    for name in ["X", "WQ", "WK", "WV", "aQ", "aK", "aV", "R"]:
        for _ in range(6):
            idx = tuple(int(rng.integers(s)) for s in x[name].shape)
            xp = {k: v.copy() for k, v in x.items()}
            xm = {k: v.copy() for k, v in x.items()}
            xp[name][idx] += eps
            xm[name][idx] -= eps
            fd = (_loss(xp, G, H, P, mask, window) - _loss(xm, G, H, P, mask, window)) / (2 * eps)
            an = g[name][idx]
            assert abs(fd - an) <= 1e-7 * max(1.0, abs(fd)), (name, idx, fd, an)


def test_empty_allowed_set_is_an_error():
    x, G = _inputs(1, 4, 4, 2, 2, seed=4)
    with pytest.raises(ValueError):
        bw.forward_and_grads(x["X"], x["WQ"], x["WK"], x["WV"], x["aQ"], x["aK"], x["aV"], x["R"],
                             2, 2, bw.MASK_WINDOW, 0, G)


# ---------------------------------------------------------------- stacked attention alone
ATT_CASES = [
    # B, L, H, d, mask, window
    (1, 6, 2, 4, bw.MASK_NONE, 0),
    (2, 7, 1, 8, bw.MASK_CAUSAL, 0),
    (1, 9, 2, 4, bw.MASK_WINDOW, 3),
    (1, 5, 1, 6, bw.MASK_WINDOW, 1),
]


def _att_inputs(B, L, H, d, seed):
    rng = np.random.default_rng(seed)
    return [rng.standard_normal((B, L, H, d)) for _ in range(4)]


@pytest.mark.parametrize("B,L,H,d,mask,window", ATT_CASES)
def test_attention_gradients_match_finite_differences(B, L, H, d, mask, window):
    Q, K, V, G = _att_inputs(B, L, H, d, seed=5)
    g = bw.attention_grads(Q, K, V, G, mask, window)
    loss = lambda q, k, v: float((G * bw.attention_grads(q, k, v, G, mask, window)["O"]).sum())
    rng = np.random.default_rng(6)
    eps = 1e-6
    for which, name in enumerate(["dQ", "dK", "dV"]):
        for _ in range(8):
            idx = tuple(int(rng.integers(s)) for s in Q.shape)
            xs_p = [Q.copy(), K.copy(), V.copy()]
            xs_m = [Q.copy(), K.copy(), V.copy()]
            xs_p[which][idx] += eps
            xs_m[which][idx] -= eps
            fd = (loss(*xs_p) - loss(*xs_m)) / (2 * eps)
            assert abs(fd - g[name][idx]) <= 1e-7 * max(1.0, abs(fd)), (name, idx, fd, g[name][idx])


@pytest.mark.parametrize("mask,window", [(bw.MASK_NONE, 0), (bw.MASK_CAUSAL, 0), (bw.MASK_WINDOW, 4)])
def test_attention_output_is_the_oracle_mha_at_one_pseudo_head(mask, window):
    # P = 1 with identity mixing and collapse: the IHA forward is per-head attention of
    # X W_Q, X W_K, X W_V over the tokens, which attention_grads computes from the projections.
    B, N, D, H = 2, 9, 8, 2
    rng = np.random.default_rng(7)
    X = rng.standard_normal((B, N, D))
    W = [rng.standard_normal((D, D)) / np.sqrt(D) for _ in range(3)]
    eye = np.eye(H)[:, :, None].copy()
    ref = oracle.forward(X, W[0], W[1], W[2], eye, eye, eye, np.eye(H), H, 1, mask, window)
    Q, K, V = [(X @ w).reshape(B, N, H, D // H) for w in W]
    O = bw.attention_grads(Q, K, V, np.zeros_like(Q), mask, window)["O"]
    np.testing.assert_allclose(O.reshape(B, N, D), ref, rtol=1e-12, atol=1e-13)


def test_attention_lse_is_the_logsumexp_of_the_visible_scores():
    from scipy.special import logsumexp
    Q, K, V, G = _att_inputs(1, 8, 1, 4, seed=8)
    lse = bw.attention_grads(Q, K, V, G, bw.MASK_WINDOW, 3)["lse"]
    for i in range(8):
        ks = [k for k in range(8) if i - 3 < k <= i]
        s = np.array([Q[0, i, 0] @ K[0, k, 0] for k in ks]) / 2.0
        assert abs(lse[0, 0, i] - logsumexp(s)) < 1e-13


def test_attention_empty_allowed_set_is_an_error():
    Q, K, V, G = _att_inputs(1, 4, 1, 4, seed=9)
    with pytest.raises(ValueError):
        bw.attention_grads(Q, K, V, G, bw.MASK_WINDOW, 0)
