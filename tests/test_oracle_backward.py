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
