"""Pins of the oracle's Nexus inner attention ("Higher-order attention mechanisms" page,
section 2: Attention_q(X) = softmax(Q Q^T / sqrt(d_k)) Q), against closed forms, torch's
scaled-dot-product attention with keys = values = queries, and invariants - none of them
computed through the oracle."""
import math

import numpy as np
import pytest
import torch

import oracle


def closed_form_orthogonal(n, d, c, mask, window):
    """Rows c * e_i (i < n <= d): row i scores c^2/sqrt(d) against itself and 0 against the
    other visible rows, so with a = exp(c^2/sqrt(d)) and v visible rows its output has
    c a / (a + v - 1) at channel i and c / (a + v - 1) at the other visible channels."""
    a = math.exp(c * c / math.sqrt(d))
    out = np.zeros((n, d))
    for i in range(n):
        if mask == oracle.MASK_NONE:
            vis = list(range(n))
        elif mask == oracle.MASK_CAUSAL:
            vis = list(range(i + 1))
        else:
            vis = list(range(max(0, i - window + 1), i + 1))
        den = a + len(vis) - 1
        for j in vis:
            out[i, j] = c * (a if j == i else 1.0) / den
    return out


@pytest.mark.parametrize("mask,window", [(oracle.MASK_NONE, 0), (oracle.MASK_CAUSAL, 0),
                                         (oracle.MASK_WINDOW, 3)])
@pytest.mark.parametrize("c", [0.5, 2.0])
def test_orthogonal_rows_closed_form(mask, window, c):
    n, d = 7, 16
    Q = np.zeros((1, n, 1, d))
    Q[0, :, 0, :n] = c * np.eye(n)
    got = oracle.nexus_inner(Q, mask, window)[0, :, 0]
    np.testing.assert_allclose(got, closed_form_orthogonal(n, d, c, mask, window), rtol=0, atol=1e-14)


@pytest.mark.parametrize("mask,window", [(oracle.MASK_NONE, 0), (oracle.MASK_CAUSAL, 0),
                                         (oracle.MASK_WINDOW, 2)])
def test_equal_rows_return_the_row(mask, window):
    q = np.random.default_rng(1).standard_normal(32)
    Q = np.tile(q, (1, 9, 2, 1))                                  # [1, 9, 2, 32]
    np.testing.assert_allclose(oracle.nexus_inner(Q, mask, window), Q, rtol=0, atol=1e-14)


def test_single_position_returns_itself():
    Q = np.random.default_rng(2).standard_normal((3, 1, 2, 8))
    np.testing.assert_allclose(oracle.nexus_inner(Q, oracle.MASK_CAUSAL), Q, rtol=0, atol=1e-15)


@pytest.mark.parametrize("causal", [False, True])
def test_matches_sdpa_with_keys_and_values_the_queries(causal):
    rng = np.random.default_rng(3)
    Q = rng.standard_normal((2, 23, 3, 16)) * 0.7
    got = oracle.nexus_inner(Q, oracle.MASK_CAUSAL if causal else oracle.MASK_NONE)
    q = torch.from_numpy(Q).permute(0, 2, 1, 3)                   # [B, H, L, d]
    ref = torch.nn.functional.scaled_dot_product_attention(q, q, q, is_causal=causal)
    np.testing.assert_allclose(got, ref.permute(0, 2, 1, 3).numpy(), rtol=0, atol=1e-12)


def test_window_beyond_length_equals_causal_and_permutation_equivariance():
    rng = np.random.default_rng(4)
    Q = rng.standard_normal((1, 15, 2, 8))
    np.testing.assert_array_equal(oracle.nexus_inner(Q, oracle.MASK_WINDOW, 100),
                                  oracle.nexus_inner(Q, oracle.MASK_CAUSAL))
    perm = rng.permutation(15)
    a = oracle.nexus_inner(Q[:, perm], oracle.MASK_NONE)
    b = oracle.nexus_inner(Q, oracle.MASK_NONE)[:, perm]
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-14)
