"""The seeded input generator: determinism, bf16 exactness and the stated distributions."""
import numpy as np

from interleaved_head_layer_amd import workloads as wl


def test_deterministic_and_bf16_exact():
    w = wl.custom(2, 33, 64, 4, 2, "window", dtype="bf16", seed=5)
    a, b = wl.make_inputs(w), wl.make_inputs(w)
    for k in a:
        assert np.array_equal(a[k], b[k])
    for k in ("X", "WQ", "WK", "WV"):
        assert np.all((a[k].view(np.uint32) & 0xFFFF) == 0), k   # bf16-representable
    assert a["aQ"].shape == (4, 4, 2) and a["R"].shape == (4, 8)


def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0, 1.0 + 2**-8, 1.0 + 3 * 2**-8, -2.5, 1.0 + 2**-9], np.float32)
    r = wl.round_to_bf16(x)
    assert list(r) == [1.0, 1.0, 1.0 + 4 * 2**-8, -2.5, 1.0]


def test_distributions_and_special_inputs():
    w = wl.custom(1, 2048, 256, 8, 2, "causal", dtype="f32", seed=9)
    x = wl.make_inputs(w)
    assert abs(x["X"].std() - 1.0) < 0.02
    assert abs(x["WQ"].std() * np.sqrt(256) - 1.0) < 0.02
    assert abs(x["aK"].std() * np.sqrt(8) - 1.0) < 0.2
    m = wl.WORKLOADS["mha_causal_bf16"]
    assert m.P == 1 and m.identity_mix
    lc = wl.WORKLOADS["iha_window_p2_n16384_longctx"]
    assert lc.window == 16384 // 4 and lc.repeated_keys == 64
    assert wl.WORKLOADS["iha_window_p4_b2_n8192_wide"].window == 1024


def test_identity_and_repeated_rows():
    w = wl.custom(1, 300, 64, 4, 1, "causal", seed=3, identity_mix=True, repeated_keys=16)
    x = wl.make_inputs(w)
    assert np.array_equal(x["aQ"][:, :, 0], np.eye(4)) and np.array_equal(x["R"], np.eye(4))
    rows = x["X"].reshape(-1, 64)
    _, counts = np.unique(rows, axis=0, return_counts=True)
    assert counts.max() == 16
    pos = x["repeated_pos"]
    assert pos.dtype == np.int64 and len(np.unique(pos)) == 16
    assert np.all(rows[pos] == rows[pos[0]])


def test_sample_tokens_cover_edges():
    w = wl.WORKLOADS["iha_window_p2_b4_n4096"]
    s = wl.sample_tokens(w, 40)
    assert s.min() == 0 and (w.N - 1) in s and (w.B * w.N - 1) in s and len(s) >= 24
