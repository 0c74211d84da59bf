"""The C-ABI library: it loads, exports every entry point include/iha.h declares, and its
host-side validation returns the documented codes before touching the GPU.  No kernel is
launched here (these run without a GPU)."""
import ctypes
import os
import re

import pytest

from interleaved_head_layer_amd import _binding as bd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    src = open(os.path.join(ROOT, "include", "iha.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(iha_[a-z_]+)\s*\(", src)))


def test_library_loads_and_exports_every_declared_symbol():
    assert os.path.exists(bd.LIB_PATH), "run __graft_entry__.build() first"
    lib = bd.load_library()
    names = declared_functions()
    assert {"iha_forward", "iha_workspace_bytes", "iha_status_str", "iha_attention",
            "iha_forward_timed", "iha_plan", "iha_attention_backward",
            "iha_attention_backward_workspace"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n


def test_probe_library_exports_its_declared_symbol():
    """The benchmark's measurement probe (include/iha_probe.h, libiha_probe.so)."""
    from interleaved_head_layer_amd import build as hb
    src = open(os.path.join(ROOT, "include", "iha_probe.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = sorted(set(re.findall(r"\b(ihp_[a-z_]+)\s*\(", src)))
    assert names == ["ihp_mfma_rate"]
    lib = ctypes.CDLL(hb.PROBE_LIB)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings():
    for code, name in enumerate(bd.STATUS_NAMES):
        assert bd.iha_status_str(code).startswith(name)


def _ws(B=2, N=100, D=256, H=2, P=2, mask="window", window=None, dtype=bd.IHA_BF16, flags=0):
    p = bd.make_problem(B, N, D, H, P, mask, window, dtype, flags)
    n = ctypes.c_size_t(0)
    return bd.load_library().iha_workspace_bytes(ctypes.byref(p), ctypes.byref(n)), n.value


def test_workspace_size_covers_the_intermediates():
    st, n = _ws()
    assert st == bd.IHA_OK
    B, N, D, P = 2, 100, 256, 2
    M, rows = B * N, B * N * P
    need = 3 * D * D * 2 + M * 2 * D * 4 + M * D * 4      # transposed W, fp32 projections
    need += 4 * rows * D * 2                               # Q~, K~, V~^T, P-bar (fp16)
    R = min(32, P * N)                                    # fp32 first rows (bf16, masked):
    R2 = min(1024, P * N)                                 # rows with fp32 attention outputs
    need += 3 * B * R * D * 4 + B * R2 * D * 4             # their q, k, v and the outputs
    assert need <= n <= need + 16 * 256
    st, n_none = _ws(mask="none")
    assert st == bd.IHA_OK and n_none < need - 3 * B * R * D * 4 - B * R2 * D * 4 + 16 * 256


@pytest.mark.parametrize("B,N,D,H,P,dtype,fused", [
    (4, 4096, 2048, 16, 2, bd.IHA_BF16, True),     # 16 heads of 128, P in {1, 2, 4}
    (2, 256, 1024, 16, 4, bd.IHA_BF16, False),     # P = 4 keeps GEMM + separate mixing
    (2, 256, 1024, 16, 1, bd.IHA_BF16, True),
    (2, 256, 1024, 16, 3, bd.IHA_BF16, False),     # P = 3
    (2, 8192, 2560, 20, 4, bd.IHA_BF16, False),    # P = 4
    (2, 8192, 2560, 20, 2, bd.IHA_BF16, True),     # 20 heads, D a multiple of 320
    (2, 256, 1280, 20, 2, bd.IHA_BF16, True),
    (2, 256, 640, 5, 2, bd.IHA_BF16, False),       # H = 5
    (2, 256, 1024, 16, 2, bd.IHA_F32, False),      # fp32 folds the mixing into the weights
])
def test_plan_and_workspace_follow_the_fused_mixing(B, N, D, H, P, dtype, fused):
    """IHA_PLAN_MIX_FUSED is set exactly for bf16 with 16 heads and D a multiple of 256, or 20
    heads and D a multiple of 320, and P in {1, 2}; then the workspace holds no fp32
    projections of all tokens."""
    p = bd.make_problem(B, N, D, H, P, "causal", None, dtype)
    assert bd.iha_plan(p) == (bd.IHA_PLAN_MIX_FUSED if fused else 0)
    n = bd.iha_workspace_bytes(p)
    stacked = 4 * B * P * N * D * 2                               # Q~ K~ V~^T, P-bar (fp16)
    if dtype == bd.IHA_BF16:
        stacked += 3 * D * D * 2                                  # transposed weights
    if dtype == bd.IHA_BF16:                                      # fp32 first rows (causal)
        R = min(32, P * N)
        stacked += B * min(1024, P * N) * D * 4                   # fp32 outputs of early rows,
        if fused:
            stacked += B * -(-R // P) * 3 * D * 4                 # their tokens' projections
        else:
            stacked += 3 * B * R * D * 4                          # their q, k, v
    fp32_proj = B * N * 3 * D * 4
    if fused:
        assert stacked <= n <= stacked + 16 * 256
    elif dtype == bd.IHA_BF16:
        assert stacked + fp32_proj <= n <= stacked + fp32_proj + 16 * 256


def test_plan_validates():
    st = bd.load_library().iha_plan(ctypes.byref(bd.make_problem(0, 64, 128, 2, 2, "causal")),
                                    ctypes.byref(ctypes.c_uint32()))
    assert st == bd.STATUS_NAMES.index("IHA_ERR_INVALID_ARG")
    assert bd.load_library().iha_plan(ctypes.byref(bd.make_problem(1, 64, 128, 2, 2, "causal")),
                                      None) == bd.STATUS_NAMES.index("IHA_ERR_INVALID_ARG")


@pytest.mark.parametrize("kw,code", [
    (dict(D=250, H=3), bd.STATUS_NAMES.index("IHA_ERR_SHAPE")),
    (dict(N=3, P=2, mask="window"), bd.STATUS_NAMES.index("IHA_ERR_EMPTY_ROW")),   # N // (2P) = 0
    (dict(window=0), bd.STATUS_NAMES.index("IHA_ERR_EMPTY_ROW")),
    (dict(D=96, H=3), bd.STATUS_NAMES.index("IHA_ERR_UNSUPPORTED")),               # d = 32 in bf16
    (dict(D=48, H=3, dtype=bd.IHA_F32), bd.IHA_OK),                                # d = 16 in fp32
    (dict(D=24, H=3, dtype=bd.IHA_F32), bd.STATUS_NAMES.index("IHA_ERR_UNSUPPORTED")),  # d = 8
    (dict(D=130 * 64, H=130), bd.STATUS_NAMES.index("IHA_ERR_UNSUPPORTED")),       # H > 64
    (dict(B=0), bd.STATUS_NAMES.index("IHA_ERR_INVALID_ARG")),
    (dict(mask=7), bd.STATUS_NAMES.index("IHA_ERR_INVALID_ARG")),
    (dict(flags=4), bd.STATUS_NAMES.index("IHA_ERR_INVALID_ARG")),
])
def test_validation_codes(kw, code):
    st, _ = _ws(**kw)
    assert st == code, (kw, bd.iha_status_str(st))


def test_forward_rejects_before_any_launch():
    """Null pointers and a short workspace are refused on the host (fake, never-dereferenced
    pointer values are enough to show it)."""
    lib = bd.load_library()
    p = bd.make_problem(1, 64, 128, 2, 2, "causal")
    fake = ctypes.c_void_p(4096)
    args = [fake] * 9
    st = lib.iha_forward(ctypes.byref(p), None, *args[:7], fake, fake, ctypes.c_size_t(1 << 40), None)
    assert st == bd.STATUS_NAMES.index("IHA_ERR_INVALID_ARG")
    st = lib.iha_forward(ctypes.byref(p), *args[:8], fake, fake, ctypes.c_size_t(16), None)
    assert st == bd.STATUS_NAMES.index("IHA_ERR_WORKSPACE")
    st = lib.iha_forward(ctypes.byref(p), *args[:8], fake, ctypes.c_void_p(4096 + 8),
                         ctypes.c_size_t(1 << 40), None)
    assert st == bd.STATUS_NAMES.index("IHA_ERR_WORKSPACE")     # misaligned
    odd = ctypes.c_void_p(4096 + 8)                               # 8-byte, not 16-byte aligned
    for k in (0, 1, 8):                                           # X, W_Q, X_out
        a = list(args[:8]) + [fake]
        a[k] = odd
        st = lib.iha_forward(ctypes.byref(p), *a, fake, ctypes.c_size_t(1 << 40), None)
        assert st == bd.STATUS_NAMES.index("IHA_ERR_INVALID_ARG"), k
    st = lib.iha_attention(1, 64, 2, 128, 0, 0, 1.0, fake, odd, fake, fake, 0, None, None)
    assert st == bd.STATUS_NAMES.index("IHA_ERR_INVALID_ARG")
    st = lib.iha_attention(1, 64, 2, 96, 0, 0, 1.0, fake, fake, fake, fake, 0, None, None)
    assert st == bd.STATUS_NAMES.index("IHA_ERR_UNSUPPORTED")
    st = lib.iha_attention(1, 64, 2, 128, 2, 0, 1.0, fake, fake, fake, fake, 0, None, None)
    assert st == bd.STATUS_NAMES.index("IHA_ERR_EMPTY_ROW")
    st = lib.iha_attention(1, 64, 2, 128, 0, 0, -1.0, fake, fake, fake, fake, 0, None, None)
    assert st == bd.STATUS_NAMES.index("IHA_ERR_INVALID_ARG")
    evs = (ctypes.c_void_p * bd.TIMED_EVENTS)()
    st = lib.iha_forward_timed(ctypes.byref(p), *args[:8], fake, fake, ctypes.c_size_t(1 << 40),
                               None, evs)
    assert st == bd.STATUS_NAMES.index("IHA_ERR_INVALID_ARG")   # null events


def test_timed_event_count_matches_header():
    """The binding's event count is the one include/iha.h declares."""
    import re
    hdr = open(os.path.join(ROOT, "include", "iha.h")).read()
    m = re.search(r"#define\s+IHA_TIMED_EVENTS\s+(\d+)", hdr)
    assert m and int(m.group(1)) == bd.TIMED_EVENTS


def test_attention_backward_workspace_and_validation():
    """Host-side only: the workspace formula (fp16 Q*scale, three padded channel-major copies,
    V^T, the fp16 forward output, fp32 lse and D) and the argument checks, which return before
    any launch."""
    lib = bd.load_library()
    n = ctypes.c_size_t(0)
    B, L, H, d = 2, 300, 3, 64
    assert lib.iha_attention_backward_workspace(B, L, H, d, ctypes.byref(n)) == 0
    up = lambda x: (x + 255) // 256 * 256
    E, Et, S = B * L * H * d, B * H * d * 320, B * H * L
    assert n.value == 3 * up(E * 2) + 3 * up(Et * 2) + 2 * up(S * 4)
    assert lib.iha_attention_backward_workspace(B, L, H, 96, ctypes.byref(n)) == bd.STATUS_NAMES.index("IHA_ERR_UNSUPPORTED")
    assert lib.iha_attention_backward_workspace(B, L, 65, d, ctypes.byref(n)) == bd.STATUS_NAMES.index("IHA_ERR_SHAPE")
    assert lib.iha_attention_backward_workspace(0, L, H, d, ctypes.byref(n)) == bd.STATUS_NAMES.index("IHA_ERR_INVALID_ARG")
    fake = ctypes.c_void_p(1 << 20)
    odd = ctypes.c_void_p((1 << 20) + 8)
    args = lambda mask, window, scale, qp=fake, ws=fake, nb=1 << 40: (
        B, L, H, d, mask, window, scale, qp, fake, fake, fake, fake, fake, fake, ws, nb, None)
    assert lib.iha_attention_backward(*args(2, 0, 1.0)) == bd.STATUS_NAMES.index("IHA_ERR_EMPTY_ROW")
    assert lib.iha_attention_backward(*args(0, 0, -1.0)) == bd.STATUS_NAMES.index("IHA_ERR_INVALID_ARG")
    assert lib.iha_attention_backward(*args(0, 0, 1.0, qp=odd)) == bd.STATUS_NAMES.index("IHA_ERR_INVALID_ARG")
    assert lib.iha_attention_backward(*args(1, 0, 1.0, ws=odd)) == bd.STATUS_NAMES.index("IHA_ERR_WORKSPACE")
    assert lib.iha_attention_backward(*args(1, 0, 1.0, nb=16)) == bd.STATUS_NAMES.index("IHA_ERR_WORKSPACE")


def test_layer_backward_workspace_and_validation():
    """Host-side checks of iha_backward, which return before any launch: bf16 only, the
    attention backward's head widths, null or misaligned pointers, a short workspace."""
    lib = bd.load_library()
    code = bd.STATUS_NAMES.index
    n = ctypes.c_size_t(0)
    p = bd.make_problem(2, 100, 256, 2, 2, "causal")
    assert lib.iha_backward_workspace(ctypes.byref(p), ctypes.byref(n)) == bd.IHA_OK
    M, D, act = 200, 256, 200 * 2 * 256
    # at least: transposed W, fp32 Y, four fp16 and three fp32 stacked tensors, bf16 high and
    # low dY (token- and channel-major), X^T twice and the concatenated W twice
    Mp = 256
    assert n.value >= (3 * D * D * 2 + M * 3 * D * 4 + 4 * act * 2 + 3 * act * 4 + M * 6 * D * 2
                       + 3 * D * 2 * Mp * 2 + D * 2 * Mp * 2 + D * 6 * D * 2)
    pf = bd.make_problem(2, 100, 256, 2, 2, "causal", dtype=bd.IHA_F32)
    assert lib.iha_backward_workspace(ctypes.byref(pf), ctypes.byref(n)) == code("IHA_ERR_UNSUPPORTED")
    p96 = bd.make_problem(1, 64, 192, 2, 2, "causal")
    assert lib.iha_backward_workspace(ctypes.byref(p96), ctypes.byref(n)) == code("IHA_ERR_UNSUPPORTED")
    pw = bd.make_problem(1, 64, 128, 2, 2, "window", 0)
    assert lib.iha_backward_workspace(ctypes.byref(pw), ctypes.byref(n)) == code("IHA_ERR_EMPTY_ROW")
    assert lib.iha_backward_workspace(ctypes.byref(p), None) == code("IHA_ERR_INVALID_ARG")
    fake = ctypes.c_void_p(1 << 20)
    odd = ctypes.c_void_p((1 << 20) + 8)
    big = ctypes.c_size_t(1 << 40)
    ptrs = [fake] * 17   # X, W_Q, W_K, W_V, alpha_Q/K/V, R, G, then the eight gradients
    for k in range(17):
        a = list(ptrs)
        a[k] = None
        assert lib.iha_backward(ctypes.byref(p), *a, fake, big, None) == code("IHA_ERR_INVALID_ARG"), k
        a[k] = odd
        assert lib.iha_backward(ctypes.byref(p), *a, fake, big, None) == code("IHA_ERR_INVALID_ARG"), k
    assert lib.iha_backward(ctypes.byref(p), *ptrs, fake, ctypes.c_size_t(16), None) == code("IHA_ERR_WORKSPACE")
    assert lib.iha_backward(ctypes.byref(p), *ptrs, odd, big, None) == code("IHA_ERR_WORKSPACE")


def test_fused_collapse_flag_validation():
    """IHA_FLAG_FUSED_COLLAPSE is accepted for bf16 problems and rejected for fp32 ones; other
    unknown flag bits stay invalid."""
    code = bd.STATUS_NAMES.index
    st, n_fused = _ws(flags=bd.IHA_FLAG_FUSED_COLLAPSE)
    assert st == bd.IHA_OK
    st, n_plain = _ws()
    assert n_fused == n_plain
    st, _ = _ws(D=64, H=4, dtype=bd.IHA_F32, flags=bd.IHA_FLAG_FUSED_COLLAPSE)
    assert st == code("IHA_ERR_UNSUPPORTED")
    st, _ = _ws(flags=4)
    assert st == code("IHA_ERR_INVALID_ARG")
