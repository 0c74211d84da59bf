#!/usr/bin/env python3
"""Throughput of the IHA forward pass on one MI355X.

Headline workload: the wide IHA layer (B 2, N 8192, D 2560, H 20, d 128, P 4), which the
workload list defines in two mask modes on the same seeded inputs.  One step is one whole
forward in window mode (W_s = N/(2P) = 1024 stacked positions) followed by one whole forward
in causal mode, inputs resident in HBM before timing; `value` is pseudo-tokens
(2 * B * P * N per step) per second over K back-to-back steps.

The line also carries: per-kernel times of each mode from HIP events recorded on the launch
stream between the kernels (a second pass of K steps; each event adds a gap of about 10 us
between kernels, so `value` comes from the pass without them), the roofline position of the
dominant kernel and of every kernel, a pass of K steps each preceded by a 512 MiB write
that flushes the caches (median of those steps), the matrix-core rate and shader clock the
chip sustains under a pure-product load (libiha_probe.so), the CPU oracle timed on a bounded
token sample with the GPU output checked against it on those tokens, the same figures for
the other full-size workloads (fewer steps), the attention backward at the 4 x 4096-token
workload's attention shape, and the layer backward (all gradients) at the headline shapes.

Work per unit (algorithmic, the count the pages' convention gives):
  attention  4 * d flops per visible (query, key) pair: QK^T and AV at 2 flops per
             multiply-add (textbook eq. 5.34), masked pairs and softmax not counted
  gemm       6 * D^2 flops per token (the three D x D projections, eq. 5.34)
  mix        bytes: 3 * D * 4 read (projected values, fp32) + 3 * P * D * 2 written
             (stacked fp16 Q~, K~, V~) per token.  Where the mixing runs in the GEMM's
             epilogue (IHA_PLAN_MIX_FUSED) the gemm step holds it and the mix step is empty
             (the first rows' fp32 mixing runs in the attention launch)
  collapse   bytes: P*H*d*e read (e = 2: the bf16 forward keeps the stacked outputs in fp16;
             4 for fp32) + H*d*4 written per token
  prep       bytes: 3*D^2*2 read + 3*D^2*2 written (bf16 weight transpose)
"""
import argparse
import ctypes
import glob
import json
import os
import statistics
import sys
import threading
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_MFMA_F16 = 2.5e15      # dense fp16 / bf16 matrix-core FLOP/s, MI355X datasheet
PEAK_MFMA_F32 = 157.3e12
PEAK_HBM = 8.0e12           # bytes/s
HEADLINE = ("iha_window_p4_b2_n8192_wide", "iha_causal_p4_b2_n8192_wide")
OTHERS = ["iha_window_p2_b4_n4096", "iha_window_p2_n16384_longctx", "mha_causal_bf16"]
STEPS = ["prep", "gemm", "mix", "attention", "first_rows", "collapse"]
BAR_BF16 = 2e-2


def allowed_pairs(L, mask, window):
    """Visible (query, key) pairs per (b, h) over L stacked rows."""
    if mask == 0:
        return L * L
    if mask == 1:
        return L * (L + 1) // 2
    W = min(window, L)
    return W * (W + 1) // 2 + (L - W) * W


def counter_traffic(workload, step):
    """HBM bytes per step of `step` from the committed rocprofv3 counter summary of
    `workload` (FETCH_SIZE and WRITE_SIZE per dispatch, scaled by the copy reference), or
    None if there is none or the kernel's source changed since the counters were taken."""
    import hashlib
    import re
    for path in glob.glob(os.path.join(ROOT, "profiles", "hbm_counters_*.md")):
        m = re.search(r"```json\n(.*?)```", open(path).read(), re.S)
        if not m:
            continue
        info = json.loads(m.group(1))
        if info.get("workload") != workload or step not in info.get("steps", {}):
            continue
        st = info["steps"][step]
        src = os.path.join(ROOT, st["source"])
        if not os.path.exists(src) or hashlib.sha256(open(src, "rb").read()).hexdigest() != st["sha256"]:
            return None
        sc = info["scale"]
        kib = sum((f * sc["FETCH_SIZE"] + w * sc["WRITE_SIZE"]) * n for f, w, n in st["kernels"].values())
        return int(kib * 1024)
    return None


def roof(kind, work, ms):
    if kind == "mfma":
        a = work / (ms * 1e-3) / 1e12
        return {"bound": "mfma", "achieved": round(a, 2), "peak": PEAK_MFMA_F16 / 1e12,
                "unit": "TFLOP/s", "frac": round(a / (PEAK_MFMA_F16 / 1e12), 4), "traffic": None}
    a = work / (ms * 1e-3) / 1e9
    return {"bound": "hbm", "achieved": round(a, 1), "peak": PEAK_HBM / 1e9, "unit": "GB/s",
            "frac": round(a / (PEAK_HBM / 1e9), 4), "traffic": None}


def kernel_rooflines(w, kms, fused):
    """Roofline entries of every step of workload `w` from its per-step times `kms`."""
    B, N, D, H, P, d = w.B, w.N, w.D, w.H, w.P, w.d
    attn_flops = 4.0 * d * B * H * allowed_pairs(P * N, w.mask, w.window)
    roofs = {"prep": roof("hbm", 3 * D * D * 2 * 2, kms["prep"]),
             "gemm": roof("mfma", 6.0 * B * N * D * D, kms["gemm"]),
             "mix": None if fused else roof("hbm", B * N * (3 * D * 4 + 3 * P * D * 2), kms["mix"]),
             "attention": roof("mfma", attn_flops, kms["attention"]),
             "collapse": roof("hbm", B * N * (P * H * d * (2 if w.dtype == "bf16" else 4) + H * d * 4)
                              + H * H * P * 4, kms["collapse"])}
    roofs = {k: v for k, v in roofs.items() if v is not None}
    for k in roofs:
        roofs[k]["traffic"] = counter_traffic(w.name, k)
        roofs[k]["ms"] = round(kms[k], 4)
    return roofs


class Forwards:
    """Device inputs of one seeded input set and the forwards of one or more mask modes of it
    (workloads with the same shapes and seed), sharing one workspace and output buffer."""

    def __init__(self, workloads):
        import torch
        import interleaved_head_layer_amd as iha
        from interleaved_head_layer_amd import workloads as wl
        self.iha, self.torch = iha, torch
        w0 = workloads[0]
        for w in workloads[1:]:
            assert (w.B, w.N, w.D, w.H, w.P, w.seed, w.dtype) == (w0.B, w0.N, w0.D, w0.H, w0.P, w0.seed, w0.dtype)
        self.ws_list = workloads
        self.x = wl.make_inputs(w0)
        dev = torch.device("cuda:0")
        dt = torch.bfloat16 if w0.dtype == "bf16" else torch.float32
        t = lambda a, d=dt: torch.from_numpy(a).to(dev).to(d).contiguous()
        self.args = [t(self.x["X"]), t(self.x["WQ"]), t(self.x["WK"]), t(self.x["WV"])] + \
                    [t(self.x[k], torch.float32) for k in ("aQ", "aK", "aV", "R")]
        dtype = iha.IHA_BF16 if w0.dtype == "bf16" else iha.IHA_F32
        self.probs = [iha.make_problem(w.B, w.N, w.D, w.H, w.P, w.mask, w.window, dtype) for w in workloads]
        self.ws = torch.empty(max(iha.iha_workspace_bytes(p) for p in self.probs), dtype=torch.uint8, device=dev)
        self.out = torch.empty((w0.B, w0.N, w0.D), dtype=torch.float32, device=dev)
        self.fused = [bool(iha.iha_plan(p) & iha.IHA_PLAN_MIX_FUSED) for p in self.probs]

    def forward(self, i, events=None, flags=0):
        w = self.ws_list[i]
        self.iha.iha_forward(*self.args, w.H, w.P, w.mask, w.window, out=self.out, workspace=self.ws,
                             events=events, flags=flags)

    def step(self):
        for i in range(len(self.ws_list)):
            self.forward(i)

    def output(self, i):
        """Output of mode i on the host (float64)."""
        import numpy as np
        self.forward(i)
        self.torch.cuda.synchronize()
        return self.out.cpu().numpy().astype(np.float64)

    def free(self):
        del self.args, self.ws, self.out
        self.torch.cuda.empty_cache()


def time_steps(fw, steps, warmup, flush_mib=512):
    """Back-to-back timing, the per-kernel event pass and the flushed pass of `fw`."""
    import numpy as np
    torch, iha = fw.torch, fw.iha
    for _ in range(warmup):
        fw.step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        fw.step()
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / steps
    # Per-kernel events (second pass).
    nm = len(fw.ws_list)
    evs = [[[torch.cuda.Event(enable_timing=True) for _ in range(iha.TIMED_EVENTS)] for _ in range(nm)]
           for _ in range(steps)]
    for per in evs:
        for e in per:
            for ev in e:
                ev.record()
    torch.cuda.synchronize()
    t2 = time.perf_counter()
    for s in range(steps):
        for i in range(nm):
            fw.forward(i, evs[s][i])
    torch.cuda.synchronize()
    ms_events = (time.perf_counter() - t2) * 1e3 / steps
    kms = [{n: float(np.mean([evs[s][i][k].elapsed_time(evs[s][i][k + 1]) for s in range(steps)]))
            for k, n in enumerate(STEPS)} for i in range(nm)]
    # Flushed pass: each step after a 512 MiB write (larger than the 256 MiB last-level cache).
    buf = torch.empty(flush_mib << 18, dtype=torch.float32, device="cuda:0")
    flushed = []
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for s in range(steps):
        buf.fill_(float(s))
        e0.record()
        fw.step()
        e1.record()
        torch.cuda.synchronize()
        flushed.append(e0.elapsed_time(e1))
    del buf
    return {"ms_step": ms_step, "ms_step_events": ms_events, "kms": kms,
            "ms_step_flushed": statistics.median(flushed)}


def oracle_sample(fw, i, ntok, seed):
    """CPU oracle on `ntok` uniformly drawn tokens of mode i (all their heads and
    pseudo-tokens, plus the key/value projections they can see), timed, and the GPU output
    of that mode compared with it on those tokens."""
    import numpy as np
    import oracle
    w = fw.ws_list[i]
    x = fw.x
    tok = np.sort(np.random.default_rng(seed).choice(w.B * w.N, min(ntok, w.B * w.N), replace=False))
    c0 = time.perf_counter()
    ref = oracle.forward(x["X"], x["WQ"], x["WK"], x["WV"], x["aQ"], x["aK"], x["aV"], x["R"],
                         w.H, w.P, w.mask, w.window, tokens=tok)
    secs = time.perf_counter() - c0
    gpu = fw.output(i).reshape(w.B * w.N, w.D)[tok]
    err = float(np.abs(gpu - ref).max())
    rms = float(np.sqrt(np.mean(ref ** 2)))
    return {"tokens": int(len(tok)), "seconds": secs, "pseudo_tokens": int(len(tok)) * w.P,
            "max_err_over_rms": err / rms}


def cpu_entry(samples, label):
    import oracle
    secs = sum(s["seconds"] for s in samples)
    pt = sum(s["pseudo_tokens"] for s in samples)
    return {"value": round(pt / secs, 2), "unit": "pseudo-tokens/s", "cores": oracle.threads(),
            "kind": "oracle",
            "sample": f"{label}: {sum(s['tokens'] for s in samples)} uniformly drawn tokens (all their heads and "
                      f"pseudo-tokens, plus the key/value projections they can see), {secs:.1f} s wall in "
                      f"IEEE double"}


def sample_sclk(stop, out):
    """Current shader clock level (MHz) from the amdgpu sysfs files, sampled until `stop`."""
    files = glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk")
    while not stop.is_set() and files:
        for f in files:
            try:
                for line in open(f):
                    if line.rstrip().endswith("*"):
                        out.append(float(line.split()[1].lower().replace("mhz", "")))
            except (OSError, ValueError, IndexError):
                pass
        time.sleep(0.01)


def probe_chip():
    """Matrix-core rate and shader clock under a pure fp16-product load (libiha_probe.so)."""
    from interleaved_head_layer_amd import build as hb
    if not os.path.exists(hb.PROBE_LIB):
        return None
    lib = ctypes.CDLL(hb.PROBE_LIB)
    d = ctypes.c_double
    lib.ihp_mfma_rate.argtypes = [ctypes.c_int, ctypes.POINTER(d), ctypes.POINTER(d), ctypes.POINTER(d)]
    lib.ihp_mfma_rate.restype = ctypes.c_int
    tf, clk, ms = d(0), d(0), d(0)
    if lib.ihp_mfma_rate(200, ctypes.byref(tf), ctypes.byref(clk), ctypes.byref(ms)) != 0:
        return None
    return {"mfma_f16_tflops": round(tf.value, 1), "frac_of_datasheet": round(tf.value * 1e12 / PEAK_MFMA_F16, 4),
            "sclk_mhz": round(clk.value, 1), "kernel_ms": round(ms.value, 1),
            "note": "pure 32x32x16 fp16 products, two waves per SIMD on every CU; clock from the "
                    "shader-clock counter against the 100 MHz constant counter"}


def copy_rate():
    """Device-to-device copy of 1 GiB (read + write bytes per second)."""
    import torch
    src = torch.ones(1 << 28, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(5):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    gbs = 5 * 2 * src.numel() * 4 / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del src, dst
    torch.cuda.empty_cache()
    return round(gbs, 1)


def run_attention_backward(w, steps, warmup):
    """Time iha_attention_backward on the stacked attention of workload `w` (L = P*N rows per
    sequence, its heads, head width, mask and window), inputs resident on the GPU.  Work is
    counted as 2.5x the forward's 4*d*(visible pairs) per head: the gradient products dV, dP,
    dQ and dK plus the recomputed scores, 2*d flops per visible pair each."""
    import torch
    import interleaved_head_layer_amd as iha

    B, H, d, L = w.B, w.H, w.D // w.H, w.P * w.N
    mask = ["none", "causal", "window"][w.mask]
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev)
    g.manual_seed(1234)
    q, k, v, go = (torch.randn((B, L, H, d), generator=g, device=dev).half() for _ in range(4))
    nbytes = ctypes.c_size_t(0)
    lib = iha.load_library()
    assert lib.iha_attention_backward_workspace(B, L, H, d, ctypes.byref(nbytes)) == 0
    ws = torch.empty(int(nbytes.value), dtype=torch.uint8, device=dev)
    call = lambda: iha.iha_attention_backward(q, k, v, go, mask, w.window, workspace=ws)
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        call()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    work = 2.5 * 4.0 * d * B * H * allowed_pairs(L, w.mask, w.window)
    del q, k, v, go, ws
    torch.cuda.empty_cache()
    return {"shape": {"B": B, "L": L, "H": H, "d": d, "mask": mask, "window": w.window},
            "ms": round(ms, 4), "steps": steps, "work_flop": work,
            "roofline": roof("mfma", work, ms),
            "note": "whole call: prep copies, forward recompute (O, lse), dQ and dK/dV kernels"}


def run_nexus_inner(B, L, H, d, mask, steps, warmup):
    """Time iha_nexus_inner (softmax(Q Q^T / sqrt(d)) Q per head) on fp16 Q [B, L, H, d];
    work: 4 * d flops per visible (query, key) pair, as for the attention step."""
    import torch
    import interleaved_head_layer_amd as iha
    g = torch.Generator(device="cuda:0")
    g.manual_seed(77)
    q = torch.randn((B, L, H, d), generator=g, device="cuda:0").half()
    out = torch.empty((B, L, H, d), dtype=torch.float32, device="cuda:0")
    lib = iha.load_library()
    nbytes = ctypes.c_size_t(0)
    assert lib.iha_nexus_inner_workspace(B, L, H, d, ctypes.byref(nbytes)) == 0
    ws = torch.empty(int(nbytes.value), dtype=torch.uint8, device="cuda:0")
    call = lambda: iha.iha_nexus_inner(q, mask, out=out, workspace=ws)
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        call()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    code = {"none": 0, "causal": 1}[mask]
    work = 4.0 * d * B * H * allowed_pairs(L, code, 0)
    del q, out, ws
    torch.cuda.empty_cache()
    return {"shape": {"B": B, "L": L, "H": H, "d": d, "mask": mask}, "ms": round(ms, 4), "steps": steps,
            "roofline": roof("mfma", work, ms),
            "note": "whole call: the channel-major copy of Q and the attention kernel"}


def run_fused_collapse_ab(w, steps):
    """A/B of the collapse placement on workload `w`: whole forwards with the separate collapse
    kernel (default) against IHA_FLAG_FUSED_COLLAPSE (the collapse in the attention epilogue
    with fp32 atomics), `steps` each after 2 warm-up forwards, alternating twice."""
    import torch
    fw = Forwards([w])
    res = {"default": [], "fused_collapse": []}
    for _ in range(2):
        for name, flags in (("default", 0), ("fused_collapse", fw.iha.IHA_FLAG_FUSED_COLLAPSE)):
            for _ in range(2):
                fw.forward(0, flags=flags)
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(steps):
                fw.forward(0, flags=flags)
            e1.record()
            torch.cuda.synchronize()
            res[name].append(e0.elapsed_time(e1) / steps)
    fw.free()
    d, f = min(res["default"]), min(res["fused_collapse"])
    return {"workload": w.name, "ms_per_forward_default": round(d, 4), "ms_per_forward_fused_collapse": round(f, 4),
            "fused_over_default": round(f / d, 2), "steps": steps,
            "note": "whole forwards; the fused collapse zeroes X~ and adds every stacked output row, "
                    "weighted by R, into all H output heads with fp32 atomics from the attention epilogue"}


def run_layer_backward(w, steps, warmup):
    """Time iha_backward (the layer's gradients dX, dW, dalpha, dR) on workload `w`, inputs
    resident on the GPU.  Work counted: the projections recomputed, dW and dX at 6 * D^2 flops
    per token each (the high/low split of dY doubles the executed products of the last two,
    not the algorithmic count), and the attention backward at 2.5x the forward's 4 * d flops
    per visible pair; the mixing, collapse and reductions over tokens are not counted."""
    import torch
    import interleaved_head_layer_amd as iha

    B, N, D, H, P, d = w.B, w.N, w.D, w.H, w.P, w.D // w.H
    mask = ["none", "causal", "window"][w.mask]
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev)
    g.manual_seed(4321)
    rnd = lambda *shape, s=1.0: torch.randn(shape, generator=g, device=dev) * s
    X = rnd(B, N, D).bfloat16()
    Ws = [rnd(D, D, s=D ** -0.5).bfloat16() for _ in range(3)]
    als = [rnd(H, H, P, s=H ** -0.5) for _ in range(3)]
    R = rnd(H, H * P, s=(H * P) ** -0.5)
    G = rnd(B, N, D)
    prob = iha.make_problem(B, N, D, H, P, mask, w.window)
    ws = torch.empty(iha.iha_backward_workspace_bytes(prob), dtype=torch.uint8, device=dev)
    call = lambda: iha.iha_backward(X, *Ws, *als, R, G, H, P, mask, w.window, workspace=ws)
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        call()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    gemm = 3 * 6.0 * D * D * B * N
    att = 2.5 * 4.0 * d * B * H * allowed_pairs(P * N, w.mask, w.window)
    out = {"shape": {"B": B, "N": N, "D": D, "H": H, "d": d, "P": P, "mask": mask, "window": w.window},
           "ms": round(ms, 4), "steps": steps, "work_flop": gemm + att,
           "gemm_flop": gemm, "attention_flop": att,
           "tokens_per_s": round(B * N / (ms * 1e-3), 1),
           "roofline": roof("mfma", gemm + att, ms),
           "workspace_bytes": int(ws.numel()),
           "note": "whole call: projections and mixing recomputed, expand through R, attention "
                   "backward, token reductions for dalpha and dR, collapse for dY, dW and dX GEMMs"}
    del X, Ws, als, R, G, ws
    torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=None,
                    help="time only this workload (one mode) instead of the headline pair")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-tokens", type=int, default=64,
                    help="tokens per mode the CPU oracle computes for the headline baseline")
    ap.add_argument("--no-extra", action="store_true", help="skip the other workloads")
    ap.add_argument("--extra-steps", type=int, default=5,
                    help="timed steps of the other workloads (at least 20 forwards, 10 backward calls)")
    ap.add_argument("--only-backward", action="store_true",
                    help="time only the attention backward of the workload's attention shape")
    ap.add_argument("--only-layer-backward", action="store_true",
                    help="time only the layer backward (iha_backward) of the workload")
    ap.add_argument("--only-fused-collapse", action="store_true",
                    help="time only the collapse-placement A/B of the workload")
    ap.add_argument("--copy-ref", type=int, default=0, metavar="MIB",
                    help="first run a plain device copy of MIB MiB (reference for HBM counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: the forward runs on one GPU; --gpus {args.gpus} is not supported "
              "(the forward shards by sequence across GPUs with no exchange)",
              file=sys.stderr)
        sys.exit(2)
    from interleaved_head_layer_amd import workloads as wl

    if args.copy_ref > 0:
        import torch
        src = torch.ones(args.copy_ref << 18, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    if args.only_backward:
        w = wl.WORKLOADS[args.workload or OTHERS[0]]
        print(json.dumps({"workload": w.name,
                          "attention_backward": run_attention_backward(w, args.steps, args.warmup)}),
              flush=True)
        return

    if args.only_fused_collapse:
        for n in ([args.workload] if args.workload else [OTHERS[0], HEADLINE[0]]):
            print(json.dumps({"fused_collapse_ab": run_fused_collapse_ab(wl.WORKLOADS[n], args.steps)}), flush=True)
        return

    if args.only_layer_backward:
        for n in ([args.workload] if args.workload else list(HEADLINE)):
            print(json.dumps({"workload": n, "layer_backward": run_layer_backward(wl.WORKLOADS[n], args.steps,
                                                                                  args.warmup)}), flush=True)
        return

    names = [args.workload] if args.workload else list(HEADLINE)
    ws = [wl.WORKLOADS[n] for n in names]
    fw = Forwards(ws)
    stop, sclk = threading.Event(), []
    th = threading.Thread(target=sample_sclk, args=(stop, sclk), daemon=True)
    th.start()
    r = time_steps(fw, args.steps, args.warmup)
    stop.set()
    th.join()
    w0 = ws[0]
    B, N, D, H, P, d = w0.B, w0.N, w0.D, w0.H, w0.P, w0.d
    modes = {}
    for i, w in enumerate(ws):
        roofs = kernel_rooflines(w, r["kms"][i], fw.fused[i])
        modes[w.name] = {"mask": ["none", "causal", "window"][w.mask], "window": w.window,
                         "ms_events": round(sum(r["kms"][i].values()), 4),
                         "kernels_ms": {k: round(v, 4) for k, v in r["kms"][i].items()},
                         "kernel_roofline": roofs, "mix_fused": fw.fused[i]}
    # Dominant kernel of the step: the longest one over all modes.
    dom_mode, dom_kernel = max(((n, k) for n in modes for k in modes[n]["kernel_roofline"]),
                               key=lambda nk: modes[nk[0]]["kernel_roofline"][nk[1]]["ms"])
    dominant = dict(modes[dom_mode]["kernel_roofline"][dom_kernel], kernel=dom_kernel, workload=dom_mode)

    cpu, parity = None, None
    if not args.no_cpu_baseline:
        samples = [oracle_sample(fw, i, args.cpu_tokens, 7 + i) for i in range(len(ws))]
        cpu = cpu_entry(samples, " + ".join(names))
        parity = {"max_err_over_rms": round(max(s["max_err_over_rms"] for s in samples), 6),
                  "bar": BAR_BF16 if w0.dtype == "bf16" else 1e-4,
                  "tokens": sum(s["tokens"] for s in samples),
                  "note": "GPU output against the oracle on the CPU-baseline tokens; RMS over those "
                          "tokens' elements (the test suite compares whole outputs)"}
    fw.free()

    extra, bwd, layer_bwd = {}, None, None
    if not args.no_extra:
        for name in OTHERS:
            if name in names:
                continue
            w = wl.WORKLOADS[name]
            f2 = Forwards([w])
            # Sub-millisecond steps: enough warm-up for the clocks to leave the idle state of
            # the CPU leg before them, and enough steps to average launch jitter.
            e = time_steps(f2, max(args.extra_steps, 20), 30)
            roofs = kernel_rooflines(w, e["kms"][0], f2.fused[0])
            dk = max(roofs, key=lambda k: roofs[k]["ms"])
            entry = {"ms_per_step": round(e["ms_step"], 4),
                     "ms_per_step_flushed": round(e["ms_step_flushed"], 4),
                     "pseudo_tokens_per_s": round(w.B * w.P * w.N / (e["ms_step"] * 1e-3), 1),
                     "roofline": dict(roofs[dk], kernel=dk),
                     "attention": roofs["attention"], "kernel_roofline": roofs,
                     "kernels_ms": {k: round(v, 4) for k, v in e["kms"][0].items()},
                     "mix_fused": f2.fused[0]}
            if not args.no_cpu_baseline:
                s = oracle_sample(f2, 0, 16, 11)
                entry["cpu_baseline"] = cpu_entry([s], name)
                entry["parity_sample_max_err_over_rms"] = round(s["max_err_over_rms"], 6)
            f2.free()
            extra[name] = entry
        bwd = run_attention_backward(wl.WORKLOADS[OTHERS[0]], max(args.extra_steps, 10), 10)
        extra["nexus_inner_causal_b4_l8192_h16"] = run_nexus_inner(4, 8192, 16, 128, "causal",
                                                                   max(args.extra_steps, 10), 5)
        layer_bwd = {n: run_layer_backward(wl.WORKLOADS[n], args.extra_steps, 2) for n in HEADLINE}
        extra["fused_collapse_ab"] = [run_fused_collapse_ab(wl.WORKLOADS[n], 3)
                                      for n in (OTHERS[0], HEADLINE[0])]

    chip = probe_chip()
    if chip is not None:
        chip["copy_gb_s"] = copy_rate()
        chip["sclk_mhz_sysfs_during_timed_steps"] = (round(statistics.median(sclk), 1) if sclk else None)
        if dominant["bound"] == "mfma":
            dominant["frac_of_measured_peak"] = round(dominant["achieved"] / chip["mfma_f16_tflops"], 4)

    pseudo_per_step = sum(w.B * w.P * w.N for w in ws)
    line = {
        "metric": "IHA fwd pseudo-tokens/s + attention TFLOP/s (% of MI355X bf16 MFMA peak)",
        "value": round(pseudo_per_step / (r["ms_step"] * 1e-3), 1), "unit": "pseudo-tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(r["ms_step"], 4),
        "ms_per_step_event_pass": round(r["ms_step_events"], 4),
        "ms_per_step_flushed": round(r["ms_step_flushed"], 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp16-mfma/fp32-acc" if w0.dtype == "bf16" else "f32", "data": "synthetic",
        "config": {"workload": " + ".join(names), "B": B, "N": N, "D": D, "H": H, "d": d, "P": P,
                   "modes": [modes[n]["mask"] for n in names],
                   "window": next((w.window for w in ws if w.mask == 2), None), "input_dtype": w0.dtype,
                   "global_batch": B, "seq_len": N, "parallelism": "none",
                   "pseudo_tokens_per_step": pseudo_per_step},
        "roofline": dominant,
        "attention": {n: modes[n]["kernel_roofline"]["attention"] for n in names},
        "modes": modes,
        "parity": parity,
        "chip": chip,
        "other_workloads": extra,
        "attention_backward": bwd,
        "layer_backward": layer_bwd,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
