"""Benchmark of the fused softmax cross-entropy hot path on one MI355X.

One step is one pass of the whole path over one batch of synthetic input:
  * ce_forward + ce_vjp on bf16 logits [2048 x 151,936] (N(0,1), uniform targets,
    g = 1): the configuration the CE fwd+VJP figure is quoted on;
  * lce_forward on bf16 H [8192 x 4096] ~ N(0,1), W [151,936 x 4096] ~ N(0, 1/D),
    uniform targets: the linear-CE configuration.
After the timed steps, lce_backward (dH, dW of the same linear-CE loss, upstream
gradient U[0.25, 2)) and kl_forward + kl_vjp (fp32 student and teacher logits
[512 x 151,936] ~ N(0, 16), the shape "One barrier short" reproduces its race on; two
copies alternate) are timed on their own loops and reported under parts/rooflines;
they are not part of the step.
Inputs are resident in HBM before the timed region.  Two copies of the logits
alternate between steps (each copy is 622 MB, larger than the 256 MB Infinity Cache,
so no step reads logits cached by the previous one).

Timing: W untimed warm-up steps, then exactly K steps bracketed by
torch.cuda.synchronize(); HIP events on the launch stream around every call give
per-kernel-call durations.  Prints ONE JSON line.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu]
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

CE_ROWS, CE_V = 2048, 151936
KL_ROWS, KL_V = 512, 151936
LCE_N, LCE_D, LCE_V = 8192, 4096, 151936
HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix, published

METRIC = "fused CE fwd+VJP ms & GB/s (% HBM peak); linear-CE fwd TFLOP/s (% MFMA)"

ROOT = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(ROOT, "softmax_cross_entropy_amd", "csrc")

# HBM traffic per launch from rocprofv3 FETCH_SIZE / WRITE_SIZE runs of this script
# (--steps 1 --warmup 0 --calibrate-copy 1024), each scaled by the same counter on a
# copy of known size; see profiles/.  Keyed by the sha256 of the kernel's source file
# and headers at measurement time: a changed kernel reports traffic null until it is measured again.
TRAFFIC = {
    "ce_forward_vjp": {
        "source_sha": "30f4ec33c2551876",
        "bytes": 1290970676
    },
    "ce_forward": {
        "source_sha": "30f4ec33c2551876",
        "bytes": 622591131
    },
    "ce_vjp": {
        "source_sha": "30f4ec33c2551876",
        "bytes": 1244995483
    },
    "lce_forward": {
        "source_sha": "c2ead97c2bc90bde",
        "bytes": 15152087151
    },
    "kl_forward": {
        "source_sha": "8178fcf06dbd3aed",
        "bytes": 622483971
    },
    "kl_vjp": {
        "source_sha": "8178fcf06dbd3aed",
        "bytes": 933636530
    },
    "ce_forward_ex": {
        "source_sha": "9c57c5ac9d01527f",
        "bytes": 622629769
    },
    "ce_vjp_ex": {
        "source_sha": "9c57c5ac9d01527f",
        "bytes": 1206069424
    },
    "ce_forward_probs": {
        "source_sha": "9c57c5ac9d01527f",
        "bytes": 622464816
    },
    "ce_vjp_probs": {
        "source_sha": "9c57c5ac9d01527f",
        "bytes": 933600435
    },
    "js_forward": {
        "source_sha": "f78dc0c5b2112634",
        "bytes": 1224776799
    },
    "js_vjp": {
        "source_sha": "f78dc0c5b2112634",
        "bytes": 936653344
    },
    "lce_backward": {
        "source_sha": "1e37de0f87323df7",
        "bytes": 55428326203
    },
    "ce_forward f32 [1048576 x 8]": {
        "source_sha": "30f4ec33c2551876",
        "bytes": 50504821
    },
    "ce_vjp f32 [1048576 x 8]": {
        "source_sha": "30f4ec33c2551876",
        "bytes": 83947084
    },
    "ce_forward f32 [65536 x 1024] offsets and -inf rows": {
        "source_sha": "30f4ec33c2551876",
        "bytes": 270329035
    },
    "ce_vjp f32 [65536 x 1024] offsets and -inf rows": {
        "source_sha": "30f4ec33c2551876",
        "bytes": 543236176
    },
    "ce_forward f16 [65536 x 1024] offsets and -inf rows": {
        "source_sha": "30f4ec33c2551876",
        "bytes": 135597286
    },
    "ce_vjp f16 [65536 x 1024] offsets and -inf rows": {
        "source_sha": "30f4ec33c2551876",
        "bytes": 271687663
    },
    "ce_forward f32 view [10, 119, 32768][:, :-1] (1180 rows)": {
        "source_sha": "30f4ec33c2551876",
        "bytes": 154859484
    },
    "ce_vjp f32 view [10, 119, 32768][:, :-1] (1180 rows)": {
        "source_sha": "30f4ec33c2551876",
        "bytes": 309565545
    },
    "ce_forward bf16 [8192 x 32000]": {
        "source_sha": "30f4ec33c2551876",
        "bytes": 525190978
    },
    "ce_vjp bf16 [8192 x 32000]": {
        "source_sha": "30f4ec33c2551876",
        "bytes": 1049705504
    },
    "ce_forward f32 [135266304 x 8]": {
        "source_sha": "30f4ec33c2551876",
        "bytes": 6567347952
    },
    "ce_vjp f32 [135266304 x 8]": {
        "source_sha": "30f4ec33c2551876",
        "bytes": 10821186773
    }
}






def source_sha(kernel):
    """sha256 (first 16 hex digits) of the kernel's source file and the two headers its
    code depends on (device helpers; launch plans and the constants kernels are built
    around), and for lce_backward also the source that lays out its chunks."""
    fname = ("lce_kernels.hip" if kernel.startswith("lce") else
             "kl_kernels.hip" if kernel.startswith("kl") else
             "js_kernels.hip" if kernel.startswith("js") else
             "ce_options.hip" if kernel.endswith(("_ex", "_probs")) else "ce_kernels.hip")
    h = hashlib.sha256()
    extra = ("lce_backward.cpp",) if kernel == "lce_backward" else ()
    for f in (fname, "device_common.h", "plan.h") + extra:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def environment(torch):
    """Where the numbers were taken: GPU, ROCm/HIP and torch versions, the source tree."""
    env = {"gpu": None, "arch": None, "hip": getattr(torch.version, "hip", None), "torch": torch.__version__,
           "rocm": None, "git_sha": None, "source_sha256": None}
    try:
        prop = torch.cuda.get_device_properties(0)
        env["gpu"] = prop.name
        env["arch"] = getattr(prop, "gcnArchName", None)
        env["cus"] = prop.multi_processor_count
    except Exception:
        pass
    try:
        with open("/opt/rocm/.info/version") as fh:
            env["rocm"] = fh.read().strip()
    except OSError:
        pass
    try:
        import subprocess
        r = subprocess.run(["git", "-C", ROOT, "rev-parse", "HEAD"], capture_output=True, text=True, timeout=10)
        if r.returncode == 0:
            env["git_sha"] = r.stdout.strip()
    except Exception:
        pass
    # the tree may travel without its git metadata: a digest of the sources that were built
    h = hashlib.sha256()
    for d in (CSRC, os.path.join(ROOT, "include")):
        for f in sorted(os.listdir(d)):
            with open(os.path.join(d, f), "rb") as fh:
                h.update(f.encode() + fh.read())
    with open(os.path.abspath(__file__), "rb") as fh:
        h.update(fh.read())
    env["source_sha256"] = h.hexdigest()[:16]
    return env


def traffic_for(kernel):
    t = TRAFFIC.get(kernel)
    if not t or t.get("source_sha") != source_sha(kernel):
        return None
    return t["bytes"]


def ce_bytes(rows, V, e):
    """Algorithmic HBM bytes per call: forward reads V*e per row and writes loss (4)
    and lse (8), reading the target (4); the VJP reads V*e plus lse, target and g
    (16 per row) and writes V*e."""
    fwd = rows * (V * e + 16)
    vjp = rows * (2 * V * e + 16)
    return fwd, vjp


# the other one-kernel workloads: rows the forward gives 512 lanes (held in registers), and
# short rows on 32 lanes (swept twice)
F_SHAPES = (("bf16 [8192 x 32000]", 8192, 32000, "bf16"), ("f32 [65536 x 1024]", 65536, 1024, "f32"))


def fused_bytes(rows, V, e):
    """Algorithmic HBM bytes of one ce_forward_vjp call: each row is read once (V*e)
    and its gradient written (V*e); per row the target and g are read (8) and the loss
    and lse written (12)."""
    return rows * (2 * V * e + 20)


def kl_bytes(rows, V, e):
    """Algorithmic HBM bytes per call: the forward reads both rows and writes kl (4)
    and the two (m, log s) pairs (16); the VJP reads both rows, the pairs and g (20)
    and writes the student gradient."""
    return rows * (2 * V * e + 20), rows * (3 * V * e + 20)


def js_bytes(rows, V, e):
    """Jensen-Shannon: the terms need both row normalisers first, so the forward reads both
    rows twice (a 1.2 MB fp32 row pair does not stay on chip) and writes js, the two pairs
    and H (24 per row); the VJP reads both rows, the pairs, H and g (24) and writes the
    gradient."""
    return rows * (4 * V * e + 24), rows * (3 * V * e + 24)


def opt_bytes(rows, V, e, ignored=0):
    """Algorithmic HBM bytes per call of the index-target options (smoothing, ignore_index,
    mean): the forward reads the logits and the target and writes loss and lse (16 per
    row; ignored rows too, whose lse is still written); the VJP reads lse and target (12)
    and writes the gradient of every row, and reads the logits of the rows that are not
    ignored (an ignored row's gradient is 0 whatever its logits).  The reduction's second
    read of loss and targets is not counted."""
    return rows * (V * e + 16), rows * (V * e + 12) + (rows - ignored) * V * e


def probs_bytes(rows, V, e):
    """Probability targets: the forward reads logits and targets and writes loss, lse and
    the weight sum (16 per row); the VJP reads both rows, lse and the weight sum (12) and
    writes the gradient."""
    return rows * (2 * V * e + 16), rows * (3 * V * e + 12)


def lce_flops(N, D, V):
    return 2.0 * N * D * V


def cpu_baseline(ce_batch, lce_inputs, lce_rows=32):
    """The float64 oracle, as it stands, on a bounded sample of the same workload."""
    from threadpoolctl import threadpool_info

    from oracle import ce as oce
    from oracle import lce as olce
    from softmax_cross_entropy_amd import inputs

    b = ce_batch
    t0 = time.perf_counter()
    for r0 in range(0, b.rows, 256):
        r1 = min(b.rows, r0 + 256)
        z = oce.decode(b.logits[r0:r1], "bf16")
        _, m, ls = oce.forward(z, b.targets[r0:r1])
        oce.grad(z, b.targets[r0:r1], b.g[r0:r1], m, ls)
    ce_s = time.perf_counter() - t0
    fwd_b, vjp_b = ce_bytes(b.rows, b.V, 2)
    H, W, y = lce_inputs
    rows = np.arange(lce_rows)
    t0 = time.perf_counter()
    olce.forward(H, W, y, rows=rows)
    lce_s = time.perf_counter() - t0
    g_up = np.random.default_rng([5, 0]).uniform(0.25, 2.0, LCE_N)
    W64 = olce.decode_bf16(W)
    t0 = time.perf_counter()
    olce.grad64(olce.decode_bf16(H[rows]), W64, y[rows], g_up[rows])
    lbw_s = time.perf_counter() - t0
    from oracle import kl as okl
    kq, kp, kg = inputs.kl_pair(32, KL_V, "f32", scale=4.0)
    t0 = time.perf_counter()
    zq, zp = kq.astype(np.float64), kp.astype(np.float64)
    okl.forward(zq, zp)
    okl.grad(zq, zp, kg)
    kl_s = time.perf_counter() - t0
    kf_b, kv_b = kl_bytes(32, KL_V, 4)
    from oracle import js as ojs
    t0 = time.perf_counter()
    ojs.forward(zq, zp)
    ojs.grad(zq, zp, kg)
    js_s = time.perf_counter() - t0
    jf_b, jv_b = js_bytes(32, KL_V, 4)
    from oracle import ce_options as oco
    y_ign = b.targets[:32].copy()
    y_ign[::16] = -100
    z = oce.decode(b.logits[:32], "bf16")
    t0 = time.perf_counter()
    oco.forward_index(z, y_ign, 0.1, -100, "mean")
    oco.grad_index(z, y_ign, 1.0, 0.1, -100, "mean")
    opt_s = time.perf_counter() - t0
    of_b, ov_b = opt_bytes(32, b.V, 2, ignored=len(range(0, 32, 16)))
    pt = inputs.prob_targets(32, KL_V, "f32", workload=20, stream=3).astype(np.float64)
    t0 = time.perf_counter()
    oco.forward_probs(zq, pt, 0.1, "mean")
    oco.grad_probs(zq, pt, 1.0, 0.1, "mean")
    probs_s = time.perf_counter() - t0
    pf_b, pv_b = probs_bytes(32, KL_V, 4)
    # the CE oracle at the other workload shapes, on a bounded sample of rows of each
    shapes = {}
    x3, y3 = inputs.strided_view_source()
    for label, (zs, ys) in (
            ("f32 [1048576 x 8], 262,144 rows", (lambda c: (c.logits[: 1 << 18], c.targets[: 1 << 18]))(
                inputs.small_v_rows())),
            ("f32 [65536 x 1024], 8,192 rows", (lambda c: (c.logits[:8192], c.targets[:8192]))(
                inputs.numerics_stress("f32"))),
            ("f32 view [10, 119, 32768][:, :-1], 256 rows",
             (np.ascontiguousarray(x3[:, :-1]).reshape(-1, x3.shape[-1])[:256], inputs.shifted_targets(y3)[:256]))):
        z = oce.decode(zs, "f32")
        t0 = time.perf_counter()
        _, m, ls = oce.forward(z, ys)
        oce.grad(z, ys, np.ones(len(ys)), m, ls)
        sec = time.perf_counter() - t0
        fb, vb = ce_bytes(len(ys), z.shape[1], 4)
        shapes[label] = {"value": (fb + vb) / sec / 1e9, "unit": "GB/s", "cores": 1, "seconds": sec}
    blas = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    return {
        "value": (fwd_b + vjp_b) / ce_s / 1e9,
        "unit": "GB/s",
        "cores": 1,
        "kind": "oracle",
        "sample": f"CE fwd+grad oracle (float64 NumPy, single-threaded) over all {b.rows} rows of the "
                  f"{b.rows}x{b.V} bf16 batch: {ce_s:.2f} s",
        "lce": {"value": lce_flops(lce_rows, LCE_D, LCE_V) / lce_s / 1e12, "unit": "TFLOP/s",
                "cores": blas, "seconds": lce_s,
                "sample": f"lce oracle (float64 BLAS matmul + CE) on {lce_rows} of {LCE_N} rows, "
                          f"all {LCE_V} columns"},
        "ce_options": {"value": (of_b + ov_b) / opt_s / 1e9, "unit": "GB/s", "cores": 1, "seconds": opt_s,
                       "sample": f"options oracle (eps 0.1, ignore_index, mean; float64 NumPy) on 32 of "
                                 f"{b.rows} rows, all {b.V} columns"},
        "js": {"value": (jf_b + jv_b) / js_s / 1e9, "unit": "GB/s", "cores": 1, "seconds": js_s,
               "sample": f"JS fwd+grad oracle (float64 NumPy) on 32 of {KL_ROWS} rows, all {KL_V} columns"},
        "ce_probs": {"value": (pf_b + pv_b) / probs_s / 1e9, "unit": "GB/s", "cores": 1, "seconds": probs_s,
                     "sample": f"probability-target oracle (eps 0.1, mean; float64 NumPy) on 32 of {KL_ROWS} rows, "
                               f"all {KL_V} columns"},
        "shapes": shapes,
        "kl": {"value": (kf_b + kv_b) / kl_s / 1e9, "unit": "GB/s", "cores": 1, "seconds": kl_s,
               "sample": f"KL fwd+grad oracle (float64 NumPy) on 32 of {KL_ROWS} rows, all {KL_V} columns"},
        "lce_backward": {"value": 3 * lce_flops(lce_rows, LCE_D, LCE_V) / lbw_s / 1e12, "unit": "TFLOP/s",
                         "cores": blas, "seconds": lbw_s,
                         "sample": f"lce gradient oracle (float64: logits, dZ, dZ W, dZ^T H) on {lce_rows} "
                                   f"of {LCE_N} rows, all {LCE_V} columns"},
        "host_cores": len(os.sched_getaffinity(0)),
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--parts", default="ce,fused,lce,lbw,kl,js,opt,probs,shapes,ceil",
                    help="comma list of ce, fused (ce_forward_vjp on the ce workload; needs ce), lce, lbw "
                         "(lce_backward), kl (kl_forward + kl_vjp), js (js_forward + "
                         "js_vjp), opt (ce_forward_ex + ce_vjp_ex), probs (ce_forward_probs + ce_vjp_probs), "
                         "shapes (ce_forward + ce_vjp at the small-vocabulary, strided and huge-row shapes), "
                         "ceil (torch's copy rate on the same GPU, beside the HBM specification)")
    ap.add_argument("--bwd-steps", type=int, default=5, help="timed lce_backward calls")
    ap.add_argument("--shape", default=None,
                    help="with shapes: only the shapes whose label contains this text (one shape per "
                         "profiler run keeps its counters apart from the other shapes)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="run one elementwise copy (torch.neg) of MIB MiB fp32 first, so a counter "
                         "profile holds a kernel of known traffic")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path (rows are "
              "independent, so each GPU would run the same kernels on its own share of the rows)",
              file=sys.stderr)
        sys.exit(2)
    parts = set(args.parts.split(","))

    def note(msg):
        # progress on stderr; stdout carries the one JSON line
        print(f"bench: {msg}", file=sys.stderr, flush=True)

    import torch

    from softmax_cross_entropy_amd import abi, inputs

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    abi.lib()

    def up(x, bf16=False):
        t = torch.from_numpy(np.ascontiguousarray(x).view(np.int16) if bf16 else x)
        return (t.view(torch.bfloat16) if bf16 else t).to(dev)

    ce_batch = lce_in = None
    if "ce" in parts:
        ce_batch = inputs.large_vocab(CE_ROWS, CE_V)
        X = [up(ce_batch.logits, True), up(ce_batch.logits, True)]
        T = up(ce_batch.targets)
        G = up(ce_batch.g)
        loss = torch.empty(CE_ROWS, device=dev)
        lse = torch.empty(CE_ROWS, 2, device=dev)
        dX = torch.empty_like(X[0])
    if "lce" in parts:
        lce_in = inputs.linear_ce(LCE_N, LCE_D, LCE_V)
        Hd, Wd, Yd = up(lce_in[0], True), up(lce_in[1], True), up(lce_in[2])
        lloss = torch.empty(LCE_N, device=dev)
        llse = torch.empty(LCE_N, 2, device=dev)
        ws = torch.empty(abi.lce_workspace_size(LCE_N, LCE_D, LCE_V), dtype=torch.uint8, device=dev)

    calib = None
    if args.calibrate_copy > 0:
        n = args.calibrate_copy * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.neg(src, out=dst)
        torch.cuda.synchronize()
        calib = {"kernel": "torch.neg fp32", "bytes_read": n * 4, "bytes_written": n * 4}
        del src, dst

    stream = torch.cuda.current_stream(dev)
    n_ev = 4
    K = args.steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(n_ev)] for _ in range(K)]

    def step(i, events=None):
        if events:
            events[0].record(stream)
        if ce_batch is not None:
            x = X[i % 2]
            abi.ce_forward(x, T, loss=loss, lse=lse)
            if events:
                events[1].record(stream)
            abi.ce_vjp(x, T, lse, G, dlogits=dX)
        if events:
            events[2].record(stream)
        if lce_in is not None:
            abi.lce_forward(Hd, Wd, Yd, loss=lloss, lse=llse, workspace=ws)
        if events:
            events[3].record(stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        step(i, ev[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    def ms(a, b):
        return [ev[i][a].elapsed_time(ev[i][b]) for i in range(K)]

    # The MI355X's 256 MB Infinity Cache sits in front of HBM.  A VJP's gradient writes
    # stay there as dirty lines after the kernel ends, so the next streaming kernel first
    # writes them back.  In the step, lce_forward's reads (15 GB through the cache) do that
    # between one step's VJP and the next step's forward.  Each pair below is timed in two
    # states: 'clean', after a 512 MiB read (outside the timed region) leaves the cache
    # holding clean lines, as in the step; and 'back to back', pairs with nothing between,
    # where every call also writes back the previous call's lines: the steady rate HBM
    # sustains for this kernel alone.
    CLEAN = torch.ones(128 << 20, dtype=torch.float32, device=dev)
    clean_out = torch.empty((), dtype=torch.float32, device=dev)

    def clean_cache():
        torch.sum(CLEAN, dim=0, out=clean_out)

    # Events bracket GPU time only if the timed calls are already queued when the first
    # event runs.  The host side of a call (argument checks, ctypes marshalling) takes tens
    # of microseconds, more than a small batch's kernel, so before each timed region a GPU
    # spin (torch.cuda._sleep) holds the stream while the host queues the events and the
    # calls behind them.  The spin touches no memory: the cache state is unchanged.
    spin_ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    torch.cuda._sleep(1000)
    spin_ev[0].record(stream)
    torch.cuda._sleep(1 << 20)
    spin_ev[1].record(stream)
    torch.cuda.synchronize()
    spin_cycles_per_ms = (1 << 20) / max(spin_ev[0].elapsed_time(spin_ev[1]), 1e-3)

    def hold(ms_):
        torch.cuda._sleep(int(spin_cycles_per_ms * ms_))

    def timed_pair(fwd, vjp, reps=K, pre=None):
        for i in range(3):
            if pre:
                pre()
            fwd(i)
            vjp(i)
        torch.cuda.synchronize()
        pev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(reps)]
        for i in range(reps):
            if pre:
                pre()
            hold(0.5)
            pev[i][0].record(stream)
            fwd(i)
            pev[i][1].record(stream)
            vjp(i)
            pev[i][2].record(stream)
        torch.cuda.synchronize()
        return (float(np.mean([e[0].elapsed_time(e[1]) for e in pev])),
                float(np.mean([e[1].elapsed_time(e[2]) for e in pev])))

    def both_states(fwd, vjp):
        return {"clean": timed_pair(fwd, vjp, pre=clean_cache), "back_to_back": timed_pair(fwd, vjp)}

    def timed_one(fn, reps=K, pre=None):
        for i in range(3):
            if pre:
                pre()
            fn(i)
        torch.cuda.synchronize()
        pev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(reps)]
        for i in range(reps):
            if pre:
                pre()
            hold(0.5)
            pev[i][0].record(stream)
            fn(i)
            pev[i][1].record(stream)
        torch.cuda.synchronize()
        return float(np.mean([e[0].elapsed_time(e[1]) for e in pev]))

    def batch_medians(fn, iters=20, batches=7, runs=3):
        # the pages' method: each run times 7 batches of `iters` back-to-back calls (one
        # pair of events per batch) and keeps the median batch; the runs' medians are given
        # with their median, min and max, and every batch's per-call time
        raw = []
        for _ in range(runs):
            per_batch = []
            for _ in range(batches):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                hold(0.15 * iters)
                e0.record(stream)
                for i in range(iters):
                    fn(i)
                e1.record(stream)
                torch.cuda.synchronize()
                per_batch.append(e0.elapsed_time(e1) / iters)
            raw.append(per_batch)
        med = sorted(sorted(r)[len(r) // 2] for r in raw)
        return {"method": f"median of {runs} runs x (median of {batches} batches x {iters} back-to-back calls)",
                "median_ms": med[len(med) // 2], "min_ms": med[0], "max_ms": med[-1], "run_medians_ms": med,
                "batch_ms": raw}

    ce_b2b = ce_batches = None
    if ce_batch is not None:
        ce_b2b = timed_pair(lambda i: abi.ce_forward(X[i % 2], T, loss=loss, lse=lse),
                            lambda i: abi.ce_vjp(X[i % 2], T, lse, G, dlogits=dX))

        def ce_pair(i):
            abi.ce_forward(X[i % 2], T, loss=loss, lse=lse)
            abi.ce_vjp(X[i % 2], T, lse, G, dlogits=dX)

        ce_batches = batch_medians(ce_pair)
    lce_batches = None
    if lce_in is not None:
        lce_batches = batch_medians(lambda i: abi.lce_forward(Hd, Wd, Yd, loss=lloss, lse=llse, workspace=ws))

    fused_ms = None
    if ce_batch is not None and "fused" in parts:
        note("ce_forward_vjp")

        def fused_call(i):
            abi.ce_forward_vjp(X[i % 2], T, G, loss=loss, lse=lse, dlogits=dX)

        fused_ms = {"clean": timed_one(fused_call, pre=clean_cache), "back_to_back": timed_one(fused_call)}
        # more shapes: bf16 [8192 x 32,000] (rows of 4000 vectors, held by 512-thread
        # workgroups) and fp32 [65,536 x 1024] (rows of 256 vectors on 32 lanes, swept
        # twice); three input copies rotate so no call finds its logits in the Infinity Cache
        fused_ms["shapes"] = []
        for label, f_rows, f_v, f_dt in F_SHAPES:
            sb = inputs.normal_rows(f_rows, f_v, f_dt, workload=90)
            SX = [up(sb.logits, f_dt == "bf16") for _ in range(3)]
            ST2, SG2 = up(sb.targets), up(sb.g)
            s_l, s_s, s_d = torch.empty(f_rows, device=dev), torch.empty(f_rows, 2, device=dev), torch.empty_like(SX[0])
            del sb

            def f2_fused(i):
                abi.ce_forward_vjp(SX[i % 3], ST2, SG2, loss=s_l, lse=s_s, dlogits=s_d)

            def f2_fwd(i):
                abi.ce_forward(SX[i % 3], ST2, loss=s_l, lse=s_s)

            def f2_vjp(i):
                abi.ce_vjp(SX[i % 3], ST2, s_s, SG2, dlogits=s_d)

            fused_ms["shapes"].append((label, f_rows, f_v, 4 if f_dt == "f32" else 2,
                                       {"clean": timed_one(f2_fused, pre=clean_cache),
                                        "back_to_back": timed_one(f2_fused),
                                        "two_calls": both_states(f2_fwd, f2_vjp)}))
            del SX, s_d

    kl_ms = None
    if "kl" in parts:
        note("kl")
        kq, kp, kg = inputs.kl_pair(KL_ROWS, KL_V, "f32", scale=4.0)
        kq2, kp2, _ = inputs.kl_pair(KL_ROWS, KL_V, "f32", scale=4.0, stream=1)
        KQ = [torch.from_numpy(kq).to(dev), torch.from_numpy(kq2).to(dev)]
        KP = [torch.from_numpy(kp).to(dev), torch.from_numpy(kp2).to(dev)]
        KG = torch.from_numpy(kg).to(dev)
        kl_o = torch.empty(KL_ROWS, device=dev)
        lq_o = torch.empty(KL_ROWS, 2, device=dev)
        lp_o = torch.empty(KL_ROWS, 2, device=dev)
        dq_o = torch.empty_like(KQ[0])
        kl_ms = both_states(lambda i: abi.kl_forward(KQ[i % 2], KP[i % 2], kl=kl_o, lse_q=lq_o, lse_p=lp_o),
                            lambda i: abi.kl_vjp(KQ[i % 2], KP[i % 2], lq_o, lp_o, KG, dq=dq_o))
        del KQ, KP, dq_o

    js_ms = None
    if "js" in parts:
        note("js")
        jq, jp, jg = inputs.kl_pair(KL_ROWS, KL_V, "f32", scale=4.0, stream=4)
        jq2, jp2, _ = inputs.kl_pair(KL_ROWS, KL_V, "f32", scale=4.0, stream=5)
        JQ = [torch.from_numpy(jq).to(dev), torch.from_numpy(jq2).to(dev)]
        JP = [torch.from_numpy(jp).to(dev), torch.from_numpy(jp2).to(dev)]
        JG = torch.from_numpy(jg).to(dev)
        j_o = torch.empty(KL_ROWS, device=dev)
        jlq = torch.empty(KL_ROWS, 2, device=dev)
        jlp = torch.empty(KL_ROWS, 2, device=dev)
        jh = torch.empty(KL_ROWS, device=dev)
        jd = torch.empty_like(JQ[0])
        js_ms = both_states(
            lambda i: abi.js_forward(JQ[i % 2], JP[i % 2], js=j_o, lse_q=jlq, lse_p=jlp, hq=jh),
            lambda i: abi.js_vjp(JQ[i % 2], JP[i % 2], jlq, jlp, jh, JG, dq=jd))
        del JQ, JP, jd

    opt_ms = None
    if "opt" in parts and ce_batch is not None:
        note("opt")
        y_ign = ce_batch.targets.copy()
        y_ign[::16] = -100
        TI = up(y_ign)
        o_tot = torch.empty(1, device=dev)
        o_cnt = torch.empty(1, dtype=torch.int64, device=dev)
        o_ws = torch.empty(abi.ce_reduce_workspace_size(), dtype=torch.uint8, device=dev)
        o_g = torch.ones(1, device=dev)
        opt_ms = both_states(
            lambda i: abi.ce_forward_ex(X[i % 2], TI, 0.1, -100, "mean", loss=loss, lse=lse, total=o_tot,
                                        count=o_cnt, workspace=o_ws),
            lambda i: abi.ce_vjp_ex(X[i % 2], TI, lse, o_g, 0.1, -100, "mean", count=o_cnt, dlogits=dX))

    probs_ms = None
    if "probs" in parts:
        note("probs")
        pz = inputs.kl_pair(KL_ROWS, KL_V, "f32", scale=4.0, stream=2)[0]
        PZ = torch.from_numpy(pz).to(dev)
        PT = torch.from_numpy(inputs.prob_targets(KL_ROWS, KL_V, "f32", workload=20, stream=3)).to(dev)
        p_loss = torch.empty(KL_ROWS, device=dev)
        p_lse = torch.empty(KL_ROWS, 2, device=dev)
        p_w = torch.empty(KL_ROWS, device=dev)
        p_tot = torch.empty(1, device=dev)
        p_cnt = torch.empty(1, dtype=torch.int64, device=dev)
        p_ws = torch.empty(abi.ce_reduce_workspace_size(), dtype=torch.uint8, device=dev)
        p_g = torch.ones(1, device=dev)
        p_d = torch.empty_like(PZ)
        probs_ms = both_states(
            lambda i: abi.ce_forward_probs(PZ, PT, 0.1, "mean", loss=p_loss, lse=p_lse, wsum=p_w, total=p_tot,
                                           count=p_cnt, workspace=p_ws),
            lambda i: abi.ce_vjp_probs(PZ, PT, p_lse, p_w, p_g, 0.1, "mean", count=p_cnt, dlogits=p_d))
        del PZ, PT, p_d

    # ce_forward + ce_vjp at the other workload shapes: the small-vocabulary layouts (one
    # lane per row for 8 classes, lane groups for 1024), the strided batch view and the
    # row count past 2**32 threads.  Each shape rotates copies of its input, at least
    # 1 GiB in all, so no input is read again from the 256 MB Infinity Cache.
    shape_ms = []
    if "shapes" in parts:
        def dev_copy(a, dt):
            t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16) if dt == "bf16" else a)
            return (t.view(torch.bfloat16) if dt == "bf16" else t).to(dev)

        def strided():
            x3, y3 = inputs.strided_view_source()
            return x3, "f32", (lambda t: t[:, :-1]), inputs.shifted_targets(y3)

        def plain(make):
            def build():
                b = make()
                return b.logits, b.dtype, (lambda t: t), b.targets
            return build

        shape_list = (
            ("f32 [1048576 x 8]", plain(inputs.small_v_rows)),
            ("f32 [65536 x 1024] offsets and -inf rows", plain(lambda: inputs.numerics_stress("f32"))),
            ("f16 [65536 x 1024] offsets and -inf rows", plain(lambda: inputs.numerics_stress("f16"))),
            ("f32 view [10, 119, 32768][:, :-1] (1180 rows)", strided),
            ("bf16 [8192 x 32000]", plain(lambda: inputs.large_vocab(8192, 32000))),
            ("f32 [135266304 x 8]", plain(inputs.huge_rows)),
        )
        for label, build in shape_list:
            if args.shape and args.shape not in label:
                continue
            note(f"shapes: {label}")
            store, dt, view_of, tgt = build()
            ncopy = max(1, -(-(1 << 30) // store.nbytes))
            views = [view_of(dev_copy(store, dt)) for _ in range(ncopy)]
            v0 = views[0]
            n_rows, V = v0.numel() // v0.shape[-1], v0.shape[-1]
            del store
            ST = torch.from_numpy(tgt).to(dev)
            SG = torch.ones(n_rows, device=dev)
            s_loss = torch.empty(n_rows, device=dev)
            s_lse = torch.empty(n_rows, 2, device=dev)
            s_d = torch.empty(v0.shape, dtype=v0.dtype, device=dev)
            tms = both_states(lambda i: abi.ce_forward(views[i % ncopy], ST, loss=s_loss, lse=s_lse),
                              lambda i: abi.ce_vjp(views[i % ncopy], ST, s_lse, SG, dlogits=s_d))
            shape_ms.append((label, n_rows, V, v0.element_size(), ncopy, tms))
            del views, v0, ST, SG, s_loss, s_lse, s_d
            torch.cuda.empty_cache()

    bwd_ms = None
    if "lbw" in parts and lce_in is not None:
        note("lbw")
        G_up = torch.from_numpy(np.random.default_rng([5, 0]).uniform(0.25, 2.0, LCE_N).astype(np.float32)).to(dev)
        dH = torch.empty(LCE_N, LCE_D, dtype=torch.float32, device=dev)
        dW = torch.empty(LCE_V, LCE_D, dtype=torch.float32, device=dev)
        # the whole vocabulary as one chunk (the workspace holds all of dZ), then chunks of
        # 8192 columns (the least workspace the call accepts): same results, both timed
        bwd_layouts = {}
        for layout, size in (("one_pass", abi.lce_backward_workspace_size_one_pass),
                             ("chunks_8192", abi.lce_backward_workspace_size)):
            bws = torch.empty(size(LCE_N, LCE_D, LCE_V), dtype=torch.uint8, device=dev)
            for _ in range(2):
                abi.lce_backward(Hd, Wd, Yd, llse, G_up, dH=dH, dW=dW, workspace=bws)
            torch.cuda.synchronize()
            bev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                   for _ in range(args.bwd_steps)]
            for e0, e1 in bev:
                e0.record(stream)
                abi.lce_backward(Hd, Wd, Yd, llse, G_up, dH=dH, dW=dW, workspace=bws)
                e1.record(stream)
            torch.cuda.synchronize()
            bwd_layouts[layout] = {"ms": float(np.mean([e0.elapsed_time(e1) for e0, e1 in bev])),
                                   "workspace_bytes": bws.numel()}
            del bws
        bwd_ms = bwd_layouts["one_pass"]["ms"]
        del dH, dW

    # A same-GPU streaming rate beside the 8 TB/s specification: torch's copy of 2 GiB of
    # fp32 (2 GiB read + 2 GiB written), best of 5.  (torch's reductions read well below
    # the HBM rate, so no read-only figure is taken from them.)
    ceiling = None
    if "ceil" in parts:
        note("ceil")
        src = torch.ones(1 << 29, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        t_copy = []
        for i in range(6):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            dst.copy_(src)
            e1.record(stream)
            torch.cuda.synchronize()
            if i:
                t_copy.append(e0.elapsed_time(e1))
        nb = src.numel() * 4
        ceiling = {"copy_GB_s": 2 * nb / (min(t_copy) * 1e-3) / 1e9, "bytes_read": nb, "bytes_written": nb,
                   "method": "torch copy_ of 2 GiB fp32, best of 5"}
        del src, dst

    step_ms = float(np.mean(ms(0, 3)))
    out = {"metric": METRIC, "n_gpus": 1, "steps": K, "warmup": args.warmup, "ms_per_step": step_ms,
           "wall_ms_per_step": wall / K * 1e3, "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "bf16", "data": "synthetic (seeded N(0,1) logits/hidden states, "
           "N(0,1/D) weights, uniform targets)"}
    cfg = {"workload": []}
    parts_out = {}
    rooflines = {}
    def rate(byts, t):
        return byts / (t * 1e-3) / 1e9

    def spread(ts):
        # per-step times of the K timed steps (ms): the value above is their mean
        raw = [float(t) for t in ts]
        ts = sorted(raw)
        return {"median_ms": float(ts[len(ts) // 2]), "min_ms": float(ts[0]), "max_ms": float(ts[-1]),
                "raw_ms": raw}

    def b2b_out(fb, vb, f, v):
        return {"fwd_ms": f, "vjp_ms": v, "ms": f + v, "GB_s": rate(fb + vb, f + v),
                "frac_hbm_peak": rate(fb + vb, f + v) / HBM_PEAK_GBS}

    def hbm_rooflines(names, byts, b2b, other, other_key):
        # the back-to-back time: the rate HBM sustains, deferred cache write-backs included
        for name, nb, t, t2 in zip(names, byts, b2b, other):
            a = rate(nb, t)
            rooflines[name] = {"bound": "hbm", "achieved": a, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                               "frac": a / HBM_PEAK_GBS, "traffic": traffic_for(name), "ms": t,
                               "timing": "back to back", other_key: t2, "algorithmic_bytes": nb}

    if ce_batch is not None:
        fwd_b, vjp_b = ce_bytes(CE_ROWS, CE_V, 2)
        f_ms = float(np.mean(ms(0, 1)))
        v_ms = float(np.mean(ms(1, 2)))
        fv_ms = float(np.mean(ms(0, 2)))
        gbs = rate(fwd_b + vjp_b, fv_ms)
        parts_out["ce_fwd_vjp"] = {"ms": fv_ms, "GB_s": gbs, "frac_hbm_peak": gbs / HBM_PEAK_GBS,
                                   "algorithmic_bytes": fwd_b + vjp_b,
                                   "fwd_ms": f_ms, "fwd_GB_s": rate(fwd_b, f_ms),
                                   "vjp_ms": v_ms, "vjp_GB_s": rate(vjp_b, v_ms),
                                   "per_step": spread(ms(0, 2)),
                                   "back_to_back": b2b_out(fwd_b, vjp_b, *ce_b2b),
                                   "batches": dict(ce_batches, GB_s=rate(fwd_b + vjp_b, ce_batches["median_ms"]))}
        hbm_rooflines(("ce_forward", "ce_vjp"), (fwd_b, vjp_b), ce_b2b, (f_ms, v_ms), "ms_in_step")
        cfg["workload"].append(f"ce_forward+ce_vjp bf16 [{CE_ROWS} x {CE_V}]")
        cfg["ce"] = {"rows": CE_ROWS, "V": CE_V, "dtype": "bf16"}
        out["value"] = gbs
        out["unit"] = "GB/s"
        if fused_ms is not None:
            ub = fused_bytes(CE_ROWS, CE_V, 2)
            tc, tb = fused_ms["clean"], fused_ms["back_to_back"]
            parts_out["ce_forward_vjp"] = {
                "ms": tc, "GB_s": rate(ub, tc), "frac_hbm_peak": rate(ub, tc) / HBM_PEAK_GBS,
                "algorithmic_bytes": ub, "in_step": False, "cache": "clean",
                "vs_two_calls_in_step": fv_ms / tc,
                "back_to_back": {"ms": tb, "GB_s": rate(ub, tb), "frac_hbm_peak": rate(ub, tb) / HBM_PEAK_GBS,
                                 "vs_two_calls": (ce_b2b[0] + ce_b2b[1]) / tb},
                "note": "one kernel for a g known before the forward: each row read from HBM once"}
            for label, f_rows, f_v, f_e, f2 in fused_ms["shapes"]:
                ub2 = fused_bytes(f_rows, f_v, f_e)
                two_c, two_b = sum(f2["two_calls"]["clean"]), sum(f2["two_calls"]["back_to_back"])
                parts_out["ce_forward_vjp"][label] = {
                    "ms": f2["clean"], "GB_s": rate(ub2, f2["clean"]), "algorithmic_bytes": ub2,
                    "two_calls_ms": two_c, "vs_two_calls": two_c / f2["clean"],
                    "back_to_back": {"ms": f2["back_to_back"], "GB_s": rate(ub2, f2["back_to_back"]),
                                     "two_calls_ms": two_b, "vs_two_calls": two_b / f2["back_to_back"]}}
            a = rate(ub, tb)
            rooflines["ce_forward_vjp"] = {"bound": "hbm", "achieved": a, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                           "frac": a / HBM_PEAK_GBS, "traffic": traffic_for("ce_forward_vjp"),
                                           "ms": tb, "timing": "back to back", "ms_clean_cache": tc,
                                           "algorithmic_bytes": ub}
    if lce_in is not None:
        l_ms = float(np.mean(ms(2, 3)))
        fl = lce_flops(LCE_N, LCE_D, LCE_V)
        tf = fl / (l_ms * 1e-3) / 1e12
        parts_out["lce_forward"] = {"ms": l_ms, "TFLOP_s": tf, "frac_mfma_bf16_peak": tf / MFMA_BF16_PEAK_TFLOPS,
                                    "flop": fl, "per_step": spread(ms(2, 3)),
                                    "batches": dict(lce_batches,
                                                    TFLOP_s=fl / (lce_batches["median_ms"] * 1e-3) / 1e12)}
        rooflines["lce_forward"] = {"bound": "mfma", "achieved": tf, "peak": MFMA_BF16_PEAK_TFLOPS,
                                    "unit": "TFLOP/s", "frac": tf / MFMA_BF16_PEAK_TFLOPS,
                                    "traffic": traffic_for("lce_forward"),
                                    "ms": l_ms, "algorithmic_flop": fl,
                                    "kernels": "lce_tile<kTileFwd> + lce_merge (one lce_forward call)",
                                    "traffic_note": "FETCH_SIZE counts L2 fills from beyond each XCD's L2 (Infinity "
                                                    "Cache or HBM): with 32 tiles of 256 x 256 in flight per XCD, each "
                                                    "W tile is filled once per XCD and each H tile once per 4 x 8 "
                                                    "super-block, 14.99 GB by the tile order; H and W are 1.31 GB"}
        cfg["workload"].append(f"lce_forward bf16 N={LCE_N} D={LCE_D} V={LCE_V}")
        cfg["lce"] = {"N": LCE_N, "D": LCE_D, "V": LCE_V, "dtype": "bf16 in, fp32 accumulate"}
        if "value" not in out:
            out["value"] = tf
            out["unit"] = "TFLOP/s"
    # ce_forward, ce_vjp, lce_forward: the kernels of the timed step
    step_kernels = [k for k in rooflines if k != "ce_forward_vjp"]
    if bwd_ms is not None:
        fl = 3 * lce_flops(LCE_N, LCE_D, LCE_V)
        tf = fl / (bwd_ms * 1e-3) / 1e12
        ch = bwd_layouts["chunks_8192"]
        parts_out["lce_backward"] = {"ms": bwd_ms, "TFLOP_s": tf, "frac_mfma_bf16_peak": tf / MFMA_BF16_PEAK_TFLOPS,
                                     "flop": fl, "calls": args.bwd_steps, "in_step": False,
                                     "layout": "one chunk over the whole vocabulary",
                                     "workspace_bytes": bwd_layouts["one_pass"]["workspace_bytes"],
                                     "chunks_8192": {"ms": ch["ms"], "TFLOP_s": fl / (ch["ms"] * 1e-3) / 1e12,
                                                     "workspace_bytes": ch["workspace_bytes"],
                                                     "note": "the least workspace the call accepts; same results"}}
        rooflines["lce_backward"] = {"bound": "mfma", "achieved": tf, "peak": MFMA_BF16_PEAK_TFLOPS,
                                     "unit": "TFLOP/s", "frac": tf / MFMA_BF16_PEAK_TFLOPS,
                                     "traffic": traffic_for("lce_backward"),
                                     "ms": bwd_ms, "algorithmic_flop": fl,
                                     "kernels": "H transposed once; the whole vocabulary as one chunk: lce_tile "
                                                "(dZ epilogue, and W transposed from its LDS stages), one lce_tile "
                                                "launch of both products (one lce_backward call)",
                                     "traffic_note": "FETCH_SIZE + WRITE_SIZE over the call's launches; writes "
                                                     "two dZ copies and W transposed, dH once, dW, H transposed"}
        cfg["lce_backward"] = {"N": LCE_N, "D": LCE_D, "V": LCE_V, "out": "fp32 dH, dW", "timed": "apart",
                               "workspace": "one chunk over the whole vocabulary"}
    for key, tms, (fb, vb), names, cfgv in (
            ("kl_fwd_vjp", kl_ms, kl_bytes(KL_ROWS, KL_V, 4), ("kl_forward", "kl_vjp"),
             {"rows": KL_ROWS, "V": KL_V, "dtype": "f32", "scale": 4.0, "timed": "apart"}),
            ("js_fwd_vjp", js_ms, js_bytes(KL_ROWS, KL_V, 4), ("js_forward", "js_vjp"),
             {"rows": KL_ROWS, "V": KL_V, "dtype": "f32", "scale": 4.0, "timed": "apart"}),
            ("ce_options", opt_ms, opt_bytes(CE_ROWS, CE_V, 2, ignored=len(range(0, CE_ROWS, 16))),
             ("ce_forward_ex", "ce_vjp_ex"),
             {"rows": CE_ROWS, "V": CE_V, "dtype": "bf16", "label_smoothing": 0.1, "ignore_index": "every 16th row",
              "reduction": "mean", "timed": "apart"}),
            ("ce_probs", probs_ms, probs_bytes(KL_ROWS, KL_V, 4), ("ce_forward_probs", "ce_vjp_probs"),
             {"rows": KL_ROWS, "V": KL_V, "dtype": "f32", "targets": "U[0,1) rows normalised to 1",
              "label_smoothing": 0.1, "reduction": "mean", "timed": "apart"})):
        if tms is None:
            continue
        f, v = tms["clean"]
        parts_out[key] = {"ms": f + v, "GB_s": rate(fb + vb, f + v),
                          "frac_hbm_peak": rate(fb + vb, f + v) / HBM_PEAK_GBS,
                          "algorithmic_bytes": fb + vb, "fwd_ms": f, "vjp_ms": v, "in_step": False,
                          "cache": "clean", "back_to_back": b2b_out(fb, vb, *tms["back_to_back"])}
        hbm_rooflines(names, (fb, vb), tms["back_to_back"], (f, v), "ms_clean_cache")
        cfg[key] = cfgv
    if shape_ms:
        shapes_out = {}
        for label, n_rows, V, e, ncopy, tms in shape_ms:
            fb, vb = ce_bytes(n_rows, V, e)
            f, v = tms["clean"]
            shapes_out[label] = {"rows": n_rows, "V": V, "ms": f + v, "GB_s": rate(fb + vb, f + v),
                                 "frac_hbm_peak": rate(fb + vb, f + v) / HBM_PEAK_GBS,
                                 "algorithmic_bytes": fb + vb, "fwd_ms": f, "vjp_ms": v, "input_copies": ncopy,
                                 "cache": "clean", "back_to_back": b2b_out(fb, vb, *tms["back_to_back"])}
            for name, nb, t, t2 in (("ce_forward", fb, tms["back_to_back"][0], f),
                                    ("ce_vjp", vb, tms["back_to_back"][1], v)):
                a = rate(nb, t)
                rooflines[f"{name} {label}"] = {"bound": "hbm", "achieved": a, "peak": HBM_PEAK_GBS,
                                                "unit": "GB/s", "frac": a / HBM_PEAK_GBS,
                                                "traffic": traffic_for(f"{name} {label}"),
                                                "ms": t, "timing": "back to back", "ms_clean_cache": t2,
                                                "algorithmic_bytes": nb}
        parts_out["shapes"] = shapes_out
        cfg["shapes"] = {"timed": "apart", "g": 1.0, "shapes": [x[0] for x in shape_ms]}
    cfg["workload"] = " + ".join(cfg["workload"])
    cfg["timing"] = ("CE parts: inside the step (after the previous step's lce_forward); parts timed apart: each "
                     "fwd+VJP pair after a 512 MiB read that leaves the Infinity Cache clean, as in the step, "
                     "and again back to back (each call also writes back the previous call's cached "
                     "gradient lines); HBM rooflines: the back-to-back times; every timed region of the "
                     "parts starts behind a GPU spin that holds the stream until the host has queued it, so "
                     "the events measure GPU time, not the host's launch cost")
    out["config"] = cfg
    out["parts"] = parts_out
    # the dominant kernel of the step by time (the parts timed apart count only without a step)
    pool = step_kernels or list(rooflines)
    dom = max(pool, key=lambda k: rooflines[k]["ms"])
    out["roofline"] = dict(rooflines[dom], kernel=dom)
    out.setdefault("value", None)
    out.setdefault("unit", None)
    if ceiling:
        for r in rooflines.values():
            if r["bound"] == "hbm":
                r["vs_torch_copy"] = r["achieved"] / ceiling["copy_GB_s"]
    out["rooflines"] = rooflines
    out["same_gpu_copy"] = ceiling
    out["env"] = environment(torch)
    if calib:
        out["calibration"] = calib
    if not args.no_cpu and ce_batch is not None and lce_in is not None:
        out["cpu_baseline"] = cpu_baseline(ce_batch, lce_in)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
