"""Throughput of the GMA forward mixer on one MI355X.

A step is one call of the full forward (parameter prep, segment aggregates, segment scan and
the chunked causal output pass) over one batch of synthetic inputs already resident in HBM.
Default workload: causal, bf16 storage / fp32 accumulation, B=1, H=16, N=65536, d_r=128,
K=128, d_v=128.  Prints one JSON line.

With --backward a step is one call of the backward instead (forward recompute and every
gradient, from a seeded dL/dO); its line carries the whole step against the peak of the matrix
cores its products run on (bf16 with split operands for bf16 storage, fp32 for fp32 storage).

The forward line also carries `copy_reference`: the rate a plain 1 GiB device copy sustains on the
same GPU (and, under `read_only`, the rate of the library's plain 1 GiB read probe), beside the
rate at which the step moves its measured HBM traffic; and `exp2_reference`: the
measured rate of the hardware exponential and the time the step's 2 K exponentials per token-head
take at it.

With --decode it times one-token causal decode steps at the workload's shape instead (mixture
from the raw parameters every step, and prepared once), and prints their latency.  With
--responsibilities it times gma_responsibilities on the workload's K_X against the HBM roof of its
own bytes (read the rows, write Gamma in fp32).

    python bench.py [--steps K] [--warmup W] [--workload I] [--backward | --decode | --responsibilities] [--no-cpu-baseline]
"""
import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "f32": 157.3}   # dense matrix peaks
METRIC = "GMA fwd tokens/sec (causal, N=64K, K=128) + % of HBM/MFMA roofline"
METRIC_BWD = "GMA backward tokens/sec (causal, N=64K, K=128) + % of matrix-core roofline"
# the same measurements at the other workloads, which the config names
METRIC_OTHER = "GMA fwd tokens/sec + % of HBM/MFMA roofline"
METRIC_BWD_OTHER = "GMA backward tokens/sec + % of matrix-core roofline"
DEFAULT_WORKLOAD = 3
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


# sources of the forward path's kernels and their launches (the backward and decode kernels and the
# exponential-rate probe live in files of their own, which the forward's code does not include)
_OTHER_PATHS = ("gma_backward", "gma_decode", "gma_probe")


def kernel_source_hash(backward: bool = False) -> str:
    """Hash of the sources that the timed path's kernels are built and launched from."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "gaussian_mixture_token_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        if not backward and name.startswith(_OTHER_PATHS):
            continue
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def algorithmic_bytes_per_token_head(w) -> int:
    # read Q_X, K_X, V once and write O once
    es = 2 if w.dtype == "bf16" else 4
    return es * (2 * w.d_route + 2 * w.d_value)


def algorithmic_flops_per_token_head(w) -> int:
    # logits of Q and K: 2 * (2 d_r) * K * 2; write Gamma_K^T V and read Gamma_Q Vt: 2 * 2 K d_v
    return 8 * w.n_comp * w.d_route + 4 * w.n_comp * w.d_value


def kernel_work_per_token_head(w, kernel: str):
    """Algorithmic (bytes, flops) per token-head of one forward kernel: the bytes the path charges it and
    the flops of the method it performs.

    causal_output: the path's bytes (it reads Q_X, V and the stored Gamma_K tiles, the size of K_X when
    K = d_r, and writes O); flops of the Q-side logits (4 K d_r), the read (2 K d_v) and the running
    state update (2 K d_v) -- the K-side logits run in the aggregate pass.  segment_aggregate reads K_X
    and V (K-side logits, write); bidir_output reads Q_X and writes O (Q-side logits, read)."""
    es = 2 if w.dtype == "bf16" else 4
    if kernel == "segment_aggregate":
        return es * (w.d_route + w.d_value), 4 * w.n_comp * w.d_route + 2 * w.n_comp * w.d_value
    if kernel == "bidir_output":
        return es * (w.d_route + w.d_value), 4 * w.n_comp * w.d_route + 2 * w.n_comp * w.d_value
    return algorithmic_bytes_per_token_head(w), 4 * w.n_comp * w.d_route + 4 * w.n_comp * w.d_value


def backward_bytes_per_token_head(w) -> int:
    # read Q_X, K_X, V, dL/dO; write dQ_X, dK_X, dV
    es = 2 if w.dtype == "bf16" else 4
    return es * (4 * w.d_route + 3 * w.d_value)


def backward_flops_per_token_head(w) -> int:
    # the forward's contractions again, then: dGamma_Q = Vt g + Z h and the sums R = Gamma_Q^T g
    # (2 K d_v each), dGamma_K = R v and dV = R^T gamma_K (2 K d_v each), and per side
    # dl [mu/s | 1/s] for dX and dl^T [x | x^2] for the parameters (4 K d_r each)
    return algorithmic_flops_per_token_head(w) + 8 * w.n_comp * w.d_value + 16 * w.n_comp * w.d_route


def load_traffic(workload_name: str, kernel: str, src_hash: str):
    """HBM bytes per launch (reads + writes) of `kernel` from the committed rocprofv3 counter runs
    (FETCH_SIZE and WRITE_SIZE scaled by a copy-kernel calibration), or None if they were taken on a
    different kernel source."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    ent = t.get(workload_name, {}).get(kernel)
    if not ent or ent.get("source_hash") != src_hash:
        return None
    return ent.get("bytes_per_launch")


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def step_traffic(w, kernels, src_hash: str):
    """Measured HBM bytes of one whole step: each kernel's counter bytes per launch times its launches
    per step, or None unless every kernel of the step has counters for the current source."""
    total = 0.0
    for name, k in kernels.items():
        b = load_traffic(w.name, name, src_hash)
        if b is None:
            return None
        total += b * k["launches_per_step"]
    return total


def cpu_baseline_backward(w, heads, dout):
    import oracle
    from gaussian_mixture_token_amd import make_inputs
    inp = make_inputs(w, heads=heads)
    oracle.build(force=False)
    threads = oracle.max_threads()
    t0 = time.perf_counter()
    oracle.backward(inp["qx"], inp["kx"], inp["v"], inp["mu"], inp["raw_var"], inp["prior_logits"], dout,
                    eps=w.eps, causal=w.causal)
    dt = time.perf_counter() - t0
    token_heads = w.batch * len(heads) * w.seq_len
    return {"value": token_heads / dt / w.heads, "unit": "tokens/s", "cores": min(threads, w.batch * len(heads)),
            "kind": "oracle", "cpu_model": cpu_model(),
            "sample": "%d of %d heads, full N=%d, %s fp64 oracle backward (threads over (batch, head)), %.1f s wall" %
                      (len(heads), w.heads, w.seq_len, "causal" if w.causal else "bidirectional", dt)}


def cpu_baseline(w, heads):
    import oracle
    sub_w = w
    from gaussian_mixture_token_amd import make_inputs
    inp = make_inputs(sub_w, heads=heads)
    oracle.build(force=False)
    threads = oracle.max_threads()
    t0 = time.perf_counter()
    oracle.forward(inp["qx"], inp["kx"], inp["v"], inp["mu"], inp["raw_var"], inp["prior_logits"],
                   eps=w.eps, causal=w.causal)
    dt = time.perf_counter() - t0
    token_heads = w.batch * len(heads) * w.seq_len
    return {"value": token_heads / dt / w.heads, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "cpu_model": cpu_model(), "sample": "%d of %d heads, full N=%d, %s fp64 oracle, %.1f s wall" %
                      (len(heads), w.heads, w.seq_len, "causal" if w.causal else "bidirectional", dt)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", type=int, default=DEFAULT_WORKLOAD)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-heads", type=int, default=4)
    ap.add_argument("--backward", action="store_true", help="time the backward pass instead of the forward")
    ap.add_argument("--decode", action="store_true",
                    help="time one-token causal decode steps (raw and prepared mixture) at the workload's B, H, "
                         "d_r, K, d_v instead of the forward")
    ap.add_argument("--responsibilities", action="store_true",
                    help="time gma_responsibilities (Gamma of every K_X row, fp32) at the workload's shape instead "
                         "of the forward, against the HBM roof of its own bytes")
    ap.add_argument("--rounds", type=int, default=None,
                    help="launch the causal pass in this many rounds over the sequence (GMA_CAUSAL_ROUNDS; "
                         "a measured-slower schedule kept for comparison)")
    ap.add_argument("--recompute", action="store_true",
                    help="causal bf16: pass a workspace without room for the stored Gamma_K tiles, so the output "
                         "pass recomputes Gamma_K from K_X (the other schedule of the same path, for comparison)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run a plain elementwise copy of 1 GiB (read 1 GiB, write 1 GiB) and exit; "
                         "its FETCH_SIZE / WRITE_SIZE counters calibrate the traffic figures")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: measures one GPU only; the library has no multi-GPU path "
              "(each (batch, head) or sequence shard would run the same single-GPU path).", file=sys.stderr)
        sys.exit(2)

    if args.rounds is not None:
        os.environ["GMA_CAUSAL_ROUNDS"] = str(args.rounds)
    import torch
    import gaussian_mixture_token_amd as gma
    from gaussian_mixture_token_amd import _lib

    dev = torch.device("cuda:0")
    if args.copy_calibration:
        x = torch.ones(1 << 28, dtype=torch.float32, device=dev)   # 1 GiB
        y = torch.empty_like(x)
        flush = torch.empty(1 << 29, dtype=torch.float32, device=dev)   # 2 GiB, evicts the 256 MB last-level cache
        for _ in range(max(args.steps, 1)):
            flush.fill_(0.0)
            torch.mul(x, 1.0, out=y)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": x.numel() * 4, "copy_calibration_bytes_written": y.numel() * 4,
                          "launches": max(args.steps, 1)}), flush=True)
        return
    lib = _lib.load()
    w = gma.workload(args.workload)
    print("bench: workload %s" % w.name, file=sys.stderr, flush=True)
    if args.decode:
        decode_line(args, w, gma, dev)
        return
    if args.responsibilities:
        resp_line(args, w, gma, dev, lib)
        return
    inp = gma.make_inputs(w)
    t = {k: v.to(dev) for k, v in inp.items()}
    del inp
    out = torch.empty(w.batch, w.heads, w.seq_len, w.d_value, dtype=w.torch_dtype, device=dev)
    prob = gma.problem(w.batch, w.heads, w.seq_len, w.d_route, w.n_comp, w.d_value, w.torch_dtype, w.eps)
    op = _lib.GMA_OP_FORWARD_CAUSAL if w.causal else _lib.GMA_OP_FORWARD_BIDIR
    ws_bytes = gma.workspace_size(prob, op)
    if args.recompute:
        ws_bytes -= 1   # one byte short of the tiles' room: the library takes the recompute schedule
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)

    def step():
        gma.forward(t["qx"], t["kx"], t["v"], t["mu"], t["raw_var"], t["prior_logits"], eps=w.eps,
                    causal=w.causal, out=out, workspace=ws)

    if args.backward:
        del out, ws
        dout = gma.make_dout(w).to(dev)
        grads = {"dqx": torch.empty_like(t["qx"]), "dkx": torch.empty_like(t["kx"]), "dv": torch.empty_like(t["v"]),
                 "dmu": torch.empty_like(t["mu"]), "draw_var": torch.empty_like(t["raw_var"]),
                 "dprior_logits": torch.empty_like(t["prior_logits"])}
        bop = _lib.GMA_OP_BACKWARD_CAUSAL if w.causal else _lib.GMA_OP_BACKWARD_BIDIR
        ws = torch.empty(gma.workspace_size(prob, bop), dtype=torch.uint8, device=dev)

        def step():   # noqa: F811
            gma.backward(t["qx"], t["kx"], t["v"], t["mu"], t["raw_var"], t["prior_logits"], dout, eps=w.eps,
                         causal=w.causal, workspace=ws, grads=grads)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    print("bench: warmup done", file=sys.stderr, flush=True)

    # timed region 1: whole steps
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    e0.record()
    for _ in range(args.steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms = e0.elapsed_time(e1)
    ms_per_step = ms / args.steps
    tokens = w.batch * w.seq_len
    value = tokens / (ms_per_step / 1e3)
    print("bench: %.3f ms/step (wall %.3f s)" % (ms_per_step, wall), file=sys.stderr, flush=True)

    # timed region 3: isolated single steps, each bracketed by its own events and followed by a
    # synchronize. "cold": a 512 MiB fill before each step evicts the last-level cache; "warm": the
    # same step run once untimed before each timed one. Median and 10th / 90th percentiles of each.
    flush = torch.empty(1 << 27, dtype=torch.float32, device=dev)
    iso = {"cold": [], "warm": []}
    for _ in range(max(args.steps, 10)):
        for kind in ("cold", "warm"):
            if kind == "cold":
                flush.fill_(1.0)
            else:
                step()
            a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a0.record()
            step()
            a1.record()
            torch.cuda.synchronize()
            iso[kind].append(a0.elapsed_time(a1))
    del flush
    step_isolated = {"flush_bytes_before_cold_steps": 1 << 29, "steps": max(args.steps, 10)}
    for kind, ts in iso.items():
        ts.sort()
        for name, f in (("median_ms", 0.5), ("p10_ms", 0.1), ("p90_ms", 0.9)):
            step_isolated["%s_%s" % (kind, name)] = ts[min(len(ts) - 1, int(f * (len(ts) - 1) + 0.5))]

    # timed region 2: the same steps with per-kernel HIP events on the launch stream
    lib.gma_timing_enable(1)
    for k in range(lib.gma_kernel_count()):
        lib.gma_timing_read(k, ctypes_double(), ctypes_int64())
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    lib.gma_timing_enable(0)
    kernels = {}
    for k in range(lib.gma_kernel_count()):
        tot, n = ctypes_double(), ctypes_int64()
        _lib.check(lib.gma_timing_read(k, tot, n))
        if n.value:
            kernels[lib.gma_kernel_name(k).decode()] = {"avg_us": 1e3 * tot.value / n.value, "launches": n.value,
                                                        "launches_per_step": n.value / args.steps}
    T = w.batch * w.heads * w.seq_len
    if args.backward:
        bwd_line(args, w, value, ms_per_step, kernels, T, dout, step_isolated)
        return
    src_hash = kernel_source_hash()
    # The roofline of the step: the path's algorithmic bytes and flops (read Q_X, K_X, V once, write O
    # once; logits of both sides, write and read) over the sustained time of back-to-back whole steps
    # (timed region 1, events on the launch stream).  `traffic`: the HBM bytes the step's kernels move,
    # from the committed counter runs of the same source.
    step_s = ms_per_step * 1e-3
    path_bytes = algorithmic_bytes_per_token_head(w) * T
    path_flops = algorithmic_flops_per_token_head(w) * T
    hbm_frac = path_bytes / step_s / 1e9 / HBM_PEAK_GBS
    mfma_frac = path_flops / step_s / 1e12 / MFMA_PEAK_TFLOPS[w.dtype]
    traffic = step_traffic(w, kernels, src_hash)
    if hbm_frac >= mfma_frac:
        roof = {"bound": "hbm", "achieved": path_bytes / step_s / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": hbm_frac, "traffic": traffic}
    else:
        roof = {"bound": "mfma", "achieved": path_flops / step_s / 1e12, "peak": MFMA_PEAK_TFLOPS[w.dtype],
                "unit": "TFLOP/s", "frac": mfma_frac, "traffic": traffic}
    roof.update({"kernel": "whole step (%s, back to back)" % ", ".join(kernels), "time_us": ms_per_step * 1e3,
                 "algorithmic_bytes_per_step": path_bytes, "algorithmic_flops_per_step": path_flops,
                 "hbm_frac": hbm_frac, "mfma_frac": mfma_frac,
                 "traffic_over_algorithmic": None if traffic is None else traffic / path_bytes})
    # The longest kernel alone, timed in region 2 (a HIP event pair around every launch): lighter duty
    # than back-to-back steps (the event packets leave gaps between kernels), so its fractions are an
    # upper bound on what the kernel sustains inside the step.
    dominant = max(kernels, key=lambda k: kernels[k]["avg_us"])
    avg_s = kernels[dominant]["avg_us"] * 1e-6
    kb, kf = kernel_work_per_token_head(w, dominant)
    dom = {"kernel": dominant, "avg_us": kernels[dominant]["avg_us"], "timing": "HIP event pair per launch",
           "algorithmic_bytes_per_launch": kb * T, "algorithmic_flops_per_launch": kf * T,
           "hbm_frac": kb * T / avg_s / 1e9 / HBM_PEAK_GBS,
           "mfma_frac": kf * T / avg_s / 1e12 / MFMA_PEAK_TFLOPS[w.dtype],
           "traffic": load_traffic(w.name, dominant, src_hash)}

    exp_ref = exp2_reference(lib, w, T, step_s)
    copy_gbs = copy_reference(dev)
    read_gbs = read_reference(dev)
    copy_ref = {"kernel": "torch copy_ of 1 GiB fp32 into 1 GiB, 20 back to back", "gbs": copy_gbs,
                "frac_of_peak": copy_gbs / HBM_PEAK_GBS,
                "read_only": {"kernel": "gma_probe_read_rate over 1 GiB (plain 16-byte loads), 10 back to back",
                              "gbs": read_gbs,
                              "frac_of_peak": read_gbs / HBM_PEAK_GBS},
                "step_traffic_gbs": None if traffic is None else traffic / step_s / 1e9,
                "step_traffic_over_copy": None if traffic is None else traffic / step_s / 1e9 / copy_gbs}

    cpu = None
    if not args.no_cpu_baseline:
        print("bench: cpu baseline (oracle)", file=sys.stderr, flush=True)
        heads = list(range(min(args.cpu_heads, w.heads)))
        cpu = cpu_baseline(w, heads)

    line = {
        "metric": METRIC if args.workload == DEFAULT_WORKLOAD else METRIC_OTHER,
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded N(0,1) inputs, N(0,1) means, U(-1,1) raw variances, N(0,0.5^2) prior logits)",
        "config": {"workload": w.name, "mode": "causal" if w.causal else "bidirectional", "batch": w.batch,
                   "heads": w.heads, "seq_len": w.seq_len, "d_route": w.d_route, "n_comp": w.n_comp,
                   "d_value": w.d_value, "eps": w.eps, "global_batch": w.batch, "parallelism": "single GPU",
                   "schedule": ("recompute Gamma_K" if args.recompute else "default")
                               + ("" if args.rounds is None else ", %d rounds" % args.rounds)},
        "roofline": roof,
        "dominant_kernel": dom,
        "copy_reference": copy_ref,
        "exp2_reference": exp_ref,
        "step_isolated": step_isolated,
        "kernels": kernels,
        "cpu_baseline": cpu,
        "source_hash": src_hash,
    }
    print(json.dumps(line), flush=True)


def copy_reference(dev, steps: int = 20) -> float:
    """GB/s of a plain device copy of 1 GiB into 1 GiB (torch's copy kernel), back to back on the current
    stream after three untimed copies: the HBM rate an ordinary streaming kernel sustains on this GPU
    next to the published peak, as context for the rate at which the step moves its own traffic."""
    import torch
    x = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    y = torch.empty_like(x)
    for _ in range(3):
        y.copy_(x)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        y.copy_(x)
    e1.record()
    torch.cuda.synchronize()
    gbs = steps * 2 * x.numel() * 4 / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del x, y
    return gbs


def read_reference(dev) -> float:
    """GB/s of the library's read-rate probe (gma_probe_read_rate: a plain grid-stride kernel of 16-byte
    loads, ten launches back to back) over 1 GiB: the rate a kernel that only reads sustains on this GPU,
    as context for passes that read far more than they write."""
    import torch
    from gaussian_mixture_token_amd import _lib
    lib = _lib.load()
    x = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    rate = ctypes.c_double(0.0)
    _lib.check(lib.gma_probe_read_rate(ctypes.c_void_p(x.data_ptr()), ctypes.c_size_t(x.numel() * 4),
                                       ctypes.byref(rate), None))
    del x
    return rate.value / 1e9


EXP2_PEAK_PER_S = 256 * 4 * 16 / 4 * 2.4e9   # CUs x SIMDs x lanes at a quarter of the full rate x clock


def exp2_reference(lib, w, T, step_s):
    """The measured rate of the hardware exponential (gma_probe_exp2_rate) beside the unit-count estimate,
    and the time the step's 2 K exponentials per token-head (the softmax of both posteriors) would take at
    it: the vector-unit floor of the step, next to its HBM and matrix-core floors."""
    import ctypes
    from gaussian_mixture_token_amd import _lib
    rate = ctypes.c_double()
    _lib.check(lib.gma_probe_exp2_rate(ctypes.byref(rate), None))
    exps = 2 * w.n_comp * T
    return {"exp2_per_s": rate.value, "estimate_per_s": EXP2_PEAK_PER_S, "exps_per_step": exps,
            "floor_us": exps / rate.value * 1e6 if rate.value > 0 else None,
            "frac_of_step": exps / rate.value / step_s if rate.value > 0 else None}


def bwd_line(args, w, value, ms_per_step, kernels, T, dout, step_isolated):
    """The backward's JSON line: the whole step against the peak of the matrix cores its products run on
    (bf16 storage: the bf16 matrix cores, each fp32 operand split into bf16 hi + lo, so about three
    MFMAs per algorithmic product; fp32 storage: the fp32 matrix cores) and, for reference, against the
    fp32 matrix-core peak and HBM."""
    step_s = ms_per_step * 1e-3
    flops = backward_flops_per_token_head(w) * T
    nbytes = backward_bytes_per_token_head(w) * T
    units = "bf16" if w.dtype == "bf16" else "f32"
    peak = MFMA_PEAK_TFLOPS[units]
    achieved = flops / step_s / 1e12
    roof = {"bound": "mfma", "achieved": achieved, "peak": peak, "unit": "TFLOP/s", "frac": achieved / peak,
            "peak_units": units + (" (split operands)" if units == "bf16" else ""),
            "fp32_frac": achieved / MFMA_PEAK_TFLOPS["f32"], "traffic": None,
            "kernel": "backward step (all kernels)",
            "algorithmic_flops_per_step": flops, "algorithmic_bytes_per_step": nbytes,
            "hbm_frac": nbytes / step_s / 1e9 / HBM_PEAK_GBS}
    cpu = None
    if not args.no_cpu_baseline:
        print("bench: cpu baseline (oracle backward)", file=sys.stderr, flush=True)
        cpu = cpu_baseline_backward(w, [0], dout[:, :1].cpu())
    line = {
        "metric": METRIC_BWD if args.workload == DEFAULT_WORKLOAD else METRIC_BWD_OTHER, "value": value, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("f32 accumulation, split-bf16 products, bf16 storage" if w.dtype == "bf16"
                  else "f32 arithmetic, f32 storage"),
        "data": "synthetic (seeded N(0,1) inputs and dL/dO, N(0,1) means, U(-1,1) raw variances, "
                "N(0,0.5^2) prior logits)",
        "config": {"workload": w.name, "pass": "backward", "mode": "causal" if w.causal else "bidirectional",
                   "batch": w.batch, "heads": w.heads, "seq_len": w.seq_len, "d_route": w.d_route,
                   "n_comp": w.n_comp, "d_value": w.d_value, "eps": w.eps, "global_batch": w.batch,
                   "parallelism": "single GPU"},
        "roofline": roof, "step_isolated": step_isolated, "kernels": kernels, "cpu_baseline": cpu,
        "source_hash": kernel_source_hash(backward=True),
    }
    print(json.dumps(line), flush=True)


def decode_line(args, w, gma, dev):
    """Per-step time of gma_decode_step (mixture from the raw parameters every step) and of
    gma_decode_step_prepared (mixture prepared once) on one token per (batch, head), state in place."""
    import torch
    w1 = w.with_(seq_len=max(args.steps, 1))
    inp = gma.make_inputs(w1)
    t = {k: v.to(dev) for k, v in inp.items()}
    st = torch.zeros(w.batch, w.heads, w.n_comp, w.d_value + 1, dtype=torch.float32, device=dev)
    out = torch.empty(w.batch, w.heads, 1, w.d_value, dtype=w.torch_dtype, device=dev)
    rows = {k: [t[k][:, :, i:i + 1].contiguous() for i in range(w1.seq_len)] for k in ("qx", "kx", "v")}
    res = {}
    for mode in ("raw", "prepared"):
        prep = gma.decode_prepare(t["raw_var"], t["prior_logits"]) if mode == "prepared" else None
        for i in range(min(args.warmup, w1.seq_len)):
            gma.decode_step(rows["qx"][i], rows["kx"][i], rows["v"][i], t["mu"], t["raw_var"], t["prior_logits"], st,
                            eps=w.eps, out=out, prepared=prep)
        st.zero_()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(w1.seq_len):
            gma.decode_step(rows["qx"][i], rows["kx"][i], rows["v"][i], t["mu"], t["raw_var"], t["prior_logits"], st,
                            eps=w.eps, out=out, prepared=prep)
        e1.record()
        torch.cuda.synchronize()
        res[mode] = e0.elapsed_time(e1) * 1e3 / w1.seq_len
        st.zero_()
    line = {"metric": "GMA causal decode step latency (one token per (batch, head), state in place)",
            "value": res["prepared"], "unit": "us/step", "n_gpus": 1, "steps": w1.seq_len, "warmup": args.warmup,
            "higher_is_better": False, "dtype": w.dtype, "data": "synthetic",
            "config": {"workload": w.name, "pass": "decode", "batch": w.batch, "heads": w.heads,
                       "d_route": w.d_route, "n_comp": w.n_comp, "d_value": w.d_value},
            "us_per_step": res}
    print(json.dumps(line), flush=True)


def resp_line(args, w, gma, dev, lib):
    """gma_responsibilities on the workload's K_X: back-to-back calls between events on the launch stream,
    against HBM (it reads d_r and writes K fp32 per row), with the copy reference of the same run."""
    import torch
    from gaussian_mixture_token_amd import _lib
    inp = gma.make_inputs(w)
    x = inp["kx"].to(dev)
    mu, rv, pl = inp["mu"].to(dev), inp["raw_var"].to(dev), inp["prior_logits"].to(dev)
    del inp
    out = torch.empty(w.batch, w.heads, w.seq_len, w.n_comp, dtype=torch.float32, device=dev)
    prob = gma.problem(w.batch, w.heads, w.seq_len, w.d_route, w.n_comp, 1, w.torch_dtype, w.eps)
    ws = torch.empty(max(gma.workspace_size(prob, _lib.GMA_OP_RESPONSIBILITIES), 1), dtype=torch.uint8, device=dev)

    def call():
        gma.responsibilities(x, mu, rv, pl, out=out, workspace=ws)

    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        call()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    lib.gma_timing_enable(1)
    for k in range(lib.gma_kernel_count()):
        lib.gma_timing_read(k, ctypes_double(), ctypes_int64())
    for _ in range(args.steps):
        call()
    torch.cuda.synchronize()
    lib.gma_timing_enable(0)
    kernels = {}
    for k in range(lib.gma_kernel_count()):
        tot, n = ctypes_double(), ctypes_int64()
        _lib.check(lib.gma_timing_read(k, tot, n))
        if n.value:
            kernels[lib.gma_kernel_name(k).decode()] = {"avg_us": 1e3 * tot.value / n.value, "launches": n.value,
                                                        "launches_per_step": n.value / args.steps}
    es = 2 if w.dtype == "bf16" else 4
    T = w.batch * w.heads * w.seq_len
    nbytes = (es * w.d_route + 4 * w.n_comp) * T
    flops = 4 * w.n_comp * w.d_route * T
    gbs = nbytes / (ms * 1e-3) / 1e9
    copy_gbs = copy_reference(dev)
    line = {"metric": "GMA responsibilities rows/sec (Gamma of every row, fp32 out) + % of HBM roofline",
            "value": T / (ms * 1e-3), "unit": "rows/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": w.dtype,
            "data": "synthetic (the workload's K_X and mixture)",
            "config": {"workload": w.name, "pass": "responsibilities", "batch": w.batch, "heads": w.heads,
                       "seq_len": w.seq_len, "d_route": w.d_route, "n_comp": w.n_comp},
            "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": gbs / HBM_PEAK_GBS, "traffic": None, "algorithmic_bytes_per_step": nbytes,
                         "algorithmic_flops_per_step": flops,
                         "mfma_frac": flops / (ms * 1e-3) / 1e12 / MFMA_PEAK_TFLOPS[w.dtype]},
            "copy_reference": {"gbs": copy_gbs, "frac_of_peak": copy_gbs / HBM_PEAK_GBS,
                               "step_over_copy": gbs / copy_gbs},
            "kernels": kernels, "source_hash": kernel_source_hash()}
    print(json.dumps(line), flush=True)


def ctypes_double():
    import ctypes
    return ctypes.c_double()


def ctypes_int64():
    import ctypes
    return ctypes.c_int64()


if __name__ == "__main__":
    main()
