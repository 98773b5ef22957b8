#!/usr/bin/env python3
"""Throughput of the MXFP4 + block-Hadamard linear-layer GEMMs on one MI355X.

One step = the whole hot path over one batch of synthetic input: for one linear layer,
  Fprop  Y  = X W^T      (X and W rotated by H16 and quantized along K, nearest-even)
  Dgrad  dX = dY W       (dY along N, W along N -- transposed quantize -- nearest-even)
  Wgrad  dW = dY^T X     (dY and X along the token axis M -- transposed -- stochastic rounding)
each as two quantize launches and one block-scaled FP4 GEMM through the C ABI
(mxfp4_quantize, mxfp4_gemm). This follows the gist.science summary of "MXFP4 LLM pretraining",
section 방법론 (Methodology): all three GEMMs in MXFP4 with the deterministic H16 rotation; the
stochastic rounding on the weight-gradient operands is the full-layer recipe of this benchmark.

Default workload: the Llama-3.1-8B QKV projection, M = 8192 tokens, K = 4096, N = 6144.
Prints ONE JSON line (rank 0). Inputs are resident in HBM before the timed region starts.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MXFP4 GEMM TFLOP/s incl. H16+quant (Fprop/Dgrad/Wgrad) + quantizer GB/s"
HBM_PEAK_GBS = 8000.0           # MI355X HBM3E, published
MXFP4_PEAK_TFLOPS = 10100.0     # MI355X dense FP4/FP6 matrix peak, published
QUANT_BYTES_PER_ELEM = 2.0 + 0.5 + 1.0 / 32.0   # bf16 in, 4-bit code out, one E8M0 byte per 32

WORKLOADS = {
    # name: (M tokens, K in_features, N out_features, description)
    "qkv": (8192, 4096, 6144, "Llama-3.1-8B QKV projection"),
    "small": (256, 512, 256, "single small layer"),
    "gateup": (8192, 4096, 28672, "Llama-3.1-8B fused gate+up projection"),
    "down": (8192, 14336, 4096, "Llama-3.1-8B down projection"),
}


def parse_args():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", choices=sorted(WORKLOADS), default="qkv")
    p.add_argument("--hadamard", type=int, default=16, choices=[0, 16, 32])
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--copy-calibration", action="store_true",
                   help="also run a plain 1 GiB device copy (reference for HBM byte counters)")
    return p.parse_args()


def source_digest():
    h = hashlib.sha256()
    for f in ("gemm.hip", "quantize.hip", "mx_device.h"):
        with open(os.path.join(ROOT, "mxfp4_block_scaled_h16_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def read_traffic(kernel, workload):
    """HBM bytes per launch from a committed counter summary, if it matches the current sources."""
    path = os.path.join(ROOT, "profiles", "%s_%s_traffic.txt" % (kernel, workload))
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                vals[k.strip()] = v.strip()
    if vals.get("source_digest") != source_digest():
        return None
    try:
        return float(vals["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


class Step:
    """Preallocated buffers and the launch sequence of one Fprop + Dgrad + Wgrad step."""

    def __init__(self, mx, torch, x, w, dy, M, K, N, h, sets):
        self.mx, self.torch = mx, torch
        self.M, self.K, self.N, self.h = M, K, N, h
        dev = x.device
        # rotate several copies of the inputs so consecutive steps do not hit in the 256 MB
        # last-level cache
        self.inputs = [(x, w, dy)] + [(x.clone(), w.clone(), dy.clone()) for _ in range(sets - 1)]
        u8 = lambda *s: torch.empty(s, dtype=torch.uint8, device=dev)  # noqa: E731
        self.fq = (u8(M, K // 2), u8(M, K // 32), u8(N, K // 2), u8(N, K // 32))
        self.dq = (u8(M, N // 2), u8(M, N // 32), u8(K, N // 2), u8(K, N // 32))
        self.wq = (u8(N, M // 2), u8(N, M // 32), u8(K, M // 2), u8(K, M // 32))
        self.y = torch.empty((M, N), dtype=torch.float32, device=dev)
        self.dx = torch.empty((M, K), dtype=torch.float32, device=dev)
        self.dw = torch.empty((N, K), dtype=torch.float32, device=dev)
        self.alpha = 1.0 / h if h else 1.0
        self.i = 0
        # launch list of one step: (name, callable)
        self.names = ["quant_rows X", "quant_rows W", "gemm Fprop",
                      "quant_rows dY", "quant_cols W", "gemm Dgrad",
                      "quant_cols dY sr", "quant_cols X sr", "gemm Wgrad"]

    def launches(self):
        mx, h = self.mx, self.h
        x, w, dy = self.inputs[self.i % len(self.inputs)]
        self.i += 1
        fq, dq, wq = self.fq, self.dq, self.wq
        return [
            lambda: mx.quantize(x, 1, h, "rne", 0, 0, fq[0], fq[1]),
            lambda: mx.quantize(w, 1, h, "rne", 0, 1, fq[2], fq[3]),
            lambda: mx.gemm(fq[0], fq[1], fq[2], fq[3], self.alpha, self.y),
            lambda: mx.quantize(dy, 1, h, "rne", 0, 0, dq[0], dq[1]),
            lambda: mx.quantize(w, 0, h, "rne", 0, 1, dq[2], dq[3]),
            lambda: mx.gemm(dq[0], dq[1], dq[2], dq[3], self.alpha, self.dx),
            lambda: mx.quantize(dy, 0, h, "sr", 0x5EED, 0, wq[0], wq[1]),
            lambda: mx.quantize(x, 0, h, "sr", 0x5EED, 1, wq[2], wq[3]),
            lambda: mx.gemm(wq[0], wq[1], wq[2], wq[3], self.alpha, self.dw),
        ]


def cpu_baseline(x, w, dy, M, K, N, h):
    """The oracle, untuned, on a bounded sample of the same step; projected to the whole step."""
    import numpy as np
    import oracle
    threads = oracle.num_threads()
    t_quant = 0.0
    sample = []
    # quantization rates, one slice per kind of launch in the step
    n_rows = min(M, 512)
    t0 = time.perf_counter()
    oracle.quantize(x[:n_rows], 1, h, 0)
    rate_rows = n_rows * K / (time.perf_counter() - t0)
    n_cols = min(N, 256)
    sl = np.ascontiguousarray(dy[:, :n_cols])
    t0 = time.perf_counter()
    oracle.quantize(sl, 0, h, 1, seed=0x5EED)
    rate_cols_sr = M * n_cols / (time.perf_counter() - t0)
    sl = np.ascontiguousarray(w[:, :n_cols]) if K >= n_cols else w
    t0 = time.perf_counter()
    oracle.quantize(sl, 0, h, 0)
    rate_cols = sl.shape[0] * sl.shape[1] / (time.perf_counter() - t0)
    sample.append("quantize: %d rows of X (rows, RNE), %d columns of dY (transposed, SR), %d columns "
                  "of W (transposed, RNE)" % (n_rows, n_cols, sl.shape[1]))
    t_quant = (M * K + N * K + M * N) / rate_rows + (N * K) / rate_cols + (M * N + M * K) / rate_cols_sr
    # GEMM rate on whole output rows of each of the three GEMMs (operands quantized outside the clock)
    rows = 16
    flops, secs = 0.0, 0.0
    for a_src, a_axis, b_src, b_axis, kc in ((x[:rows], 1, w, 1, K),
                                             (dy[:rows], 1, w, 0, N),
                                             (None, 0, x, 0, M)):
        if a_src is None:
            a = oracle.quantize(np.ascontiguousarray(dy[:, :rows]), 0, h, 1, seed=0x5EED)
        else:
            a = oracle.quantize(a_src, a_axis, h, 0)
        b = oracle.quantize(b_src, b_axis, h, 1 if a_src is None else 0, seed=0x5EED, stream=1)
        t0 = time.perf_counter()
        c = oracle.gemm(*a, *b, alpha=1.0 / h if h else 1.0)
        secs += time.perf_counter() - t0
        flops += 2.0 * c.shape[0] * c.shape[1] * kc
    rate_gemm = flops / secs
    sample.append("GEMM: %d output rows of each of Fprop, Dgrad, Wgrad (%.2f GFLOP)" % (rows, flops / 1e9))
    step_flops = 3 * 2.0 * M * N * K
    t_step = t_quant + step_flops / rate_gemm
    return {"value": step_flops / t_step / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": "; ".join(sample) + "; projected to the whole step",
            "gemm_gflops": rate_gemm / 1e9, "quantize_melem_s": rate_rows / 1e6,
            "step_seconds_projected": t_step}


def main():
    args = parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py runs on exactly one GPU: this build has no multi-GPU path "
              "(the sharding plan is written up in DESIGN.md). Use --gpus 1.", file=sys.stderr)
        return 2
    import numpy as np
    import torch
    import mxfp4_block_scaled_h16_amd as mx
    from synth import inputs

    M, K, N, desc = WORKLOADS[args.workload]
    h = args.hadamard
    xh, wh, dyh = inputs.linear_inputs(M, K, N, seed=0)
    to_dev = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()  # noqa: E731
    x, w, dy = to_dev(xh), to_dev(wh), to_dev(dyh)
    in_bytes = 2 * (M * K + N * K + M * N)
    sets = max(1, min(8, -(-(1 << 30) // in_bytes)))
    step = Step(mx, torch, x, w, dy, M, K, N, h, sets)
    torch.cuda.synchronize()

    for _ in range(args.warmup):
        for f in step.launches():
            f()
    torch.cuda.synchronize()

    # timed region: K steps, per-launch HIP events on the stream the kernels run on
    stream = torch.cuda.current_stream()
    n_launch = len(step.names)
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(n_launch + 1)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        ev = events[s]
        ev[0].record(stream)
        for i, f in enumerate(step.launches()):
            f()
            ev[i + 1].record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps

    per_launch = np.array([[events[s][i].elapsed_time(events[s][i + 1]) for i in range(n_launch)]
                           for s in range(args.steps)])  # ms
    avg_ms = per_launch.mean(0)
    gemm_flops = 2.0 * M * N * K
    step_flops = 3 * gemm_flops
    value = step_flops / (ms_per_step * 1e-3) / 1e12

    kernels = {}
    quant_elems = [M * K, N * K, None, M * N, N * K, None, M * N, M * K, None]
    for name, t, e in zip(step.names, avg_ms, quant_elems):
        entry = {"us": round(float(t) * 1e3, 2)}
        if e is None:
            entry["tflops"] = round(gemm_flops / (t * 1e-3) / 1e12, 1)
        else:
            entry["gbs"] = round(e * QUANT_BYTES_PER_ELEM / (t * 1e-3) / 1e9, 1)
        kernels[name] = entry

    gemm_idx = [2, 5, 8]
    gemm_avg_s = float(avg_ms[gemm_idx].mean()) * 1e-3
    achieved = gemm_flops / gemm_avg_s / 1e12
    traffic = read_traffic("gemm", args.workload)
    roofline = {"bound": "mfma", "achieved": round(achieved, 1), "peak": MXFP4_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / MXFP4_PEAK_TFLOPS, 4), "traffic": traffic,
                "kernel": "gemm_mxfp4 (average over the step's Fprop, Dgrad and Wgrad launches)",
                "algorithmic_per_launch": "2*M*N*K = %.1f GFLOP" % (gemm_flops / 1e9)}

    q_idx = [0, 1, 3, 4, 6, 7]
    q_bytes = sum(quant_elems[i] for i in q_idx) * QUANT_BYTES_PER_ELEM
    q_time = float(sum(avg_ms[i] for i in q_idx)) * 1e-3
    quantizer = {"gbs": round(q_bytes / q_time / 1e9, 1), "frac_of_hbm": round(q_bytes / q_time / 1e9 / HBM_PEAK_GBS, 4),
                 "bytes_per_elem": QUANT_BYTES_PER_ELEM, "us_per_step": round(q_time * 1e6, 1)}

    if args.copy_calibration:
        buf = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        buf2 = torch.empty_like(buf)
        buf2.copy_(buf)
        torch.cuda.synchronize()

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(xh, wh, dyh, M, K, N, h)

    line = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "mxfp4",
        "data": "synthetic",
        "config": {"workload": "%s Fprop+Dgrad+Wgrad, M=%d tokens, K=%d, N=%d, H%d, MXFP4 RNE "
                               "(SR on Wgrad operands)" % (desc, M, K, N, h),
                   "M": M, "K": K, "N": N, "hadamard": h, "input_sets": sets},
        "roofline": roofline, "quantizer": quantizer, "kernels": kernels, "cpu_baseline": cpu,
        "source_digest": source_digest(),
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
