#!/usr/bin/env python3
"""Throughput of the MXFP4 + block-Hadamard linear-layer GEMMs on one MI355X.

One step = the whole hot path over one batch of synthetic input. For each linear projection of
the workload it runs the passes the workload names:
  Fprop  Y  = X W^T      (X and W rotated and quantized along K, nearest-even)
  Dgrad  dX = dY W       (dY along N, W along N -- transposed quantize -- nearest-even)
  Wgrad  dW = dY^T X     (dY and X along the token axis M -- transposed -- Philox stochastic
                          rounding on both operands)
Every pass is quantize launches plus one block-scaled FP4 GEMM through the C ABI
(mxfp4_quantize, mxfp4_gemm); an activation read by several projections is quantized once per
axis. This follows the gist.science summary "기술 요약: MXFP4 를 활용한 대규모 언어 모델 사전
학습", section 방법론 (Methodology): all three GEMMs in MXFP4 behind the deterministic H16
rotation; stochastic rounding on the weight-gradient operands is the full-layer recipe here.

Default workload: one Llama-3.1-8B decoder layer at 8192 tokens, all 7 projections (q 4096->4096,
k and v 4096->1024, o 4096->4096, gate and up 4096->14336, down 14336->4096) x Fprop + Dgrad +
Wgrad, H16, nearest rounding for Fprop and Dgrad and Philox stochastic rounding on both Wgrad
operands: 21 GEMMs per step. `--workload qkv` runs the QKV projection alone (M = 8192, K = 4096,
N = 6144), `small`, `gateup` and `down` the other single-projection configurations.
Prints ONE JSON line. Inputs are resident in HBM before the timed region starts.
"""
import argparse
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
DUAL_BYTES_PER_ELEM = 2.0 + 2 * (0.5 + 1.0 / 32.0)  # one read, both quantizations written

# name: (description, [(projection, K, N)], input of each projection, passes, tokens)
LLAMA_PROJ = [("q", 4096, 4096), ("k", 4096, 1024), ("v", 4096, 1024), ("o", 4096, 4096),
              ("gate", 4096, 14336), ("up", 4096, 14336), ("down", 14336, 4096)]
LLAMA_INPUT = {"q": "attn_in", "k": "attn_in", "v": "attn_in", "o": "o_in", "gate": "mlp_in",
               "up": "mlp_in", "down": "down_in"}
WORKLOADS = {
    "qkv": ("Llama-3.1-8B QKV projection Fprop+Dgrad+Wgrad", [("qkv", 4096, 6144)], "FDW", 8192),
    "qkv_fprop": ("Llama-3.1-8B QKV projection Fprop", [("qkv", 4096, 6144)], "F", 8192),
    "small": ("single small layer Fprop+Dgrad+Wgrad", [("small", 512, 256)], "FDW", 256),
    "gateup": ("Llama-3.1-8B fused gate+up projection Fprop+Dgrad", [("gateup", 4096, 28672)], "FD", 8192),
    "down": ("Llama-3.1-8B down projection Wgrad", [("down", 14336, 4096)], "W", 8192),
    "layer": ("Llama-3.1-8B decoder layer, 7 projections x Fprop+Dgrad+Wgrad", LLAMA_PROJ, "FDW", 8192),
}


def parse_args():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", choices=sorted(WORKLOADS), default="layer")
    p.add_argument("--hadamard", type=int, default=16, choices=[0, 16, 32])
    p.add_argument("--rht", action="store_true",
                   help="randomized Hadamard: a sign diagonal keyed by each GEMM's seed before H")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--settle", type=float, default=1.0,
                   help="seconds of untimed steps before the warm-up (GPU clock ramp)")
    p.add_argument("--no-library-baselines", action="store_true",
                   help="skip the vendor GEMM baselines (hipBLASLt FP8 per tensor and MXFP8 at every GEMM "
                        "shape of the step, on the step's operands)")
    p.add_argument("--separate-quant", action="store_true",
                   help="one quantizer launch per axis instead of one dual launch per tensor")
    p.add_argument("--no-graph", action="store_true",
                   help="launch every kernel of the timed steps from the host instead of replaying each step "
                        "as one captured HIP graph")
    p.add_argument("--no-group", action="store_true",
                   help="one GEMM launch per product, also for same-shape products of one input (k and v, "
                        "gate and up), which otherwise share a grouped launch per pass; and one quantizer "
                        "launch per tensor, where back-to-back dual quantizations otherwise share one")
    p.add_argument("--no-ceilings", action="store_true",
                   help="skip the measured HBM and matrix-core ceilings")
    p.add_argument("--copy-calibration", action="store_true",
                   help="also run a plain 1 GiB device copy (reference for HBM byte counters)")
    return p.parse_args()


class Plan:
    """Buffers and the ordered launch list of one step (quantize and GEMM launches)."""

    def __init__(self, mx, torch, workload, h, sets, dual=True, host=None, group=True, tokens=None):
        import numpy as np
        from synth import inputs
        desc, projs, passes, M = WORKLOADS[workload]
        M = M if tokens is None else int(tokens)   # tests run the layer at fewer tokens
        self.mx, self.torch, self.h, self.passes, self.M = mx, torch, h, passes, M
        self.dual = dual
        self.group = group
        # h may carry the randomized-Hadamard or orthonormal flags; alpha undoes the factor of the
        # size alone (the orthonormal rotation leaves none)
        hs = h & ~(mx.RHT | mx.ORTHO)
        self.alpha = 1.0 if (h & mx.ORTHO) or not hs else 1.0 / hs
        dev = "cuda"
        to_dev = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)  # noqa: E731
        # host tensors (bf16 bit patterns), drawn by the shared seeded recipe
        if host is not None:
            acts, per_proj = host["acts"], host["proj"]
            self.host = host
            inp = {projs[0][0]: "x"}
        elif workload == "layer":
            acts, per_proj = inputs.llama_layer_inputs(seed=0, tokens=M)
            self.host = {"acts": acts, "proj": per_proj}
            inp = LLAMA_INPUT
        else:
            (name, K, N), = projs
            if workload == "down":
                dy, x = inputs.down_wgrad(seed=0, m=M, n=N, k=K)
                w = inputs.weights(np.random.default_rng(1), N, K)
            else:
                x, w, dy = inputs.linear_inputs(M, K, N, seed=0)
            acts, per_proj = {"x": x}, {name: (w, dy)}
            self.host = {"acts": acts, "proj": per_proj}
            inp = {name: "x"}
        self.desc = desc
        # device copies: `sets` rotated copies so consecutive steps do not hit in the 256 MB cache
        self.sets = []
        for s in range(sets):
            d_acts = {k: to_dev(v) for k, v in acts.items()}
            d_proj = {k: (to_dev(w), to_dev(dy)) for k, (w, dy) in per_proj.items()}
            self.sets.append((d_acts, d_proj))
        u8 = lambda *s: torch.empty(s, dtype=torch.uint8, device=dev)  # noqa: E731
        f32 = lambda *s: torch.empty(s, dtype=torch.float32, device=dev)  # noqa: E731
        # quantized operand buffers (reused every step); contractions that are multiples of 512
        # use the tiled layout, as the library's linear entry points do
        self.q = {}
        self.layout = {}

        def qbuf(key, outer, L):
            tiled = L % 512 == 0
            rows = -(-outer // 256) * 256 if tiled else outer
            self.q[key] = (u8(rows, L // 2), u8(rows, L // 32))
            self.layout[key] = "tiled" if tiled else "rows"
        for a, x in acts.items():
            K = x.shape[1]
            if "F" in passes:
                qbuf((a, "rows"), M, K)
            if "W" in passes:
                qbuf((a, "cols"), K, M)
        self.out = {}
        self.ops = []       # (label, kind, callable-builder, work) per launch; kind in quant/gemm
        self.projs = projs
        for name, K, N in projs:
            a = inp[name]
            if "F" in passes:
                qbuf((name, "w_rows"), N, K)
                self.out[(name, "F")] = f32(M, N)
            if "D" in passes:
                qbuf((name, "dy_rows"), M, N)
                qbuf((name, "w_cols"), K, N)
                self.out[(name, "D")] = f32(M, K)
            if "W" in passes:
                qbuf((name, "dy_cols"), N, M)
                self.out[(name, "W")] = f32(N, K)
        # split-K workspaces of the products with few output tiles (allocated once, outside timing)
        self.ws = {}
        for key, c in self.out.items():
            kc = {"F": None, "D": None, "W": None}[key[1]]
            name = key[0]
            K, N = next((k, n) for nm, k, n in projs if nm == name)
            kc = K if key[1] == "F" else (N if key[1] == "D" else M)
            need = mx.gemm_workspace_bytes(c.shape[0], c.shape[1], kc)
            self.ws[key] = torch.empty(need, dtype=torch.uint8, device=dev) if need else None
        self._build(inp)

    def _build(self, inp):
        """Launch order: per projection its passes, each preceded by the quantizations it needs
        that have not run yet. A tensor quantized along both axes in the step (X, W, dY when the
        passes need both) gets one dual launch, placed where its first output is needed, unless
        the plan was built with separate quantizer launches."""
        M = self.M
        quants = []   # (label, src, key, axis, rounding, seed, stream, dst, elems), in first-use order
        seen = set()

        def need(label, src, key, axis, rnd, seed, stream, dst, elems):
            if dst not in seen:
                seen.add(dst)
                quants.append((label, src, key, axis, rnd, seed, stream, dst, elems))
            return dst
        # projections that read one input with weights of one shape (k and v, gate and up) run
        # each pass as one grouped launch, unless the plan was built without grouping
        groups = []
        for name, K, N in self.projs:
            last = groups[-1] if groups else None
            if self.group and last and (inp[last[0][0]], last[0][1], last[0][2]) == (inp[name], K, N):
                last.append((name, K, N))
            else:
                groups.append([(name, K, N)])
        steps = []    # (label, [(qa, qb, out)], flops), each after the quantizations it needs
        for members in groups:
            names = "+".join(m[0] for m in members)
            for pas, pname in (("F", "Fprop"), ("D", "Dgrad"), ("W", "Wgrad")):
                if pas not in self.passes:
                    continue
                prods, flops = [], 0.0
                for name, K, N in members:
                    a = inp[name]
                    if pas == "F":
                        qa = need("x", "act", a, 1, "rne", 0, 0, (a, "rows"), M * K)
                        qb = need("W", "w", name, 1, "rne", 0, 1, (name, "w_rows"), N * K)
                    elif pas == "D":
                        qa = need("dY", "dy", name, 1, "rne", 0, 0, (name, "dy_rows"), M * N)
                        qb = need("W", "w", name, 0, "rne", 0, 1, (name, "w_cols"), N * K)
                    else:
                        qa = need("dY", "dy", name, 0, "sr", 0x5EED, 0, (name, "dy_cols"), M * N)
                        qb = need("x", "act", a, 0, "sr", 0x5EED, 1, (a, "cols"), M * K)
                    prods.append((qa, qb, (name, pas)))
                    flops += 2.0 * M * N * K
                steps.append(("gemm %s %s" % (pname, names), prods, flops))
        by_dst = {q[7]: q for q in quants}
        by_src = {}
        for q in quants:
            by_src.setdefault((q[1], q[2]), []).append(q)
        ops, done = [], set()

        def emit(dst):
            if dst in done:
                return
            q = by_dst[dst]
            both = by_src[(q[1], q[2])]
            if self.dual and len(both) == 2:
                q1 = next(t for t in both if t[3] == 1)
                q0 = next(t for t in both if t[3] == 0)
                tensor = q[2] if q[1] == "act" else "%s_%s" % (q[0], q[2])
                ops.append(("quant_dual %s" % tensor, "dual", ((q1, q0),), q[8]))
                done.add(q1[7])
                done.add(q0[7])
            else:
                tensor = q[2] if q[1] == "act" else "%s_%s" % (q[0], q[2])
                ops.append(("quant_%s %s%s" % ("rows" if q[3] == 1 else "cols", tensor,
                                                 " sr" if q[4] == "sr" else ""), "quant", q, q[8]))
                done.add(dst)
        for label, prods, flops in steps:
            for qa, qb, _ in prods:
                emit(qa)
                emit(qb)
            ops.append((label, "gemm", tuple(prods), flops))
        if self.group:
            # launches that run back to back share one: dual quantizations (an activation and the
            # weight of the product that reads it, k and v, gate and up), and GEMMs of one output
            # shape and contraction (the Dgrad and Wgrad of a layer with as many tokens as outputs)
            merged = []
            for op in ops:
                last = merged[-1] if merged else None
                same = last is not None and last[1] == op[1] and len(last[2]) + len(op[2]) <= 8 and (
                    op[1] == "dual" or (op[1] == "gemm" and self.gemm_shape(last[2][0][2]) ==
                                        self.gemm_shape(op[2][0][2])))
                if same:
                    prefix = "quant_dual " if op[1] == "dual" else "gemm "
                    merged[-1] = (last[0] + "+" + op[0][len(prefix):], op[1], last[2] + op[2], last[3] + op[3])
                else:
                    merged.append(op)
            ops = merged
        self.op_list = ops

    def gemm_shape(self, okey):
        """(output rows, output columns, contraction) of the GEMM that writes okey."""
        name, pas = okey
        K, N = next((k, n) for nm, k, n in self.projs if nm == name)
        return {"F": (self.M, N, K), "D": (self.M, K, N), "W": (N, K, self.M)}[pas]

    def _tensor(self, d_acts, d_proj, q):
        src, key = q[1], q[2]
        return d_acts[key] if src == "act" else d_proj[key][0 if src == "w" else 1]

    def launches(self, step_index):
        mx, h, alpha = self.mx, self.h, self.alpha
        d_acts, d_proj = self.sets[step_index % len(self.sets)]
        calls = []
        for label, kind, spec, work in self.op_list:
            if kind == "quant":
                t = self._tensor(d_acts, d_proj, spec)
                _, _, _, axis, rnd, seed, stream, dst, _ = spec
                q, s = self.q[dst]
                calls.append(lambda t=t, axis=axis, rnd=rnd, seed=seed, stream=stream, q=q, s=s, lay=self.layout[dst]:
                             mx.quantize(t, axis, h, rnd, seed, stream, q, s, layout=lay))
            elif kind == "dual":
                items = []
                for q1, q0 in spec:
                    t = self._tensor(d_acts, d_proj, q1)
                    o1 = dict(rounding=q1[4], seed=q1[5], stream_id=q1[6], layout=self.layout[q1[7]],
                              q=self.q[q1[7]][0], scales=self.q[q1[7]][1])
                    o0 = dict(rounding=q0[4], seed=q0[5], stream_id=q0[6], layout=self.layout[q0[7]],
                              q=self.q[q0[7]][0], scales=self.q[q0[7]][1])
                    items.append((t, o1, o0))
                if len(items) == 1:
                    calls.append(lambda it=items[0]: mx.quantize_dual(it[0], h, it[1], it[2]))
                else:
                    calls.append(lambda items=items: mx.quantize_dual_grouped(items, h))
            elif len(spec) == 1:
                (qa, qb, out), = spec
                calls.append(lambda qa=self.q[qa], qb=self.q[qb], c=self.out[out], lay=self.layout[qa], ws=self.ws[out]:
                             mx.gemm(qa[0], qa[1], qb[0], qb[1], alpha, c, layout=lay, workspace=ws))
            else:
                items = [(*self.q[qa], *self.q[qb]) for qa, qb, _ in spec]
                outs = [self.out[out] for _, _, out in spec]
                calls.append(lambda items=items, outs=outs, lay=self.layout[spec[0][0]]:
                             mx.gemm_grouped(items, alpha, outs=outs, layout=lay))
        return calls


def _profile_values(name, source):
    """key: value lines and table rows of a committed counter summary under profiles/, if it was
    taken with `source` (a file of the HIP library) as it is now; otherwise None."""
    import hashlib
    path = os.path.join(ROOT, "profiles", name)
    src = os.path.join(ROOT, "mxfp4_block_scaled_h16_amd", "csrc", source)
    if not os.path.exists(path):
        return None
    vals, rows = {}, []
    with open(path) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            if "|" in line:
                rows.append([c.strip() for c in line.split("|")])
            elif ":" in line:
                k, v = line.split(":", 1)
                vals[k.strip()] = v.strip()
    with open(src, "rb") as f:
        digest = hashlib.sha256(f.read()).hexdigest()[:16]
    if vals.get("source_digest") != digest:
        return None
    return vals, rows


def gemm_algorithmic_bytes(rows_a, rows_b, kc):
    """HBM bytes a GEMM must move: both operands once (codes 1/2 B and scales 1/32 B per element,
    17/32 B in all) and the FP32 output once."""
    return int((rows_a + rows_b) * kc * 17 // 32 + 4 * rows_a * rows_b)


def measured_traffic(workload):
    """HBM bytes per GEMM launch of the step, averaged over its GEMM launches, from the committed
    FETCH_SIZE / WRITE_SIZE summary of this workload, if it was taken with the GEMM source as it
    is now (otherwise None)."""
    got = _profile_values("gemm_mxfp4_%s_step_hbm_bytes.txt" % workload, "gemm.hip")
    if got is None:
        return None
    try:
        return float(got[0]["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


# CUs x SIMDs x lanes per clock x clock: 78.6 T lane-ops/s. A SIMD issues a 32-bit wave64 VALU
# instruction every two clocks (the published 157.3 TFLOP/s FP32 vector rate counts an FMA as two
# operations; a probe of dependent-free adds measured 2.2 clocks per wave64 instruction).
VALU_LANE_OPS_PEAK = 256 * 4 * 32 * 2.4e9


def measured_mfma_busy(workload):
    """The fraction of SIMD cycles the matrix cores were busy during the step's GEMM launches
    (SQ_VALU_MFMA_BUSY_CYCLES over GRBM_GUI_ACTIVE x 1024 SIMDs), from the committed SQ summary
    of this workload, if it was taken with the GEMM source as it is now (otherwise None)."""
    got = _profile_values("gemm_mxfp4_%s_step_sq_counters.txt" % workload, "gemm.hip")
    if got is None:
        return None
    try:
        return float(got[0]["mfma_busy_step"])
    except (KeyError, ValueError):
        return None


def quantizer_valu(workload, plan, avg_ms):
    """The stochastic-rounding quantizer launches against the VALU roofline: VALU instructions
    per wavefront and wavefronts per launch from the committed SQ counter summary of this
    workload (taken with the quantizer source as it is now, else None), times 64 lanes, over the
    launch's duration in this run, against 256 CUs x 4 SIMDs x 32 lanes per clock x 2.4 GHz.
    Counts every VALU instruction as one issue slot; the 64-bit multiply-adds of Philox take
    about 2.8 slots each (measured), so the VALU is busier than this says."""
    got = _profile_values("quant_%s_step_sq_counters.txt" % workload, "quantize.hip")
    if got is None:
        return None
    counts = {}
    for row in got[1]:
        if len(row) >= 3 and row[0] not in ("launch", ""):
            try:
                counts[row[0]] = (float(row[1]), float(row[2]))   # waves, VALU instructions per wave
            except ValueError:
                pass
    launches, ops_total, t_total = {}, 0.0, 0.0
    for (label, kind, spec, _), t in zip(plan.op_list, avg_ms):
        if kind != "dual" or label not in counts:
            continue
        if not any(q[4] == "sr" for pair in spec for q in pair):
            continue
        waves, per_wave = counts[label]
        ops = waves * per_wave * 64
        launches[label] = {"valu_giga_lane_ops": round(ops / 1e9, 2),
                           "frac": round(ops / (float(t) * 1e-3) / VALU_LANE_OPS_PEAK, 4)}
        ops_total += ops
        t_total += float(t) * 1e-3
    if not launches:
        return None
    return {"bound": "valu", "achieved": round(ops_total / t_total / 1e12, 2), "peak": round(VALU_LANE_OPS_PEAK / 1e12, 2),
            "unit": "T lane-ops/s", "frac": round(ops_total / t_total / VALU_LANE_OPS_PEAK, 4),
            "launches": launches, "counters": "profiles/quant_%s_step_sq_counters.txt" % workload}


def quantization_error(plan, rows=8):
    """Error of the method itself (MXFP4 with the step's rotation and rounding against the exact
    product): for each GEMM of the last step, ||C - C_exact|| / ||C_exact|| (Frobenius) over
    `rows` evenly spaced output rows, C_exact the binary64 product of the unquantized bf16
    inputs (numpy on the host, outside any timed region)."""
    import numpy as np
    f64 = {}

    def host64(key, a):
        if key not in f64:
            f64[key] = (np.asarray(a, dtype=np.uint32) << 16).view(np.float32).astype(np.float64)
        return f64[key]
    acts, per_proj = plan.host["acts"], plan.host["proj"]
    out = {}
    products = [(qa, qb, okey) for _, kind, spec, _ in plan.op_list if kind == "gemm" for qa, qb, okey in spec]
    for qa, qb, okey in products:
        name, pas = okey
        label = "gemm %s %s" % ({"F": "Fprop", "D": "Dgrad", "W": "Wgrad"}[pas], name)
        w = host64(("w", name), per_proj[name][0])
        dy = host64(("dy", name), per_proj[name][1])
        akey = qb[0] if pas == "W" else qa[0]
        x = host64(("x", akey), acts[akey]) if pas in "FW" else None
        got = plan.out[okey]
        idx = np.linspace(0, got.shape[0] - 1, rows).round().astype(np.int64)
        c = got[plan.torch.from_numpy(idx).to(got.device)].cpu().numpy().astype(np.float64)
        if pas == "F":
            ref = x[idx] @ w.T
        elif pas == "D":
            ref = dy[idx] @ w
        else:
            ref = dy[:, idx].T @ x
        out[label] = round(float(np.linalg.norm(c - ref) / np.linalg.norm(ref)), 5)
    out["rows_sampled"] = rows
    out["reference"] = "binary64 product of the unquantized bf16 inputs"
    return out


GEMM_ROWS = 1024  # output rows of the oracle GEMM the CPU baseline times (about 15 s on 16 cores)


def cpu_model():
    """The host CPU's model name (Linux /proc/cpuinfo), or None."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(plan, h):
    """The oracle, untuned, on a bounded sample of the same step, projected to the whole step."""
    import numpy as np
    import oracle
    t_begin = time.perf_counter()
    threads = oracle.num_threads()
    acts, per_proj = plan.host["acts"], plan.host["proj"]
    # quantization rate: one whole operand per launch kind (rows of an activation, the transposed
    # SR quantization of dY, the transposed RNE quantization of W)
    any_act = next(iter(acts.values()))
    name0 = plan.projs[0][0]
    w0, dy0 = per_proj[name0]
    rows = any_act.shape[0]
    t0 = time.perf_counter()
    oracle.quantize(np.ascontiguousarray(any_act), 1, h, oracle.RNE)
    rate_rows = any_act.size / (time.perf_counter() - t0)
    t0 = time.perf_counter()
    oracle.quantize(dy0, 0, h, oracle.SR, seed=0x5EED)
    rate_cols_sr = dy0.size / (time.perf_counter() - t0)
    t0 = time.perf_counter()
    oracle.quantize(w0, 0, h, oracle.RNE)
    rate_cols = w0.size / (time.perf_counter() - t0)
    t_quant = 0.0
    for label, kind, spec, work in plan.op_list:
        for q in ([x for pair in spec for x in pair] if kind == "dual" else (spec,) if kind == "quant" else ()):
            axis, rnd = q[3], q[4]
            rate = rate_rows if axis == 1 else (rate_cols_sr if rnd == "sr" else rate_cols)
            t_quant += work / rate
    # GEMM rate: the first GEMM_ROWS output rows of the first projection's Fprop-shaped product
    qa = oracle.quantize(np.ascontiguousarray(any_act[:GEMM_ROWS]), 1, h, oracle.RNE)
    qb = oracle.quantize(w0, 1, h, oracle.RNE, stream=1) if w0.shape[1] == any_act.shape[1] else None
    if qb is None:
        qa = oracle.quantize(np.ascontiguousarray(dy0[:GEMM_ROWS]), 1, h, oracle.RNE)
        qb = oracle.quantize(w0, 0, h, oracle.RNE, stream=1)
    t0 = time.perf_counter()
    c = oracle.gemm(*qa, *qb, alpha=oracle.alpha_for(h))
    secs = time.perf_counter() - t0
    rate_gemm = 2.0 * c.shape[0] * c.shape[1] * qa[0].shape[1] * 2 / secs
    step_flops = sum(work for label, kind, spec, work in plan.op_list if kind == "gemm")
    t_step = t_quant + step_flops / rate_gemm
    return {"value": step_flops / t_step / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": ("quantize all %d rows of an activation (RNE, along rows), all of dY %s (transposed, SR) "
                       "and all of W %s (transposed, RNE); GEMM %d output rows of %s; projected to the whole "
                       "step" % (rows, "x".join(map(str, dy0.shape)), "x".join(map(str, w0.shape)),
                                 c.shape[0], name0)),
            "cpu_seconds": round(time.perf_counter() - t_begin, 2),
            "gemm_gflops": rate_gemm / 1e9, "quantize_melem_s": rate_rows / 1e6,
            "quantize_gbs": rate_rows * QUANT_BYTES_PER_ELEM / 1e9, "cpu_model": cpu_model(),
            "step_seconds_projected": t_step}


class TimingEvents:
    """HIP timing events created with hipEventDisableSystemFence, recorded on the stream the
    kernels run on. Recording a default event also writes back and invalidates the caches
    (a system-scope fence), which after every launch adds several microseconds and flushes the
    dirty output lines of the previous kernel; these events only take timestamps."""
    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self):
        import ctypes
        self.ct = ctypes
        # the HIP runtime already loaded by torch and libmxfp4
        self.hip = ctypes.CDLL("libamdhip64.so.7")
        self.hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.events = []

    def create(self):
        e = self.ct.c_void_p()
        st = self.hip.hipEventCreateWithFlags(self.ct.byref(e), self.DISABLE_SYSTEM_FENCE)
        if st != 0:
            raise RuntimeError("hipEventCreateWithFlags failed (%d)" % st)
        self.events.append(e)
        return e

    def record(self, e, stream):
        st = self.hip.hipEventRecord(e, stream)
        if st != 0:
            raise RuntimeError("hipEventRecord failed (%d)" % st)

    def elapsed_ms(self, a, b):
        v = self.ct.c_float()
        st = self.hip.hipEventElapsedTime(self.ct.byref(v), a, b)
        if st != 0:
            raise RuntimeError("hipEventElapsedTime failed (%d)" % st)
        return v.value

    def close(self):
        for e in self.events:
            self.hip.hipEventDestroy(e)
        self.events = []


def capture_steps(plan):
    """One HIP graph per input set (torch.cuda.CUDAGraph), each holding every launch of one step
    on that set, after one eager run of the step on a side stream. The library launches only
    kernels (no memset, copy or allocation) on the stream it is given: the capture stream here."""
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graphs = []
    with torch.cuda.stream(side):
        for i in range(len(plan.sets)):
            for f in plan.launches(i):
                f()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for i in range(len(plan.sets)):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for f in plan.launches(i):
                f()
        graphs.append(g)
    torch.cuda.synchronize()
    return graphs


def step_runner(plan, graphs):
    """f(step index) that runs one step: a graph replay, or the eager launches."""
    if graphs:
        return lambda s: graphs[s % len(graphs)].replay()

    def eager(s):
        for f in plan.launches(s):
            f()
    return eager


def settle(plan, seconds, graphs=None):
    """Untimed steps until `seconds` of wall time have passed: the GPU leaves its idle clock
    state only after some tens of milliseconds of sustained load (a cold start measured 10-15%
    slower than the steady state of a training loop). Returns the number of steps run."""
    import torch
    run = step_runner(plan, graphs)
    n, t_end = 0, time.perf_counter() + seconds
    while time.perf_counter() < t_end:
        run(n)
        n += 1
        torch.cuda.synchronize()
    return n


def run_timed(plan, steps, warmup, graphs=None):
    """W untimed warm-up steps, then EXACTLY K timed steps bracketed by device synchronizations
    (host clock, no per-launch instrumentation; each step one graph replay when `graphs` holds
    the captured steps), then K more steps launched from the host with fence-free HIP events
    around every launch on the launch stream for the per-kernel durations.
    Returns (ms per step of the timed steps, average ms of each launch of the step, ms of each
    instrumented step from its first launch's start to its last launch's end)."""
    import numpy as np
    import torch
    run = step_runner(plan, graphs)
    for s in range(warmup):
        run(s)
    calls = [plan.launches(s) for s in range(steps)]
    torch.cuda.synchronize()
    if graphs:
        t0 = time.perf_counter()
        for s in range(steps):
            graphs[s % len(graphs)].replay()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
    else:
        t0 = time.perf_counter()
        for s in range(steps):
            for f in calls[s]:
                f()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
    ev = TimingEvents()
    stream = torch.cuda.current_stream().cuda_stream
    n_launch = len(plan.op_list)
    marks = [[ev.create() for _ in range(n_launch + 1)] for _ in range(steps)]
    torch.cuda.synchronize()
    for s in range(steps):
        ev.record(marks[s][0], stream)
        for i, f in enumerate(calls[s]):
            f()
            ev.record(marks[s][i + 1], stream)
    torch.cuda.synchronize()
    per_launch = np.array([[ev.elapsed_ms(marks[s][i], marks[s][i + 1]) for i in range(n_launch)]
                           for s in range(steps)])
    per_step = np.array([ev.elapsed_ms(marks[s][0], marks[s][n_launch]) for s in range(steps)])
    ev.close()
    return (t1 - t0) * 1e3 / steps, per_launch.mean(0), per_step


def machine_ceilings(settle_s=0.25, reps=10):
    """Practical ceilings of this board, measured in the same run with the plain kernels of
    libmxfp4_ceiling.so: streaming HBM read, write and copy of 1 GiB buffers (16-byte accesses,
    GB/s of bytes moved), and the scaled FP4 MFMA loop on register-resident operands that change
    every round, one 8-wavefront workgroup per compute unit (TFLOP/s). Each is settled for
    `settle_s` seconds, then `reps` launches are timed with fence-free events."""
    import torch
    from mxfp4_block_scaled_h16_amd import ceiling
    ev = TimingEvents()
    stream = torch.cuda.current_stream().cuda_stream
    nbytes = 1 << 30
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    ceiling.write(src, 0x5A5AA5A5)  # every lane's XOR of equal 16-byte words is 0, never 1
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    msink = torch.empty(cus * 512, dtype=torch.float32, device="cuda")
    iters = 3000
    cases = [
        ("hbm_read_gbs", lambda: ceiling.read(src, 1, sink), nbytes),
        ("hbm_write_gbs", lambda: ceiling.write(dst, 0x01234567), nbytes),
        ("hbm_copy_gbs", lambda: ceiling.copy(src, dst), 2 * nbytes),
        ("mfma_fp4_tflops", lambda: ceiling.mfma(cus, iters, 7, msink), cus * iters * ceiling.MFMA_FLOPS_PER_ROUND),
    ]
    out = {}
    for name, f, work in cases:
        t_end = time.perf_counter() + settle_s
        while time.perf_counter() < t_end:
            f()
            torch.cuda.synchronize()
        a, b = ev.create(), ev.create()
        ev.record(a, stream)
        for _ in range(reps):
            f()
        ev.record(b, stream)
        torch.cuda.synchronize()
        t = ev.elapsed_ms(a, b) * 1e-3 / reps
        out[name] = round(work / t / (1e12 if name.startswith("mfma") else 1e9), 1)
    ev.close()
    if not bool(torch.isfinite(msink).all()):
        raise RuntimeError("matrix-core ceiling kernel produced non-finite sums")
    out["note"] = ("measured in this run: 1 GiB streaming read / write / copy (copy counts read + write bytes); "
                   "scaled FP4 32x32x64 MFMA loop, %d workgroups x 8 wavefronts, operands changing every round"
                   % cus)
    del src, dst, msink
    return out


def step_entry_points(plan, steps, warmup, settle_s=0.25):
    """The same step through the library's training-step calls (mxfp4_linear_forward, then
    mxfp4_linear_backward: X, W and dY each quantized once along both axes, three GEMMs), on the
    plan's inputs, workspaces allocated once outside the timed region. Host clock over K steps."""
    import torch
    mx = plan.mx
    if plan.passes != "FDW" or len(plan.projs) != 1:
        return None
    name, K, N = plan.projs[0]
    M = plan.M
    ws = torch.empty(mx.step_workspace_bytes(M, K, N), dtype=torch.uint8, device="cuda")
    y = torch.empty((M, N), dtype=torch.float32, device="cuda")
    dx = torch.empty((M, K), dtype=torch.float32, device="cuda")
    dw = torch.empty((N, K), dtype=torch.float32, device="cuda")

    def step(i):
        d_acts, d_proj = plan.sets[i % len(plan.sets)]
        x = d_acts[next(iter(d_acts))]
        w, dy = d_proj[name]
        mx.linear_forward(x, w, plan.h, "rne", "rne", "sr", 0x5EED, workspace=ws, out=y)
        mx.linear_backward(dy, K, ws, plan.h, "rne", "rne", "sr", 0x5EED, dx=dx, dw=dw)
    t_end, i = time.perf_counter() + settle_s, 0
    while time.perf_counter() < t_end:
        step(i)
        i += 1
        torch.cuda.synchronize()
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(i)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    flops = 3 * 2.0 * M * N * K
    return {"calls": "mxfp4_linear_forward + mxfp4_linear_backward", "ms_per_step": round(ms, 4),
            "tflops": round(flops / (ms * 1e-3) / 1e12, 1)}


def gemm_operands_bf16(plan, okey):
    """The bf16 device operands (A [rows_A, Kc], B [rows_B, Kc], both contiguous) of one GEMM of
    the plan, from its first input set: Fprop A = X, B = W; Dgrad A = dY, B = W^T; Wgrad A = dY^T,
    B = X^T."""
    name, pas = okey
    d_acts, d_proj = plan.sets[0]
    w, dy = d_proj[name]
    key = LLAMA_INPUT.get(name)
    x = d_acts[key] if key in d_acts else d_acts["x"]
    if pas == "F":
        return x, w
    if pas == "D":
        return dy, w.t().contiguous()
    return dy.t().contiguous(), x.t().contiguous()


def fp8_per_tensor(t):
    """FP8 E4M3 codes of t with one binary32 scale: amax / 448 (the largest E4M3 value)."""
    import torch
    amax = t.float().abs().max().clamp(min=1e-30)
    scale = (amax / 448.0).float()
    return (t.float() / scale).clamp(-448.0, 448.0).to(torch.float8_e4m3fn), scale


def mxfp8(t):
    """MXFP8 (E4M3 elements, one E8M0 scale per 32 along the rows): the shared exponent is
    floor(log2 amax) - 8 (the largest E4M3 exponent), elements saturate at 448."""
    import torch
    rows, kc = t.shape
    blk = t.float().reshape(rows, kc // 32, 32)
    amax = blk.abs().amax(-1).clamp(min=2.0 ** -126)
    e = torch.floor(torch.log2(amax)) - 8
    e = e.clamp(-127, 127)
    codes = (blk / torch.exp2(e)[..., None]).clamp(-448.0, 448.0).reshape(rows, kc).to(torch.float8_e4m3fn)
    return codes, (e + 127).to(torch.uint8).view(torch.float8_e8m0fnu)


def vendor_gemm(kind, a, b):
    """The vendor (hipBLASLt) product A B^T in bf16 for FP8 operands of fp8_per_tensor ("fp8") or
    mxfp8 ("mxfp8"); a and b are (codes, scale) pairs."""
    import torch
    return torch._scaled_mm(a[0], b[0].t(), scale_a=a[1], scale_b=b[1], out_dtype=torch.bfloat16)


def library_baselines(plan, avg_ms, steps, settle_s=0.1):
    """Vendor GEMMs (hipBLASLt through torch._scaled_mm) at every GEMM shape of the step, on the
    step's own operands converted to FP8 E4M3 once, outside timing: per-tensor FP8 and MXFP8
    (E8M0 scale per 32). The FP8 form of the method's step is the pages' baseline; these are its
    GEMMs alone (bf16 output, half the bytes of this library's FP32 output). Each shape is
    settled for `settle_s` seconds, then timed over K launches (host clock). A grouped launch's
    time is shared evenly among its products."""
    out = {"output": "bf16", "operands": "the step's bf16 operands, converted once outside timing", "gemms": {}}
    ours_s, tot = 0.0, {"fp8_per_tensor": 0.0, "mxfp8": 0.0}
    for (label, kind, spec, work), t in zip(plan.op_list, avg_ms):
        if kind != "gemm":
            continue
        ours_s += float(t) * 1e-3
        for okey in (p[2] for p in spec):
            library_baseline_entry(out, tot, plan, okey, float(t) / len(spec), len(spec), steps, settle_s)
    out["step_gemm_ms"] = {"this_library_mxfp4": round(ours_s * 1e3, 4),
                           "fp8_per_tensor": round(tot["fp8_per_tensor"] * 1e3, 4),
                           "mxfp8": round(tot["mxfp8"] * 1e3, 4)}
    return out


def library_baseline_entry(out, tot, plan, okey, t_ms, group, steps, settle_s):
    """Time the vendor GEMMs of one product (okey) and add its entry to out["gemms"]."""
    import torch
    A, B = gemm_operands_bf16(plan, okey)
    label = "gemm %s %s" % ({"F": "Fprop", "D": "Dgrad", "W": "Wgrad"}[okey[1]], okey[0])
    entry = {"shape": "%dx%dx%d" % (A.shape[0], B.shape[0], A.shape[1]),
             "this_library_us": round(t_ms * 1e3, 2)}
    if group > 1:
        entry["this_library_grouped"] = "1/%d of one launch for %d products" % (group, group)
    for name, conv, vk in (("fp8_per_tensor", fp8_per_tensor, "fp8"), ("mxfp8", mxfp8, "mxfp8")):
        try:
            a, b = conv(A), conv(B)
            f = lambda a=a, b=b, vk=vk: vendor_gemm(vk, a, b)  # noqa: E731
            t_end = time.perf_counter() + settle_s
            while time.perf_counter() < t_end:
                f()
                torch.cuda.synchronize()
            t0 = time.perf_counter()
            for _ in range(steps):
                f()
            torch.cuda.synchronize()
            us = (time.perf_counter() - t0) * 1e6 / steps
            entry[name + "_us"] = round(us, 2)
            tot[name] += us * 1e-6
            del a, b
        except Exception as e:  # a baseline the runtime does not offer is reported, not fatal
            entry[name + "_error"] = str(e)[:160]
            tot[name] = float("nan")
    del A, B
    out["gemms"][label] = entry


def main():
    args = parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py runs on exactly one GPU: this library has no multi-GPU path. Use --gpus 1.",
              file=sys.stderr)
        return 2
    import numpy as np
    import torch
    import mxfp4_block_scaled_h16_amd as mx

    if args.rht and args.hadamard == 0:
        print("--rht needs --hadamard 16 or 32", file=sys.stderr)
        return 2
    h = args.hadamard | (mx.RHT if args.rht else 0)
    hsize = args.hadamard
    rot_name = ("RHT%d" if args.rht else "H%d") % hsize
    desc, projs, passes, M = WORKLOADS[args.workload]
    in_bytes = 0
    for name, K, N in projs:
        in_bytes += 2 * (N * K + M * N)
    in_bytes += 2 * M * sum(K for name, K, N in projs)
    sets = max(1, min(8, -(-(1 << 30) // in_bytes)))
    plan = Plan(mx, torch, args.workload, h, sets, dual=not args.separate_quant, group=not args.no_group)
    torch.cuda.synchronize()
    graphs = None if args.no_graph else capture_steps(plan)

    settle_steps = settle(plan, args.settle, graphs)
    ms_per_step, avg_ms, step_ms = run_timed(plan, args.steps, args.warmup, graphs)
    step_flops = sum(w for _, kind, _, w in plan.op_list if kind == "gemm")
    value = step_flops / (ms_per_step * 1e-3) / 1e12

    kernels = {}
    gemm_flops, gemm_s, q_bytes, q_s, gemm_bytes = 0.0, 0.0, 0.0, 0.0, 0
    for (label, kind, spec, work), t in zip(plan.op_list, avg_ms):
        entry = {"us": round(float(t) * 1e3, 2)}
        if kind == "gemm":
            entry["tflops"] = round(work / (t * 1e-3) / 1e12, 1)
            ra, rb = plan.out[spec[0][2]].shape
            kc = int(round(work / (2.0 * ra * rb * len(spec))))
            entry["shape"] = "%dx%dx%d" % (ra, rb, kc)
            if len(spec) > 1:
                entry["products"] = len(spec)
            entry["algorithmic_bytes"] = gemm_algorithmic_bytes(ra, rb, kc) * len(spec)
            gemm_flops += work
            gemm_s += float(t) * 1e-3
            gemm_bytes += entry["algorithmic_bytes"]
        else:
            nbytes = work * (DUAL_BYTES_PER_ELEM if kind == "dual" else QUANT_BYTES_PER_ELEM)
            entry["gbs"] = round(nbytes / (t * 1e-3) / 1e9, 1)
            entry["algorithmic_bytes"] = int(nbytes)
            q_bytes += nbytes
            q_s += float(t) * 1e-3
        kernels[label] = entry

    n_gemm = sum(1 for _, kind, _, _ in plan.op_list if kind == "gemm")
    achieved = gemm_flops / gemm_s / 1e12
    roofline = {"bound": "mfma", "achieved": round(achieved, 1), "peak": MXFP4_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / MXFP4_PEAK_TFLOPS, 4),
                "traffic": measured_traffic(args.workload),
                "mfma_busy": measured_mfma_busy(args.workload),
                "kernel": "gemm_mxfp4_pipelined (%d launches per step; achieved = GEMM FLOPs / GEMM time)" % n_gemm,
                "algorithmic_per_launch": "2*M*N*K = %.1f GFLOP average" % (gemm_flops / n_gemm / 1e9),
                "algorithmic_bytes_per_launch": int(gemm_bytes / n_gemm)}
    quantizer = {"gbs": round(q_bytes / q_s / 1e9, 1), "frac_of_hbm": round(q_bytes / q_s / 1e9 / HBM_PEAK_GBS, 4),
                 "bytes_per_elem": {"single": QUANT_BYTES_PER_ELEM, "dual": DUAL_BYTES_PER_ELEM},
                 "launches": "dual" if plan.dual else "separate", "us_per_step": round(q_s * 1e6, 1)}

    # the Fprop configuration taken literally (X and W along K, nearest rounding, one GEMM), timed
    # in the same run on the same inputs
    fprop = None
    if args.workload == "qkv" and "F" in passes:
        fplan = Plan(mx, torch, "qkv_fprop", h, sets, dual=False, host=plan.host)
        settle(fplan, min(args.settle, 0.25))
        f_ms, f_avg, _ = run_timed(fplan, args.steps, args.warmup)
        f_flops = sum(w for _, kind, _, w in fplan.op_list if kind == "gemm")
        f_gemm_s = sum(float(t) * 1e-3 for (_, kind, _, _), t in zip(fplan.op_list, f_avg) if kind == "gemm")
        f_q_s = sum(float(t) * 1e-3 for (_, kind, _, _), t in zip(fplan.op_list, f_avg) if kind != "gemm")
        fprop = {"workload": "Llama-3.1-8B QKV projection Fprop only, M=8192 K=4096 N=6144, %s, MXFP4 RNE" % rot_name,
                 "ms_per_step": round(f_ms, 4), "tflops": round(f_flops / (f_ms * 1e-3) / 1e12, 1),
                 "gemm_tflops": round(f_flops / f_gemm_s / 1e12, 1), "quant_us": round(f_q_s * 1e6, 1),
                 "launches": [label for label, _, _, _ in fplan.op_list]}
        del fplan

    entry = step_entry_points(plan, args.steps, args.warmup) if args.workload == "qkv" else None

    baselines = None
    if not args.no_library_baselines and passes == "FDW":
        baselines = library_baselines(plan, avg_ms, args.steps)
    valu = quantizer_valu(args.workload, plan, avg_ms)
    if valu is not None:
        quantizer["valu"] = valu

    if args.copy_calibration:
        buf = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        buf2 = torch.empty_like(buf)
        buf2.copy_(buf)
        torch.cuda.synchronize()

    ceilings = None
    if not args.no_ceilings:
        ceilings = machine_ceilings()
        roofline["ceiling"] = ceilings["mfma_fp4_tflops"]
        roofline["frac_of_ceiling"] = round(achieved / ceilings["mfma_fp4_tflops"], 4)
        quantizer["frac_of_copy_ceiling"] = round(q_bytes / q_s / 1e9 / ceilings["hbm_copy_gbs"], 4)

    qerr = quantization_error(plan, rows=8 if len(plan.op_list) < 12 else 4)
    cpu = None if args.no_cpu_baseline else cpu_baseline(plan, h)

    sizes = ", ".join("%s K=%d N=%d" % (n, k, nn) for n, k, nn in projs)
    line = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "mxfp4",
        "data": "synthetic",
        "config": {"workload": "%s, M=%d tokens, %s, %s, MXFP4 RNE (Philox SR on Wgrad operands)"
                               % (desc, M, sizes, rot_name),
                   "M": M, "hadamard": hsize, "randomized_hadamard": bool(args.rht), "passes": passes,
                   "input_sets": sets},
        "timing": {"settle_s": args.settle, "settle_steps": settle_steps,
                   "value": ("host clock over the K timed steps, each one replay of the step captured as one HIP "
                             "graph, no per-launch instrumentation" if graphs else
                             "host clock over the K timed steps launched from the host, no per-launch "
                             "instrumentation"),
                   "kernels": "a second pass of K steps launched from the host with fence-free HIP events around "
                              "every launch",
                   "instrumented_step_ms": {"median": round(float(np.median(step_ms)), 4),
                                            "min": round(float(step_ms.min()), 4),
                                            "max": round(float(step_ms.max()), 4)}},
        "roofline": roofline, "quantizer": quantizer, "kernels": kernels, "cpu_baseline": cpu,
    }
    if fprop is not None:
        line["fprop_only"] = fprop
    line["quantization_error"] = qerr
    if entry is not None:
        line["step_entry_points"] = entry
    if ceilings is not None:
        line["ceilings"] = ceilings
    if baselines is not None:
        line["library_baselines"] = baselines
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
