"""Seeded synthetic inputs shaped like the Llama-3.1-8B linear layers (shared by tests and bench).

This module holds no quantization, rotation or GEMM arithmetic: it only draws random tensors
and rounds them to bfloat16 bit patterns. The training workload of the method (Llama-3.1-8B
pretraining on C4 under MLPerf settings; gist.science summary of "MXFP4 LLM pretraining",
section 방법론 / Methodology) is not available here; these draws stand in for its activations,
weights and gradients, with outlier activation channels and heavy-tailed gradients because the
summary names activation and gradient outliers as what amplifies quantization error
(section 문제 제기 / Problem statement).

Recipe (every tensor): numpy.random.default_rng(seed), draws in the order listed per workload,
float32 values rounded to bfloat16 by round-to-nearest-even, returned as uint16 bit patterns.
  X  ~ N(0, 1), with round(0.001 * K) channels (columns) multiplied by 50 before rounding
  W  ~ N(0, 0.02^2)
  dY ~ 1e-3 * Student-t(nu = 3)
"""
import numpy as np


def bf16_bits(a) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return uint16 bit patterns."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    bits = a.view(np.uint32).astype(np.uint64)
    rounded = (bits + 0x7FFF + ((bits >> 16) & 1)) >> 16
    nan = np.isnan(a)
    out = rounded.astype(np.uint16)
    if nan.any():
        out[nan] = 0x7FC0
    return out


def bf16_to_f32(b) -> np.ndarray:
    """Widen bfloat16 bit patterns to float32 (exact)."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def normal(rng, shape, std=1.0) -> np.ndarray:
    v = rng.standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        v *= np.float32(std)
    return v


def student_t(rng, shape, nu=3.0, scale=1e-3) -> np.ndarray:
    return (rng.standard_t(nu, size=shape) * scale).astype(np.float32)


def activations(rng, m, k, outliers=True) -> np.ndarray:
    """X[m, k] ~ N(0,1) with round(0.001 k) outlier channels scaled by 50 (as bf16 bits)."""
    x = normal(rng, (m, k))
    if outliers:
        n_out = int(round(0.001 * k))
        if n_out:
            cols = rng.choice(k, size=n_out, replace=False)
            x[:, cols] *= np.float32(50.0)
    return bf16_bits(x)


def weights(rng, n, k) -> np.ndarray:
    return bf16_bits(normal(rng, (n, k), 0.02))


def grads(rng, m, n) -> np.ndarray:
    return bf16_bits(student_t(rng, (m, n)))


# Llama-3.1-8B projection shapes (in_features K, out_features N), 8192 tokens per batch.
LLAMA31_8B_PROJECTIONS = {
    "q": (4096, 4096), "k": (4096, 1024), "v": (4096, 1024), "o": (4096, 4096),
    "gate": (4096, 14336), "up": (4096, 14336), "down": (14336, 4096),
}


def linear_inputs(m, k, n, seed=0, outliers=True):
    """X[m,k], W[n,k], dY[m,n] for one linear layer, drawn in that order."""
    rng = np.random.default_rng(seed)
    x = normal(rng, (m, k))
    w = weights(rng, n, k)
    dy = grads(rng, m, n)
    if outliers:
        n_out = int(round(0.001 * k))
        if n_out:
            cols = rng.choice(k, size=n_out, replace=False)
            x[:, cols] *= np.float32(50.0)
    return bf16_bits(x), w, dy


def small_fprop(seed=0):
    """X 256x512 ~ N(0,1), W 256x512 ~ N(0, 0.02^2): the small single-GEMM case."""
    rng = np.random.default_rng(seed)
    x = bf16_bits(normal(rng, (256, 512)))
    w = weights(rng, 256, 512)
    return x, w


def down_wgrad(seed=0, m=8192, n=4096, k=14336):
    """dY[m, n] (heavy-tailed) and X[m, k] ~ N(0,1): the down-projection weight gradient."""
    rng = np.random.default_rng(seed)
    dy = grads(rng, m, n)
    x = bf16_bits(normal(rng, (m, k)))
    return dy, x


# The projections of one decoder layer grouped by the activation they read: q, k, v share the
# attention input, gate and up share the MLP input.
LLAMA31_8B_INPUT_OF = {"q": "attn_in", "k": "attn_in", "v": "attn_in", "o": "o_in",
                       "gate": "mlp_in", "up": "mlp_in", "down": "down_in"}


def llama_layer_inputs(seed=0, tokens=8192):
    """Inputs of every linear projection of one Llama-3.1-8B decoder layer at `tokens` tokens.

    Draw order: the activations attn_in, o_in, mlp_in (each N(0,1) with outlier channels) and
    down_in (N(0,1)); then per projection in LLAMA31_8B_PROJECTIONS order its W ~ N(0, 0.02^2)
    and its dY ~ 1e-3 Student-t(3). Returns (acts: name -> X[tokens, K] bits,
    per_proj: name -> (W[N, K] bits, dY[tokens, N] bits)).
    """
    rng = np.random.default_rng(seed)
    acts = {}
    for name, k in (("attn_in", 4096), ("o_in", 4096), ("mlp_in", 4096)):
        acts[name] = activations(rng, tokens, k, outliers=True)
    acts["down_in"] = activations(rng, tokens, 14336, outliers=False)
    per_proj = {}
    for name, (k, n) in LLAMA31_8B_PROJECTIONS.items():
        per_proj[name] = (weights(rng, n, k), grads(rng, tokens, n))
    return acts, per_proj
