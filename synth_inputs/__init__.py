"""Seeded synthetic inputs for the SharQ linear-layer path.

This module is shared by the CPU oracle's tests and by the HIP path's tests
and benchmark.  It holds no step of the method itself: it only draws random
activations, weights and norm gains, and rounds them to bfloat16 bit patterns.

The workloads stand in for the activations of the models evaluated in
"SharQ: Bridging Activation Sparsity and FP4 Quantization for LLM Inference"
(arXiv:2606.26587), abstract, sentence 7 (Llama-3.1-8B and others).  Neither
the weights nor the evaluation data are available, so the shapes follow
Llama-3.1-8B's linear layers (hidden 4096, QKV 6144, MLP 14336, gate+up 28672)
and a few channels are scaled up to model the input-dependent outliers that
the abstract (sentence 1) says dominate FP4 block scales.

Recipe (every config):
  * ``rng = numpy.random.default_rng(seed_x)``; draw the base values in
    float64 (``rng.standard_normal``, ``rng.standard_t`` ...);
  * ``rng.choice(K, n_out, replace=False)`` picks the outlier channels
    (columns k, shared by all rows), whose float64 values are multiplied by
    the outlier factor;
  * the float64 array is cast to float32 (round to nearest even) and then to
    bfloat16 by round-to-nearest-even on the float32 bits.
  * W uses its own ``default_rng(seed_w)`` and ``normal(0, 0.02, (N, K))``.
  * gamma (when asked for a non-unit one) is ``1 + 0.1 * N(0,1)`` from
    ``default_rng(seed_x + 500)``.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

MXFP4 = 0
NVFP4 = 1


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    m: int
    k: int
    n: int
    dist: str            # "normal" | "student_t4" | "silu_like"
    n_outlier: int
    outlier_scale: float
    norm: bool
    fmt: int
    seed_x: int
    seed_w: int


# The five Llama-3.1-8B-shaped workloads (tiny check, QKV prefill, MLP down
# prefill, decode gate+up, large NVFP4-style prefill).
WORKLOADS = {
    "tiny": Workload("tiny", 16, 256, 256, "normal", 4, 40.0, True, MXFP4, 1, 1001),
    "qkv_prefill": Workload("qkv_prefill", 2048, 4096, 6144, "student_t4", 41, 50.0, True, MXFP4, 2, 1002),
    "down_prefill": Workload("down_prefill", 2048, 14336, 4096, "silu_like", 72, 30.0, False, MXFP4, 3, 1003),
    "decode_gate_up": Workload("decode_gate_up", 16, 4096, 28672, "student_t4", 41, 50.0, True, MXFP4, 4, 1004),
    "nvfp4_prefill": Workload("nvfp4_prefill", 8192, 4096, 14336, "student_t4", 41, 50.0, True, NVFP4, 5, 1005),
}


# The four linear layers of one Llama-3.1-8B decoder layer, in order, for the
# layer-chain benchmark: (K, N, input distribution, outlier channels, outlier
# factor, RMSNorm before it).  QKV and gate+up read the residual stream
# through an RMSNorm (heavy-tailed, with outlier channels, as qkv_prefill);
# O reads the attention output (no norm; plain normal values); down reads
# SiLU(gate) * up (as down_prefill).
LAYER_LINEARS = {
    "qkv": (4096, 6144, "student_t4", 41, 50.0, True),
    "o": (4096, 4096, "normal", 0, 1.0, False),
    "gate_up": (4096, 28672, "student_t4", 41, 50.0, True),
    "down": (14336, 4096, "silu_like", 72, 30.0, False),
}


def layer_workload(linear: str, m: int, fmt: int = MXFP4) -> Workload:
    """One linear of the decoder-layer chain with m tokens (2048: prefill, 16:
    decode); seeds 20 + i for X and 1020 + i for W, i the linear's position."""
    i = list(LAYER_LINEARS).index(linear)
    k, n, dist, n_out, factor, norm = LAYER_LINEARS[linear]
    return Workload(f"layer_{linear}_m{m}", m, k, n, dist, n_out, factor, norm, fmt, 20 + i, 1020 + i)


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values (finite) to bfloat16, nearest-even, as uint16 bits."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    lsb = (u >> 16) & np.uint32(1)
    lsb += np.uint32(0x7FFF)
    lsb += u                      # no wrap-around for finite inputs
    lsb >>= np.uint32(16)
    return lsb.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _base(rng: np.random.Generator, dist: str, m: int, k: int) -> np.ndarray:
    if dist == "normal":
        return rng.standard_normal((m, k))
    if dist == "student_t4":
        return rng.standard_t(4.0, (m, k))
    if dist == "silu_like":
        # two independent draws a * sigmoid(b); a is drawn first
        a = rng.standard_normal((m, k))
        b = rng.standard_normal((m, k))
        return a / (1.0 + np.exp(-b))
    raise ValueError(f"unknown distribution {dist!r}")


def activations(dist: str, m: int, k: int, n_outlier: int, outlier_scale: float,
                seed: int) -> np.ndarray:
    """bf16 bits [m, k] of a seeded activation tensor with outlier channels."""
    rng = np.random.default_rng(seed)
    x = _base(rng, dist, m, k)
    if n_outlier > 0:
        cols = rng.choice(k, n_outlier, replace=False)
        x[:, cols] *= outlier_scale
    return f32_to_bf16_bits(x.astype(np.float32))


def weights(n: int, k: int, seed: int, std: float = 0.02) -> np.ndarray:
    """bf16 bits [n, k] of a seeded N(0, std) weight matrix."""
    rng = np.random.default_rng(seed)
    return f32_to_bf16_bits(rng.normal(0.0, std, (n, k)).astype(np.float32))


def gamma(k: int, seed: Optional[int]) -> np.ndarray:
    """bf16 bits [k] of an RMSNorm gain: all ones when seed is None."""
    if seed is None:
        return f32_to_bf16_bits(np.ones(k, dtype=np.float32))
    rng = np.random.default_rng(seed)
    return f32_to_bf16_bits((1.0 + 0.1 * rng.standard_normal(k)).astype(np.float32))


# Magnitudes of the E2M1 element format (OCP Microscaling v1.0).
E2M1_GRID = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)


def fp4_grid(rows: int, k: int, exp2: int, seed: int) -> np.ndarray:
    """bf16 bits [rows, k] of values drawn uniformly from the signed E2M1 grid
    times 2^exp2: a uniform 4-bit index from ``default_rng(seed)``, bit 3 the
    sign and bits 0-2 the magnitude's place in E2M1_GRID.  Block-scaled FP4
    holds every 32-block of such values exactly, and their products and sums
    stay exact in fp32 for the sizes used here, so these inputs make a GEMM's
    result independent of its summation order."""
    rng = np.random.default_rng(seed)
    idx = rng.integers(0, 16, (rows, k), dtype=np.uint8)
    mags = np.asarray(E2M1_GRID, dtype=np.float64) * 2.0 ** exp2
    table = f32_to_bf16_bits(np.concatenate([mags, -mags]).astype(np.float32))   # exact in bf16
    return table[idx]


def gate_up_output(m: int, f: int, seed: int, n_outlier: int = 72, outlier_scale: float = 30.0):
    """fp32 gate and up [m, f] standing in for the gate+up projection's output
    in front of the down projection: gate ~ N(0, 2^2), up ~ N(0, 1) with
    n_outlier up channels scaled by outlier_scale (drawn in that order from
    ``default_rng(seed)``, cast to float32)."""
    rng = np.random.default_rng(seed)
    g = 2.0 * rng.standard_normal((m, f))
    u = rng.standard_normal((m, f))
    if n_outlier > 0:
        u[:, rng.choice(f, n_outlier, replace=False)] *= outlier_scale
    return g.astype(np.float32), u.astype(np.float32)


# One mixture-of-experts layer of Qwen3-30B-A3B (hidden 2048, 128 experts of
# intermediate size 768, 8 experts a token): the grouped dual GEMM workload.
MOE_QWEN3_30B_A3B = {"hidden": 2048, "intermediate": 768, "experts": 128, "top_k": 8}


def moe_routing(tokens: int, experts: int, top_k: int, seed: int):
    """Seeded top-k routing: logits N(0, 1) [tokens, experts] plus a per-expert
    bias N(0, 0.5^2) (uneven expert loads), each token's top_k experts.
    Returns (row_index int32 [tokens * top_k]: the token of each (token,
    expert) pair, pairs sorted by expert then token; offsets int64
    [experts + 1]: expert e's pairs are rows offsets[e] .. offsets[e + 1])."""
    rng = np.random.default_rng(seed)
    logits = rng.standard_normal((tokens, experts)) + 0.5 * rng.standard_normal(experts)
    top = np.argsort(-logits, axis=1, kind="stable")[:, :top_k]
    tok = np.repeat(np.arange(tokens), top_k)
    exp = top.reshape(-1)
    order = np.lexsort((tok, exp))
    counts = np.bincount(exp, minlength=experts)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    return tok[order].astype(np.int32), offsets


def workload_x(w: Workload, m: Optional[int] = None) -> np.ndarray:
    return activations(w.dist, w.m if m is None else m, w.k, w.n_outlier, w.outlier_scale, w.seed_x)


def workload_w(w: Workload, n: Optional[int] = None) -> np.ndarray:
    return weights(w.n if n is None else n, w.k, w.seed_w)


def workload_gamma(w: Workload) -> Optional[np.ndarray]:
    return gamma(w.k, None) if w.norm else None


def outlier_count(frac: float, k: int) -> int:
    return int(round(frac * k))
