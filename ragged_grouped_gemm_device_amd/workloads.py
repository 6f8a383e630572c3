"""Seeded synthetic workloads for the dropless MoE expert MLP.

This module only draws random inputs and describes workload shapes. It holds
none of the method's arithmetic (no routing, layout, GEMM, activation or
quantization), so both the CPU oracle and the GPU path may use it.

Every tensor is drawn from numpy's PCG64 in float32 and, where the path takes
bf16, rounded to the nearest bf16 (ties to even) and returned as raw uint16
bit patterns. Sub-streams come from ``SeedSequence(seed).spawn`` in the fixed
order x, logits, W1, W2, dO.

Workload shapes follow the pages' descriptions:
  * "tiny": a correctness-sized MoE (top-2 over 8 experts).
  * "balanced": the grouped-GEMM microbenchmark shape on the NVIDIA CuTe DSL
    fusion-kernel page, section on published evidence (8 experts, 4096
    tokens per expert, K=8192, N=4096, BF16). The router logits carry a +64
    bias on expert t // 4096, so softmax top-1 routes exactly 4096 tokens to
    each expert with weight 1.0 in fp32.
  * "skewed": one GPU's share of a fine-grained MoE (32 local experts, top-8,
    d=7168, n=2048) with a Zipf-shaped expert bias so that several experts
    receive no tokens (the empty groups of the Transformer Engine page,
    section on the three components).
  * "train": a GPT-OSS-like training step (32 experts, top-4, d=n=2880).
  * "skewed-large": the skewed recipe at T=32768 (permuted tensors of 3.8 GB).
  * "mxfp8": the balanced shape with 1 % of activations scaled by 50.
"""
from __future__ import annotations

import dataclasses
import numpy as np


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    T: int          # tokens
    k: int          # experts per token
    E: int          # local experts
    d: int          # model dim
    n: int          # expert hidden dim (FC1 produces 2n = gate + up)
    seed: int
    routing: str    # "normal" | "balanced" | "zipf"
    x_std: float = 1.0
    w_std: float = 0.02
    outlier_p: float = 0.0
    outlier_scale: float = 1.0

    @property
    def M(self) -> int:
        return self.T * self.k


WORKLOADS = {
    "tiny": Workload("tiny", T=256, k=2, E=8, d=128, n=64, seed=1001, routing="normal"),
    "balanced": Workload("balanced", T=32768, k=1, E=8, d=8192, n=2048, seed=1002,
                         routing="balanced", w_std=0.01),
    "skewed": Workload("skewed", T=16384, k=8, E=32, d=7168, n=2048, seed=1003, routing="zipf"),
    "train": Workload("train", T=8192, k=4, E=32, d=2880, n=2880, seed=1004, routing="normal"),
    # the skewed shape at twice the tokens: every permuted [M_cap, d] tensor is 3.8 GB,
    # past what 32-bit byte offsets address from one base
    "skewed-large": Workload("skewed-large", T=32768, k=8, E=32, d=7168, n=2048, seed=1006,
                             routing="zipf"),
    "mxfp8": Workload("mxfp8", T=32768, k=1, E=8, d=8192, n=2048, seed=1005, routing="balanced",
                      w_std=0.01, outlier_p=0.01, outlier_scale=50.0),
}


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); return uint16 bits.

    Input preparation only (finite inputs): the GPU path receives bf16 tensors.
    """
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _normal_bf16(rng: np.random.Generator, shape, std: float, chunk: int = 1 << 24) -> np.ndarray:
    out = np.empty(int(np.prod(shape)), dtype=np.uint16)
    for s in range(0, out.size, chunk):
        e = min(out.size, s + chunk)
        v = rng.standard_normal(e - s, dtype=np.float32)
        if std != 1.0:
            v *= np.float32(std)
        out[s:e] = f32_to_bf16_bits(v)
    return out.reshape(shape)


def _streams(seed: int):
    return [np.random.Generator(np.random.PCG64(s)) for s in np.random.SeedSequence(seed).spawn(5)]


def make_logits(w: Workload, rng: np.random.Generator) -> np.ndarray:
    logits = rng.standard_normal((w.T, w.E), dtype=np.float32)
    if w.routing == "balanced":
        per = w.T // w.E
        logits[np.arange(w.T), np.arange(w.T) // per] += np.float32(64.0)
    elif w.routing == "zipf":
        # Zipf(1.2) log-popularity at inverse temperature 3 over a seeded
        # permutation of expert ranks: b_e = -3 * 1.2 * ln(rank_e).
        rank = rng.permutation(w.E) + 1
        bias = (-3.0 * 1.2 * np.log(rank.astype(np.float64))).astype(np.float32)
        logits += bias[None, :]
    return logits


def make_inputs(w: Workload, parts=("x", "logits", "w1", "w2", "dout")) -> dict:
    """Return the seeded inputs of a workload as numpy arrays.

    x    uint16 bf16 bits [T, d]
    logits float32 [T, E]
    w1   uint16 bf16 bits [E, d, 2n]  (gate/up interleaved by construction)
    w2   uint16 bf16 bits [E, n, d]
    dout uint16 bf16 bits [T, d]
    """
    rx, rl, r1, r2, rd = _streams(w.seed)
    out = {}
    if "x" in parts:
        x = _normal_bf16(rx, (w.T, w.d), w.x_std)
        if w.outlier_p > 0:
            sel = rx.random((w.T, w.d)) < w.outlier_p
            xf = bf16_bits_to_f32(x)
            xf[sel] *= np.float32(w.outlier_scale)
            x = f32_to_bf16_bits(xf)
        out["x"] = x
    if "logits" in parts:
        out["logits"] = make_logits(w, rl)
    if "w1" in parts:
        out["w1"] = _normal_bf16(r1, (w.E, w.d, 2 * w.n), w.w_std)
    if "w2" in parts:
        out["w2"] = _normal_bf16(r2, (w.E, w.n, w.d), w.w_std)
    if "dout" in parts:
        out["dout"] = _normal_bf16(rd, (w.T, w.d), 1.0)
    return out


def small(name: str, T: int, k: int, E: int, d: int, n: int, seed: int, routing: str = "normal",
          w_std: float = 0.02) -> Workload:
    """A custom-shaped workload for parity tests (same recipe, other sizes)."""
    return Workload(name, T=T, k=k, E=E, d=d, n=n, seed=seed, routing=routing, w_std=w_std)
