"""Seeded synthetic inputs for the GGUF quantized-matmul path.

This module only draws random numbers and names the workload shapes.  It
holds none of the method's arithmetic (no quantization, no dot products), so
both the CPU oracle's tests and the GPU path may take their inputs from it.

Distributions and shapes follow the pages' SmolLM2-135M workloads
("GGUF" page, section on running a GGUF in candle: hidden 576, 9 query heads
and 3 KV heads of dim 64, FFN 1536, vocabulary 49152, a 37-token prompt plus
270 generated tokens) with trained weights replaced by N(0, 0.02) draws and
activations by N(0, 1) draws.  Every array comes from NumPy's PCG64
``default_rng(seed).standard_normal`` in float64, scaled, then cast to float32.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Tuple

import numpy as np

W_SIGMA = 0.02

# Projection shapes of one SmolLM2-135M layer as (name, N=out, K=in).
SMOLLM2_LAYER = (
    ("q", 576, 576),
    ("k", 192, 576),
    ("v", 192, 576),
    ("o", 576, 576),
    ("gate", 1536, 576),
    ("up", 1536, 576),
    ("down", 576, 1536),
)
SMOLLM2_LAYERS = 30
SMOLLM2_VOCAB = 49152
SMOLLM2_HIDDEN = 576
PREFILL_TOKENS = 37 + 270  # prompt plus teacher-forced tokens


def normal_f32(seed: int, shape: Tuple[int, ...], scale: float = 1.0) -> np.ndarray:
    """float32 array of N(0, scale^2) draws from PCG64(seed)."""
    g = np.random.default_rng(seed)
    return (g.standard_normal(shape) * scale).astype(np.float32)


def weights_f32(seed: int, n: int, k: int) -> np.ndarray:
    return normal_f32(seed, (n, k), W_SIGMA)


def acts_f32(seed: int, m: int, k: int, scale: float = 1.0) -> np.ndarray:
    return normal_f32(seed, (m, k), scale)


@dataclass(frozen=True)
class Problem:
    """One y = x . W^T problem: which weights, which activations."""
    name: str
    n: int
    k: int
    m: int
    w_seed: int
    x_seed: int
    x_scale: float = 1.0
    x_rows_of: int = 0  # >0: x is the first m rows of an x drawn with this many rows

    def weights(self) -> np.ndarray:
        return weights_f32(self.w_seed, self.n, self.k)

    def acts(self) -> np.ndarray:
        rows = self.x_rows_of if self.x_rows_of > 0 else self.m
        x = acts_f32(self.x_seed, rows, self.k, self.x_scale)
        return np.ascontiguousarray(x[: self.m])


def c1_q_proj() -> Problem:
    """576x576 q_proj-shaped GEMV, one token."""
    return Problem("q_proj 576x576 M=1", 576, 576, 1, 101, 102)


def c2_lm_head() -> Problem:
    """Tied lm_head GEMV: 49152x576, one token, x scaled by 0.5."""
    return Problem("lm_head 49152x576 M=1", 49152, 576, 1, 201, 202, 0.5)


def c3_ffn_down(m: int) -> Problem:
    """ffn_down 576x1536 (6 super-blocks of 256 per row), M in {1, 37}."""
    assert m in (1, 37)
    return Problem(f"ffn_down 576x1536 M={m}", 576, 1536, m, 301, 302, 1.0, 37)


def c4_prefill() -> List[Problem]:
    """All 30 layers' projections plus the tied lm_head, M=307 tokens."""
    out = []
    for layer in range(SMOLLM2_LAYERS):
        for p, (name, n, k) in enumerate(SMOLLM2_LAYER):
            out.append(Problem(f"L{layer}.{name} {n}x{k} M=307", n, k, PREFILL_TOKENS,
                               4000 + 10 * layer + p, 4500 + 10 * layer + p))
    out.append(Problem("lm_head 49152x576 M=307", SMOLLM2_VOCAB, SMOLLM2_HIDDEN,
                       PREFILL_TOKENS, 4999, 4998))
    return out


C5_N, C5_K, C5_LAYERS, C5_MMAX = 14336, 4096, 8, 512


def c5_layer(layer: int, m: int) -> Problem:
    """HBM-resident scale-up: 14336x4096, 8 stacked layers, M in {1, 8, 512}."""
    return Problem(f"scaleup L{layer} 14336x4096 M={m}", C5_N, C5_K, m,
                   5000 + layer, 5100, 1.0, C5_MMAX)


def integer_acts(seed: int, m: int, k: int, block: int) -> np.ndarray:
    """Integer-valued activations in [-127, 127] whose every `block`-long run
    along a row contains +127 or -127 (so an absmax/127 scale is exactly 1)."""
    g = np.random.default_rng(seed)
    x = g.integers(-127, 128, size=(m, k)).astype(np.float32)
    nb = k // block
    pos = g.integers(0, block, size=(m, nb))
    sgn = np.where(g.integers(0, 2, size=(m, nb)) == 0, -1.0, 1.0).astype(np.float32)
    for r in range(m):
        for b in range(nb):
            x[r, b * block + pos[r, b]] = 127.0 * sgn[r, b]
    return x


def tie_rows(seed: int, k: int) -> np.ndarray:
    """Two activation rows built around the quantizers' tie rules (values only).

    Row 0: every 32-value block holds 127 (so an absmax/127 scale is exactly
    1) and the half-way values 2.5, -2.5, 0.5 beside N(0,1) draws.  Row 1:
    every 256-value block holds +8 and -8 at offsets 5 and 9 (the order of the
    signs alternating from block to block) above N(0, 0.25) draws, so its two
    largest magnitudes tie with opposite signs."""
    x = np.stack([normal_f32(seed, (k,)), normal_f32(seed + 1, (k,), 0.5)])
    for b in range(k // 32):
        x[0, 32 * b: 32 * b + 4] = [127.0, 2.5, -2.5, 0.5]
    for sb in range(k // 256):
        s = 1.0 if sb % 2 == 0 else -1.0
        x[1, 256 * sb + 5], x[1, 256 * sb + 9] = 8.0 * s, -8.0 * s
    return x


def random_bytes(seed: int, n: int) -> np.ndarray:
    return np.random.default_rng(seed).integers(0, 256, size=n, dtype=np.uint8)
