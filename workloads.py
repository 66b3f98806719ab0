"""Seeded synthetic inputs for the W4A16 GEMM (shared by tests and bench).

This module draws raw inputs only -- fp16 activations, integer codes 0..15,
integer zeros 0..15 and fp16 scales -- and holds none of the method's
arithmetic (no packing, no dequantization, no product).  Both the GPU path and
the CPU oracle start from what it returns.

The workloads stand in for the only one the source pages measure: Llama-2-7B
decode at batch 1..128 (lmdeploy PR "[Feature] Blazing fast W4A16 inference",
benchmark table), with batch mapped to M and the Llama-2 7B / 70B linear-layer
shapes as (N, K).  There is no checkpoint; values are random and only their
distributions are modelled.

Draw order, fixed: X (fp32 N(0,1), optional x20 outlier columns, then RNE to
fp16), codes (uniform 0..15, [N, K]), zeros (uniform 0..15, [N, G]; skipped
when symmetric), scales (fp64 U[0.002, 0.02] then RNE to fp16, [N, G]).
"""
from __future__ import annotations

import zlib
from dataclasses import dataclass

import numpy as np

# Llama-2 linear-layer shapes (N, K).
LLAMA7B_SHAPES = {
    "o_proj": (4096, 4096),
    "qkv": (12288, 4096),
    "gate_up": (22016, 4096),
    "down": (4096, 11008),
}
LLAMA70B_SHAPES = {
    "qkv": (10240, 8192),
    "o_proj": (8192, 8192),
    "gate_up": (57344, 8192),
    "down": (8192, 28672),
}
DECODE_M = (1, 4, 8, 16, 32)
PREFILL_M = (64, 128, 256, 512, 2048)
L70B_M = (1, 16, 128, 1024)
EDGE_M = (1, 7, 33, 257)
EDGE_G = (32, 64, 128, 256)


@dataclass
class Case:
    X: np.ndarray        # fp16 [M, K]
    codes: np.ndarray    # uint8 [N, K], values 0..15
    zeros: np.ndarray    # uint8 [N, G] or None when symmetric
    scales: np.ndarray   # fp16 [N, G]
    K: int
    g: int
    symmetric: bool

    @property
    def M(self):
        return self.X.shape[0]

    @property
    def N(self):
        return self.codes.shape[0]

    @property
    def G(self):
        return -(-self.K // self.g)

    def with_m(self, M):
        return Case(self.X[:M], self.codes, self.zeros, self.scales, self.K,
                    self.g, self.symmetric)


def shape_seed(family: str, N: int, K: int, g: int, symmetric: bool) -> int:
    """Seed of one (workload family, shape, group size, symmetry) case."""
    tag = f"w4a16/{family}/N{N}/K{K}/g{g}/{'sym' if symmetric else 'asym'}"
    return zlib.crc32(tag.encode())


def draw(M: int, N: int, K: int, g: int, symmetric: bool, seed: int,
         outliers: bool = False, scale_lo: float = 0.002,
         scale_hi: float = 0.02) -> Case:
    rng = np.random.default_rng(seed)
    x32 = rng.standard_normal((M, K), dtype=np.float32)
    if outliers:
        n_out = int(round(0.01 * K))
        cols = rng.choice(K, size=n_out, replace=False)
        x32[:, cols] *= np.float32(20.0)
    X = x32.astype(np.float16)
    codes = rng.integers(0, 16, size=(N, K), dtype=np.uint8)
    G = -(-K // g)
    zeros = None if symmetric else rng.integers(0, 16, size=(N, G), dtype=np.uint8)
    scales = rng.uniform(scale_lo, scale_hi, size=(N, G)).astype(np.float16)
    return Case(X, codes, zeros, scales, K, g, symmetric)


def exact_family(M: int, N: int, K: int, g: int, symmetric: bool, seed: int) -> Case:
    """Inputs whose exact product is representable in fp32 for any summation
    order: X integers in [-3, 3]; scales 2^-e with e drawn per group in 4..7;
    codes and zeros uniform 0..15.  Every partial sum is a multiple of 2^-7
    below 2^17 in magnitude for K <= 28672."""
    rng = np.random.default_rng(seed)
    X = rng.integers(-3, 4, size=(M, K)).astype(np.float16)
    codes = rng.integers(0, 16, size=(N, K), dtype=np.uint8)
    G = -(-K // g)
    zeros = None if symmetric else rng.integers(0, 16, size=(N, G), dtype=np.uint8)
    e = rng.integers(4, 8, size=(N, G))
    scales = np.ldexp(1.0, -e).astype(np.float16)
    return Case(X, codes, zeros, scales, K, g, symmetric)


def tiny_case() -> Case:
    """M=4, K=512, N=512, g=128, asymmetric, seed 0."""
    return draw(4, 512, 512, 128, False, seed=0)


# ---------------------------------------------------------------------------
# fp16 weights for the quantizer (the step upstream of the GEMM).
# ---------------------------------------------------------------------------
WEIGHT_KINDS = ("normal", "outliers", "extremes", "positive", "sparse", "constant")


def draw_weight(N: int, K: int, kind: str, seed: int) -> np.ndarray:
    """fp16 [N, K] weight (values drawn in fp64, then RNE to fp16):
    normal    N(0, 0.02^2), the scale of a trained linear layer;
    outliers  normal with 1% of entries x300;
    extremes  random sign * 2^U{-24..15} * U[1, 1.99): the whole fp16 range,
              subnormals included;
    positive  |N(0, 1)| + 1 (no zero or negative value in a group);
    sparse    N(0, 1) with 90% of entries 0;
    constant  each row one value (every group constant; some rows all 0)."""
    rng = np.random.default_rng(seed)
    if kind == "normal":
        W = rng.standard_normal((N, K)) * 0.02
    elif kind == "outliers":
        W = rng.standard_normal((N, K)) * 0.02
        W[rng.random((N, K)) < 0.01] *= 300
    elif kind == "extremes":
        W = (rng.choice([-1.0, 1.0], (N, K)) * np.ldexp(1.0, rng.integers(-24, 16, (N, K)))
             * rng.uniform(1.0, 1.99, (N, K)))
    elif kind == "positive":
        W = np.abs(rng.standard_normal((N, K))) + 1.0
    elif kind == "sparse":
        W = rng.standard_normal((N, K))
        W[rng.random((N, K)) < 0.9] = 0.0
    elif kind == "constant":
        v = rng.standard_normal((N, 1))
        v[rng.random((N, 1)) < 0.25] = 0.0
        W = np.repeat(v, K, axis=1)
    else:
        raise ValueError(kind)
    return W.astype(np.float16)


def draw_tie_weight(N: int, K: int, g: int, symmetric: bool, seed: int) -> np.ndarray:
    """fp16 [N, K] weight dense in exact rounding ties for a quantizer with
    group size g: per row and group, a step s = m * 2^e (m odd in 33..63, e in
    -22..-6, so every multiple below is an exact fp16 value); the group's
    first two columns are -7 s and 8 s (7 s when symmetric), which make s the
    group's scale under a range / 15 (max / 7) rule; the other columns are
    (k + 1/2) s or k s with k uniform in -7..6, half each."""
    rng = np.random.default_rng(seed)
    G = -(-K // g)
    m = rng.integers(16, 32, (N, G)) * 2 + 1
    e = rng.integers(-22, -5, (N, G))
    step = np.ldexp(m.astype(np.float64), e)
    gi = np.arange(K) // g
    k = rng.integers(-7, 7, (N, K)).astype(np.float64)
    half = rng.random((N, K)) < 0.5
    W = (k + np.where(half, 0.5, 0.0)) * step[:, gi]
    first = np.arange(K) % g == 0
    W[:, first] = -7 * step
    second = np.arange(K) % g == 1
    W[:, second] = (7 if symmetric else 8) * step[:, gi[second]]
    out = W.astype(np.float16)
    assert np.array_equal(out.astype(np.float64), W)
    return out


# ---------------------------------------------------------------------------
# bfloat16 inputs (the bf16 variant): the same draws, encoded as bfloat16 bit
# patterns (uint16) by round-to-nearest-even of the fp32 value.
# ---------------------------------------------------------------------------
def f32_to_bf16_bits(x) -> np.ndarray:
    """Input encoding: float32 values -> bfloat16 bit patterns, nearest-even
    (finite inputs)."""
    u = np.ascontiguousarray(np.asarray(x, np.float32)).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


@dataclass
class CaseBF16:
    X: np.ndarray        # bf16 bits [M, K]
    codes: np.ndarray    # uint8 [N, K]
    zeros: np.ndarray    # uint8 [N, G] or None when symmetric
    scales: np.ndarray   # bf16 bits [N, G]
    K: int
    g: int
    symmetric: bool

    @property
    def M(self):
        return self.X.shape[0]

    @property
    def N(self):
        return self.codes.shape[0]


def draw_bf16(M: int, N: int, K: int, g: int, symmetric: bool, seed: int) -> CaseBF16:
    """As draw(), in the same order, with X and scales encoded as bfloat16."""
    rng = np.random.default_rng(seed)
    G = -(-K // g)
    X = f32_to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
    codes = rng.integers(0, 16, (N, K), dtype=np.uint8)
    zeros = None if symmetric else rng.integers(0, 16, (N, G), dtype=np.uint8)
    scales = f32_to_bf16_bits(rng.uniform(0.002, 0.02, (N, G)).astype(np.float32))
    return CaseBF16(X, codes, zeros, scales, K, g, symmetric)


def exact_family_bf16(M: int, N: int, K: int, g: int, symmetric: bool, seed: int) -> CaseBF16:
    """Integer X in [-3, 3] and power-of-two scales 2^-e (e in 4..7), as
    bfloat16: every product and partial sum is exact in fp32."""
    rng = np.random.default_rng(seed)
    G = -(-K // g)
    X = f32_to_bf16_bits(rng.integers(-3, 4, (M, K)).astype(np.float32))
    codes = rng.integers(0, 16, (N, K), dtype=np.uint8)
    zeros = None if symmetric else rng.integers(0, 16, (N, G), dtype=np.uint8)
    scales = f32_to_bf16_bits(np.ldexp(1.0, -rng.integers(4, 8, (N, G))).astype(np.float32))
    return CaseBF16(X, codes, zeros, scales, K, g, symmetric)
