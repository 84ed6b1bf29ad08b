"""Seeded synthetic inputs for the decoder-block workloads.

Shared by the CPU oracle's tests and by the GPU path's tests and benchmark.
This module holds shapes, value distributions, the random draw order and the
rounding of drawn values to a storage dtype; none of the block's arithmetic
lives here.

Draw recipe (one numpy PCG64 generator per call, seeded by ``seed``):
  training step: x, W_qkv, W_o, W_fc, W_proj, dY, in that order, each drawn as
    float64 ``standard_normal``; weights are then multiplied by 0.02
    (N(0, 0.02) weights, N(0, 1) activations and upstream gradients);
  decode step: x_new, W_qkv, W_o, W_fc, W_proj, K cache, V cache, then the
    cache lengths (all equal to ``cache_len``, or uniform integers in
    [ragged_lo, ragged_hi] when ``ragged``).
Each value is rounded to the storage dtype (float32: IEEE round-to-nearest-
even; bfloat16: float64 -> float32 -> bfloat16, both steps round to nearest
even).  The float64 copy returned next to the storage bits holds exactly the
rounded value, so the oracle and the GPU consume the same numbers.
"""
from __future__ import annotations

import dataclasses
import numpy as np

__all__ = [
    "BlockShape", "DecodeShape", "HeadShape", "WORKLOADS", "DECODE_WORKLOADS", "HEAD_WORKLOADS",
    "from_depth", "round_to", "to_storage", "from_storage",
    "make_block_inputs", "make_decode_inputs", "make_head_inputs", "ragged_lengths",
]


@dataclasses.dataclass(frozen=True)
class BlockShape:
    """Sizes of one decoder-block training step.

    B sequences of T tokens, width C = H*D, H heads of D = 128, MLP width F.
    dtype: 'f32' or 'bf16' (operand/storage type); gemm: 'native' or 'fp8'
    (the linear layers' GEMMs take OCP e4m3 operands with per-tensor scales).
    """
    B: int
    T: int
    C: int
    H: int
    F: int
    D: int = 128
    eps: float = 1e-6
    rope_base: float = 10000.0
    dtype: str = "bf16"
    gemm: str = "native"
    window: int = 0          # attention window (0: causal over the whole sequence)
    n_kv_head: int = 0       # key/value heads (0: as many as query heads)

    @property
    def G(self) -> int:
        return self.n_kv_head or self.H

    @property
    def N(self) -> int:
        return self.B * self.T

    def replace(self, **kw) -> "BlockShape":
        return dataclasses.replace(self, **kw)


@dataclasses.dataclass(frozen=True)
class DecodeShape:
    """Sizes of one KV-cache decode step: B sequences, one new token each,
    caches of capacity S_max per (sequence, head)."""
    B: int
    C: int
    H: int
    F: int
    S_max: int
    D: int = 128
    eps: float = 1e-6
    rope_base: float = 10000.0
    dtype: str = "bf16"
    window: int = 0
    n_kv_head: int = 0

    @property
    def G(self) -> int:
        return self.n_kv_head or self.H


@dataclasses.dataclass(frozen=True)
class HeadShape:
    """Sizes of the language-model head and loss: N final rows of width C,
    vocabulary V (a multiple of 64)."""
    N: int
    C: int
    V: int
    eps: float = 1e-6
    dtype: str = "bf16"


def from_depth(depth: int, aspect: int = 64, head_dim: int = 128) -> tuple[int, int, int]:
    """Width, heads and MLP width from the depth knob: width is depth*aspect
    rounded up to a multiple of the head size, heads = width/head size, MLP
    width = 4*width (nanochat README translation on the flicky.cc page,
    section on the single --depth knob, step 1; 4x MLP per the block)."""
    C = -(-depth * aspect // head_dim) * head_dim
    return C, C // head_dim, 4 * C


def _shape(depth: int, B: int, T: int, **kw) -> BlockShape:
    C, H, F = from_depth(depth)
    return BlockShape(B=B, T=T, C=C, H=H, F=F, **kw)


# The named workloads (sizes and distributions as the benchmark's configs
# state them; d20 is the speedrun width of the pages).
WORKLOADS = {
    "d6_f32": _shape(6, B=1, T=512, dtype="f32"),
    "d12_bf16": _shape(12, B=8, T=2048),
    "d20_bf16": _shape(20, B=32, T=2048),
    "d26_fp8": _shape(26, B=16, T=2048, gemm="fp8"),
    # a short-window layer of the SSSL pattern: window T/4
    "d20_bf16_swa": _shape(20, B=32, T=2048, window=512),
    # grouped-query attention at d20: ten query heads on two key/value heads
    "d20_bf16_gqa": _shape(20, B=32, T=2048, n_kv_head=2),
}
_C20, _H20, _F20 = from_depth(20)
HEAD_WORKLOADS = {
    # the d20 batch of 32 x 2048 tokens under a 65,536-token vocabulary
    "d20_head": HeadShape(N=32 * 2048, C=_C20, V=65536),
}
DECODE_WORKLOADS = {
    "d20_decode": DecodeShape(B=64, C=_C20, H=_H20, F=_F20, S_max=2049),
    "d20_decode_gqa": DecodeShape(B=64, C=_C20, H=_H20, F=_F20, S_max=2049, n_kv_head=2),
}


def round_to(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round float64 values to ``dtype`` ('f64', 'f32', 'bf16'); returns
    float64 holding the rounded values exactly."""
    x = np.asarray(x, dtype=np.float64)
    if dtype == "f64":
        return x.copy()
    x32 = x.astype(np.float32)
    if dtype == "f32":
        return x32.astype(np.float64)
    if dtype == "bf16":
        return from_storage(_bf16_bits(x32), "bf16")
    raise ValueError(dtype)


def _bf16_bits(x32: np.ndarray) -> np.ndarray:
    bits = x32.view(np.uint32).astype(np.uint64)
    bias = 0x7FFF + ((bits >> 16) & 1)
    return ((bits + bias) >> 16).astype(np.uint16)


def to_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    """Storage array for ``dtype``: float32 values, or bfloat16 bit patterns
    as uint16."""
    x32 = np.asarray(x, dtype=np.float64).astype(np.float32)
    if dtype == "f32":
        return x32
    if dtype == "bf16":
        return _bf16_bits(x32)
    raise ValueError(dtype)


def from_storage(bits: np.ndarray, dtype: str) -> np.ndarray:
    """Inverse of :func:`to_storage` (exact), as float64."""
    if dtype == "f32":
        return np.asarray(bits, dtype=np.float32).astype(np.float64)
    if dtype == "bf16":
        u32 = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
        return u32.view(np.float32).astype(np.float64)
    raise ValueError(dtype)


def make_block_inputs(shape: BlockShape, seed: int = 0) -> dict[str, np.ndarray]:
    """x [B,T,C], W_qkv [(H+2G)D,C] (3C without grouping), W_o [C,C],
    W_fc [F,C], W_proj [C,F], dy [B,T,C], float64 arrays holding values
    already rounded to shape.dtype."""
    B, T, C, F = shape.B, shape.T, shape.C, shape.F
    rng = np.random.default_rng(seed)
    out = {}
    for name, dims, scale in (
        ("x", (B, T, C), 1.0),
        ("w_qkv", ((shape.H + 2 * shape.G) * shape.D, C), 0.02),
        ("w_o", (C, C), 0.02),
        ("w_fc", (F, C), 0.02),
        ("w_proj", (C, F), 0.02),
        ("dy", (B, T, C), 1.0),
    ):
        v = rng.standard_normal(dims)
        if scale != 1.0:
            v *= scale
        out[name] = round_to(v, shape.dtype)
    return out


def ragged_lengths(B: int, lo: int, hi: int, seed: int = 0) -> np.ndarray:
    """B cache lengths, uniform integers in [lo, hi], from their own stream
    (default_rng(seed + 1))."""
    return np.random.default_rng(seed + 1).integers(lo, hi, size=B, endpoint=True).astype(np.int32)


def make_decode_inputs(shape: DecodeShape, seed: int = 0, cache_len: int | None = None,
                       ragged: bool = False, ragged_lo: int = 128,
                       ragged_hi: int | None = None) -> dict[str, np.ndarray]:
    """x [B,C], four weights, k_cache/v_cache [B,G,S_max,D] ~ N(0,1) and
    int32 lengths [B].  Slots at and beyond a sequence's length hold drawn
    values too (they must not influence the result)."""
    B, C, H, F, S, D = shape.B, shape.C, shape.H, shape.F, shape.S_max, shape.D
    G = shape.G
    rng = np.random.default_rng(seed)
    out = {}
    for name, dims, scale in (
        ("x", (B, C), 1.0),
        ("w_qkv", ((H + 2 * G) * D, C), 0.02),
        ("w_o", (C, C), 0.02),
        ("w_fc", (F, C), 0.02),
        ("w_proj", (C, F), 0.02),
        ("k_cache", (B, G, S, D), 1.0),
        ("v_cache", (B, G, S, D), 1.0),
    ):
        v = rng.standard_normal(dims)
        if scale != 1.0:
            v *= scale
        out[name] = round_to(v, shape.dtype)
    hi = S - 1 if ragged_hi is None else ragged_hi
    if ragged:
        lens = ragged_lengths(B, ragged_lo, hi, seed)
    else:
        lens = np.full(B, S - 1 if cache_len is None else cache_len)
    if np.any(lens + 1 > S) or np.any(lens < 0):
        raise ValueError("cache lengths must satisfy 0 <= len <= S_max-1")
    out["cache_len"] = lens.astype(np.int32)
    return out


def block_param_count(C: int, F: int) -> int:
    """Weights of one block: W_qkv 3C*C, W_o C*C, W_fc F*C, W_proj C*F."""
    return 3 * C * C + C * C + 2 * F * C


def make_head_inputs(shape: HeadShape, seed: int = 0, uncounted: float = 0.05,
                     counted_rows=None) -> dict[str, np.ndarray]:
    """x [N,C] ~ N(0,1) (final residual rows), w_lm [V,C] ~ N(0, 0.02), and
    int32 targets [N] uniform in [0, V).  A fraction `uncounted` of the rows
    get the target -1 (not counted); with `counted_rows` given, only those
    rows keep a target in [0, V)."""
    N, C, V = shape.N, shape.C, shape.V
    rng = np.random.default_rng(seed)
    out = {"x": round_to(rng.standard_normal((N, C)), shape.dtype),
           "w_lm": round_to(rng.standard_normal((V, C)) * 0.02, shape.dtype)}
    t = rng.integers(0, V, size=N)
    if counted_rows is not None:
        keep = np.zeros(N, dtype=bool)
        keep[list(counted_rows)] = True
        t = np.where(keep, t, -1)
    else:
        t = np.where(rng.random(N) < uncounted, -1, t)
    out["targets"] = t.astype(np.int32)
    return out
