"""Seeded synthetic inputs for LSH attention (shared by the tests, the
benchmark and the smoke check).

This module draws random numbers and stores them; it holds none of the
method's arithmetic.  Every workload is reproducible from (seed, stream):

    stream 0  qk noise            N(0, 1), float32
    stream 1  v                   N(0, 1), float32
    stream 2  rotations           N(0, 1), float32, shape [H][R][B/2][d]
    stream 3  cluster centres     N(0, 1), float32, shape [n_clusters][d]
    stream 4  cluster assignment  uniform integers in [0, n_clusters)

Mixture inputs (imbalanced buckets) are qk = centre[c] + spread * noise with
one set of centres per tensor, shared across batch and heads.  bf16 tensors
are the float32 draws rounded to nearest-even; they are handed to both the
GPU path (as bf16 bit patterns) and the oracle (upcast exactly).
"""
from __future__ import annotations

import dataclasses

import numpy as np


def rng(seed: int, stream: int) -> np.random.Generator:
    return np.random.default_rng([int(seed), int(stream)])


def normal(seed: int, stream: int, shape) -> np.ndarray:
    return rng(seed, stream).standard_normal(shape, dtype=np.float32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest, ties to even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float32 (exact)."""
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(
        np.float32)


@dataclasses.dataclass(frozen=True)
class Workload:
    """One problem size.  Layouts: qk, v [batch][heads][seq_len][head_dim];
    rot [heads][rounds][n_buckets/2][head_dim]."""
    name: str
    batch: int
    heads: int
    seq_len: int
    head_dim: int
    n_buckets: int
    n_rounds: int
    chunk_len: int
    causal: bool
    self_mask: bool
    dtype: str                 # "f32" or "bf16": storage of qk, v and rot
    seed: int
    n_clusters: int = 0        # 0: qk ~ N(0,1); else Gaussian mixture
    spread: float = 0.3
    # local chunked attention (no hashing): chunks before / after each chunk in
    # its window; None for the LSH workloads
    look_before: "int | None" = None
    look_after: "int | None" = None
    # storage of the per-round outputs between the attention and the combine:
    # "f32" rows, or "f16_scaled" (bf16 inputs only); "auto" = f16_scaled for
    # bf16 inputs, f32 for fp32 inputs
    o_format: str = "auto"

    @property
    def o16(self) -> bool:
        """Per-round outputs stored as scaled fp16 rows."""
        return self.dtype == "bf16" and self.o_format in ("auto", "f16_scaled")

    @property
    def is_local(self) -> bool:
        return self.look_before is not None

    @property
    def tokens(self) -> int:
        return self.batch * self.seq_len

    @property
    def token_rounds(self) -> int:
        return self.batch * self.heads * self.seq_len * self.n_rounds

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five benchmark shapes (all with d = 64, chunk = 64 and B = L / chunk).
WORKLOADS = {
    "tiny": Workload("tiny", 1, 1, 1024, 64, 16, 1, 64, False, True, "f32", 1),
    "small": Workload("small", 4, 8, 4096, 64, 64, 2, 64, True, True, "bf16", 2),
    "medium": Workload("medium", 1, 8, 16384, 64, 256, 4, 64, True, True, "bf16", 3,
                       n_clusters=32),
    "long": Workload("long", 1, 8, 65536, 64, 1024, 8, 64, True, True, "bf16", 4),
    "verylong": Workload("verylong", 1, 4, 524288, 64, 8192, 2, 64, True, True, "bf16", 5,
                         n_clusters=256),
    # local chunked attention: one chunk of look-back and one of look-ahead
    # (encoder-style, so not causal), the headline shape otherwise
    "local_long": Workload("local_long", 1, 8, 65536, 64, 1, 1, 64, False, True, "bf16", 6,
                           look_before=1, look_after=1),
}


def _storage(x32: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return bf16_bits(x32)
    if dtype == "f32":
        return np.ascontiguousarray(x32, dtype=np.float32)
    raise ValueError(f"unknown dtype {dtype!r}")


def to_f64(stored: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 value of a stored tensor."""
    if dtype == "bf16":
        return bf16_to_f32(stored).astype(np.float64)
    return np.asarray(stored, dtype=np.float64)


def make_inputs(w: Workload) -> dict:
    """Stored tensors {'qk', 'v', 'rot'} (uint16 bf16 bits or float32)."""
    shape = (w.batch, w.heads, w.seq_len, w.head_dim)
    if w.n_clusters > 0:
        centres = normal(w.seed, 3, (w.n_clusters, w.head_dim))
        assign = rng(w.seed, 4).integers(0, w.n_clusters, size=shape[:3])
        qk = centres[assign]
        qk += np.float32(w.spread) * normal(w.seed, 0, shape)
    else:
        qk = normal(w.seed, 0, shape)
    v = normal(w.seed, 1, shape)
    half = w.n_buckets // 2
    rot = normal(w.seed, 2, (w.heads, w.n_rounds, half, w.head_dim))
    return {"qk": _storage(qk, w.dtype), "v": _storage(v, w.dtype),
            "rot": _storage(rot, w.dtype)}


# ---------------------------------------------------------------- layer
@dataclasses.dataclass(frozen=True)
class LayerWorkload:
    """One reversible layer: residual stream [batch][seq_len][d_model] fp32,
    heads = d_model / 64, LSH attention with n_buckets / n_rounds, FFN hidden
    width d_ff evaluated ffn_chunk tokens at a time (0 = all)."""
    name: str
    batch: int
    seq_len: int
    d_model: int
    d_ff: int
    n_buckets: int
    n_rounds: int
    causal: bool
    self_mask: bool
    ffn_chunk: int
    seed: int

    @property
    def heads(self) -> int:
        return self.d_model // 64


LAYER_WORKLOADS = {
    # the headline attention shape inside one layer: 8 heads of 64 features,
    # a 4x feed-forward expansion evaluated 32,768 tokens at a time
    "layer_long": LayerWorkload("layer_long", 1, 65536, 512, 2048, 1024, 8, True, True, 32768, 8),
}


def make_layer_inputs(w: LayerWorkload) -> dict:
    """Seeded inputs of one layer: x1, x2 fp32 ~ N(0, 1); weights bf16 bit
    patterns ~ N(0, 1/fan_in) stored [out][in]; biases fp32 ~ N(0, 0.1^2);
    rotations bf16 ~ N(0, 1) [H][R][B/2][64].  Streams 10..19 of the seed."""
    D, F, H = w.d_model, w.d_ff, w.heads
    shape = (w.batch, w.seq_len, D)

    def wmat(stream, n_out, n_in):
        return bf16_bits(normal(w.seed, stream, (n_out, n_in)) / np.float32(np.sqrt(n_in)))

    return {
        "x1": normal(w.seed, 10, shape),
        "x2": normal(w.seed, 11, shape),
        "w_qk": wmat(12, D, D),
        "w_v": wmat(13, D, D),
        "w_o": wmat(14, D, D),
        "rot": bf16_bits(normal(w.seed, 15, (H, w.n_rounds, w.n_buckets // 2, 64))),
        "w_1": wmat(16, F, D),
        "b_1": normal(w.seed, 17, (F,)) * np.float32(0.1),
        "w_2": wmat(18, D, F),
        "b_2": normal(w.seed, 19, (D,)) * np.float32(0.1),
    }
