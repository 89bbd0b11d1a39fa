"""Seeded synthetic inputs for the fp16 TN GEMM and attention workloads.

This module is shared by the tests, the benchmark and the smoke check.  It
holds no GEMM arithmetic: it only turns a seed into fp16 / fp32 tensors of
the shapes and value distributions of the workloads, so that the HIP path
and the CPU oracle can be fed the very same stored bits.

Generator: SplitMix64 (Steele, Lea and Flood, "Fast Splittable Pseudorandom
Number Generators", OOPSLA 2014), used as a counter-based stream: draw i of
a stream with start state s is mix64(s + (i + 1) * GAMMA).  Each tensor of a
workload has its own stream, started at mix64(seed XOR (tensor_id << 32)).

Value maps (all computed in float64 and then rounded to the storage type
with numpy's round-to-nearest-even cast):
  uniform : 2 * ((x >> 11) * 2^-53) - 1              in [-1, 1)
  normal  : Box-Muller on two draws, cos branch        N(0, 1)
  integer : (x mod 7) - 3                              in {-3, ..., 3}
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)

TENSOR_A, TENSOR_B, TENSOR_C = 0, 1, 2
TENSOR_Q, TENSOR_K, TENSOR_V = 3, 4, 5


def mix64(z: np.ndarray) -> np.ndarray:
    """SplitMix64 output function (the variant-13 finaliser)."""
    z = np.asarray(z, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = (z ^ (z >> np.uint64(30))) * _M1
        z = (z ^ (z >> np.uint64(27))) * _M2
    return z ^ (z >> np.uint64(31))


def stream(seed: int, tensor_id: int, n: int) -> np.ndarray:
    """n draws of the SplitMix64 stream of one tensor, as uint64."""
    s0 = mix64(np.array([(seed ^ (tensor_id << 32)) & 0xFFFFFFFFFFFFFFFF],
                        dtype=np.uint64))[0]
    with np.errstate(over="ignore"):
        ctr = np.arange(1, n + 1, dtype=np.uint64) * GAMMA + s0
    return mix64(ctr)


def _unit53(x: np.ndarray) -> np.ndarray:
    return (x >> np.uint64(11)).astype(np.float64) * (2.0 ** -53)


def uniform_pm1(seed: int, tensor_id: int, n: int) -> np.ndarray:
    return 2.0 * _unit53(stream(seed, tensor_id, n)) - 1.0


def normal01(seed: int, tensor_id: int, n: int) -> np.ndarray:
    x = stream(seed, tensor_id, 2 * n)
    u1 = ((x[0::2] >> np.uint64(11)).astype(np.float64) + 1.0) * (2.0 ** -53)
    u2 = _unit53(x[1::2])
    return np.sqrt(-2.0 * np.log(u1)) * np.cos(2.0 * math.pi * u2)


def small_ints(seed: int, tensor_id: int, n: int) -> np.ndarray:
    x = stream(seed, tensor_id, n)
    return (x % np.uint64(7)).astype(np.int64).astype(np.float64) - 3.0


def make(kind: str, shape, seed: int, tensor_id: int, dtype=np.float16,
         scale: float = 1.0) -> np.ndarray:
    """A tensor of `shape`, filled in row-major order from one stream."""
    n = int(np.prod(shape)) if len(shape) else 1
    if kind == "uniform":
        v = uniform_pm1(seed, tensor_id, n)
    elif kind == "normal":
        v = normal01(seed, tensor_id, n)
    elif kind == "int":
        v = small_ints(seed, tensor_id, n)
    else:
        raise ValueError(f"unknown value kind {kind!r}")
    if scale != 1.0:
        v = v * scale
    return v.astype(dtype).reshape(shape)


@dataclass
class Workload:
    """One GEMM problem: D = alpha * A @ B^T + beta * C, batched."""
    name: str
    batch: int
    M: int
    N: int
    K: int
    alpha: float
    beta: float
    out_dtype: str                      # "f16" or "f32"
    A: np.ndarray = field(repr=False)   # (batch, M, K) float16
    B: np.ndarray = field(repr=False)   # (batch, N, K) float16
    C: np.ndarray | None = field(repr=False, default=None)  # (batch, M, N)

    @property
    def flops(self) -> int:
        return 2 * self.batch * self.M * self.N * self.K

    @property
    def algorithmic_bytes(self) -> int:
        es = 2 if self.out_dtype == "f16" else 4
        b = 2 * self.batch * (self.M * self.K + self.N * self.K)
        b += es * self.batch * self.M * self.N
        if self.beta != 0.0:
            b += es * self.batch * self.M * self.N
        return b


def _np_out(out_dtype: str):
    return np.float16 if out_dtype == "f16" else np.float32


def build(name: str, batch: int, M: int, N: int, K: int, alpha: float,
          beta: float, out_dtype: str, kind: str, seed: int,
          scale: float = 1.0, c_kind: str = "uniform") -> Workload:
    A = make(kind, (batch, M, K), seed, TENSOR_A, np.float16, scale)
    B = make(kind, (batch, N, K), seed, TENSOR_B, np.float16, scale)
    C = None
    if beta != 0.0:
        C = make(c_kind, (batch, M, N), seed, TENSOR_C, _np_out(out_dtype))
    return Workload(name, batch, M, N, K, alpha, beta, out_dtype, A, B, C)


SEED_BASE = 0x5EED0000

# The five workloads of the fp16 TN GEMM study, by number.  `int_values`
# swaps the A/B value distribution for small integers in {-3..3}, whose
# products and partial sums are exact in fp32 (bit-exact comparison).
WORKLOADS = {
    "c1_256": dict(batch=1, M=256, N=256, K=256, alpha=1.0, beta=0.0,
                   out_dtype="f16", kind="uniform", num=1),
    "c2_1024": dict(batch=1, M=1024, N=1024, K=1024, alpha=1.5, beta=0.5,
                    out_dtype="f32", kind="uniform", num=2),
    "c3_4096": dict(batch=1, M=4096, N=4096, K=4096, alpha=1.0, beta=0.0,
                    out_dtype="f16", kind="uniform", num=3),
    "c4a_ragged": dict(batch=1, M=1000, N=1030, K=1000, alpha=1.0, beta=0.0,
                       out_dtype="f32", kind="normal", num=4,
                       scale=1.0 / math.sqrt(1000)),
    "c4b_skinny": dict(batch=1, M=128, N=4096, K=8192, alpha=1.0, beta=0.0,
                       out_dtype="f32", kind="normal", num=4,
                       scale=1.0 / math.sqrt(8192)),
    "c5_qk": dict(batch=64, M=1024, N=1024, K=64, alpha=0.125, beta=0.0,
                  out_dtype="f32", kind="normal", num=5),
    # not one of the five: 17 x 17 tiles of 256, one wave plus a tail
    "tail_4352": dict(batch=1, M=4352, N=4352, K=4096, alpha=1.0, beta=0.0,
                      out_dtype="f16", kind="uniform", num=6),
}


def workload(name: str, int_values: bool = False) -> Workload:
    cfg = dict(WORKLOADS[name])
    num = cfg.pop("num")
    scale = cfg.pop("scale", 1.0)
    kind = cfg.pop("kind")
    if int_values:
        kind, scale = "int", 1.0
    seed = SEED_BASE + num + (0x100 if int_values else 0)
    if name == "c4b_skinny":
        seed += 0x10      # 4a and 4b share a workload number
    return build(name + ("_int" if int_values else ""), scale=scale,
                 kind=kind, seed=seed, **cfg)


def workload_shape(name: str) -> Workload:
    """The workload's sizes, alpha, beta and output type, without its data
    (A, B and C are None): for code that needs only the shape."""
    cfg = dict(WORKLOADS[name])
    return Workload(name, cfg["batch"], cfg["M"], cfg["N"], cfg["K"],
                    cfg["alpha"], cfg["beta"], cfg["out_dtype"], None, None,
                    None)


@dataclass
class AttentionWorkload:
    """One attention forward problem, O = softmax(scale * Q K^T) V, over
    `batch` independent heads."""
    name: str
    batch: int
    Lq: int
    Lk: int
    d: int
    scale: float
    out_dtype: str                      # "f16" or "f32"
    Q: np.ndarray = field(repr=False)   # (batch, Lq, d) float16
    K: np.ndarray = field(repr=False)   # (batch, Lk, d) float16
    V: np.ndarray = field(repr=False)   # (batch, Lk, d) float16

    @property
    def flops(self) -> int:
        """The two products: 2 * Lq * Lk * d for the scores, as many for
        P V."""
        return 4 * self.batch * self.Lq * self.Lk * self.d

    @property
    def algorithmic_bytes(self) -> int:
        es = 2 if self.out_dtype == "f16" else 4
        return self.batch * self.d * (2 * (self.Lq + 2 * self.Lk)
                                      + es * self.Lq)


# Attention workloads: the score product of the head-dimension-64 study
# (64 heads of 1024 queries and keys) completed into the forward pass, and
# a small ragged case.  Q, K and V are standard normal, as the score
# product's operands are.
ATTENTION_WORKLOADS = {
    "attn_small": dict(batch=2, Lq=200, Lk=300, d=64, scale=0.125,
                       out_dtype="f16", num=0x61),
    "attn_64x1024": dict(batch=64, Lq=1024, Lk=1024, d=64, scale=0.125,
                         out_dtype="f16", num=0x62),
}


def attention_workload(name: str, out_dtype: str | None = None,
                       magnitude: float = 1.0) -> AttentionWorkload:
    cfg = dict(ATTENTION_WORKLOADS[name])
    seed = SEED_BASE + cfg.pop("num")
    if out_dtype is not None:
        cfg["out_dtype"] = out_dtype
    b, Lq, Lk, d = cfg["batch"], cfg["Lq"], cfg["Lk"], cfg["d"]
    Q = make("normal", (b, Lq, d), seed, TENSOR_Q, np.float16, magnitude)
    K = make("normal", (b, Lk, d), seed, TENSOR_K, np.float16, magnitude)
    V = make("normal", (b, Lk, d), seed, TENSOR_V, np.float16)
    return AttentionWorkload(name, Q=Q, K=K, V=V, **cfg)
