"""Seeded synthetic inputs for the rotated W4A4 linear layer.

This module only draws random numbers and names shapes; it holds none of the
method's arithmetic (no rotation, no quantization, no GEMM).  Both the CPU
oracle tests and the GPU path take their inputs from here.

Workloads (shapes follow the LLaMA-2-7B / LLaMA-2-70B projections the pages
quantize; distributions add outlier channels and a massive-activation pivot
token, the failure case FlatQuant's article describes in its section 2.2):

  tiny     X [16, 256] N(0,1), 4 outlier channels x50; W [256, 256] N(0, 0.02);
           full 256-point Walsh-Hadamard; seed 0.
  llama7b  X [2048, 4096] N(0,1), 16 outlier channels x30, token 0 x100;
           W [4096, 4096] N(0, 0.02); full 4096-point Walsh-Hadamard.
  gsr      X as llama7b (own seed); W [11008, 4096]; block-diagonal of 64
           sequency-ordered 64x64 Walsh blocks; activation clip ratio 0.9.
  flat     X as llama7b (own seed); P1, P2 = I + N(0,1)/64 (64x64, fp32);
           per-channel scale s ~ U(0.5, 2); activation clip ratio 0.95;
           W [4096, 4096].
  quik     X [T, 8192] N(0,1), 256 outlier columns x40 kept in fp16, T = 4096
           (prefill) or the first 8 rows of it (decode); W [28672, 8192];
           asymmetric per-token INT4 on the 7936 normal columns.
  kv       the KV cache of one LLaMA-2-7B attention layer over 2048 tokens,
           32 heads of 128 channels: keys [2048, 4096] N(0,1) with 16
           outlier channels x30, values [2048, 4096] N(0,1); keys take R3
           (a 128-point Walsh-Hadamard per head), both are quantized
           group-wise asymmetric INT4 with groups of 128 channels.
  quik8_down  the LLaMA-2-70B down projection in QUIK's 8-bit form:
           X [4096, 28672] N(0,1) with 896 outlier columns x40 kept in fp16
           (256 per 8192 input features, scaled to 28672), W [8192, 28672];
           per-token asymmetric INT8 activations, per-channel INT8 weights.
  quik8_decode  the same layer at decode: the first 8 rows of that X.

Draw order per workload (numpy Generator, PCG64): outlier channel indices
(choice without replacement, sorted), X (standard normal, scaled, cast to fp16
once with round-to-nearest-even), W (standard normal x 0.02, cast to fp16),
then the affine factors and channel scales for "flat", the values for "kv".
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

__all__ = ["Workload", "WORKLOADS", "get", "make_inputs", "make_activations",
           "make_weights", "make_affine"]


@dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    T: int
    K: int
    N: int
    rot: str                      # "hadamard" | "gsr" | "kron" | "none" | "r3"
    block: int = 0                # GSR block size; r3: head size = quantization group
    n1: int = 0                   # Kronecker factor sizes (K == n1 * n2)
    n2: int = 0
    clip_x: float = 1.0           # activation clip ratio
    clip_w: float = 1.0           # weight clip ratio
    asym: bool = False            # asymmetric per-token activations (QUIK)
    n_outlier_ch: int = 0         # channels scaled by outlier_mult
    outlier_mult: float = 1.0
    pivot_mult: float = 1.0       # token 0 multiplier
    n_out: int = 0                # fp16-kept outlier columns (QUIK)
    bits: int = 4                 # code width of activations and weights
    decode_rows: int = 0          # >0: the decode variant keeps the first rows
    extra: dict = field(default_factory=dict)

    @property
    def k_int(self) -> int:
        """Columns that go through the INT4 path."""
        return self.K - self.n_out


WORKLOADS = {
    "tiny": Workload("tiny", 0, 16, 256, 256, "hadamard",
                     n_outlier_ch=4, outlier_mult=50.0),
    "llama7b": Workload("llama7b", 1, 2048, 4096, 4096, "hadamard",
                        n_outlier_ch=16, outlier_mult=30.0, pivot_mult=100.0),
    "gsr": Workload("gsr", 2, 2048, 4096, 11008, "gsr", block=64, clip_x=0.9,
                    n_outlier_ch=16, outlier_mult=30.0, pivot_mult=100.0),
    "flat": Workload("flat", 3, 2048, 4096, 4096, "kron", n1=64, n2=64,
                     clip_x=0.95, n_outlier_ch=16, outlier_mult=30.0,
                     pivot_mult=100.0),
    "quik_prefill": Workload("quik_prefill", 4, 4096, 8192, 28672, "none",
                             asym=True, n_outlier_ch=256, outlier_mult=40.0,
                             n_out=256),
    "quik_decode": Workload("quik_decode", 4, 4096, 8192, 28672, "none",
                            asym=True, n_outlier_ch=256, outlier_mult=40.0,
                            n_out=256, decode_rows=8),
    "kv": Workload("kv", 5, 2048, 4096, 0, "r3", block=128, asym=True,
                   n_outlier_ch=16, outlier_mult=30.0),
    "quik8_down": Workload("quik8_down", 6, 4096, 28672, 8192, "none", asym=True,
                           n_outlier_ch=896, outlier_mult=40.0, n_out=896, bits=8),
    "quik8_decode": Workload("quik8_decode", 6, 4096, 28672, 8192, "none", asym=True,
                             n_outlier_ch=896, outlier_mult=40.0, n_out=896, bits=8, decode_rows=8),
}


def get(name: str) -> Workload:
    return WORKLOADS[name]


def _rng(wl: Workload) -> np.random.Generator:
    return np.random.default_rng(wl.seed)


def make_activations(wl: Workload, T: int | None = None, K: int | None = None,
                     rng: np.random.Generator | None = None):
    """X fp16 [T, K] and the sorted outlier channel indices (int32).

    T and K may be overridden to draw a smaller instance of the same recipe
    (used by tests that need many tiles plus a ragged tail quickly).
    """
    rng = _rng(wl) if rng is None else rng
    T = wl.T if T is None else T
    K = wl.K if K is None else K
    n_ch = min(wl.n_outlier_ch, K)
    idx = np.sort(rng.choice(K, size=n_ch, replace=False)).astype(np.int32)
    x = rng.standard_normal((T, K))
    if n_ch:
        x[:, idx] *= wl.outlier_mult
    if T > 0 and wl.pivot_mult != 1.0:
        x[0] *= wl.pivot_mult
    x16 = x.astype(np.float16)
    if wl.decode_rows:
        x16 = np.ascontiguousarray(x16[: wl.decode_rows])
    return x16, idx


def make_weights(wl: Workload, N: int | None = None, K: int | None = None,
                 rng: np.random.Generator | None = None) -> np.ndarray:
    """W fp16 [N, K] ~ N(0, 0.02)."""
    N = wl.N if N is None else N
    K = wl.K if K is None else K
    rng = _rng(wl) if rng is None else rng
    w = rng.standard_normal((N, K)) * 0.02
    return w.astype(np.float16)


def make_affine(wl: Workload, rng: np.random.Generator, n1: int | None = None,
                n2: int | None = None):
    """P1 [n1,n1], P2 [n2,n2] = I + N(0,1)/n (fp32), channel scale s [n1*n2] ~ U(0.5, 2) (fp32)."""
    n1 = wl.n1 if n1 is None else n1
    n2 = wl.n2 if n2 is None else n2
    p1 = (np.eye(n1) + rng.standard_normal((n1, n1)) / n1).astype(np.float32)
    p2 = (np.eye(n2) + rng.standard_normal((n2, n2)) / n2).astype(np.float32)
    s = rng.uniform(0.5, 2.0, size=n1 * n2).astype(np.float32)
    return p1, p2, s


def make_inputs(name: str, T: int | None = None, K: int | None = None,
                N: int | None = None, with_weights: bool = True,
                n1: int | None = None, n2: int | None = None,
                seed: int | None = None) -> dict:
    """All seeded inputs of one workload, drawn in the documented order.

    T, K, N (and n1, n2 for the affine workload, K == n1 * n2) shrink the
    instance for quick tests; ``seed`` replaces the workload's seed.
    """
    wl = get(name)
    rng = np.random.default_rng(wl.seed if seed is None else seed)
    x, idx = make_activations(wl, T=T, K=K, rng=rng)
    out = {"x": x, "outlier_ch": idx, "wl": wl}
    if with_weights:
        out["w"] = make_weights(wl, N=N, K=K, rng=rng)
    if wl.rot == "kron":
        out["p1"], out["p2"], out["s"] = make_affine(wl, rng, n1, n2)
    if wl.rot == "r3":
        out["v"] = rng.standard_normal(x.shape).astype(np.float16)
    return out
