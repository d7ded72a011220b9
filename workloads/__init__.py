"""Seeded synthetic inputs for the FP8 runtime chain.

This module only draws random tensors; it holds none of the method's
arithmetic (no amax, scale, cast or GEMM).  Both the CPU oracle and the HIP
library are fed from it.  Arrays are numpy: float32, or bfloat16 carried as
``uint16`` bit patterns (rounded to nearest even from float32 by torch's CPU
cast).  The random source is numpy's Philox4x32-10 counter-based generator,
keyed by ``42 + 1000 * config + tensor_id``; a draw of more than 2^22
elements is made of 2^22-element chunks, chunk i from that generator's
stream jumped i + 1 times (drawn on several threads, the same values
whatever their number).

The five workloads stand in for the LLM linear layers the pages discuss (a
decode-time linear, a 72B-class MLP up-projection at prefill, a backward GEMM
under the hybrid E5M2/E4M3 recipe with delayed scaling, and a block-scaled
layer); the pages measured real models, which are not used here.
"""
from __future__ import annotations

import concurrent.futures
import dataclasses
import os

import numpy as np

BASE_SEED = 42


def case_seed(*parts) -> int:
    """A seed that depends only on the text of ``parts`` (CRC-32 of their repr):
    the same in every process, unlike ``hash`` of tuples holding ``str`` or
    ``None``, which Python salts per process."""
    import zlib

    return zlib.crc32(repr(parts).encode()) & 0x7FFFFFFF


def rng(config: int, tensor_id: int) -> np.random.Generator:
    return np.random.Generator(np.random.Philox(key=BASE_SEED + 1000 * config + tensor_id))


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest even (torch CPU cast)."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


CHUNK = 1 << 22  # elements per independent stream of a large draw


def _workers() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _chunked(g: np.random.Generator, shape, fill) -> np.ndarray:
    """A float32 array of `shape` filled chunk by chunk: chunk i (CHUNK elements,
    the last one shorter) comes from its own stream, g's bit generator jumped
    i + 1 times, so the values depend on the seed and CHUNK only, not on the
    number of threads.  Arrays of at most CHUNK elements are one draw from g."""
    n = int(np.prod(shape))
    out = np.empty(n, np.float32)
    if n <= CHUNK:
        fill(g, out)
        return out.reshape(shape)
    bg = g.bit_generator
    starts = range(0, n, CHUNK)

    def one(i):
        fill(np.random.Generator(bg.jumped(i + 1)), out[i * CHUNK:(i + 1) * CHUNK])

    with concurrent.futures.ThreadPoolExecutor(_workers()) as ex:
        list(ex.map(one, range(len(starts))))
    return out.reshape(shape)


def normal(g: np.random.Generator, shape, std: float = 1.0) -> np.ndarray:
    x = _chunked(g, shape, lambda gi, o: gi.standard_normal(o.shape, dtype=np.float32, out=o))
    if std != 1.0:
        x *= np.float32(std)
    return x


def student_t3(g: np.random.Generator, shape) -> np.ndarray:
    """Student-t with 3 degrees of freedom: Z / sqrt(chi2_3 / 3), Z and the
    chi-square drawn in the same chunk stream."""
    def fill(gi, o):
        z = gi.standard_normal(o.shape, dtype=np.float32)
        chi = gi.chisquare(3, size=o.shape).astype(np.float32)
        o[:] = z / np.sqrt(chi / np.float32(3.0))

    return _chunked(g, shape, fill)


# --------------------------------------------------------------------------
# Workload recipes.  Sizes default to the full shapes; smaller shapes with the
# same recipe serve the oracle-sized parity cases.

@dataclasses.dataclass
class C1Tiny:
    """Per-tensor dynamic E4M3: X 256x1024 fp32 N(0,1) with 4 entries at +-400;
    W 256x1024 fp32 N(0, 0.02) (per-output-channel E4M3); GEMM X[0:64] W^T, K=1024."""
    rows: int = 256
    K: int = 1024
    N: int = 256
    M_gemm: int = 64

    def make(self):
        g = rng(1, 0)
        x = normal(g, (self.rows, self.K))
        pos = rng(1, 1).choice(self.rows * self.K, size=4, replace=False)
        sign = np.where(rng(1, 2).integers(0, 2, size=4) == 0, -1.0, 1.0).astype(np.float32)
        x.reshape(-1)[pos] = np.float32(400.0) * sign
        w = normal(rng(1, 3), (self.N, self.K), 0.02)
        return {"x": x, "w": w}


@dataclasses.dataclass
class C2Decode:
    """Decode linear: A bf16 16x8192 N(0,1), 1% of columns (82) x30, per-token E4M3;
    W bf16 8192x8192 N(0, 0.02) per-output-channel E4M3; bias bf16 N(0, 0.1)."""
    M: int = 16
    N: int = 8192
    K: int = 8192

    def make(self):
        a = normal(rng(2, 0), (self.M, self.K))
        ncols = max(1, int(round(0.01 * self.K)))
        cols = rng(2, 1).choice(self.K, size=ncols, replace=False)
        a[:, cols] *= np.float32(30.0)
        w = normal(rng(2, 2), (self.N, self.K), 0.02)
        bias = normal(rng(2, 3), (self.N,), 0.1)
        return {"a": to_bf16_bits(a), "w": to_bf16_bits(w), "bias": to_bf16_bits(bias),
                "outlier_cols": np.sort(cols)}


@dataclasses.dataclass
class C3Prefill:
    """72B-class MLP up-projection at prefill: X bf16 4096x8192 = 0.5 * t(3), per-tensor
    dynamic E4M3; W bf16 29568x8192 N(0, 0.02), per-tensor static E4M3; out bf16."""
    M: int = 4096
    N: int = 29568
    K: int = 8192

    def make_x(self):
        return to_bf16_bits(np.float32(0.5) * student_t3(rng(3, 0), (self.M, self.K)))

    def make_w(self):
        return to_bf16_bits(normal(rng(3, 1), (self.N, self.K), 0.02))

    def make(self):
        return {"x": self.make_x(), "w": self.make_w()}


@dataclasses.dataclass
class C4Delayed:
    """Hybrid-recipe backward GEMM under delayed scaling: per step t, G_t bf16
    8192x8192 = N(0,1) * sigma_t with sigma_t = exp(z_t), z_t ~ N(0,1); one seeded
    spike step in [1, steps-1] multiplies G by 100.  E5M2 with a 16-entry amax
    history.  W bf16 8192x8192 N(0, 0.02), per-tensor E4M3.  Output fp32."""
    M: int = 8192
    N: int = 8192
    K: int = 8192
    steps: int = 32
    history: int = 16

    def sigmas(self):
        z = rng(4, 0).standard_normal(self.steps)
        sig = np.exp(z)
        n_spikes = max(1, int(round(0.02 * self.steps)))
        spike_steps = rng(4, 1).choice(np.arange(1, self.steps), size=n_spikes, replace=False)
        sig[spike_steps] *= 100.0
        return sig.astype(np.float32), np.sort(spike_steps)

    def make_g(self, t: int):
        sig, _ = self.sigmas()
        return to_bf16_bits(normal(rng(4, 100 + t), (self.M, self.K)) * sig[t])

    def make_w(self):
        return to_bf16_bits(normal(rng(4, 2), (self.N, self.K), 0.02))


@dataclasses.dataclass
class C5Block:
    """Block-scaled E4M3 GEMM M=8192, K=7168, N=18432: A bf16 N(0,1) with 1x128
    group scales; W bf16 N(0, 0.02) with 128x128 block scales; out bf16.  The
    variant uses 1x32 power-of-two (round-up) scales on both operands."""
    M: int = 8192
    N: int = 18432
    K: int = 7168

    def make_a(self):
        return to_bf16_bits(normal(rng(5, 0), (self.M, self.K)))

    def make_w(self):
        return to_bf16_bits(normal(rng(5, 1), (self.N, self.K), 0.02))

    def make(self):
        return {"a": self.make_a(), "w": self.make_w()}


def sample_points(M: int, N: int, seed: int, n_random: int = 32768, n_rows: int = 8,
                  n_cols: int = 8):
    """GEMM output sample: n_rows full rows + n_cols full columns + n_random points."""
    g = rng(99, seed)
    rows = g.choice(M, size=min(n_rows, M), replace=False)
    cols = g.choice(N, size=min(n_cols, N), replace=False)
    m_idx = np.concatenate([np.repeat(rows, N), np.repeat(np.arange(M), len(cols)),
                            g.integers(0, M, n_random)]).astype(np.int64)
    n_idx = np.concatenate([np.tile(np.arange(N), len(rows)), np.tile(cols, M),
                            g.integers(0, N, n_random)]).astype(np.int64)
    return m_idx, n_idx


def ceil_div(a: int, b: int) -> int:
    return -(-a // b)


__all__ = ["C1Tiny", "C2Decode", "C3Prefill", "C4Delayed", "C5Block", "rng", "to_bf16_bits",
           "normal", "student_t3", "sample_points", "ceil_div"]
