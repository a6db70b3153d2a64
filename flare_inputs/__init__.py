"""Seeded synthetic inputs for the FLARE / FLARE++ forward operator.

This module is shared by the tests, the benchmark and the CPU oracle's callers.
It holds no part of the operator's arithmetic: it only draws Gaussian numbers,
scales them, and rounds them to the storage type.

Storage convention (both sides read the very same bits):
  * fp32 tensors are numpy ``float32`` arrays;
  * bf16 tensors are numpy ``uint16`` arrays holding the bf16 bit patterns.

Recipe: numpy PCG64 streams ``default_rng([seed, tensor_id, chunk])`` with
tensor_id 0/1/2 for Q/K/V, drawing ``standard_normal(float32)`` in C order in
chunks of ``CHUNK`` elements; each value is multiplied by the tensor's scale in
float32 and then rounded to nearest-even into bf16 when the dtype is bf16.

The workload table mirrors the shapes and value distributions that the FLARE
pages run on (PDE meshes up to one million points on one GPU, and
long-sequence classification); the datasets themselves are not used, and
i.i.d. Gaussians of the same shapes stand in for them.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass

import numpy as np

CHUNK = 1 << 22  # elements per independent PCG64 stream

F32 = "f32"
BF16 = "bf16"


@dataclass(frozen=True)
class Workload:
    """One synthetic workload: shape, storage type, value scales and operator."""

    name: str
    B: int
    H: int
    N: int
    M: int
    D: int
    dtype: str
    q_scale: float
    kv_scale: float
    op: str  # "forward" (FLARE) or "pp_forward" (FLARE++)
    seed: int

    @property
    def bh(self) -> int:
        return self.B * self.H

    def shapes(self):
        return (self.H, self.M, self.D), (self.B, self.H, self.N, self.D)


# Five headline workloads and one at the largest M. Q scales: 0.02*sqrt(D) for the mesh workload (latent init
# N(0, 0.02^2) of the FLARE page, step 1, seen through a sqrt(D) head width),
# 0.5 for the others; K and V are unit Gaussians everywhere.
WORKLOADS = {
    1: Workload("tiny-fp32", 1, 4, 1024, 32, 16, F32, 1.0, 1.0, "forward", 1),
    2: Workload("pde-mesh-65k", 4, 8, 65536, 128, 32, BF16, 0.02 * math.sqrt(32.0), 1.0, "forward", 2),
    3: Workload("long-seq-4k", 32, 8, 4096, 64, 64, BF16, 0.5, 1.0, "forward", 3),
    4: Workload("large-mesh-1m", 1, 16, 1048576, 256, 64, BF16, 0.5, 1.0, "forward", 4),
    5: Workload("flarepp-262k", 2, 8, 262144, 128, 64, BF16, 0.5, 1.0, "pp_forward", 5),
    # the top of the FLARE page's latent range ("Key Hyperparameters": M up
    # to 512): not one of the five headline configurations
    6: Workload("latents-512", 1, 8, 262144, 512, 64, BF16, 0.5, 1.0, "forward", 6),
    # the same latent count at the widest head (D = 128): the decode's latents
    # do not fit in one CU's LDS there, so it runs over two latent ranges
    7: Workload("latents-512-d128", 1, 8, 131072, 512, 128, BF16, 0.5, 1.0, "forward", 7),
}


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); return uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = u + 0x7FFF + ((u >> 16) & 1)
    return (u >> 16).astype(np.uint16)


def _draw(seed: int, tensor_id: int, n: int, scale: float, dtype: str, threads: int) -> np.ndarray:
    out_dt = np.float32 if dtype == F32 else np.uint16
    out = np.empty(n, dtype=out_dt)
    nchunks = (n + CHUNK - 1) // CHUNK

    def one(c: int) -> None:
        lo = c * CHUNK
        hi = min(n, lo + CHUNK)
        z = np.random.default_rng([seed, tensor_id, c]).standard_normal(hi - lo, dtype=np.float32)
        if scale != 1.0:
            z *= np.float32(scale)
        out[lo:hi] = z if dtype == F32 else f32_to_bf16_bits(z)

    if nchunks == 1 or threads <= 1:
        for c in range(nchunks):
            one(c)
    else:
        with ThreadPoolExecutor(max_workers=threads) as ex:
            list(ex.map(one, range(nchunks)))
    return out


def default_threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def make_inputs(B: int, H: int, N: int, M: int, D: int, dtype: str, q_scale: float = 1.0,
                kv_scale: float = 1.0, seed: int = 0, threads: int | None = None):
    """Return (Q[H,M,D], K[B,H,N,D], V[B,H,N,D]) as float32 or bf16-bit arrays."""
    if dtype not in (F32, BF16):
        raise ValueError(f"dtype must be {F32!r} or {BF16!r}")
    t = default_threads() if threads is None else threads
    q = _draw(seed, 0, H * M * D, q_scale, dtype, t).reshape(H, M, D)
    k = _draw(seed, 1, B * H * N * D, kv_scale, dtype, t).reshape(B, H, N, D)
    v = _draw(seed, 2, B * H * N * D, kv_scale, dtype, t).reshape(B, H, N, D)
    return q, k, v


def workload_inputs(w: Workload, threads: int | None = None):
    return make_inputs(w.B, w.H, w.N, w.M, w.D, w.dtype, w.q_scale, w.kv_scale, w.seed, threads)


def recipe() -> str:
    return ("numpy PCG64 default_rng([seed, tensor_id(0=Q,1=K,2=V), chunk]) standard_normal(float32) "
            f"in chunks of {CHUNK} elements, scaled in float32, rounded to nearest-even for bf16")
