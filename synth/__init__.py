"""Seeded synthetic inputs for W12 tests and benchmarks.

This module only draws random numbers and rounds them to BF16 once. It holds
none of the W12 arithmetic (no window choice, no packing, no GEMM), so both the
oracle-side tests and the GPU path may consume what it produces.

Recipe (the workloads of SpecPilot, arXiv 2611.02501, are projections and the
LM head of a 27B target at hidden size 5120; its checkpoints are not available,
so per-output-channel Gaussian weights of the same shapes stand in for them):

* weights: row i of a matrix is ``N(0, s_i^2)`` in fp32 with
  ``s_i = base * lognormal(0, sigma)``; then a Bernoulli(``outlier_rate``)
  subset of entries is multiplied by 2**12; then a Bernoulli(``zero_rate``)
  subset is set to +0.0; then, for the escape-stress workload, a
  Bernoulli(0.1) subset of rows is made bimodal by multiplying each of its
  entries by 2**8 with probability 0.5; finally every entry is rounded to BF16
  (round to nearest even) once.
* activations: fp32 ``N(0, 1)`` rounded to BF16.

Rows are generated in blocks of ``ROW_BLOCK`` rows, each block from its own
PCG64 stream seeded with ``SeedSequence([seed, block])``; the result does not
depend on how many threads generate it.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

ROW_BLOCK = 256
SEED_BASE = 20261202


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 values to BF16 (nearest, ties to even); return uint16 bits.

    Inputs here are finite (the generator never makes inf or NaN)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


@dataclass(frozen=True)
class MatrixSpec:
    name: str
    n: int  # out features (rows)
    k: int  # in features (columns)


@dataclass(frozen=True)
class Workload:
    index: int
    title: str
    matrices: tuple
    ms: tuple
    scale_base: float = 0.02
    scale_sigma: float = 0.5
    outlier_rate: float = 1e-4
    zero_rate: float = 1e-4
    bimodal_rows: float = 0.0
    extra: dict = field(default_factory=dict)


_H = 5120
WORKLOADS = {
    0: Workload(0, "single 1024x1024 matrix",
                (MatrixSpec("w", 1024, 1024),), (1,)),
    1: Workload(1, "MLP GEMMs at hidden 5120",
                (MatrixSpec("gate", 17408, _H), MatrixSpec("up", 17408, _H),
                 MatrixSpec("down", _H, 17408)), (1, 4, 8, 16, 32)),
    2: Workload(2, "one decoder layer's linears at hidden 5120",
                (MatrixSpec("q", 6144, _H), MatrixSpec("k", 1024, _H),
                 MatrixSpec("v", 1024, _H), MatrixSpec("o", _H, 6144),
                 MatrixSpec("gate", 17408, _H), MatrixSpec("up", 17408, _H),
                 MatrixSpec("down", _H, 17408)), (32, 64)),
    3: Workload(3, "LM head 151936x5120",
                (MatrixSpec("lm_head", 151936, _H),), (1, 16, 32),
                scale_base=0.015, scale_sigma=0.3),
    4: Workload(4, "Q pass and escape stress on the MLP shapes",
                (MatrixSpec("gate", 17408, _H), MatrixSpec("up", 17408, _H),
                 MatrixSpec("down", _H, 17408)), (32,),
                outlier_rate=1e-2, bimodal_rows=0.1),
}


def matrix_seed(workload: int, matrix_index: int) -> int:
    return SEED_BASE + 100 * workload + matrix_index


def _weight_block(seed, blk, rows, k, wl: Workload):
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, blk])))
    s = (wl.scale_base * rng.lognormal(0.0, wl.scale_sigma, size=rows)).astype(np.float32)
    w = rng.standard_normal((rows, k), dtype=np.float32)
    w *= s[:, None]
    if wl.outlier_rate > 0:
        w[rng.random((rows, k), dtype=np.float32) < wl.outlier_rate] *= np.float32(4096.0)
    if wl.zero_rate > 0:
        w[rng.random((rows, k), dtype=np.float32) < wl.zero_rate] = np.float32(0.0)
    if wl.bimodal_rows > 0:
        brow = rng.random(rows) < wl.bimodal_rows
        if brow.any():
            sub = w[brow]
            sub[rng.random(sub.shape, dtype=np.float32) < 0.5] *= np.float32(256.0)
            w[brow] = sub
    return f32_to_bf16_bits(w)


def make_weights(n: int, k: int, wl: Workload, seed: int, threads: int | None = None,
                 rows: slice | None = None) -> np.ndarray:
    """BF16 bits ``uint16[n, k]`` (or only the row range ``rows``, which must
    start and stop on ``ROW_BLOCK`` boundaries or at ``n``)."""
    r0, r1 = (0, n) if rows is None else (rows.start or 0, rows.stop if rows.stop is not None else n)
    assert r0 % ROW_BLOCK == 0 and (r1 % ROW_BLOCK == 0 or r1 == n) and 0 <= r0 <= r1 <= n
    out = np.empty((r1 - r0, k), dtype=np.uint16)
    blocks = list(range(r0 // ROW_BLOCK, (r1 + ROW_BLOCK - 1) // ROW_BLOCK))

    def work(b):
        a = b * ROW_BLOCK
        z = min(a + ROW_BLOCK, n)
        out[a - r0:z - r0] = _weight_block(seed, b, z - a, k, wl)

    nthreads = threads or min(16, os.cpu_count() or 1)
    if len(blocks) == 1 or nthreads == 1:
        for b in blocks:
            work(b)
    else:
        with ThreadPoolExecutor(nthreads) as ex:
            list(ex.map(work, blocks))
    return out


def workload_matrix(workload: int, matrix_index: int, **kw) -> np.ndarray:
    wl = WORKLOADS[workload]
    spec = wl.matrices[matrix_index]
    return make_weights(spec.n, spec.k, wl, matrix_seed(workload, matrix_index), **kw)


def make_activations(m: int, k: int, seed: int) -> np.ndarray:
    """BF16 bits ``uint16[m, k]`` of N(0, 1) activations."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 7777])))
    return f32_to_bf16_bits(rng.standard_normal((m, k), dtype=np.float32))


def activation_seed(workload: int, matrix_index: int, m: int) -> int:
    return SEED_BASE + 100 * workload + 10 * matrix_index + 1000 * m + 50_000


def plain_gaussian(n: int, k: int, seed: int, scale: float = 0.02, sigma: float = 0.5) -> np.ndarray:
    """Per-channel Gaussian weights with no injected outliers or zeros."""
    wl = Workload(-1, "plain", (MatrixSpec("w", n, k),), (1,), scale_base=scale,
                  scale_sigma=sigma, outlier_rate=0.0, zero_rate=0.0)
    return make_weights(n, k, wl, seed)


def random_bits(shape, seed: int) -> np.ndarray:
    """Uniformly random 16-bit patterns (every class: normals, zeros,
    subnormals, infinities, NaNs)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return rng.integers(0, 1 << 16, size=shape, dtype=np.uint16)


def all_bf16_patterns(k: int = 512) -> np.ndarray:
    """All 65,536 BF16 bit patterns in a ``[65536 // k, k]`` matrix."""
    assert 65536 % k == 0
    return np.arange(65536, dtype=np.uint32).astype(np.uint16).reshape(65536 // k, k)
