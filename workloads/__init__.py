"""Seeded synthetic inputs for the classifier-head cross-entropy workloads.

This module only draws random numbers and rounds them to the storage type; it
holds none of the loss arithmetic.  Both the CPU oracle tests and the GPU path
consume the same arrays, so both sides see bit-identical operands.

Workloads (shapes follow the head shapes the Cut Cross-Entropy pages discuss:
Llama 3.x and Gemma 2 classifier heads, mlx-cross-entropy README, "The problem"
table and "Performance" section):

  tiny      N=256   D=64   V=1000    fp32  e~N(0,1), c~N(0,1)/sqrt(D), uniform targets, 10% ignored
  llama1b   N=2048  D=2048 V=128256  bf16  e~N(0,1), c~N(0,0.02^2), uniform targets, 5% ignored
  gemma2b   N=4096  D=2304 V=256000  bf16  "trained-like" e (see below), Zipf(1.1) targets, none ignored
  llama8b   N=4096  D=4096 V=128256  bf16  e~N(0,1), c~N(0,0.02^2), uniform targets, none ignored
  long8b    N=16384 D=4096 V=128256  bf16  trained-like e, Zipf(1.1) targets, 3% ignored
  llama8b_pad25  as llama8b (seed 6) with 25% of the rows ignored (padding)

"trained-like" literal construction: e_i = 3 * c_{y_i}/||c_{y_i}|| * sqrt(D) + N(0, I).
The "calibrated" variants (gemma2b_cal, long8b_cal) instead use
e_i = (ln V + 2) * c_{y_i}/||c_{y_i}||^2 + N(0, I), which puts the target logit
near ln V + 2 so the softmax is peaked but the loss is not zero in fp32.

Draw order is fixed: c, then targets, then the ignored rows, then e.  Every
large array is drawn in fixed row blocks, each from its own child of the
seed's SeedSequence, so the values do not depend on how many threads draw them.
bf16 storage is produced by round-to-nearest-even of the fp32 draw; the arrays
returned are fp32 arrays whose values are exactly representable in bf16.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

IGNORE_INDEX = -100
_BLOCK_ROWS = 4096


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round an fp32 array to the nearest bf16 value (ties to even), kept as fp32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    r = (u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))) & np.uint32(0xFFFF0000)
    return r.view(np.float32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Upper 16 bits of fp32 values that are exactly bf16 (the bf16 bit pattern)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    return (x.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def _normal_rows(ss: np.random.SeedSequence, rows: int, cols: int, std: float,
                 threads: int | None = None) -> np.ndarray:
    """rows x cols N(0, std^2) fp32 drawn in fixed row blocks from children of ss."""
    nblk = max(1, math.ceil(rows / _BLOCK_ROWS))
    children = ss.spawn(nblk)
    out = np.empty((rows, cols), dtype=np.float32)

    def fill(b: int) -> None:
        r0 = b * _BLOCK_ROWS
        r1 = min(rows, r0 + _BLOCK_ROWS)
        g = np.random.default_rng(children[b])
        blk = out[r0:r1]
        g.standard_normal(out=blk, dtype=np.float32)
        if std != 1.0:
            blk *= np.float32(std)

    nthr = threads or min(16, len(os.sched_getaffinity(0)))
    if nblk == 1 or nthr <= 1:
        for b in range(nblk):
            fill(b)
    else:
        with ThreadPoolExecutor(nthr) as ex:
            list(ex.map(fill, range(nblk)))
    return out


def zipf_targets(rng: np.random.Generator, n: int, V: int, s: float = 1.1) -> np.ndarray:
    """Finite Zipf over the vocabulary: P(k) proportional to k^-s for k=1..V, id = k-1."""
    k = np.arange(1, V + 1, dtype=np.float64)
    p = k ** (-s)
    cdf = np.cumsum(p)
    cdf /= cdf[-1]
    u = rng.random(n)
    return np.minimum(np.searchsorted(cdf, u, side="right"), V - 1).astype(np.int64)


@dataclass
class Workload:
    name: str
    N: int
    D: int
    V: int
    dtype: str              # "f32" or "bf16": the storage type of e and c
    e_mode: str             # "normal", "trained", "calibrated"
    e_std: float
    c_std: float
    targets: str            # "uniform" or "zipf"
    ignore_frac: float
    seed: int
    reduction: str = "mean"
    notes: str = ""
    extra: dict = field(default_factory=dict)


WORKLOADS: dict[str, Workload] = {
    "tiny": Workload("tiny", 256, 64, 1000, "f32", "normal", 1.0, 1.0 / 8.0, "uniform", 0.10, 1),
    "llama1b": Workload("llama1b", 2048, 2048, 128256, "bf16", "normal", 1.0, 0.02, "uniform", 0.05, 2),
    "gemma2b": Workload("gemma2b", 4096, 2304, 256000, "bf16", "trained", 1.0, 0.02, "zipf", 0.0, 3),
    "gemma2b_cal": Workload("gemma2b_cal", 4096, 2304, 256000, "bf16", "calibrated", 1.0, 0.02, "zipf", 0.0, 3),
    "llama8b": Workload("llama8b", 4096, 4096, 128256, "bf16", "normal", 1.0, 0.02, "uniform", 0.0, 4,
                        reduction="none"),
    "long8b": Workload("long8b", 16384, 4096, 128256, "bf16", "trained", 1.0, 0.02, "zipf", 0.03, 5),
    "long8b_cal": Workload("long8b_cal", 16384, 4096, 128256, "bf16", "calibrated", 1.0, 0.02, "zipf", 0.03, 5),
    # the 8B head with a quarter of the rows padding (variable-length batches)
    "llama8b_pad25": Workload("llama8b_pad25", 4096, 4096, 128256, "bf16", "normal", 1.0, 0.02, "uniform", 0.25, 6),
    # the widest head the 32-bit buffer offsets take whole: D = 8192 (a 70B-class
    # model), the classifier 2.1 GB, just under 2^31 bytes
    "wide8192": Workload("wide8192", 1024, 8192, 128256, "bf16", "normal", 1.0, 0.02, "uniform", 0.05, 7),
    # a classifier beyond 2^31 bytes (Gemma-2-27B's head: 256000 x 4608 bf16,
    # 2.4 GB), which the backward takes in vocabulary chunks
    "gemma27b_1k": Workload("gemma27b_1k", 1024, 4608, 256000, "bf16", "normal", 1.0, 0.02, "uniform", 0.05, 8),
    # 64K tokens on the 8B head: eight vocabulary chunks in the backward
    "long64k": Workload("long64k", 65536, 4096, 128256, "bf16", "normal", 1.0, 0.02, "uniform", 0.03, 9),
}


def generate(w: Workload, threads: int | None = None) -> dict:
    """Draw (e, c, targets) for a workload.

    Returns a dict with fp32 arrays e [N, D], c [V, D] (bf16-exact when
    w.dtype == "bf16"), int64 targets [N] with round(ignore_frac*N) rows set to
    IGNORE_INDEX, and the workload's metadata.
    """
    ss = np.random.SeedSequence(w.seed)
    ss_c, ss_t, ss_i, ss_e = ss.spawn(4)
    c = _normal_rows(ss_c, w.V, w.D, w.c_std, threads)
    if w.dtype == "bf16":
        c = round_to_bf16(c)
    rng_t = np.random.default_rng(ss_t)
    if w.targets == "uniform":
        t = rng_t.integers(0, w.V, size=w.N, dtype=np.int64)
    elif w.targets == "zipf":
        t = zipf_targets(rng_t, w.N, w.V)
    else:
        raise ValueError(w.targets)
    n_ign = int(round(w.ignore_frac * w.N))
    y = t.copy()
    if n_ign:
        rows = np.random.default_rng(ss_i).choice(w.N, size=n_ign, replace=False)
        t[rows] = IGNORE_INDEX
    e = _normal_rows(ss_e, w.N, w.D, w.e_std, threads)
    if w.e_mode != "normal":
        # Direction of the (pre-masking) target's classifier row, scaled.
        cy = c[y].astype(np.float32)
        nrm2 = np.einsum("ij,ij->i", cy, cy, dtype=np.float64).astype(np.float32)
        if w.e_mode == "trained":
            scale = np.float32(3.0 * math.sqrt(w.D)) / np.sqrt(nrm2)
        elif w.e_mode == "calibrated":
            scale = np.float32(math.log(w.V) + 2.0) / nrm2
        else:
            raise ValueError(w.e_mode)
        e += cy * scale[:, None]
        del cy
    if w.dtype == "bf16":
        e = round_to_bf16(e)
    return {"e": e, "c": c, "targets": t, "workload": w, "ignore_index": IGNORE_INDEX,
            "n_ignored": n_ign}


def custom(N: int, D: int, V: int, dtype: str = "bf16", *, seed: int = 0, e_std: float = 1.0,
           c_std: float = 0.02, targets: str = "uniform", ignore_frac: float = 0.0,
           e_mode: str = "normal", reduction: str = "mean", threads: int | None = None) -> dict:
    """Same recipe as the named workloads at arbitrary (small) sizes."""
    w = Workload(f"custom_{N}x{D}x{V}", N, D, V, dtype, e_mode, e_std, c_std, targets,
                 ignore_frac, seed, reduction=reduction)
    return generate(w, threads)


def bias(V: int, dtype: str = "bf16", *, seed: int = 0, std: float = 0.5, block_offsets=None) -> np.ndarray:
    """Seeded classifier bias [V] ~ N(0, std^2), rounded to bf16 for bf16
    problems.  `block_offsets` {(v0, v1): value} adds a constant to vocab ranges
    (e.g. a strongly negative block, which the gradient filter then drops)."""
    rng = np.random.default_rng(np.random.SeedSequence([seed, 0xB1A5]))
    b = (rng.standard_normal(V) * std).astype(np.float32)
    for (v0, v1), val in (block_offsets or {}).items():
        b[v0:v1] += np.float32(val)
    return round_to_bf16(b) if dtype == "bf16" else b


def get(name: str, threads: int | None = None) -> dict:
    return generate(WORKLOADS[name], threads)
