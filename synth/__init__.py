"""Seeded synthetic inputs for the cross-entropy workloads.

This module holds input generation only -- none of the method's arithmetic.
It is the one piece shared by the oracle-side tests and the GPU-side tests and
bench, so both sides always see the same bytes.

Every row is addressable on its own: logits row ``i`` of a workload comes from
``numpy.random.default_rng([seed, 0, i])``, so a checker can regenerate any
sampled row without materialising the whole matrix.

Workload shapes follow the pages: the Megatron-LM vocab-parallel CE table
(sequence 2048, batch 1, a "128K" vocabulary read as 131072), the Liger CE
micro-bench setup (S=2048, B=4, with the 151,936-token vocabulary of the
Qwen3 model on the same page) and the Muse Glimmer dimensions (hidden 6656,
vocabulary 202,048).  Value distributions are synthetic.
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

IGNORE_INDEX = -100


@dataclasses.dataclass(frozen=True)
class CEWorkload:
    name: str
    seed: int
    n: int
    V: int
    dtype: str              # "f32" or "bf16"
    sigma: float
    ignore_frac: float
    label_smoothing: float = 0.0
    softcap: float = 0.0
    reduction: str = "mean"
    grad_out: float = 1.0
    spike: float = 0.0      # added at the label column of a share of valid rows
    spike_frac: float = 0.0
    quant_frac: float = 0.0  # rows rounded to integers in [-4, 4] (argmax ties)
    want_argmax: bool = False

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2


@dataclasses.dataclass(frozen=True)
class FLCEWorkload:
    name: str
    seed: int
    n: int
    H: int
    V: int
    hidden_scale: float     # output multiplier folded into hidden
    w_sigma: float
    ignore_frac: float
    softcap: float = 0.0
    label_smoothing: float = 0.0
    reduction: str = "mean"
    grad_out: float = 1.0
    chunk: int = 1024


# The five workloads.
C1 = CEWorkload("ce_f32_256x4096", 1001, 256, 4096, "f32", 1.0, 0.10)
C2 = CEWorkload("ce_bf16_2048x131072", 1002, 2048, 131072, "bf16", 2.0, 0.05)
C3 = CEWorkload("ce_bf16_8192x151936_smooth0.1", 1003, 8192, 151936, "bf16", 3.0, 0.02,
                label_smoothing=0.1, grad_out=0.5, spike=8.0, spike_frac=0.3)
C4 = CEWorkload("ce_bf16_4096x202048_softcap30_argmax", 1004, 4096, 202048, "bf16", 10.0, 0.03,
                softcap=30.0, quant_frac=0.1, want_argmax=True)
C5 = FLCEWorkload("flce_bf16_4096x6656x202048", 1005, 4096, 6656, 202048, 0.5, 0.02, 0.05,
                  softcap=30.0, chunk=1024)
# Reduced fused-linear shape the oracle checks in full.
C5_SMALL = FLCEWorkload("flce_bf16_256x512x8192", 1005, 256, 512, 8192, 0.5, 0.02, 0.05,
                        softcap=30.0, chunk=64)

WORKLOADS = {w.name: w for w in (C1, C2, C3, C4)}
FLCE_WORKLOADS = {w.name: w for w in (C5, C5_SMALL)}

# The vocabulary sweep of the cross-entropy op (bench only): sequence 2048 x batch 4 tokens over
# vocabularies from 4K to 128K (the Liger CE micro-bench's setup), one vocabulary-parallel rank's
# shard of the 128K vocabulary at 8, 4 and 2 ranks ([2048, 16384], [2048, 32768], [2048, 65536]),
# and an odd vocabulary (50257, the GPT-2 tokenizer's size), whose rows do not start on 16-byte
# boundaries.  sigma 2, 5% ignored, mean reduction.
SWEEP = {w.name: w for w in (
    [CEWorkload(f"ce_bf16_8192x{v}", 1100 + i, 8192, v, "bf16", 2.0, 0.05)
     for i, v in enumerate((4096, 16384, 32768, 65536, 131072))]
    + [CEWorkload("ce_bf16_2048x16384", 1110, 2048, 16384, "bf16", 2.0, 0.05),
       CEWorkload("ce_bf16_2048x50257", 1111, 2048, 50257, "bf16", 2.0, 0.05),
       CEWorkload("ce_bf16_2048x32768", 1112, 2048, 32768, "bf16", 2.0, 0.05),
       CEWorkload("ce_bf16_2048x65536", 1113, 2048, 65536, "bf16", 2.0, 0.05)])}
ALL_CE_WORKLOADS = {**WORKLOADS, **SWEEP}


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns, round to nearest even (inputs are finite)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _first_of_permutation(seed_seq, population: np.ndarray, count: int) -> np.ndarray:
    perm = np.random.default_rng(seed_seq).permutation(population.size)
    return population[perm[:count]]


def labels(w: CEWorkload | FLCEWorkload) -> np.ndarray:
    """int64 labels, uniform in [0, V), with round(ignore_frac * n) rows set to -100."""
    y = np.random.default_rng([w.seed, 1]).integers(0, w.V, w.n).astype(np.int64)
    n_ign = int(round(w.ignore_frac * w.n))
    ign = _first_of_permutation([w.seed, 2], np.arange(w.n), n_ign)
    y[ign] = IGNORE_INDEX
    return y


def row_features(w: CEWorkload, y: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Boolean masks over rows: which rows get the label spike, which rows are quantised."""
    spike = np.zeros(w.n, dtype=bool)
    if w.spike_frac > 0:
        valid_rows = np.nonzero(y != IGNORE_INDEX)[0]
        k = int(round(w.spike_frac * valid_rows.size))
        spike[_first_of_permutation([w.seed, 3], valid_rows, k)] = True
    quant = np.zeros(w.n, dtype=bool)
    if w.quant_frac > 0:
        k = int(round(w.quant_frac * w.n))
        quant[_first_of_permutation([w.seed, 4], np.arange(w.n), k)] = True
    return spike, quant


def logits_row_f32(w: CEWorkload, i: int, y_i: int, spike: bool, quant: bool) -> np.ndarray:
    x = np.random.default_rng([w.seed, 0, int(i)]).standard_normal(w.V, dtype=np.float32)
    x *= np.float32(w.sigma)
    if spike and 0 <= y_i < w.V:
        x[y_i] += np.float32(w.spike)
    if quant:
        x = np.clip(np.rint(x), -4.0, 4.0).astype(np.float32)
    return x


def logits_rows(w: CEWorkload, rows, y: np.ndarray | None = None, out: np.ndarray | None = None,
                ld: int | None = None, threads: int | None = None) -> np.ndarray:
    """Stored logits for the given rows: float32, or uint16 bf16 bit patterns.

    When ``ld`` > V the returned rows are padded with ``ld - V`` extra columns set to a
    sentinel (0x7FC1 for bf16 / the float32 NaN 0x7FC00001), so a checker can see that the
    padding was left untouched.
    """
    if y is None:
        y = labels(w)
    spike, quant = row_features(w, y)
    rows = np.asarray(rows, dtype=np.int64)
    ld = w.V if ld is None else int(ld)
    dt = np.float32 if w.dtype == "f32" else np.uint16
    if out is None:
        out = np.empty((rows.size, ld), dtype=dt)
    if ld > w.V:
        if w.dtype == "f32":
            out[:, w.V:] = np.array([0x7FC00001], dtype=np.uint32).view(np.float32)[0]
        else:
            out[:, w.V:] = np.uint16(0x7FC1)

    def fill(k: int) -> None:
        i = int(rows[k])
        x = logits_row_f32(w, i, int(y[i]), bool(spike[i]), bool(quant[i]))
        out[k, :w.V] = x if w.dtype == "f32" else f32_to_bf16_bits(x)

    nthr = threads or min(16, os.cpu_count() or 1)
    if rows.size >= 64 and nthr > 1:
        with ThreadPoolExecutor(nthr) as ex:
            list(ex.map(fill, range(rows.size)))
    else:
        for k in range(rows.size):
            fill(k)
    return out


def logits(w: CEWorkload, y: np.ndarray | None = None, ld: int | None = None) -> np.ndarray:
    return logits_rows(w, np.arange(w.n), y=y, ld=ld)


def flce_hidden_rows(w: FLCEWorkload, rows) -> np.ndarray:
    """bf16 bits of hidden rows: RNE(N(0,1)) times the output multiplier (a power of two, exact)."""
    rows = np.asarray(rows, dtype=np.int64)
    out = np.empty((rows.size, w.H), dtype=np.uint16)
    mult = np.float32(w.hidden_scale)
    for k, i in enumerate(rows):
        x = np.random.default_rng([w.seed, 5, int(i)]).standard_normal(w.H, dtype=np.float32)
        out[k] = f32_to_bf16_bits(bf16_bits_to_f32(f32_to_bf16_bits(x)) * mult)
    return out


def flce_weight_rows(w: FLCEWorkload, rows, threads: int | None = None) -> np.ndarray:
    rows = np.asarray(rows, dtype=np.int64)
    out = np.empty((rows.size, w.H), dtype=np.uint16)
    sig = np.float32(w.w_sigma)

    def fill(k: int) -> None:
        x = np.random.default_rng([w.seed, 6, int(rows[k])]).standard_normal(w.H, dtype=np.float32)
        out[k] = f32_to_bf16_bits(x * sig)

    nthr = threads or min(16, os.cpu_count() or 1)
    if rows.size >= 256 and nthr > 1:
        with ThreadPoolExecutor(nthr) as ex:
            list(ex.map(fill, range(rows.size)))
    else:
        for k in range(rows.size):
            fill(k)
    return out
