"""CPU oracle for vocabulary-wide cross-entropy (fp64).

TEST INFRASTRUCTURE ONLY: the tests, ``__graft_entry__.smoke()`` and the
bench's ``cpu_baseline`` leg may import this package; the product path (the
HIP library and its binding) never does.  It shares no code with the GPU path.

The arithmetic lives in ``lce_oracle.c`` (plain fp64 C, one OpenMP loop over
rows).  This module only marshals numpy arrays into it and builds it with gcc.
The definitions it follows are cited in the C file's header.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "lce_oracle.c")
_LIB = os.path.join(_HERE, "liblce_oracle.so")

RED_NONE, RED_MEAN, RED_SUM = 0, 1, 2
_REDUCTIONS = {"none": RED_NONE, "mean": RED_MEAN, "sum": RED_SUM}
_DTYPES = {"f32": 0, "bf16": 1, "f64": 2}


def build(verbose: bool = False) -> str:
    """Compile the oracle with gcc (IEEE semantics: no fast-math, no FMA contraction)."""
    cmd = ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-fPIC", "-shared",
           "-std=c11", "-Wall", "-o", _LIB, _SRC, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    return _LIB


def _ptr(a):
    return None if a is None else ctypes.c_void_p(a.ctypes.data)


def _dtype_code(arr: np.ndarray) -> int:
    if arr.dtype == np.uint16:
        return _DTYPES["bf16"]  # raw bf16 bit patterns
    if arr.dtype == np.float32:
        return _DTYPES["f32"]
    if arr.dtype == np.float64:
        return _DTYPES["f64"]
    raise TypeError(f"oracle takes uint16 (bf16 bits), float32 or float64 logits, not {arr.dtype}")


def _grad_out_array(grad_out, reduction: int, n: int):
    if grad_out is None:
        return None
    g = np.ascontiguousarray(np.asarray(grad_out, dtype=np.float64).reshape(-1))
    want = n if reduction == RED_NONE else 1
    if g.size != want:
        raise ValueError(f"grad_out must have {want} element(s), got {g.size}")
    return g


class Oracle:
    """One loaded build of the oracle library (the default build, or a test's own copy)."""

    def __init__(self, lib_path: str = _LIB):
        if lib_path == _LIB and not os.path.exists(_LIB):
            build()
        lib = ctypes.CDLL(lib_path)
        p = ctypes.c_void_p
        i64 = ctypes.c_int64
        lib.lce_oracle_ce.restype = ctypes.c_int
        lib.lce_oracle_ce.argtypes = [p, i64, ctypes.c_int, p, i64, i64, i64, ctypes.c_double,
                                      ctypes.c_double, ctypes.c_int, p, p, i64, p, p, p, p, ctypes.c_int]
        lib.lce_oracle_reduce_loss.restype = ctypes.c_double
        lib.lce_oracle_reduce_loss.argtypes = [p, i64, i64, ctypes.c_int]
        lib.lce_oracle_round_bf16.restype = None
        lib.lce_oracle_round_bf16.argtypes = [p, p, i64]
        lib.lce_oracle_count.restype = None
        lib.lce_oracle_count.argtypes = [p, i64, i64, i64, p, p]
        lib.lce_oracle_flce.restype = ctypes.c_int
        lib.lce_oracle_flce.argtypes = [p, p, p, i64, i64, i64, i64, ctypes.c_double, ctypes.c_double,
                                        ctypes.c_int, p, p, p, p, p, p, ctypes.c_int]
        lib.lce_oracle_row_stats.restype = ctypes.c_int
        lib.lce_oracle_row_stats.argtypes = [p, i64, ctypes.c_int, p, i64, i64, i64, ctypes.c_double, p, i64, p, p,
                                             p, ctypes.c_int]
        if lib.lce_oracle_abi_version() != 2:
            raise RuntimeError("stale liblce_oracle.so; rebuild it")
        self.lib = lib

    def ce(self, logits: np.ndarray, labels: np.ndarray, *, V: int | None = None, ignore_index: int = -100,
           label_smoothing: float = 0.0, softcap: float = 0.0, reduction: str = "mean",
           grad_out=None, rows=None, want_grad: bool = True, nthreads: int = 0) -> dict:
        """Cross-entropy forward + backward by definition, in fp64.

        logits: [n, ld] uint16 (bf16 bits), float32 or float64; the first V columns are the row.
        rows:   optional row indices to evaluate (counts n_valid/n_bad still cover all rows).
        Returns loss_tok [len(rows)], argmax, counts {n_valid, n_correct(rows), n_bad},
        loss_out (only when all rows were evaluated) and grad [len(rows), V] fp64 (unrounded).
        """
        lib = self.lib
        logits = np.ascontiguousarray(logits)
        if logits.ndim != 2:
            raise ValueError("logits must be 2-D")
        n, ld = logits.shape
        V = ld if V is None else int(V)
        labels = np.ascontiguousarray(labels, dtype=np.int64)
        if labels.shape != (n,):
            raise ValueError("labels must be [n]")
        red = _REDUCTIONS[reduction]
        g = _grad_out_array(grad_out, red, n)
        if rows is None:
            rows_arr = None
            nrows = n
        else:
            rows_arr = np.ascontiguousarray(rows, dtype=np.int64)
            nrows = rows_arr.size
        loss = np.zeros(nrows, dtype=np.float64)
        amax = np.zeros(nrows, dtype=np.int64)
        grad = np.zeros((nrows, V), dtype=np.float64) if want_grad else None
        counts = np.zeros(3, dtype=np.int64)
        rc = lib.lce_oracle_ce(_ptr(logits), ld, _dtype_code(logits), _ptr(labels), n, V, int(ignore_index),
                               float(label_smoothing), float(softcap), red, _ptr(g), _ptr(rows_arr), nrows,
                               _ptr(loss), _ptr(amax), _ptr(grad), _ptr(counts), int(nthreads))
        if rc != 0:
            raise ValueError("lce_oracle_ce rejected its arguments")
        out = {"loss_tok": loss, "argmax": amax, "counts": counts, "grad": grad}
        if rows is None:
            out["loss_out"] = lib.lce_oracle_reduce_loss(_ptr(loss), n, int(counts[0]), red)
        return out

    def reduce_loss(self, loss_tok: np.ndarray, n_valid: int, reduction: str) -> float:
        lib = self.lib
        lt = np.ascontiguousarray(loss_tok, dtype=np.float64)
        return lib.lce_oracle_reduce_loss(_ptr(lt), lt.size, int(n_valid), _REDUCTIONS[reduction])

    def count(self, labels: np.ndarray, V: int, ignore_index: int = -100) -> tuple[int, int]:
        lib = self.lib
        lab = np.ascontiguousarray(labels, dtype=np.int64)
        nv = ctypes.c_int64(0)
        nb = ctypes.c_int64(0)
        lib.lce_oracle_count(_ptr(lab), lab.size, int(V), int(ignore_index), ctypes.byref(nv), ctypes.byref(nb))
        return nv.value, nb.value

    def row_stats(self, logits: np.ndarray, labels: np.ndarray, *, V: int | None = None, ignore_index: int = -100,
                  softcap: float = 0.0, rows=None, nthreads: int = 0) -> dict:
        """Per-row log-sum-exp, target log-probability (0 for ignored rows) and entropy of the softmax over
        the (capped) logits, in fp64 (labs-molt PR "Enable Liger layers": action log-probabilities and
        entropy)."""
        logits = np.ascontiguousarray(logits)
        n, ld = logits.shape
        V = ld if V is None else int(V)
        labels = np.ascontiguousarray(labels, dtype=np.int64)
        rows_arr = None if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
        nrows = n if rows is None else rows_arr.size
        lse = np.zeros(nrows)
        logp = np.zeros(nrows)
        ent = np.zeros(nrows)
        rc = self.lib.lce_oracle_row_stats(_ptr(logits), ld, _dtype_code(logits), _ptr(labels), n, V,
                                           int(ignore_index), float(softcap), _ptr(rows_arr), nrows, _ptr(lse),
                                           _ptr(logp), _ptr(ent), int(nthreads))
        if rc != 0:
            raise ValueError("lce_oracle_row_stats rejected its arguments")
        return {"lse": lse, "logp": logp, "entropy": ent}

    def round_bf16(self, x: np.ndarray) -> np.ndarray:
        """fp64 -> bf16 bit patterns (uint16), round to nearest even, in one step."""
        lib = self.lib
        src = np.ascontiguousarray(x, dtype=np.float64)
        out = np.empty(src.shape, dtype=np.uint16)
        lib.lce_oracle_round_bf16(_ptr(src), _ptr(out), src.size)
        return out

    def flce(self, hidden: np.ndarray, weight: np.ndarray, labels: np.ndarray, *, ignore_index: int = -100,
             label_smoothing: float = 0.0, softcap: float = 0.0, reduction: str = "mean", grad_out=None,
             nthreads: int = 0) -> dict:
        """Fused linear cross-entropy by definition (fp64, no chunking).

        hidden [n, H] and weight [V, H] are bf16 bit patterns (uint16).  Returns loss_tok, loss_out,
        grad_hidden [n, H] and grad_weight [V, H] in fp64, and counts.
        """
        lib = self.lib
        hidden = np.ascontiguousarray(hidden, dtype=np.uint16)
        weight = np.ascontiguousarray(weight, dtype=np.uint16)
        n, H = hidden.shape
        V, H2 = weight.shape
        if H2 != H:
            raise ValueError("hidden and weight disagree on H")
        labels = np.ascontiguousarray(labels, dtype=np.int64)
        red = _REDUCTIONS[reduction]
        g = _grad_out_array(grad_out, red, n)
        loss = np.zeros(n, dtype=np.float64)
        loss_out = ctypes.c_double(0.0)
        dh = np.zeros((n, H), dtype=np.float64)
        dw = np.zeros((V, H), dtype=np.float64)
        counts = np.zeros(3, dtype=np.int64)
        rc = lib.lce_oracle_flce(_ptr(hidden), _ptr(weight), _ptr(labels), n, H, V, int(ignore_index),
                                 float(label_smoothing), float(softcap), red, _ptr(g), _ptr(loss),
                                 ctypes.byref(loss_out), _ptr(dh), _ptr(dw), _ptr(counts), int(nthreads))
        if rc != 0:
            raise ValueError("lce_oracle_flce rejected its arguments")
        return {"loss_tok": loss, "loss_out": loss_out.value, "grad_hidden": dh, "grad_weight": dw,
                "counts": counts}


def flce_sampled(orc: "Oracle", hidden: np.ndarray, weight: np.ndarray, labels: np.ndarray, tokens, vocab_rows, *,
                 ignore_index: int = -100, label_smoothing: float = 0.0, softcap: float = 0.0,
                 reduction: str = "mean", grad_out: float = 1.0, block: int = 256, nthreads: int = 0) -> dict:
    """Fused linear cross-entropy at sizes where the plain-loop definition is too slow (Liger-Kernel PR
    "Add Liger Kernel support for Muse Glimmer", Summary / Memory): the logits Z = H W^T of every token in
    fp64 by a library matmul (bf16 inputs are exact in fp64), the per-token loss and gradient G by the
    oracle's own row routine on those fp64 logits, then dH = G W for the sampled tokens and dW = G^T H for
    the sampled vocabulary rows, both in fp64.  The mean is over every valid label (reduction 'mean' or
    'sum'; grad_out is the scalar upstream gradient).

    Returns loss_tok [n], loss_out, counts, grad_hidden [len(tokens), H], grad_weight [len(vocab_rows), H]
    and zmax [n], the largest |z| of each token's (capped) logits.
    """
    hidden = np.ascontiguousarray(hidden, dtype=np.uint16)
    weight = np.ascontiguousarray(weight, dtype=np.uint16)
    labels = np.ascontiguousarray(labels, dtype=np.int64)
    n, H = hidden.shape
    V = weight.shape[0]
    tokens = np.asarray(tokens, dtype=np.int64)
    vocab_rows = np.asarray(vocab_rows, dtype=np.int64)
    h64 = (hidden.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    w64 = (weight.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    n_valid, n_bad = orc.count(labels, V, ignore_index)
    if reduction == "mean":
        scale = grad_out / n_valid if n_valid > 0 else 0.0
    elif reduction == "sum":
        scale = grad_out
    else:
        raise ValueError("flce_sampled covers the mean and sum reductions")
    loss = np.zeros(n)
    zmax = np.zeros(n)
    gw = np.zeros((vocab_rows.size, H))
    g_tok = np.zeros((tokens.size, V))
    for b0 in range(0, n, block):
        b1 = min(n, b0 + block)
        z = h64[b0:b1] @ w64.T
        zmax[b0:b1] = np.abs(softcap * np.tanh(z / softcap) if softcap > 0 else z).max(axis=1)
        # the row routine with reduction 'sum' and the upstream gradient set to the call's scale gives
        # the per-token losses and s_i (softmax - target) of these rows
        o = orc.ce(z, labels[b0:b1], V=V, ignore_index=ignore_index, label_smoothing=label_smoothing,
                   softcap=softcap, reduction="sum", grad_out=[scale], want_grad=True, nthreads=nthreads)
        loss[b0:b1] = o["loss_tok"]
        g = o["grad"]
        gw += g[:, vocab_rows].T @ h64[b0:b1]
        sel = np.flatnonzero((tokens >= b0) & (tokens < b1))
        g_tok[sel] = g[tokens[sel] - b0]
    gh = g_tok @ w64
    loss_out = orc.reduce_loss(loss, n_valid, reduction)
    return {"loss_tok": loss, "loss_out": loss_out, "counts": np.array([n_valid, 0, n_bad]),
            "grad_hidden": gh, "grad_weight": gw, "zmax": zmax}


def flce_rows(orc: "Oracle", hidden: np.ndarray, weight: np.ndarray, labels: np.ndarray, *, tokens=None,
              ignore_index: int = -100, label_smoothing: float = 0.0, softcap: float = 0.0,
              grad_scale: float | None = None, block: int = 256, nthreads: int = 0) -> dict:
    """Per-token row outputs of the fused linear cross-entropy (Liger-Kernel PR "Add Liger Kernel
    support for Muse Glimmer", Summary: loss and token accuracy without the logits; labs-molt PR
    "Enable Liger layers": log-probabilities and entropy): the logits Z = H W^T of the chosen tokens
    in fp64 by a library matmul (bf16 inputs are exact in fp64), then the oracle's row routines on them.

    Returns, per token: loss_tok (reduction 'none', with the given smoothing), argmax (first index of
    the raw logits), lse, logp, entropy, and gap = the largest raw logit minus the largest at any other
    index; with grad_scale s, also grad_hidden = G W for these tokens, G = s (p - t) dz/dx being the
    row routine's gradient (s = the upstream gradient over the mean's denominator, or as given).
    """
    hidden = np.ascontiguousarray(hidden, dtype=np.uint16)
    weight = np.ascontiguousarray(weight, dtype=np.uint16)
    labels = np.ascontiguousarray(labels, dtype=np.int64)
    n = hidden.shape[0]
    V = weight.shape[0]
    tokens = np.arange(n) if tokens is None else np.asarray(tokens, dtype=np.int64)
    h64 = (hidden.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    w64 = (weight.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    out = {k: np.zeros(tokens.size) for k in ("loss_tok", "lse", "logp", "entropy", "gap")}
    out["argmax"] = np.zeros(tokens.size, dtype=np.int64)
    if grad_scale is not None:
        out["grad_hidden"] = np.zeros((tokens.size, hidden.shape[1]))
    for b0 in range(0, tokens.size, block):
        sel = tokens[b0:b0 + block]
        z = h64[sel] @ w64.T
        y = labels[sel]
        # reduction 'sum' with the upstream gradient set to the scale: per-token losses and s (p - t)
        o = orc.ce(z, y, V=V, ignore_index=ignore_index, label_smoothing=label_smoothing, softcap=softcap,
                   reduction="sum", grad_out=[1.0 if grad_scale is None else grad_scale],
                   want_grad=grad_scale is not None, nthreads=nthreads)
        if grad_scale is not None:
            out["grad_hidden"][b0:b0 + block] = o["grad"] @ w64
        st = orc.row_stats(z, y, V=V, ignore_index=ignore_index, softcap=softcap, nthreads=nthreads)
        out["loss_tok"][b0:b0 + block] = o["loss_tok"]
        out["argmax"][b0:b0 + block] = o["argmax"]
        for k in ("lse", "logp", "entropy"):
            out[k][b0:b0 + block] = st[k]
        top = z[np.arange(sel.size), o["argmax"]]
        rest = z.copy()
        rest[np.arange(sel.size), o["argmax"]] = -np.inf
        out["gap"][b0:b0 + block] = top - rest.max(axis=1) if V > 1 else np.inf
    return out


_default: Oracle | None = None


def default() -> Oracle:
    """The oracle built from lce_oracle.c next to this file (built on first use)."""
    global _default
    if _default is None:
        _default = Oracle()
    return _default


def ce(*a, **k):
    return default().ce(*a, **k)


def flce(*a, **k):
    return default().flce(*a, **k)


def round_bf16(x):
    return default().round_bf16(x)


def count(*a, **k):
    return default().count(*a, **k)


def reduce_loss(*a, **k):
    return default().reduce_loss(*a, **k)
