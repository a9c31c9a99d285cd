"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each ``pin_*`` takes an ``oracle.Oracle`` and raises AssertionError when the
oracle disagrees with a closed form, an invariant, a brute-force count, central
finite differences, a hand-derived fixture (tests/golden) or an independent
library definition (PyTorch's fp64 ``cross_entropy``, which the Liger CE page's
"Test setup" names as the same operation).

The pins are plain functions so that ``test_oracle_mutants.py`` can run all of
them against copies of the oracle with a planted mistake and check that every
planted mistake is caught by at least one pin.
"""
from __future__ import annotations

import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import synth
import torch
import torch.nn.functional as F

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")

REDS = ("none", "mean", "sum")


def _close(a, b, atol, rtol=0.0, what=""):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    err = np.abs(a - b)
    lim = atol + rtol * np.abs(b)
    if not np.all(err <= lim):
        k = int(np.argmax(err - lim))
        raise AssertionError(f"{what}: max violation at flat index {k}: got {a.reshape(-1)[k]!r}, "
                             f"want {b.reshape(-1)[k]!r} (|err|={err.reshape(-1)[k]:.3e})")


def _scale(reduction, grad_out, i, n_valid):
    if reduction == "none":
        return 1.0 if grad_out is None else float(np.asarray(grad_out).reshape(-1)[i])
    g = 1.0 if grad_out is None else float(np.asarray(grad_out).reshape(-1)[0])
    if reduction == "mean":
        return g / n_valid if n_valid else 0.0
    return g


# ----------------------------------------------------------------------------- closed forms

def pin_uniform_rows(orc):
    """Constant rows: p_j = 1/V, so loss = ln V for every eps (and every cap, since a
    constant row stays constant after T*tanh(x/T)); the gradient is
    scale*(1/V - (1-eps)[j==y] - eps/V)*chain."""
    for V in (1, 2, 7, 4096):
        for eps in (0.0, 0.1, 1.0):
            for T in (0.0, 30.0):
                n = 3
                c = np.array([[0.0], [1.25], [-3.5]])
                x = np.repeat(c, V, axis=1)
                y = np.array([0, V - 1, V // 2], dtype=np.int64)
                o = orc.ce(x, y, label_smoothing=eps, softcap=T, reduction="sum", grad_out=[0.75])
                _close(o["loss_tok"], [math.log(V)] * n, 1e-12, 1e-13, f"uniform loss V={V}")
                for i in range(n):
                    chain = 1.0 - math.tanh(c[i, 0] / T) ** 2 if T > 0 else 1.0
                    want = np.full(V, 1.0 / V - eps / V)
                    want[y[i]] -= 1.0 - eps
                    _close(o["grad"][i], 0.75 * want * chain, 1e-14, 1e-12, f"uniform grad V={V} eps={eps} T={T}")


def pin_v2_closed_form(orc):
    """V=2, eps=0: loss = log(1 + e^(z_o - z_y)), d/dz_o = sigmoid(z_o - z_y) = -d/dz_y."""
    rng = np.random.default_rng(11)
    x = rng.normal(0, 3, size=(6, 2))
    y = np.array([0, 1, 1, 0, 1, 0], dtype=np.int64)
    o = orc.ce(x, y, reduction="sum")
    for i in range(6):
        d = x[i, 1 - y[i]] - x[i, y[i]]
        _close(o["loss_tok"][i], math.log1p(math.exp(d)), 1e-13, 1e-13, "V=2 loss")
        sig = 1.0 / (1.0 + math.exp(-d))
        _close(o["grad"][i, 1 - y[i]], sig, 1e-14, 1e-13, "V=2 grad other")
        _close(o["grad"][i, y[i]], -sig, 1e-14, 1e-13, "V=2 grad label")


def pin_v1(orc):
    """V=1: the only class has probability 1, loss 0 and gradient 0 (any eps)."""
    for eps in (0.0, 0.5):
        o = orc.ce(np.array([[3.0], [-2.0]]), np.array([0, 0]), label_smoothing=eps, reduction="sum")
        _close(o["loss_tok"], [0.0, 0.0], 1e-15, 0, "V=1 loss")
        _close(o["grad"], np.zeros((2, 1)), 1e-15, 0, "V=1 grad")


def pin_golden_fixtures(orc):
    """Hand-derived worked cases in tests/golden/closed_forms.json (exact expressions)."""
    with open(os.path.join(GOLDEN, "closed_forms.json")) as f:
        cases = json.load(f)["cases"]
    env = {"log": math.log, "exp": math.exp, "tanh": math.tanh, "atanh": math.atanh, "F": Fraction}
    for c in cases:
        x = np.array([[float(eval(s, env)) for s in c["logits"]]])
        T = float(eval(c["softcap"], env))
        o = orc.ce(x, np.array([c["label"]]), label_smoothing=float(eval(c["eps"], env)), softcap=T,
                   reduction="sum", grad_out=[float(eval(c["grad_out"], env))])
        _close(o["loss_tok"][0], float(eval(c["loss"], env)), 1e-14, 1e-13, c["name"] + " loss")
        _close(o["grad"][0], [float(eval(s, env)) for s in c["grad"]], 1e-14, 1e-13, c["name"] + " grad")
        _close(o["argmax"][0], c["argmax"], 0, 0, c["name"] + " argmax")


# ----------------------------------------------------------------------------- invariants

def pin_rowsum_zero(orc):
    """Without a cap, sum_j dloss/dz_j = 1 - (1-eps) - eps = 0 on every valid row."""
    rng = np.random.default_rng(12)
    for eps in (0.0, 0.3, 1.0):
        x = rng.normal(0, 4, size=(8, 33))
        y = rng.integers(0, 33, 8)
        o = orc.ce(x, y, label_smoothing=eps, reduction="sum")
        _close(o["grad"].sum(axis=1), np.zeros(8), 1e-14, 0, f"row sum eps={eps}")
        if np.all(np.abs(o["grad"]) < 1e-12):
            raise AssertionError("gradient vanished")


def pin_shift_invariance(orc):
    """Without a cap, adding a constant to a row changes neither loss nor gradient."""
    rng = np.random.default_rng(13)
    x = rng.normal(0, 2, size=(5, 19))
    y = rng.integers(0, 19, 5)
    a = orc.ce(x, y, label_smoothing=0.2)
    b = orc.ce(x + 7.5, y, label_smoothing=0.2)
    _close(b["loss_tok"], a["loss_tok"], 1e-12, 1e-12, "shift loss")
    _close(b["grad"], a["grad"], 1e-15, 1e-10, "shift grad")


def pin_smoothing_identity(orc):
    """loss = (1-eps)(-log p_y) + (eps/V) sum_j (-log p_j), with log p from a log-sum-exp
    computed here by numpy (logaddexp.reduce)."""
    rng = np.random.default_rng(14)
    for eps in (0.0, 0.1, 0.7):
        x = rng.normal(0, 3, size=(6, 25))
        y = rng.integers(0, 25, 6)
        o = orc.ce(x, y, label_smoothing=eps, reduction="none")
        logp = x - np.logaddexp.reduce(x, axis=1, keepdims=True)
        want = (1 - eps) * -logp[np.arange(6), y] + (eps / 25) * (-logp).sum(axis=1)
        _close(o["loss_tok"], want, 1e-12, 1e-12, f"smoothing identity eps={eps}")


def pin_reductions(orc):
    """sum = mean * n_valid; none scales each row's gradient by its own upstream value."""
    rng = np.random.default_rng(15)
    x = rng.normal(0, 2, size=(9, 11))
    y = rng.integers(0, 11, 9)
    y[[2, 5]] = -100
    m = orc.ce(x, y, reduction="mean")
    s = orc.ce(x, y, reduction="sum")
    _close(s["loss_out"], m["loss_out"] * 7, 1e-12, 1e-12, "sum = mean * n_valid")
    _close(s["grad"], m["grad"] * 7, 1e-15, 1e-12, "sum grad = mean grad * n_valid")
    g = rng.normal(size=9)
    nn = orc.ce(x, y, reduction="none", grad_out=g)
    _close(nn["grad"], s["grad"] * g[:, None], 1e-15, 1e-12, "none grad = g_i * sum grad")


def pin_rows_subset(orc):
    """Evaluating a subset of rows reproduces those rows of the full evaluation, and the
    mean scale still uses n_valid over all rows."""
    rng = np.random.default_rng(16)
    x = rng.normal(0, 2, size=(10, 13))
    y = rng.integers(0, 13, 10)
    y[[1, 4]] = -100
    full = orc.ce(x, y)
    rows = np.array([7, 1, 3])
    sub = orc.ce(x, y, rows=rows)
    _close(sub["loss_tok"], full["loss_tok"][rows], 0, 0, "subset loss")
    _close(sub["grad"], full["grad"][rows], 0, 0, "subset grad")
    if sub["counts"][0] != 8 or full["counts"][0] != 8:
        raise AssertionError("n_valid must cover all rows")


def pin_dtype_loading(orc):
    """bf16 bit patterns and float32 inputs are read exactly; padding columns [V, ld) are
    never read (they hold NaN here)."""
    rng = np.random.default_rng(17)
    f = rng.normal(0, 2, size=(4, 9)).astype(np.float32)
    bits = (f.view(np.uint32) >> 16).astype(np.uint16)
    widened = (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    y = np.array([0, 8, 3, -100])
    a = orc.ce(bits, y, label_smoothing=0.1)
    b = orc.ce(widened, y, label_smoothing=0.1)
    _close(a["loss_tok"], b["loss_tok"], 0, 0, "bf16 load")
    _close(a["grad"], b["grad"], 0, 0, "bf16 load grad")
    c = orc.ce(f, y, label_smoothing=0.1)
    d = orc.ce(f.astype(np.float64), y, label_smoothing=0.1)
    _close(c["grad"], d["grad"], 0, 0, "f32 load")
    pad = np.full((4, 12), np.nan, dtype=np.float32)
    pad[:, :9] = f
    e = orc.ce(pad, y, V=9, label_smoothing=0.1)
    _close(e["grad"], c["grad"], 0, 0, "padded rows")
    _close(e["loss_tok"], c["loss_tok"], 0, 0, "padded rows loss")


# ----------------------------------------------------------------------------- masks, argmax

def pin_ignore_and_bad_labels(orc):
    """ignore_index rows and out-of-range labels give zero loss and zero gradient, are left out
    of the mean, and are counted (n_valid, n_bad)."""
    rng = np.random.default_rng(18)
    x = rng.normal(0, 2, size=(7, 6))
    y = np.array([1, -100, 5, 6, -7, 0, -100])
    o = orc.ce(x, y)
    if tuple(o["counts"][[0, 2]]) != (3, 2):
        raise AssertionError(f"counts {o['counts']}")
    bad = np.array([1, 3, 4, 6])
    _close(o["loss_tok"][bad], np.zeros(4), 0, 0, "masked loss")
    _close(o["grad"][bad], np.zeros((4, 6)), 0, 0, "masked grad")
    keep = np.array([0, 2, 5])
    ref = orc.ce(x[keep], y[keep])
    _close(o["loss_out"], ref["loss_out"], 1e-13, 1e-13, "mean excludes masked rows")
    _close(o["grad"][keep], ref["grad"], 1e-16, 1e-13, "valid-row grads")


def pin_all_ignored(orc):
    """Mean over zero valid tokens: loss 0 and all-zero gradient (torch would give NaN)."""
    x = np.random.default_rng(19).normal(size=(3, 5))
    o = orc.ce(x, np.array([-100, -100, -100]))
    if o["loss_out"] != 0.0 or np.any(o["grad"] != 0.0) or o["counts"][0] != 0:
        raise AssertionError("all-ignored mean must be 0 with zero gradient")


def _first_argmax(row):
    best = 0
    for j in range(1, len(row)):
        if row[j] > row[best]:
            best = j
    return best


def pin_argmax_bruteforce(orc):
    """argmax = smallest index of the row maximum over the raw values, for every row; token
    accuracy counts valid rows whose argmax is the label."""
    rng = np.random.default_rng(20)
    x = np.clip(np.rint(rng.normal(0, 3, size=(40, 17))), -4, 4)   # many ties
    x[0] = 0.0
    x[1] = [-0.0 if j % 2 else 0.0 for j in range(17)]               # signed zeros tie
    x[2, :] = -4.0
    x[2, 16] = -3.0
    x[3, :] = 2.0
    y = rng.integers(0, 17, 40)
    y[[5, 9]] = -100
    for i in range(40):
        if i % 3 == 0:
            y[i] = _first_argmax(x[i])
    for T in (0.0, 30.0):
        o = orc.ce(x, y, softcap=T)
        want = np.array([_first_argmax(r) for r in x])
        if not np.array_equal(o["argmax"], want):
            raise AssertionError(f"argmax mismatch at rows {np.nonzero(o['argmax'] != want)[0]}")
        if not np.array_equal(o["argmax"], torch.argmax(torch.tensor(x), dim=1).numpy()):
            raise AssertionError("argmax disagrees with torch.argmax (first maximal index)")
        valid = (y >= 0) & (y < 17)
        if o["counts"][1] != int(np.sum(valid & (want == y))):
            raise AssertionError("n_correct")


# ----------------------------------------------------------------------------- library pins

def _torch_ce(x, y, eps, T, reduction, grad_out, V=None):
    t = torch.tensor(x, dtype=torch.float64, requires_grad=True)
    z = T * torch.tanh(t / T) if T > 0 else t
    yy = torch.tensor(y)
    loss = F.cross_entropy(z, yy, ignore_index=-100, label_smoothing=eps, reduction=reduction)
    if reduction == "none":
        g = torch.ones(len(y), dtype=torch.float64) if grad_out is None else torch.tensor(grad_out)
        (loss * g).sum().backward()
    else:
        g = 1.0 if grad_out is None else float(np.asarray(grad_out).reshape(-1)[0])
        (loss * g).backward()
    return loss.detach().numpy(), t.grad.numpy()


def pin_torch_library(orc):
    """PyTorch fp64 cross_entropy (+ autograd) for every reduction, several eps, with ignored
    rows and an upstream gradient."""
    rng = np.random.default_rng(21)
    for V in (3, 50):
        x = rng.normal(0, 3, size=(12, V))
        y = rng.integers(0, V, 12)
        y[[0, 7]] = -100
        for eps in (0.0, 0.1, 1.0):
            for red in REDS:
                g = rng.normal(size=12) if red == "none" else [0.5]
                o = orc.ce(x, y, label_smoothing=eps, reduction=red, grad_out=g)
                tl, tg = _torch_ce(x, y, eps, 0.0, red, g)
                got = o["loss_tok"] if red == "none" else o["loss_out"]
                _close(got, tl, 1e-12, 1e-12, f"torch loss V={V} eps={eps} {red}")
                _close(o["grad"], tg, 1e-15, 1e-11, f"torch grad V={V} eps={eps} {red}")


def pin_torch_softcap(orc):
    """Softcap composes: CE_T(x) = CE(T*tanh(x/T)); autograd supplies the chain factor."""
    rng = np.random.default_rng(22)
    x = rng.normal(0, 10, size=(10, 40))
    y = rng.integers(0, 40, 10)
    y[3] = -100
    for T in (30.0, 2.5):
        for eps in (0.0, 0.2):
            o = orc.ce(x, y, softcap=T, label_smoothing=eps)
            tl, tg = _torch_ce(x, y, eps, T, "mean", None)
            _close(o["loss_out"], tl, 1e-12, 1e-12, f"softcap loss T={T}")
            _close(o["grad"], tg, 1e-16, 1e-11, f"softcap grad T={T}")
    # a very large cap is the identity up to O((x/T)^2)
    a = orc.ce(x, y, softcap=1e7)
    b = orc.ce(x, y)
    _close(a["loss_tok"], b["loss_tok"], 1e-9, 0, "T -> inf")


# ----------------------------------------------------------------------------- finite differences

def pin_finite_differences(orc):
    """Central differences of the objective J (mean/sum: g * loss_out; none: sum_i g_i loss_i)
    match the analytic gradient on tiny inputs, for every eps / cap / reduction."""
    rng = np.random.default_rng(23)
    h = 1e-6
    for red in REDS:
        for eps in (0.0, 0.25):
            for T in (0.0, 3.0):
                n, V = 4, 6
                x = rng.normal(0, 2, size=(n, V))
                y = rng.integers(0, V, n)
                y[2] = -100
                g = rng.normal(size=n) if red == "none" else [rng.normal()]
                o = orc.ce(x, y, label_smoothing=eps, softcap=T, reduction=red, grad_out=g)

                def J(xx):
                    r = orc.ce(xx, y, label_smoothing=eps, softcap=T, reduction=red, want_grad=False)
                    if red == "none":
                        return float(np.dot(r["loss_tok"], g))
                    return float(r["loss_out"] * g[0])

                fd = np.zeros_like(x)
                for i in range(n):
                    for j in range(V):
                        xp = x.copy()
                        xm = x.copy()
                        xp[i, j] += h
                        xm[i, j] -= h
                        fd[i, j] = (J(xp) - J(xm)) / (2 * h)
                _close(o["grad"], fd, 1e-7, 0, f"FD red={red} eps={eps} T={T}")


# ----------------------------------------------------------------------------- rounding

def pin_bf16_rounding(orc):
    """fp64 -> bf16 round-to-nearest-even: torch's float32 -> bfloat16 cast on float32
    inputs, exact midpoints tie to even, just-off-midpoint values go to the nearer side,
    the subnormal spacing 2^-133, overflow to infinity and signed zero."""
    rng = np.random.default_rng(24)
    f = (rng.standard_normal(20000) * np.exp(rng.uniform(-80, 80, 20000))).astype(np.float32)
    want = torch.tensor(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = orc.round_bf16(f.astype(np.float64))
    if not np.array_equal(got, want):
        raise AssertionError("bf16 rounding differs from torch on float32 inputs")
    # midpoints between adjacent bf16 values a < b: ties go to the even significand
    bits = np.array([0x3F80, 0x3F81, 0x4000, 0x0080, 0x0001, 0x7F7E], dtype=np.uint32)
    lo = (bits << 16).view(np.float32).astype(np.float64)
    hi = ((bits + 1) << 16).view(np.float32).astype(np.float64)
    mid = (lo + hi) / 2
    r = orc.round_bf16(mid)
    even = np.where(bits % 2 == 0, bits, bits + 1).astype(np.uint16)
    if not np.array_equal(r, even):
        raise AssertionError(f"ties-to-even: got {r}, want {even}")
    up = orc.round_bf16(mid + (hi - lo) * 1e-6)
    dn = orc.round_bf16(mid - (hi - lo) * 1e-6)
    if not (np.array_equal(up, (bits + 1).astype(np.uint16)) and np.array_equal(dn, bits.astype(np.uint16))):
        raise AssertionError("off-midpoint rounding")
    if orc.round_bf16(np.array([2.0 ** -133 * 5.49]))[0] != 5:
        raise AssertionError("subnormal spacing")
    if orc.round_bf16(np.array([2.0 ** 128]))[0] != 0x7F80 or orc.round_bf16(np.array([-0.0]))[0] != 0x8000:
        raise AssertionError("overflow / signed zero")


# ----------------------------------------------------------------------------- fused linear

def _bf16_bits(a):
    f = np.asarray(a, dtype=np.float32)
    return (f.view(np.uint32) >> 16).astype(np.uint16)


def _from_bits(b):
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def pin_flce_zero_hidden(orc):
    """hidden = 0: Z = 0, loss = ln V, grad_weight = 0 and
    grad_hidden_i = scale * (1-eps) * (mean_v W_v - W_{y_i}) (the cap's chain factor is 1 at 0)."""
    rng = np.random.default_rng(25)
    n, H, V = 5, 8, 12
    Wb = _bf16_bits(rng.normal(0, 0.5, size=(V, H)))
    W = _from_bits(Wb)
    y = np.array([3, -100, 0, 11, 7])
    for eps, T in ((0.0, 0.0), (0.3, 30.0)):
        o = orc.flce(np.zeros((n, H), np.uint16), Wb, y, label_smoothing=eps, softcap=T)
        _close(o["loss_tok"][[0, 2, 3, 4]], [math.log(V)] * 4, 1e-13, 1e-13, "flce h=0 loss")
        _close(o["grad_weight"], np.zeros((V, H)), 0, 0, "flce h=0 dW")
        scale = 1.0 / 4
        for i in range(n):
            want = np.zeros(H) if y[i] < 0 else scale * (1 - eps) * (W.mean(axis=0) - W[y[i]])
            _close(o["grad_hidden"][i], want, 1e-15, 1e-12, "flce h=0 dH")


def pin_flce_composition(orc):
    """FLCE equals CE on the materialised Z = hidden * weight^T (numpy fp64 matmul), with
    grad_hidden = G * W and grad_weight = G^T * hidden (chain rule of the product)."""
    rng = np.random.default_rng(26)
    n, H, V = 9, 16, 40
    Hb = _bf16_bits(rng.normal(0, 1, size=(n, H)))
    Wb = _bf16_bits(rng.normal(0, 0.3, size=(V, H)))
    Hd, Wd = _from_bits(Hb), _from_bits(Wb)
    y = rng.integers(0, V, n)
    y[4] = -100
    for eps, T, red in ((0.0, 0.0, "mean"), (0.1, 30.0, "sum"), (0.0, 2.0, "none")):
        g = rng.normal(size=n) if red == "none" else [0.7]
        o = orc.flce(Hb, Wb, y, label_smoothing=eps, softcap=T, reduction=red, grad_out=g)
        Z = Hd @ Wd.T
        c = orc.ce(Z, y, label_smoothing=eps, softcap=T, reduction=red, grad_out=g)
        _close(o["loss_tok"], c["loss_tok"], 1e-13, 1e-13, "flce loss = ce(HW^T)")
        _close(o["loss_out"], c["loss_out"], 1e-13, 1e-13, "flce reduced loss")
        _close(o["grad_hidden"], c["grad"] @ Wd, 1e-15, 1e-11, "flce dH = G W")
        _close(o["grad_weight"], c["grad"].T @ Hd, 1e-15, 1e-11, "flce dW = G^T H")
        if not np.array_equal(o["counts"], c["counts"]):
            raise AssertionError("flce counts")


# ----------------------------------------------------------------------------- row statistics

def pin_row_stats_closed_forms(orc):
    """Constant rows: lse = c + ln V, entropy = ln V, log p_y = -ln V.  V = 2: lse = log(e^a + e^b),
    entropy = the binary entropy of sigmoid(a - b).  Ignored rows give log p = 0 but keep their entropy."""
    for V in (1, 2, 7, 1000):
        x = np.full((3, V), 1.75)
        y = np.array([0, V - 1, -100])
        o = orc.row_stats(x, y)
        _close(o["lse"], np.full(3, 1.75 + math.log(V)), 1e-13, 1e-13, f"uniform lse V={V}")
        _close(o["entropy"], np.full(3, math.log(V)), 1e-12, 1e-13, f"uniform entropy V={V}")
        _close(o["logp"], np.array([-math.log(V), -math.log(V), 0.0]), 1e-13, 1e-13, f"uniform logp V={V}")
    a, b = 1.3, -0.4
    o = orc.row_stats(np.array([[a, b]]), np.array([1]))
    pa = 1.0 / (1.0 + math.exp(b - a))
    _close(o["lse"], [math.log(math.exp(a) + math.exp(b))], 1e-14, 0, "V=2 lse")
    _close(o["logp"], [math.log(1.0 - pa)], 1e-14, 0, "V=2 logp")
    _close(o["entropy"], [-(pa * math.log(pa) + (1 - pa) * math.log(1 - pa))], 1e-14, 0, "V=2 entropy")


def pin_row_stats_torch(orc):
    """PyTorch fp64 logsumexp, log_softmax at the target and Categorical entropy, with and without the
    softcap (applied to the logits first), on rows of mixed scale; row subsets and bf16 loading."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(31)
    x = rng.normal(0, 4, size=(9, 300))
    x[2] *= 20.0
    y = rng.integers(0, 300, 9)
    y[4] = -100
    for T in (0.0, 30.0, 3.0):
        t = torch.from_numpy(x)
        z = T * torch.tanh(t / T) if T > 0 else t
        lse = torch.logsumexp(z, dim=1).numpy()
        lsm = torch.log_softmax(z, dim=1).numpy()
        ent = torch.distributions.Categorical(logits=z).entropy().numpy()
        o = orc.row_stats(x, y, softcap=T)
        _close(o["lse"], lse, 1e-13, 1e-12, f"torch lse T={T}")
        want = np.array([lsm[i, y[i]] if y[i] >= 0 else 0.0 for i in range(9)])
        _close(o["logp"], want, 1e-13, 1e-12, f"torch logp T={T}")
        _close(o["entropy"], ent, 1e-12, 1e-12, f"torch entropy T={T}")
    rows = np.array([8, 0, 4])
    sub = orc.row_stats(x, y, rows=rows)
    full = orc.row_stats(x, y)
    _close(sub["entropy"], full["entropy"][rows], 0, 0, "row subset")
    xb = synth.f32_to_bf16_bits(x.astype(np.float32))
    xb64 = synth.bf16_bits_to_f32(xb).astype(np.float64)
    _close(orc.row_stats(xb, y)["lse"], orc.row_stats(xb64, y)["lse"], 0, 0, "bf16 loading")


def pin_row_stats_match_loss(orc):
    """Without smoothing the per-token loss is -log p_y, and lse - z_y; the entropy of a row equals the
    label-smoothing loss term (1/V) sum_j (-log p_j) only for the uniform row, where both are ln V."""
    rng = np.random.default_rng(32)
    x = rng.normal(0, 2, size=(6, 40))
    y = rng.integers(0, 40, 6)
    y[1] = -100
    for T in (0.0, 7.0):
        o = orc.row_stats(x, y, softcap=T)
        c = orc.ce(x, y, softcap=T, want_grad=False)
        _close(-o["logp"], c["loss_tok"], 1e-13, 1e-13, f"logp vs loss T={T}")


PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
