"""GPU parity of rows that do not start on a 16-byte boundary against the fp64 oracle.

Odd V, a row stride that is not a multiple of the 16-byte vector, or a logits base that is
not 16-byte aligned: the persistent row kernel then reads each row through the aligned
window that holds it, masks the neighbouring rows' elements in the window's first and last
vector and stores the row's own elements of those vectors one at a time.  Every case
compares the whole buffer, so a store into a neighbouring row (or into padding) fails it.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from parity import check_bf16_grad, check_f32_grad, check_loss, row_scales, smoothing_allowance
from test_gpu_ce import DEV, _labels, from_dev, make_logits, run_and_check, to_dev

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU visible to torch", allow_module_level=True)

import vocabulary_cross_entropy_row_amd as lce  # noqa: E402

# (n, V, ld, dtype): odd V for each window size the unaligned families take (1, 2, 4, 8, 12
# and 16 rounds of 1024 vectors), a stride that breaks the alignment of a multiple-of-8 V,
# and the GPT-2 vocabulary; 300 rows put the walk past its static rows
UA_SHAPES = [
    (64, 1001, 1001, "bf16"),
    (300, 9001, 9001, "bf16"),
    (40, 30011, 30011, "bf16"),
    (300, 50257, 50257, "bf16"),
    (24, 90001, 90001, "bf16"),
    (12, 130003, 130003, "bf16"),
    (64, 4096, 4101, "bf16"),
    (64, 1001, 1001, "f32"),
    (80, 30001, 30001, "f32"),
    (16, 50003, 50005, "f32"),
]


@pytest.mark.parametrize("n,V,ld,dt", UA_SHAPES, ids=[f"{s[0]}x{s[1]}ld{s[2]}{s[3]}" for s in UA_SHAPES])
@pytest.mark.parametrize("feat", ["plain", "smooth_sum", "cap_argmax_none", "all"])
def test_unaligned_rows(n, V, ld, dt, feat):
    rng = np.random.default_rng([n, V, ld, len(dt), len(feat), 3])
    x = make_logits(rng, n, V, ld, dt, sigma=4.0 if "cap" in feat or feat == "all" else 2.0)
    if ld > V:
        x[:, V:] = np.uint16(0x7FC1) if dt == "bf16" else np.float32(np.nan)
    y = _labels(rng, n, V, bad=2 if feat == "all" else 0)
    kw = dict(plain=dict(), smooth_sum=dict(eps=0.1, red="sum", grad_out=[0.5]),
              cap_argmax_none=dict(T=5.0, red="none", grad_out=rng.normal(size=n), want_argmax=True),
              all=dict(eps=0.2, T=30.0, red="mean", grad_out=[1.5], want_argmax=True))[feat]
    run_and_check(x, y, V, **kw)


@pytest.mark.parametrize("V,dt", [(50257, "bf16"), (8191, "f32")], ids=["bf16-50257", "f32-8191"])
def test_unaligned_targets_at_window_edges(V, dt):
    """Targets on a row's first and last elements (which share a vector with the row before or
    after), and on round boundaries of the window."""
    E = 8 if dt == "bf16" else 4
    R = 1024 * E
    cand = {0, 1, E - 2, E - 1, E, R - 1, R, R + 1, V - E - 1, V - E, V - 2, V - 1}
    y = np.array(sorted(c for c in cand if 0 <= c < V), dtype=np.int64)
    y = np.concatenate([y, y[::-1]])    # both orders: every target sees several window offsets
    n = len(y)
    rng = np.random.default_rng([V, 53])
    x = make_logits(rng, n, V, V, dt)
    run_and_check(x, y, V, want_argmax=True)
    run_and_check(x, y, V, eps=0.2, T=10.0, red="none", grad_out=rng.normal(size=n))


@pytest.mark.parametrize("c0", [1, 3, 7], ids=["col1", "col3", "col7"])
def test_unaligned_base_view(c0):
    """Logits that start c0 elements into an allocation (a column slice): every row's window
    starts before the row; the columns around the slice are never written."""
    rng = np.random.default_rng([c0, 54])
    n, V, ld = 96, 16384, 16400
    x = make_logits(rng, n, V, ld, "bf16")
    y = _labels(rng, n, V)
    buf = to_dev(x)
    res = lce.lce_ce_fwd_bwd(buf[:, c0:c0 + V], torch.from_numpy(y).to(DEV), label_smoothing=0.1, want_argmax=True)
    torch.cuda.synchronize()
    out = from_dev(buf)
    xs = np.ascontiguousarray(x[:, c0:c0 + V])
    o = oracle.ce(xs, y, V=V, label_smoothing=0.1, want_grad=True)
    check_loss(res.loss_tok.cpu().numpy(), o["loss_tok"], "loss_tok")
    check_loss(float(res.loss_out.cpu()[0]), o["loss_out"], "loss_out")
    assert np.array_equal(res.argmax.cpu().numpy(), o["argmax"])
    allow = smoothing_allowance(row_scales("mean", None, y, V), 0.1, V)
    check_bf16_grad(out[:, c0:c0 + V], o["grad"], oracle.default(), allow=allow)
    keep = np.ones(ld, dtype=bool)
    keep[c0:c0 + V] = False
    assert np.array_equal(out[:, keep].view(np.uint16), x[:, keep].view(np.uint16)), "columns outside the view written"


@pytest.mark.parametrize("want_argmax", [False, True], ids=["plain", "argmax"])
def test_unaligned_ignored_rows_next_to_live_ones(want_argmax):
    """Without the argmax, ignored rows are zeroed at the end of the call, each next to rows
    whose gradient is already written; zeroing an ignored row's window must leave its
    neighbours' elements in the shared vectors alone."""
    rng = np.random.default_rng(55)
    n, V = 1500, 9001
    x = make_logits(rng, n, V, V, "bf16")
    y = rng.integers(0, V, n).astype(np.int64)
    y[400::3] = -100            # every third row past the static ones
    y[1000:1040] = -100         # and a run
    res, out = run_and_check(x, y, V, want_argmax=want_argmax, rows=np.arange(0, n, 7))
    ign = y == -100
    assert np.all(out[ign].view(np.int16) & 0x7FFF == 0)
    # rows next to ignored ones, in full
    live = np.where(~ign & (np.roll(ign, 1) | np.roll(ign, -1)))[0][:60]
    o = oracle.ce(x, y, V=V, rows=live, want_grad=True)
    check_bf16_grad(out[live], o["grad"], oracle.default())


def test_unaligned_f32_large_magnitudes():
    """fp32 rows with logits of magnitude ~1e3 on an odd stride: the exponent is formed
    relative to the exact row max, as on aligned rows."""
    rng = np.random.default_rng(56)
    n, V, ld = 32, 4099, 4103
    x = (rng.standard_normal((n, ld)) * 1000.0).astype(np.float32)
    y = _labels(rng, n, V)
    res, out = run_and_check(x, y, V)
    o = oracle.ce(x, y, V=V, want_grad=True)
    check_f32_grad(out[:, :V], o["grad"], row_scales("mean", None, y, V))
