"""GPU parity of the half-row kernel (two workgroups per row) against the fp64 oracle.

Rows of 122,888 to 153,600 bf16 columns (61,444 to 76,800 fp32) take this kernel: each half
row is reduced by one workgroup of a pair and the two exchange their halves' statistics
through workspace records.  The cases cover rows drawn past the static ones, halves of
unequal length, targets on either side of the half boundary, every feature combination,
ignored-row runs the leader's draws step over, stale workspace records, and replays.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from test_gpu_ce import DEV, _labels, from_dev, make_logits, run_and_check, to_dev

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU visible to torch", allow_module_level=True)

import vocabulary_cross_entropy_row_amd as lce  # noqa: E402

# (n, V, dtype): 300 rows are more than the 128 pairs' static rows (rows are then drawn); the
# widths span the kernel's range: exact 9-round halves, an odd vector count (the second half
# one vector shorter), the widest (10 full rounds) and narrowest rows, fp32, and fewer rows
# than pairs
HALF_SHAPES = [
    (300, 131072, "bf16"),
    (257, 138232, "bf16"),
    (130, 153600, "bf16"),
    (96, 122888, "bf16"),
    (200, 65536, "f32"),
    (3, 151936, "bf16"),
]


@pytest.mark.parametrize("n,V,dt", HALF_SHAPES, ids=[f"{s[0]}x{s[1]}{s[2]}" for s in HALF_SHAPES])
@pytest.mark.parametrize("feat", ["plain", "smooth_sum", "cap_argmax_none", "all"])
def test_half_rows(n, V, dt, feat):
    rng = np.random.default_rng([n, V, len(dt), len(feat), 7])
    x = make_logits(rng, n, V, V, dt, sigma=4.0 if "cap" in feat or feat == "all" else 2.0)
    y = _labels(rng, n, V, bad=2 if feat == "all" else 0)
    kw = dict(plain=dict(), smooth_sum=dict(eps=0.1, red="sum", grad_out=[0.5]),
              cap_argmax_none=dict(T=5.0, red="none", grad_out=rng.normal(size=n), want_argmax=True),
              all=dict(eps=0.2, T=30.0, red="mean", grad_out=[1.5], want_argmax=True))[feat]
    run_and_check(x, y, V, **kw)


@pytest.mark.parametrize("V,dt", [(131072, "bf16"), (138232, "bf16"), (65536, "f32")],
                         ids=["bf16-131072", "bf16-138232", "f32-65536"])
def test_half_targets_at_the_split(V, dt):
    """Targets on the last element of the first half and the first of the second, on round
    boundaries of either half and on the row's ends: the half holding the target keeps it out
    of its sum and hands its logit to the other."""
    E = 8 if dt == "bf16" else 4
    nvec = V // E
    hv0 = (nvec + 1) // 2
    R = 960 * E
    b = hv0 * E
    cand = {0, 1, E - 1, R - 1, R, b - E, b - 1, b, b + 1, b + E, b + R - 1, b + R, V - E, V - 1}
    y = np.array(sorted(c for c in cand if 0 <= c < V), dtype=np.int64)
    n = len(y)
    rng = np.random.default_rng([V, 52])
    x = make_logits(rng, n, V, V, dt)
    run_and_check(x, y, V, want_argmax=True)
    run_and_check(x, y, V, eps=0.2, T=10.0, red="none", grad_out=rng.normal(size=n))


@pytest.mark.parametrize("pattern", ["long_ignored_runs", "all_ignored", "bad_labels"])
@pytest.mark.parametrize("want_argmax", [False, True], ids=["plain", "argmax"])
def test_half_draws_and_ignored_rows(pattern, want_argmax):
    """1024 rows: the leaders draw most of them.  Without the argmax a draw steps over every
    ignored row (however long the run) and the rows are zeroed at the end of the call; with it
    they are carried through with scale 0.  Sampled rows against the oracle, ignored rows all
    zero, the reduced loss and counts over every row."""
    rng = np.random.default_rng(31)
    n, V = 1024, 131072
    x = make_logits(rng, n, V, V, "bf16")
    y = rng.integers(0, V, n).astype(np.int64)
    if pattern == "all_ignored":
        y[:] = -100
    elif pattern == "long_ignored_runs":
        y[300:] = -100
        y[300::97] = rng.integers(0, V, len(y[300::97]))
    else:
        y[rng.permutation(n)[:40]] = V + 5
        y[rng.permutation(n)[:30]] = -100
    rows = np.unique(np.concatenate([np.arange(0, n, 37), np.arange(n - 5, n), np.arange(250, 262)]))
    res, out = run_and_check(x, y, V, want_argmax=want_argmax, rows=rows)
    ign = (y == -100) | (y < 0) | (y >= V)
    assert np.all(out[ign].view(np.int16) & 0x7FFF == 0)
    assert np.all(res.loss_tok.cpu().numpy()[ign] == 0.0)


@pytest.mark.parametrize("want_argmax", [False, True], ids=["plain", "argmax"])
def test_half_workspace_contents_do_not_matter(want_argmax):
    """The exchange records carry a key of the launch and the step, so a workspace of 0xFF
    bytes, of random bytes, or holding records that match an earlier call on another stream
    gives bitwise the results of a zeroed one; every finished call leaves the counter words at 0."""
    rng = np.random.default_rng(13)
    n, V = 600, 131072
    x = make_logits(rng, n, V, V, "bf16")
    y = _labels(rng, n, V)
    wsb = lce.lce_ce_workspace_bytes(n, V)
    fills = {"zero": torch.zeros(wsb, dtype=torch.uint8, device=DEV),
             "ff": torch.full((wsb,), 0xFF, dtype=torch.uint8, device=DEV),
             "random": torch.from_numpy(rng.integers(0, 256, wsb, dtype=np.uint8)).to(DEV)}
    outs = {}
    for name, ws in fills.items():
        buf = to_dev(x)
        res = lce.lce_ce_fwd_bwd(buf, torch.from_numpy(y).to(DEV), want_argmax=want_argmax, workspace=ws)
        torch.cuda.synchronize()
        outs[name] = [from_dev(buf), res.loss_tok.cpu().numpy(), res.loss_out.cpu().numpy(), res.counts.cpu().numpy()]
        if want_argmax:
            outs[name].append(res.argmax.cpu().numpy())
        assert ws[:256].view(torch.int64)[[0, 8, 16]].cpu().tolist() == [0, 0, 0], name
    # the same workspace reused by calls on two streams, one after the other
    ws = fills["zero"]
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    for s in (s1, s2, s1):
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            buf = to_dev(x)
            res = lce.lce_ce_fwd_bwd(buf, torch.from_numpy(y).to(DEV), want_argmax=want_argmax, workspace=ws)
        s.synchronize()
        o = [from_dev(buf), res.loss_tok.cpu().numpy(), res.loss_out.cpu().numpy(), res.counts.cpu().numpy()]
        if want_argmax:
            o.append(res.argmax.cpu().numpy())
        outs[f"stream{id(s)}"] = o
    for name, o in outs.items():
        for a, b in zip(outs["zero"], o):
            assert np.array_equal(np.asarray(a).view(np.uint8), np.asarray(b).view(np.uint8)), name
    run_and_check(x, y, V, want_argmax=want_argmax, rows=np.arange(0, n, 59))


def test_half_replays_are_bitwise_equal():
    """Which pair takes which row changes from call to call; the outputs do not."""
    rng = np.random.default_rng(17)
    n, V = 2048, 131072
    x = make_logits(rng, n, V, V, "bf16")
    y = _labels(rng, n, V, ignore_frac=0.05)
    ref = None
    for _ in range(4):
        buf = to_dev(x)
        res = lce.lce_ce_fwd_bwd(buf, torch.from_numpy(y).to(DEV), label_smoothing=0.1)
        torch.cuda.synchronize()
        got = [from_dev(buf), res.loss_tok.cpu().numpy(), res.loss_out.cpu().numpy(), res.counts.cpu().numpy()]
        if ref is None:
            ref = got
        else:
            for a, b in zip(ref, got):
                assert np.array_equal(np.asarray(a).view(np.uint8), np.asarray(b).view(np.uint8))
        del buf
    o = oracle.ce(x, y, V=V, label_smoothing=0.1, want_grad=False)
    from parity import check_loss
    check_loss(float(ref[2][0]), o["loss_out"], "loss_out")
