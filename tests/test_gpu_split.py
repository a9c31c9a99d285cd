"""GPU parity of the split cross-entropy (lce_ce_stats / lce_ce_combine / lce_ce_grad) against the
fp64 oracle, through the C ABI.

One shard is the forward / deferred-backward split; several shards of one matrix on this GPU are
the vocabulary-parallel layout (each shard a column slice; the stats records are what ranks would
exchange).  Tolerances: integers exact; loss, lse and log p_y within 1e-4 max(1, |o|) (the fp32 loss
rule); entropy within 1e-4 max(1, |lse|) -- it is lse - E_p[z], a difference of two fp32 terms of
size |lse|; gradients by the same bf16 2-ulp / fp32 rules as the fused kernel.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import synth
from parity import check_bf16_grad, check_f32_grad, check_loss, row_scales, smoothing_allowance

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU visible to torch", allow_module_level=True)

import vocabulary_cross_entropy_row_amd as lce  # noqa: E402

DEV = torch.device("cuda:0")


def to_dev(x: np.ndarray):
    if x.dtype == np.uint16:
        return torch.from_numpy(x.view(np.int16)).to(DEV).view(torch.bfloat16)
    return torch.from_numpy(x).to(DEV)


def from_dev(t) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def run_split(x: np.ndarray, y: np.ndarray, V: int, widths, *, eps=0.0, T=0.0, red="mean", grad_out=None):
    """stats of every shard, one combine, then the gradient of every shard in place."""
    buf = to_dev(x)
    lab = torch.from_numpy(y.astype(np.int64)).to(DEV)
    offs = np.concatenate([[0], np.cumsum(widths)]).astype(int)
    assert offs[-1] == V
    stats = torch.stack([lce.lce_ce_stats(buf[:, offs[k]:offs[k + 1]], lab, v_offset=int(offs[k]), softcap=T)
                         for k in range(len(widths))]).contiguous()
    rows = lce.lce_ce_combine(stats, lab, V, label_smoothing=eps, reduction=red)
    g = None
    if grad_out is not None:
        g = torch.from_numpy(np.asarray(grad_out, dtype=np.float32).reshape(-1)).to(DEV)
    for k in range(len(widths)):
        lce.lce_ce_grad(buf[:, offs[k]:offs[k + 1]], lab, V, rows, v_offset=int(offs[k]), label_smoothing=eps,
                        softcap=T, reduction=red, grad_out=g)
    torch.cuda.synchronize()
    return rows, buf


def check_split(x, y, V, widths, *, eps=0.0, T=0.0, red="mean", grad_out=None, rows_sel=None):
    n = x.shape[0]
    rows, buf = run_split(x, y, V, widths, eps=eps, T=T, red=red, grad_out=grad_out)
    orc = oracle.default()
    o = orc.ce(x, y, V=V, label_smoothing=eps, softcap=T, reduction=red, grad_out=grad_out, rows=rows_sel)
    st = orc.row_stats(x, y, V=V, softcap=T, rows=rows_sel)
    idx = np.arange(n) if rows_sel is None else np.asarray(rows_sel)
    check_loss(rows.loss_tok.cpu().numpy()[idx], o["loss_tok"], "loss_tok")
    check_loss(rows.lse.cpu().numpy()[idx], st["lse"], "lse")
    check_loss(rows.logprob.cpu().numpy()[idx], st["logp"], "logprob")
    ent = rows.entropy.cpu().numpy()[idx].astype(np.float64)
    lim = 1e-4 * np.maximum(1.0, np.abs(st["lse"]))
    assert np.all(np.abs(ent - st["entropy"]) <= lim), f"entropy off by {np.max(np.abs(ent - st['entropy'])):.3e}"
    assert np.array_equal(rows.argmax.cpu().numpy()[idx], o["argmax"]), "argmax differs"
    nv, nb = orc.count(y, V)
    counts = rows.counts.cpu().numpy()
    assert counts[0] == nv and counts[2] == nb
    if rows_sel is None:
        assert counts[1] == o["counts"][1]
        want = o["loss_out"] if red != "none" else 0.0
        check_loss(float(rows.loss_out.cpu()[0]), want, "loss_out")
    out = from_dev(buf)[idx, :V]
    scales = row_scales(red, grad_out, y, V)[idx]
    if x.dtype == np.uint16:
        n_allow = check_bf16_grad(out, o["grad"], orc, allow=smoothing_allowance(scales, eps, V))
        assert n_allow <= max(4, out.size // 1000)
    else:
        check_f32_grad(out, o["grad"], scales)
    return rows


def _labels(rng, n, V, ignore_frac=0.1, bad=0):
    y = rng.integers(0, V, n).astype(np.int64)
    y[rng.permutation(n)[: int(round(ignore_frac * n))]] = -100
    if bad:
        pos = rng.permutation(n)[:bad]
        y[pos[::2]] = V + 3
        y[pos[1::2]] = -7
    return y


CASES = [  # n, V, dtype, shard widths
    (32, 8488, "bf16", [8488]),
    (32, 8488, "bf16", [2048, 4096, 2344]),
    (16, 32768, "bf16", [4096] * 8),
    (24, 6000, "f32", [2000, 4000]),
    (8, 131072, "bf16", [16384] * 8),
    (40, 1000, "bf16", [8, 992]),
]
FEATS = {
    "plain": dict(),
    "smooth_sum": dict(eps=0.1, red="sum", grad_out=[0.5]),
    "cap_none": dict(T=5.0, red="none"),
    "all": dict(eps=0.2, T=30.0, red="mean", grad_out=[-1.5]),
    "strong_cap": dict(eps=0.1, T=0.5, red="sum", grad_out=[2.0]),   # tanh saturated for most logits
}


@pytest.mark.parametrize("widths", [[4096], [1024, 1024, 2048], [512] * 8], ids=["tp1", "tp3", "tp8"])
def test_split_large_magnitudes(widths):
    """bf16 logits ~N(0, 1000^2) with +1e4 spikes (target on and off them), plain, smoothed and
    softcapped: statistics that underflow across shards, a one-hot softmax, saturated tanh."""
    V = sum(widths)
    rng = np.random.default_rng([V, len(widths), 61])
    n = 10
    x = (rng.standard_normal((n, V)) * 1000.0).astype(np.float32)
    y = rng.integers(0, V, n).astype(np.int64)
    sp = rng.integers(0, V, n)
    for i in range(5, n):
        x[i, sp[i]] = 1.0e4
    y[5:7] = sp[5:7]
    xb = synth.f32_to_bf16_bits(x)
    check_split(xb, y, V, widths)
    check_split(xb, y, V, widths, eps=0.1, red="sum", grad_out=[0.5])
    check_split(xb, y, V, widths, T=30.0)


@pytest.mark.parametrize("n,V,dt,widths", CASES, ids=[f"{c[0]}x{c[1]}{c[2]}_tp{len(c[3])}" for c in CASES])
@pytest.mark.parametrize("feat", list(FEATS))
def test_split_matrix(n, V, dt, widths, feat):
    rng = np.random.default_rng([n, V, len(widths), len(feat)])
    x = (rng.standard_normal((n, V)) * (4.0 if "cap" in feat or feat == "all" else 2.0)).astype(np.float32)
    x = synth.f32_to_bf16_bits(x) if dt == "bf16" else x
    y = _labels(rng, n, V, bad=2 if feat == "all" else 0)
    kw = dict(FEATS[feat])
    if feat == "cap_none":
        kw["grad_out"] = rng.normal(size=n)   # per-token, both signs
    check_split(x, y, V, widths, **kw)


def test_split_argmax_tie_across_shards():
    """Equal maxima in two shards: the smaller global index wins, whichever shard holds it."""
    rng = np.random.default_rng(5)
    n, V = 6, 4096
    x = rng.normal(size=(n, V)).astype(np.float32)
    for i, (a, b) in enumerate([(10, 3000), (2047, 2048), (0, 4095), (1500, 2600), (100, 101), (4000, 2100)]):
        x[i, a] = x[i, b] = 9.0
    xb = synth.f32_to_bf16_bits(x)
    y = rng.integers(0, V, n)
    rows = check_split(xb, y, V, [2048, 2048])
    want = [10, 2047, 0, 1500, 100, 2100]
    assert rows.argmax.cpu().numpy().tolist() == want


def test_split_matches_fused():
    """One shard, deferred backward: the same loss and gradient as the fused in-place call."""
    rng = np.random.default_rng(6)
    n, V = 64, 16384
    x = synth.f32_to_bf16_bits((rng.standard_normal((n, V)) * 3).astype(np.float32))
    y = _labels(rng, n, V)
    rows, buf = run_split(x, y, V, [V], eps=0.1, T=30.0, grad_out=[0.5])
    fbuf = to_dev(x)
    res = lce.lce_ce_fwd_bwd(fbuf, torch.from_numpy(y).to(DEV), label_smoothing=0.1, softcap=30.0,
                             grad_out=torch.tensor([0.5], device=DEV))
    torch.cuda.synchronize()
    assert torch.allclose(rows.loss_tok, res.loss_tok, rtol=1e-5, atol=1e-5)
    diff = (buf.float() - fbuf.float()).abs().max().item()
    assert diff <= 2.0 ** -7 * fbuf.float().abs().max().item(), diff


def test_split_edge_cases():
    rng = np.random.default_rng(8)
    V = 64
    x = synth.f32_to_bf16_bits(rng.normal(size=(5, V)).astype(np.float32))
    check_split(x, np.full(5, -100), V, [32, 32])                  # all ignored: zeros, loss 0
    check_split(x, np.array([0, 63, 31, 32, 5]), V, [32, 32])      # targets at shard edges
    check_split(x[:1], np.array([7]), V, [8] * 8)                   # one row, eight shards
    # n = 0
    z = torch.zeros((0, V), dtype=torch.bfloat16, device=DEV)
    lab = torch.zeros(0, dtype=torch.int64, device=DEV)
    st = lce.lce_ce_stats(z, lab)
    rows = lce.lce_ce_combine(st, lab, V)
    lce.lce_ce_grad(z, lab, V, rows)
    torch.cuda.synchronize()
    assert rows.counts.cpu().tolist() == [0, 0, 0] and float(rows.loss_out.cpu()[0]) == 0.0


@pytest.mark.parametrize("n,widths", [(1025, [32, 32]), (3000, [24, 40, 64]), (2048, [16] * 8),
                                        (4099, [8] * 16), (16385, [64]), (20000, [32, 32])])
def test_split_combine_many_rows(n, widths):
    """More rows than one workgroup covers in a pass (the combine then spreads over many workgroups
    and the last one folds the counts and the loss): every output against the oracle, on the one- and
    many-workgroup forms (the first runs when argmax is not asked for), with counts holding stale and
    arbitrary words before the call, twice in a row, the second call smaller."""
    rng = np.random.default_rng([n, len(widths)])
    V = int(sum(widths))
    offs = np.concatenate([[0], np.cumsum(widths)]).astype(int)
    orc = oracle.default()
    for m, fill in ((n, [-1, -1, -1]), (n - 517, [3, 12345, 9])):
        x = synth.f32_to_bf16_bits((rng.standard_normal((m, V)) * 3).astype(np.float32))
        y = _labels(rng, m, V, bad=6)
        buf, lab = to_dev(x), torch.from_numpy(y).to(DEV)
        stats = torch.stack([lce.lce_ce_stats(buf[:, offs[k]:offs[k + 1]], lab, v_offset=int(offs[k]))
                             for k in range(len(widths))]).contiguous()
        f = lambda: torch.empty(m, dtype=torch.float32, device=DEV)  # noqa: E731
        res = []
        for with_argmax in (True, True, False):
            out = lce.SplitRows(f(), f(), f(), torch.empty(1, dtype=torch.float32, device=DEV), f(), f(),
                                torch.empty(m, dtype=torch.int64, device=DEV) if with_argmax else None,
                                torch.tensor(fill, dtype=torch.int64, device=DEV))
            res.append(lce.lce_ce_combine(stats, lab, V, label_smoothing=0.05, out=out))
        torch.cuda.synchronize()
        o = orc.ce(x, y, V=V, label_smoothing=0.05, want_grad=False)
        st = orc.row_stats(x, y, V=V)
        nv, nb = orc.count(y, V)
        for r in res:
            check_loss(r.loss_tok.cpu().numpy(), o["loss_tok"], "loss_tok")
            check_loss(r.lse.cpu().numpy(), st["lse"], "lse")
            check_loss(r.logprob.cpu().numpy(), st["logp"], "logprob")
            ent = r.entropy.cpu().numpy().astype(np.float64)
            assert np.all(np.abs(ent - st["entropy"]) <= 1e-4 * np.maximum(1.0, np.abs(st["lse"])))
            check_loss(float(r.loss_out.cpu()[0]), o["loss_out"], "loss_out")
            assert r.counts.cpu().tolist() == [nv, int(o["counts"][1]), nb]
        assert np.array_equal(res[0].argmax.cpu().numpy(), o["argmax"]), "argmax differs"
        for name in ("lse", "one_minus_py", "loss_tok", "logprob", "entropy", "argmax", "loss_out"):
            assert torch.equal(getattr(res[0], name), getattr(res[1], name)), f"{name} differs between calls"
        for name in ("lse", "one_minus_py", "loss_tok", "logprob", "entropy"):
            assert torch.equal(getattr(res[0], name), getattr(res[2], name)), f"{name}: forms differ"


def test_split_graph_replay():
    """Eight shards' stats, the many-workgroup combine and the gradients captured in one graph: every
    replay (fresh logits, counts holding other words in between) gives the eager result bit for bit."""
    rng = np.random.default_rng(31)
    n, tp, ws = 2048, 8, 1024
    V = tp * ws
    x = synth.f32_to_bf16_bits((rng.standard_normal((n, V)) * 3).astype(np.float32))
    y = _labels(rng, n, V, bad=4)
    pristine, lab = to_dev(x), torch.from_numpy(y).to(DEV)
    bufs = [torch.empty((n, ws), dtype=torch.bfloat16, device=DEV) for _ in range(tp)]
    stats = torch.empty((tp, n, 8), dtype=torch.float32, device=DEV)
    f = lambda: torch.empty(n, dtype=torch.float32, device=DEV)  # noqa: E731
    rows = lce.SplitRows(f(), f(), f(), torch.empty(1, dtype=torch.float32, device=DEV), f(), f(),
                         torch.empty(n, dtype=torch.int64, device=DEV), torch.empty(3, dtype=torch.int64, device=DEV))
    go = torch.full((1,), 0.5, dtype=torch.float32, device=DEV)

    def reset():
        for k in range(tp):
            bufs[k].copy_(pristine[:, k * ws:(k + 1) * ws])
        rows.counts.fill_(-1)

    def call():
        st = torch.cuda.current_stream()
        for k in range(tp):
            lce.lce_ce_stats(bufs[k], lab, v_offset=k * ws, stats=stats[k], stream=st)
        lce.lce_ce_combine(stats, lab, V, label_smoothing=0.1, out=rows, stream=st)
        for k in range(tp):
            lce.lce_ce_grad(bufs[k], lab, V, rows, v_offset=k * ws, label_smoothing=0.1, grad_out=go, stream=st)

    def snapshot():
        return [from_dev(b) for b in bufs] + [getattr(rows, a).cpu().numpy() for a in
                                              ("lse", "one_minus_py", "loss_tok", "loss_out", "logprob", "entropy",
                                               "argmax", "counts")]

    reset()
    call()
    torch.cuda.synchronize()
    want = snapshot()
    o = oracle.ce(x, y, V=V, label_smoothing=0.1, want_grad=False)
    check_loss(float(want[tp + 3][0]), o["loss_out"], "loss_out")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        reset()
        call()   # warm-up on the side stream before capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for _ in range(3):
        reset()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(want, snapshot()):
            assert np.array_equal(np.asarray(a).view(np.uint8), np.asarray(b).view(np.uint8))


@pytest.mark.slow
@pytest.mark.parametrize("tp", [1, 8])
def test_split_full_size(tp):
    """bf16 [2048, 131072] as 1 and 8 vocabulary shards: sampled rows element by element, the reduced
    loss and counts over every row."""
    w = synth.C2
    y = synth.labels(w)
    x = synth.logits(w, y)
    rng = np.random.default_rng(0)
    sel = np.unique(np.concatenate([rng.choice(w.n, 16, replace=False), np.flatnonzero(y == -100)[:2], [0, w.n - 1]]))
    rows = check_split(x, y, w.V, [w.V // tp] * tp, rows_sel=sel)
    o = oracle.ce(x, y, V=w.V, want_grad=False)
    check_loss(float(rows.loss_out.cpu()[0]), o["loss_out"], "loss_out")
    assert int(rows.counts.cpu()[1]) == int(o["counts"][1])


@pytest.mark.parametrize("red", ["mean", "sum", "none"])
def test_deferred_autograd(red):
    """The autograd form: forward is a read-only sweep, backward writes the gradient in place with the
    upstream gradient it receives; a second backward through the same graph is refused."""
    rng = np.random.default_rng([9, len(red)])
    n, V, eps, T = 48, 8192, 0.1, 30.0
    xb = synth.f32_to_bf16_bits((rng.standard_normal((n, V)) * 4).astype(np.float32))
    y = _labels(rng, n, V)
    x = to_dev(xb).clone().requires_grad_()
    lab = torch.from_numpy(y).to(DEV)
    loss, logp, ent, am, counts = lce.cross_entropy(x, lab, label_smoothing=eps, softcap=T, reduction=red)
    before = from_dev(x.detach())
    assert np.array_equal(before, xb), "the forward must not write the logits"
    if red == "none":
        w = rng.normal(size=n)
        (loss * torch.from_numpy(w).to(DEV, torch.float32)).sum().backward(retain_graph=True)
        grad_out = w
    else:
        (loss * 0.5).backward(retain_graph=True)
        grad_out = [0.5]
    assert x.grad is not None and x.grad.dtype == torch.bfloat16
    orc = oracle.default()
    o = orc.ce(xb, y, V=V, label_smoothing=eps, softcap=T, reduction=red, grad_out=grad_out)
    got = loss.detach().cpu().numpy()
    check_loss(got if red == "none" else float(got), o["loss_tok"] if red == "none" else o["loss_out"], "loss")
    st = orc.row_stats(xb, y, V=V, softcap=T)
    check_loss(logp.cpu().numpy(), st["logp"], "logprob")
    assert np.array_equal(am.cpu().numpy(), o["argmax"])
    scales = row_scales(red, grad_out, y, V)
    n_allow = check_bf16_grad(from_dev(x.grad), o["grad"], orc, allow=smoothing_allowance(scales, eps, V))
    assert n_allow <= max(4, n * V // 1000)
    with pytest.raises(RuntimeError, match="second time"):
        (loss.sum() if red == "none" else loss).backward()
