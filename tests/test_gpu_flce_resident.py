"""GPU parity of the tile-resident fused linear cross-entropy (lce_flce_forward / lce_flce_backward)
against the fp64 oracle, through the C ABI.

The logits are fp32 sums of exact bf16 products, never rounded to bf16.  Their accumulation error is
far below the loss tolerance at the workloads' magnitudes, so the per-token loss, log-sum-exp,
log p_y and entropy, and the reduced loss, are held to 1e-4 max(1, |value|) of the oracle on the
exact logits.  The argmax is a decision taken on these logits: each logit differs from the exact one
by at most delta_i = H 2^-24 max_j sum_k |h_ik w_jk| (the summation bound for H terms in any order),
so the argmax must equal the oracle's where the oracle's top-2 gap exceeds 2 delta_i, and elsewhere
be a column whose exact logit is within 2 delta_i of the maximum; n_correct must count the kernel's
own argmax.  One stress test (logits of magnitude ~1e3 to 3e4, where the fp32 accumulation error
itself exceeds 1e-4 of a near-zero loss) is held to that summation bound instead: 2 delta_i for
loss, LSE and log p_y, 4 delta_i for entropy.  Gradients: relative L2 <= 1e-2.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import synth
from parity import bits_to_f64

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU visible to torch", allow_module_level=True)

import vocabulary_cross_entropy_row_amd as lce  # noqa: E402

DEV = torch.device("cuda:0")
REL_L2 = 1e-2


def bf16_tensor(bits: np.ndarray):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(DEV).view(torch.bfloat16)


def rel_l2(a: np.ndarray, b: np.ndarray) -> float:
    nb = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / nb) if nb > 0 else float(np.linalg.norm(a))


def logit_bound(hb, wb) -> np.ndarray:
    H = hb.shape[1]
    return H * 2.0 ** -24 * (np.abs(bits_to_f64(hb)) @ np.abs(bits_to_f64(wb)).T).max(axis=1)


def gen(n, H, V, seed, wsig=0.05, hsig=1.0, ignore=0.05):
    rng = np.random.default_rng(seed)
    hb = synth.f32_to_bf16_bits((rng.standard_normal((n, H)) * hsig).astype(np.float32))
    wb = synth.f32_to_bf16_bits((rng.standard_normal((V, H)) * wsig).astype(np.float32))
    y = rng.integers(0, V, n).astype(np.int64)
    y[rng.permutation(n)[: int(round(ignore * n))]] = -100
    return hb, wb, y


def run_resident(hb, wb, y, *, eps=0.0, T=0.0, red="mean", grad_out=None, chunk=64):
    h, w = bf16_tensor(hb), bf16_tensor(wb)
    lab = torch.from_numpy(y).to(DEV)
    rows = lce.lce_flce_forward(h, w, lab, label_smoothing=eps, softcap=T, reduction=red)
    g = None
    if grad_out is not None:
        g = torch.from_numpy(np.asarray(grad_out, dtype=np.float32).reshape(-1)).to(DEV)
    gh, gw = lce.lce_flce_backward(h, w, lab, rows, label_smoothing=eps, softcap=T, reduction=red, grad_out=g,
                                   chunk_tokens=chunk)
    torch.cuda.synchronize()
    return rows, gh, gw


def check_rows(rows, hb, wb, y, *, eps=0.0, T=0.0, red="mean", summation_bound=False):
    """Forward outputs against the oracle; returns the per-token logit bound delta_i.  With
    summation_bound the real-valued outputs are held to multiples of delta_i instead of
    1e-4 max(1, |value|) (the large-magnitude stress test)."""
    orc = oracle.default()
    V = wb.shape[0]
    ro = oracle.flce_rows(orc, hb, wb, y, softcap=T)
    o = orc.flce(hb, wb, y, label_smoothing=eps, softcap=T, reduction=red, grad_out=None)
    d = logit_bound(hb, wb)
    tol = lambda ref: 1e-4 * np.maximum(1.0, np.abs(ref))  # noqa: E731
    errs = {}
    for name, got_t, ref, mult in (("lse", rows.lse, ro["lse"], 2), ("log p_y", rows.logprob, ro["logp"], 2),
                                   ("entropy", rows.entropy, ro["entropy"], 4),
                                   ("loss_tok", rows.loss_tok, o["loss_tok"], 2)):
        got = got_t.cpu().numpy().astype(np.float64)
        err = np.abs(got - ref)
        lim = mult * d + tol(ro["lse"]) if summation_bound else tol(ref)
        assert np.all(err <= lim), f"{name} beyond its tolerance at {np.flatnonzero(err > lim)[:5]}: {err[err > lim][:5]}"
        errs[name] = float(err.max()) if err.size else 0.0
    am = rows.argmax.cpu().numpy()
    firm = ro["gap"] > 2 * d
    assert np.array_equal(am[firm], ro["argmax"][firm]), "argmax differs where the top-2 gap is clear"
    Z = bits_to_f64(hb) @ bits_to_f64(wb).T
    zk = Z[np.arange(y.size), am]
    assert np.all(zk >= Z.max(axis=1) - 2 * d), "argmax is not within the bound of the maximum"
    valid = (y != -100) & (y >= 0) & (y < V)
    counts = rows.counts.cpu().numpy()
    nv, nb = orc.count(y, V)
    assert counts[0] == nv and counts[2] == nb
    assert counts[1] == int(np.sum(valid & (am == y))), "n_correct does not count the argmax"
    if red != "none":
        got = float(rows.loss_out.cpu()[0])
        if summation_bound:
            lim = (2 * d + tol(o["loss_tok"]))[valid]
            lim = lim.mean() if red == "mean" and valid.any() else lim.sum()
        else:
            lim = 1e-4 * max(1.0, abs(o["loss_out"]))
        assert abs(got - o["loss_out"]) <= lim, f"loss_out {got!r} vs {o['loss_out']!r}"
    print("  max errors: " + ", ".join(f"{k} {v:.2e}" for k, v in errs.items()))
    return d


def check_resident(hb, wb, y, *, eps=0.0, T=0.0, red="mean", grad_out=None, chunk=64, summation_bound=False):
    rows, gh, gw = run_resident(hb, wb, y, eps=eps, T=T, red=red, grad_out=grad_out, chunk=chunk)
    check_rows(rows, hb, wb, y, eps=eps, T=T, red=red, summation_bound=summation_bound)
    o = oracle.flce(hb, wb, y, label_smoothing=eps, softcap=T, reduction=red, grad_out=grad_out)
    e_h = rel_l2(bits_to_f64(gh.view(torch.int16).cpu().numpy().view(np.uint16)), o["grad_hidden"])
    e_w = rel_l2(gw.cpu().numpy().astype(np.float64), o["grad_weight"])
    assert e_h <= REL_L2, f"grad_hidden rel L2 {e_h:.3e}"
    assert e_w <= REL_L2, f"grad_weight rel L2 {e_w:.3e}"
    return rows, gh, gw, e_h, e_w


def test_resident_reduced_workload():
    """The fused-linear workload's recipe at a size the oracle runs in full: H 512, V 8192, 256 tokens,
    softcap 30, 5% ignored; backward in chunks of 64."""
    w = synth.C5_SMALL
    y = synth.labels(w)
    hb = synth.flce_hidden_rows(w, np.arange(w.n))
    wb = synth.flce_weight_rows(w, np.arange(w.V))
    *_, e_h, e_w = check_resident(hb, wb, y, T=w.softcap, chunk=w.chunk)
    print(f"rel L2 dH {e_h:.2e} dW {e_w:.2e}")


SHAPES = [
    # n, H, V, chunk, eps, T, red   -- partial tiles in every dimension, K tails, partial last chunk
    (300, 520, 1000, 64, 0.1, 0.0, "sum"),
    (130, 256, 4096, 130, 0.0, 5.0, "none"),
    (77, 136, 520, 32, 0.0, 30.0, "mean"),
    (1, 64, 512, 1024, 0.0, 0.0, "mean"),
    (512, 1024, 3072, 256, 0.2, 30.0, "mean"),
    (257, 72, 264, 100, 0.05, 0.0, "mean"),
    (200, 264, 2056, 64, 0.1, 0.1, "sum"),     # strong cap: tanh saturated for most logits
]


@pytest.mark.parametrize("n,H,V,chunk,eps,T,red", SHAPES, ids=[f"{s[0]}x{s[1]}x{s[2]}c{s[3]}" for s in SHAPES])
def test_resident_shapes(n, H, V, chunk, eps, T, red):
    hb, wb, y = gen(n, H, V, seed=n * 7 + H + 1)
    g = np.random.default_rng(2).normal(size=n) if red == "none" else [0.75]
    check_resident(hb, wb, y, eps=eps, T=T, red=red, grad_out=g, chunk=chunk)


@pytest.mark.parametrize("eps,red", [(0.0, "mean"), (0.1, "sum")])
def test_resident_large_magnitudes(eps, red):
    """Logits of sigma ~1000 over four 256-column tiles, and rows 0-15 whose target logit is a 3e4 spike
    (one-hot rows, entropy ~0).  Each tile's weights share the rounding of max * log2(e) (about 2^-9 at
    these magnitudes); the target's weight is formed exactly when the records are merged, so the target
    must stay out of both tile sums -- inside the e sum it would move the entropy by |z_y| * 2^-9."""
    n, H, V = 64, 256, 1024
    hb, wb, y = gen(n, H, V, seed=31, wsig=62.5)
    w64 = bits_to_f64(wb)
    for i in range(16):
        if y[i] < 0:
            y[i] = 5 + i
        hb[i] = synth.f32_to_bf16_bits((w64[y[i]] * (3.0e4 / float(w64[y[i]] @ w64[y[i]]))).astype(np.float32))
    check_resident(hb, wb, y, eps=eps, red=red, grad_out=[0.5], chunk=64, summation_bound=True)


def test_resident_argmax_ties_and_accuracy():
    """Duplicate weight rows make exact logit ties: the first index wins; accuracy counts it."""
    hb, wb, y = gen(96, 128, 768, seed=5, wsig=0.2)
    wb[300] = wb[17]
    wb[700] = wb[17]
    wb[511] = wb[256]           # the two column halves of one tile
    hb[:40] = synth.f32_to_bf16_bits((bits_to_f64(wb[17]) * 3.0).astype(np.float32))[None, :]
    hb[40:60] = synth.f32_to_bf16_bits((bits_to_f64(wb[256]) * 3.0).astype(np.float32))[None, :]
    y[:20] = 17
    y[20:30] = 300
    y[40:50] = 256
    rows, *_ = run_resident(hb, wb, y)
    check_rows(rows, hb, wb, y)
    am = rows.argmax.cpu().numpy()
    assert (am[:40] == 17).all() and (am[40:60] == 256).all()


def test_resident_matches_chunked():
    """The same inputs through lce_flce_fwd_bwd (bf16-rounded logits): losses within the bf16 bound,
    gradients close."""
    hb, wb, y = gen(200, 256, 2048, seed=9)
    rows, gh, gw = run_resident(hb, wb, y, eps=0.1, T=30.0)
    res = lce.lce_flce_fwd_bwd(bf16_tensor(hb), bf16_tensor(wb), torch.from_numpy(y).to(DEV), label_smoothing=0.1,
                               softcap=30.0, chunk_tokens=64)
    torch.cuda.synchronize()
    zmax = np.abs(30.0 * np.tanh(bits_to_f64(hb) @ bits_to_f64(wb).T / 30.0)).max(axis=1)
    diff = np.abs(rows.loss_tok.cpu().numpy().astype(np.float64) - res.loss_tok.cpu().numpy())
    assert np.all(diff <= 2 * 2.0 ** -9 * zmax + 1e-4 * (1 + np.abs(res.loss_tok.cpu().numpy())))
    assert rel_l2(gw.cpu().numpy(), res.grad_weight.cpu().numpy()) <= REL_L2
    assert rel_l2(gh.float().cpu().numpy(), res.grad_hidden.float().cpu().numpy()) <= REL_L2
    assert torch.equal(rows.counts[[0, 2]].cpu(), res.counts[[0, 2]].cpu())


def test_resident_edge_cases():
    # every label ignored: zero loss, zero gradients
    hb, wb, y = gen(40, 64, 256, seed=3)
    y[:] = -100
    rows, gh, gw = run_resident(hb, wb, y)
    assert rows.counts.cpu().tolist() == [0, 0, 0] and float(rows.loss_out.cpu()[0]) == 0.0
    assert not gh.float().abs().any() and not gw.abs().any()
    # out-of-range labels are counted and treated as ignored
    hb, wb, y = gen(40, 64, 256, seed=4)
    y[:3] = [256, -5, 1000]
    rows, gh, gw = run_resident(hb, wb, y)
    check_rows(rows, hb, wb, y)
    assert int(rows.counts.cpu()[2]) == 3
    # n = 0: counts zero, grad_weight overwritten with zeros
    w = bf16_tensor(gen(1, 64, 256, seed=6)[1])
    h = torch.zeros((0, 64), dtype=torch.bfloat16, device=DEV)
    lab = torch.zeros(0, dtype=torch.int64, device=DEV)
    rows = lce.lce_flce_forward(h, w, lab)
    gw = torch.full((256, 64), 7.0, device=DEV)
    lce.lce_flce_backward(h, w, lab, rows, grad_weight=gw)
    torch.cuda.synchronize()
    assert rows.counts.cpu().tolist() == [0, 0, 0] and float(rows.loss_out.cpu()[0]) == 0.0
    assert not gw.abs().any()


def test_resident_deterministic():
    hb, wb, y = gen(300, 520, 1000, seed=12)
    a = run_resident(hb, wb, y, T=30.0)
    b = run_resident(hb, wb, y, T=30.0)
    assert torch.equal(a[0].loss_tok, b[0].loss_tok) and torch.equal(a[0].argmax, b[0].argmax)
    assert torch.equal(a[1], b[1]) and torch.equal(a[2], b[2])


@pytest.mark.parametrize("red", ["mean", "none"])
def test_linear_cross_entropy_autograd(red):
    """The autograd form: gradients arrive with the upstream gradient of the caller's graph."""
    hb, wb, y = gen(130, 256, 1000, seed=13)
    h = bf16_tensor(hb).clone().requires_grad_()
    w = bf16_tensor(wb).clone().requires_grad_()
    lab = torch.from_numpy(y).to(DEV)
    loss, logp, ent, am, counts = lce.linear_cross_entropy(h, w, lab, softcap=30.0, reduction=red, chunk_tokens=64)
    if red == "none":
        g = np.random.default_rng(3).normal(size=y.size)
        (loss * torch.from_numpy(g).to(DEV, torch.float32)).sum().backward()
    else:
        g = [0.5]
        (loss * 0.5).backward()
    torch.cuda.synchronize()
    o = oracle.flce(hb, wb, y, softcap=30.0, reduction=red, grad_out=g)
    assert h.grad.dtype == torch.bfloat16 and w.grad.dtype == torch.bfloat16
    assert rel_l2(h.grad.float().cpu().numpy(), o["grad_hidden"]) <= REL_L2
    assert rel_l2(w.grad.float().cpu().numpy(), o["grad_weight"]) <= REL_L2


@pytest.mark.slow
@pytest.mark.timeout(900)
def test_resident_full_size_sampled():
    """The fused-linear workload at full size (hidden 4096 x 6656, weight 202048 x 6656, T = 30) in the
    bench's launch configuration (backward in chunks of 1024, default workspace), against the fp64
    oracle: every token's loss and the mean loss within 1e-4 max(1, |loss|); on sampled tokens, one
    by one, lse, log p_y and entropy within 1e-4 max(1, |value|), argmax (gap-aware) and grad_hidden
    rows; sampled grad_weight rows (the sampled tokens' labels included); over every token, counts
    and n_correct from the kernel's own argmax."""
    w = synth.C5
    y = synth.labels(w)
    hb = synth.flce_hidden_rows(w, np.arange(w.n))
    wb = synth.flce_weight_rows(w, np.arange(w.V))
    print(f"\n  inputs ready: hidden {hb.shape}, weight {wb.shape}", flush=True)
    rows, gh, gw = run_resident(hb, wb, y, T=w.softcap, chunk=w.chunk)
    orc = oracle.default()
    nv, nb = orc.count(y, w.V)
    rng = np.random.default_rng(98)
    tok = np.unique(np.concatenate([rng.choice(w.n, 30, replace=False), np.flatnonzero(y == -100)[:2],
                                    [0, w.n - 1]]))
    voc = np.unique(np.concatenate([rng.choice(w.V, 64, replace=False), y[tok][y[tok] >= 0]]))
    ro = oracle.flce_rows(orc, hb, wb, y, tokens=tok, softcap=w.softcap, block=64)
    o = oracle.flce_sampled(orc, hb, wb, y, tok, voc, softcap=w.softcap)
    print("  oracle done", flush=True)
    lt = rows.loss_tok.cpu().numpy().astype(np.float64)
    err = np.abs(lt - o["loss_tok"])
    assert np.all(err <= 1e-4 * np.maximum(1.0, np.abs(o["loss_tok"]))), f"loss_tok beyond 1e-4: {err.max():.3e}"
    got = float(rows.loss_out.cpu()[0])
    assert abs(got - o["loss_out"]) <= 1e-4 * max(1.0, abs(o["loss_out"])), f"loss_out {got!r} vs {o['loss_out']!r}"
    for name, k in (("lse", "lse"), ("logprob", "logp"), ("entropy", "entropy")):
        g = getattr(rows, name).cpu().numpy()[tok].astype(np.float64)
        assert np.all(np.abs(g - ro[k]) <= 1e-4 * np.maximum(1.0, np.abs(ro[k]))), f"{name} beyond 1e-4"
    d = w.H * 2.0 ** -24 * (np.abs(bits_to_f64(hb[tok])) @ np.abs(bits_to_f64(wb)).T).max(axis=1)
    am = rows.argmax.cpu().numpy()
    firm = ro["gap"] > 2 * d
    assert np.array_equal(am[tok][firm], ro["argmax"][firm])
    counts = rows.counts.cpu().numpy()
    valid = (y != -100) & (y >= 0) & (y < w.V)
    assert counts[0] == nv and counts[2] == nb and counts[1] == int(np.sum(valid & (am == y)))
    e_h = rel_l2(bits_to_f64(gh[torch.from_numpy(tok).to(DEV)].view(torch.int16).cpu().numpy().view(np.uint16)),
                 o["grad_hidden"])
    e_w = rel_l2(gw[torch.from_numpy(voc).to(DEV)].cpu().numpy().astype(np.float64), o["grad_weight"])
    print(f"  loss_tok max err {err.max():.2e}, loss_out err {abs(got - o['loss_out']):.2e}, "
          f"rel L2 dH {e_h:.2e} dW {e_w:.2e} (oracle)", flush=True)
    assert e_h <= REL_L2 and e_w <= REL_L2
