"""GPU parity of the fused linear cross-entropy (lce_flce_fwd_bwd) against the fp64 oracle.

The call forms the logits in fp32 with bf16 MFMA and stores them as bf16 for the row kernel, so
its losses are those of the bf16-rounded logits.  The reference for them is the oracle's row
routine on RNE_bf16 of the exact logits (two oracle functions, composed here): per-token and
reduced loss within 1e-4 max(1, |loss|).  Both sides round the same exact value, except where the
fp32 accumulation error carries a logit across a bf16 rounding boundary (for the target logit,
about one token in 10^4); such a token's loss may move by one bf16 step of its target logit, so
at most one token in 200 (at least one) may instead meet the worst-case bound of bf16 logits
against the exact-logit oracle, 2 2^-9 max_j |z_ij| + 1e-4 max(1, |loss|).  At full size the
reduced loss is also held to 1e-4 max(1, |loss|) of the exact-logit oracle (the bf16 rounding of
single logits averages out over ~3.9K tokens).  Gradients: relative L2 <= 1e-2 (grad_hidden,
grad_weight).  Counts: exact.
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


def run_flce(hb, wb, y, *, eps=0.0, T=0.0, red="mean", grad_out=None, chunk=64, group_chunks=None):
    g = None
    if grad_out is not None:
        g = torch.from_numpy(np.asarray(grad_out, dtype=np.float32).reshape(-1)).to(DEV)
    ws = None
    if group_chunks is not None:
        n, H = hb.shape
        ws = torch.zeros(lce.lce_flce_workspace_bytes_grouped(n, H, wb.shape[0], chunk, group_chunks),
                         dtype=torch.uint8, device=DEV)
    res = lce.lce_flce_fwd_bwd(bf16_tensor(hb), bf16_tensor(wb), torch.from_numpy(y).to(DEV), label_smoothing=eps,
                               softcap=T, reduction=red, grad_out=g, chunk_tokens=chunk, workspace=ws)
    torch.cuda.synchronize()
    return res


def bf16_logit_reference(hb, wb, y, *, eps=0.0, T=0.0, red="mean", grad_out=None):
    """The oracle's losses of the bf16-rounded exact logits, and each token's worst-case bound of
    bf16 logits against the exact-logit losses (2 2^-9 max_j |z_ij|)."""
    orc = oracle.default()
    V = wb.shape[0]
    Z = bits_to_f64(hb) @ bits_to_f64(wb).T          # exact: bf16 products, fp64 sums
    ob = orc.ce(orc.round_bf16(Z), y, V=V, label_smoothing=eps, softcap=T, reduction=red, grad_out=grad_out,
                want_grad=False)
    zc = T * np.tanh(Z / T) if T > 0 else Z
    return ob, 2.0 * 2.0 ** -9 * np.abs(zc).max(axis=1)


def check_loss_tok(lt, ob_loss, exact_loss, worst):
    """Per-token loss within 1e-4 max(1, |loss|) of the bf16-logit reference; at most one token in
    200 (at least one) may instead be within the worst-case bf16 bound of the exact-logit loss."""
    lt = np.asarray(lt, dtype=np.float64)
    err = np.abs(lt - ob_loss)
    off = err > 1e-4 * np.maximum(1.0, np.abs(ob_loss))
    assert np.count_nonzero(off) <= max(1, lt.size // 200), \
        f"{np.count_nonzero(off)} tokens beyond 1e-4 max(1, |loss|), first {np.flatnonzero(off)[:5]}: {err[off][:5]}"
    far = off & (np.abs(lt - exact_loss) > worst + 1e-4 * np.maximum(1.0, np.abs(exact_loss)))
    assert not far.any(), f"loss_tok beyond the bf16-logit bound at {np.flatnonzero(far)[:5]}"
    return float(err.max()) if err.size else 0.0, int(np.count_nonzero(off))


def check_flce(hb, wb, y, *, eps=0.0, T=0.0, red="mean", grad_out=None, chunk=64, group_chunks=None):
    res = run_flce(hb, wb, y, eps=eps, T=T, red=red, grad_out=grad_out, chunk=chunk, group_chunks=group_chunks)
    o = oracle.flce(hb, wb, y, label_smoothing=eps, softcap=T, reduction=red, grad_out=grad_out)
    assert res.counts.cpu().tolist() == [int(o["counts"][0]), 0, int(o["counts"][2])]
    ob, worst = bf16_logit_reference(hb, wb, y, eps=eps, T=T, red=red, grad_out=grad_out)
    e_max, n_off = check_loss_tok(res.loss_tok.cpu().numpy(), ob["loss_tok"], o["loss_tok"], worst)
    if red != "none":
        got = float(res.loss_out.cpu()[0])
        assert abs(got - ob["loss_out"]) <= 1e-4 * max(1.0, abs(ob["loss_out"])), \
            f"loss_out {got!r} vs {ob['loss_out']!r}"
    print(f"  loss_tok max err {e_max:.2e} ({n_off} tokens on the worst-case bound)")
    dh = res.grad_hidden.view(torch.int16).cpu().numpy().view(np.uint16)
    e_h = rel_l2(bits_to_f64(dh), o["grad_hidden"])
    e_w = rel_l2(res.grad_weight.cpu().numpy().astype(np.float64), o["grad_weight"])
    assert e_h <= REL_L2, f"grad_hidden rel L2 {e_h:.3e}"
    assert e_w <= REL_L2, f"grad_weight rel L2 {e_w:.3e}"
    return res, o, e_h, e_w


def gen(n, H, V, seed, wsig=0.05, hsig=1.0, ignore=0.05):
    rng = np.random.default_rng(seed)
    hb = synth.f32_to_bf16_bits((rng.standard_normal((n, H)) * hsig).astype(np.float32))
    wb = synth.f32_to_bf16_bits((rng.standard_normal((V, H)) * wsig).astype(np.float32))
    y = rng.integers(0, V, n).astype(np.int64)
    y[rng.permutation(n)[: int(round(ignore * n))]] = -100
    return hb, wb, y


def test_flce_reduced_workload():
    """The fused-linear workload's recipe at a size the oracle runs in full: H 512, V 8192,
    256 tokens in chunks of 64, softcap 30, 5% ignored."""
    w = synth.C5_SMALL
    y = synth.labels(w)
    hb = synth.flce_hidden_rows(w, np.arange(w.n))
    wb = synth.flce_weight_rows(w, np.arange(w.V))
    _, _, e_h, e_w = check_flce(hb, wb, y, T=w.softcap, chunk=w.chunk)
    print(f"rel L2 dH {e_h:.2e} dW {e_w:.2e}")


SHAPES = [
    # n, H, V, chunk, eps, T, red   -- partial GEMM tiles in every dimension, partial last chunk
    (300, 520, 1000, 64, 0.1, 0.0, "sum"),
    (130, 256, 4096, 130, 0.0, 5.0, "none"),
    (77, 136, 520, 32, 0.0, 30.0, "mean"),
    (1, 64, 512, 1024, 0.0, 0.0, "mean"),
    (512, 1024, 3072, 256, 0.2, 30.0, "mean"),
    (200, 264, 2056, 64, 0.1, 0.1, "sum"),     # strong cap: tanh saturated for most logits
]


@pytest.mark.parametrize("n,H,V,chunk,eps,T,red", SHAPES, ids=[f"{s[0]}x{s[1]}x{s[2]}c{s[3]}" for s in SHAPES])
def test_flce_shapes(n, H, V, chunk, eps, T, red):
    hb, wb, y = gen(n, H, V, seed=n * 7 + H)
    g = np.random.default_rng(1).normal(size=n) if red == "none" else [0.75]
    check_flce(hb, wb, y, eps=eps, T=T, red=red, grad_out=g, chunk=chunk)


@pytest.mark.parametrize("group_chunks", [1, 2])
def test_flce_grad_weight_groups(group_chunks):
    """A smaller workspace splits grad_weight into several passes (the later ones accumulate into it);
    the result matches the oracle and the one-pass result."""
    hb, wb, y = gen(300, 520, 1000, seed=21)
    _, o, _, _ = check_flce(hb, wb, y, eps=0.1, T=30.0, chunk=64, group_chunks=group_chunks)
    one_pass = run_flce(hb, wb, y, eps=0.1, T=30.0, chunk=64)
    grouped = run_flce(hb, wb, y, eps=0.1, T=30.0, chunk=64, group_chunks=group_chunks)
    assert rel_l2(grouped.grad_weight.cpu().numpy(), one_pass.grad_weight.cpu().numpy()) < 1e-5
    assert torch.equal(grouped.grad_hidden, one_pass.grad_hidden)


def wt_workspace_bytes(n, H, V, chunk):
    """The default workspace plus room for W^T (2 H V bytes, rounded up to 256)."""
    return lce.lce_flce_workspace_bytes(n, H, V, chunk) + (2 * H * V + 255) // 256 * 256


@pytest.mark.parametrize("n,H,V", [(300, 520, 1000), (130, 136, 4104)])
def test_flce_weight_read_in_place(n, H, V):
    """The default workspace has no room for W^T, so the grad_hidden GEMM reads W in place (k-major
    operand, transposing LDS reads); a workspace with room for W^T reads it K-contiguous instead.  The
    same eight k values reach every lane in the same order, so the results are bitwise equal, and
    match the oracle."""
    hb, wb, y = gen(n, H, V, seed=n + V)
    _, o, _, _ = check_flce(hb, wb, y, eps=0.1, T=30.0, chunk=64)
    in_place = run_flce(hb, wb, y, eps=0.1, T=30.0, chunk=64)
    ws = torch.empty(wt_workspace_bytes(n, H, V, 64), dtype=torch.uint8, device=DEV)
    with_wt = lce.lce_flce_fwd_bwd(bf16_tensor(hb), bf16_tensor(wb), torch.from_numpy(y).to(DEV), label_smoothing=0.1,
                                   softcap=30.0, chunk_tokens=64, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(in_place.grad_hidden, with_wt.grad_hidden)
    assert torch.equal(in_place.grad_weight, with_wt.grad_weight)
    assert torch.equal(in_place.loss_tok, with_wt.loss_tok)


def test_flce_chunk_invariance():
    """The chunk size changes only the order of fp32 accumulation in grad_weight."""
    hb, wb, y = gen(192, 256, 2048, seed=5)
    outs = [run_flce(hb, wb, y, chunk=c) for c in (192, 64, 50)]
    for r in outs[1:]:
        assert np.allclose(r.loss_tok.cpu().numpy(), outs[0].loss_tok.cpu().numpy(), rtol=0, atol=1e-6)
        assert rel_l2(r.grad_weight.cpu().numpy(), outs[0].grad_weight.cpu().numpy()) < 1e-5


def test_flce_all_ignored_and_empty():
    hb, wb, y = gen(40, 64, 256, seed=9)
    res = run_flce(hb, wb, np.full(40, -100, dtype=np.int64))
    assert float(res.loss_out.cpu()[0]) == 0.0
    assert torch.count_nonzero(res.grad_weight).item() == 0
    assert torch.count_nonzero(res.grad_hidden.float()).item() == 0
    # n = 0: grad_weight is still overwritten (with zeros)
    gw = torch.full((256, 64), 7.0, device=DEV)
    lce.lce_flce_fwd_bwd(torch.zeros((0, 64), dtype=torch.bfloat16, device=DEV), bf16_tensor(wb),
                         torch.zeros(0, dtype=torch.int64, device=DEV), grad_weight=gw)
    torch.cuda.synchronize()
    assert torch.count_nonzero(gw).item() == 0


def test_flce_deterministic():
    hb, wb, y = gen(128, 256, 1024, seed=11)
    a = run_flce(hb, wb, y, chunk=48)
    b = run_flce(hb, wb, y, chunk=48)
    assert torch.equal(a.grad_weight, b.grad_weight)
    assert torch.equal(a.grad_hidden, b.grad_hidden)
    assert torch.equal(a.loss_tok, b.loss_tok)


def test_flce_clobbered_workspace():
    """The fused linear call's workspace is caller-clobbered: a workspace full of 0xFF bytes
    (the chunk row kernel's completion and row counters included) gives bitwise the results
    of a zeroed one."""
    hb, wb, y = gen(300, 256, 4096, seed=12)
    n, H = hb.shape
    wsb = lce.lce_flce_workspace_bytes(n, H, wb.shape[0], 64)
    outs = []
    for fill in (0, 0xFF):
        ws = torch.full((wsb,), fill, dtype=torch.uint8, device=DEV)
        res = lce.lce_flce_fwd_bwd(bf16_tensor(hb), bf16_tensor(wb), torch.from_numpy(y).to(DEV), chunk_tokens=64,
                                   workspace=ws)
        torch.cuda.synchronize()
        outs.append(res)
    for name in ("loss_tok", "loss_out", "grad_hidden", "grad_weight", "counts"):
        assert torch.equal(getattr(outs[0], name), getattr(outs[1], name)), name


@pytest.mark.parametrize("group_chunks", [None, 2])
def test_flce_graph_replay(group_chunks):
    """The fused call captured in a HIP graph (torch's stream capture).  Its transposes run on a
    second stream forked from and joined back to the caller's, so the graph holds both; every
    replay, with eager work and host syncs in between, gives bitwise the eager result."""
    hb, wb, y = gen(300, 256, 4096, seed=13)
    n, H = hb.shape
    V = wb.shape[0]
    h, w, lab = bf16_tensor(hb), bf16_tensor(wb), torch.from_numpy(y).to(DEV)
    wsb = (lce.lce_flce_workspace_bytes(n, H, V, 64) if group_chunks is None
           else lce.lce_flce_workspace_bytes_grouped(n, H, V, 64, group_chunks))
    ws = torch.zeros(wsb, dtype=torch.uint8, device=DEV)
    out = dict(loss_tok=torch.empty(n, dtype=torch.float32, device=DEV),
               loss_out=torch.empty(1, dtype=torch.float32, device=DEV),
               grad_hidden=torch.empty((n, H), dtype=torch.bfloat16, device=DEV),
               grad_weight=torch.empty((V, H), dtype=torch.float32, device=DEV),
               counts=torch.empty(3, dtype=torch.int64, device=DEV))
    go = torch.full((1,), 0.5, dtype=torch.float32, device=DEV)

    def call():
        lce.lce_flce_fwd_bwd(h, w, lab, label_smoothing=0.1, softcap=30.0, grad_out=go, chunk_tokens=64,
                             workspace=ws, stream=torch.cuda.current_stream(), **out)

    call()
    torch.cuda.synchronize()
    want = {k: v.clone() for k, v in out.items()}
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call()   # warm-up on another stream before capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for _ in range(3):
        for v in out.values():
            v.fill_(7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k, v in out.items():
            assert torch.equal(v, want[k]), k


def test_flce_two_host_threads():
    """Two host threads call the fused entry point at once, each on its own stream with its own
    workspace and outputs (and the binding's second stream of its own thread).  Every call gives
    bitwise the result of the same call made alone."""
    import threading
    cases = []
    for seed in (21, 22):
        hb, wb, y = gen(200, 256, 2048, seed=seed)
        h, w, lab = bf16_tensor(hb), bf16_tensor(wb), torch.from_numpy(y).to(DEV)
        ws = torch.zeros(lce.lce_flce_workspace_bytes(200, 256, 2048, 64), dtype=torch.uint8, device=DEV)
        alone = lce.lce_flce_fwd_bwd(h, w, lab, softcap=30.0, chunk_tokens=64, workspace=ws)
        torch.cuda.synchronize()
        cases.append((h, w, lab, ws, alone))
    errors = []

    def worker(k):
        try:
            h, w, lab, ws, alone = cases[k]
            st = torch.cuda.Stream()
            with torch.cuda.stream(st):
                for _ in range(4):
                    res = lce.lce_flce_fwd_bwd(h, w, lab, softcap=30.0, chunk_tokens=64, workspace=ws, stream=st)
                    st.synchronize()
                    for name in ("loss_tok", "loss_out", "grad_hidden", "grad_weight", "counts"):
                        if not torch.equal(getattr(res, name), getattr(alone, name)):
                            errors.append(f"thread {k}: {name}")
        except Exception as exc:  # noqa: BLE001
            errors.append(f"thread {k}: {exc!r}")

    threads = [threading.Thread(target=worker, args=(k,)) for k in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads), "a thread did not finish"
    assert not errors, errors


def test_flce_second_stream_choices():
    """The transposes on this thread's second stream (the default), on a stream the caller names,
    or on the caller's stream alone, and the call on a stream other than the current one (which is
    kept busy meanwhile): bitwise the same results."""
    hb, wb, y = gen(300, 256, 4096, seed=17)
    h, w, lab = bf16_tensor(hb), bf16_tensor(wb), torch.from_numpy(y).to(DEV)
    names = ("loss_tok", "loss_out", "grad_hidden", "grad_weight", "counts")
    ref = lce.lce_flce_fwd_bwd(h, w, lab, label_smoothing=0.1, softcap=30.0, chunk_tokens=64)
    torch.cuda.synchronize()
    mine = torch.cuda.Stream()
    for aux in (None, mine):
        res = lce.lce_flce_fwd_bwd(h, w, lab, label_smoothing=0.1, softcap=30.0, chunk_tokens=64, aux_stream=aux)
        torch.cuda.synchronize()
        for k in names:
            assert torch.equal(getattr(res, k), getattr(ref, k)), (aux, k)
    big = torch.randn(4096, 4096, device=DEV)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    for _ in range(8):
        big = big @ big.T / 64.0
    res = lce.lce_flce_fwd_bwd(h, w, lab, label_smoothing=0.1, softcap=30.0, grad_out=1.0, chunk_tokens=64, stream=s)
    s.synchronize()
    for k in names:
        assert torch.equal(getattr(res, k), getattr(ref, k)), ("other stream", k)
    torch.cuda.synchronize()


def test_flce_capture_beside_an_eager_call():
    """One thread captures the fused call into a graph with a second stream it names; before the
    capture ends, another thread makes an eager call naming the same second stream.  That stream
    is then being captured into the first thread's graph, so the eager call runs on its own
    stream alone and stays out of the graph.  The eager result and every replay of the graph are
    bitwise the results of the call made alone."""
    import threading
    hb, wb, y = gen(200, 256, 2048, seed=23)
    n, H = hb.shape
    V = wb.shape[0]
    h, w, lab = bf16_tensor(hb), bf16_tensor(wb), torch.from_numpy(y).to(DEV)
    names = ("loss_tok", "loss_out", "grad_hidden", "grad_weight", "counts")

    def outputs():
        return dict(loss_tok=torch.empty(n, dtype=torch.float32, device=DEV),
                    loss_out=torch.empty(1, dtype=torch.float32, device=DEV),
                    grad_hidden=torch.empty((n, H), dtype=torch.bfloat16, device=DEV),
                    grad_weight=torch.empty((V, H), dtype=torch.float32, device=DEV),
                    counts=torch.empty(3, dtype=torch.int64, device=DEV))

    alone = lce.lce_flce_fwd_bwd(h, w, lab, softcap=30.0, chunk_tokens=64, aux_stream=None)
    torch.cuda.synchronize()
    shared_aux = torch.cuda.Stream()
    cap_out, eager_out = outputs(), outputs()
    cap_ws = torch.empty(lce.lce_flce_workspace_bytes(n, H, V, 64), dtype=torch.uint8, device=DEV)
    eager_ws = torch.empty_like(cap_ws)
    cap_stream, eager_stream = torch.cuda.Stream(), torch.cuda.Stream()
    torch.cuda.synchronize()
    inside, eager_done = threading.Event(), threading.Event()
    errors = []
    graph = torch.cuda.CUDAGraph()

    def capturer():
        try:
            with torch.cuda.stream(cap_stream):
                lce.lce_flce_fwd_bwd(h, w, lab, softcap=30.0, chunk_tokens=64, workspace=cap_ws,
                                     aux_stream=shared_aux, **cap_out)   # warm-up
            cap_stream.synchronize()
            with torch.cuda.graph(graph, stream=cap_stream, capture_error_mode="thread_local"):
                lce.lce_flce_fwd_bwd(h, w, lab, softcap=30.0, chunk_tokens=64, workspace=cap_ws,
                                     aux_stream=shared_aux, **cap_out)
                inside.set()
                if not eager_done.wait(120):
                    errors.append("the eager call did not finish")
        except Exception as exc:  # noqa: BLE001
            errors.append(f"capture: {exc!r}")
            inside.set()

    def eager():
        try:
            if not inside.wait(120):
                errors.append("the capture did not start")
                return
            lce.lce_flce_fwd_bwd(h, w, lab, softcap=30.0, chunk_tokens=64, workspace=eager_ws,
                                 aux_stream=shared_aux, stream=eager_stream, **eager_out)
            eager_stream.synchronize()
        except Exception as exc:  # noqa: BLE001
            errors.append(f"eager: {exc!r}")
        finally:
            eager_done.set()

    threads = [threading.Thread(target=capturer), threading.Thread(target=eager)]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=180)
    assert not any(t.is_alive() for t in threads), "a thread did not finish"
    assert not errors, errors
    for k in names:
        assert torch.equal(eager_out[k], getattr(alone, k)), ("eager", k)
    for _ in range(2):
        for v in cap_out.values():
            v.fill_(7)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for k in names:
            assert torch.equal(cap_out[k], getattr(alone, k)), ("replay", k)


@pytest.mark.slow
@pytest.mark.timeout(900)
def test_flce_full_size_sampled():
    """The fused-linear workload at full size (hidden 4096 x 6656, weight 202048 x 6656, T = 30) in the
    bench's launch configuration (chunks of 1024, default workspace): exact counts, the mean loss within
    1e-4 max(1, |loss|) of the exact-logit oracle, 48 sampled tokens' losses against the oracle on
    their bf16-rounded logits, and sampled grad_hidden rows and grad_weight rows (the sampled tokens'
    labels included) within 1e-2 relative L2, against the fp64 oracle."""
    w = synth.C5
    y = synth.labels(w)
    hb = synth.flce_hidden_rows(w, np.arange(w.n))
    wb = synth.flce_weight_rows(w, np.arange(w.V))
    print(f"\n  inputs ready: hidden {hb.shape}, weight {wb.shape}", flush=True)
    res = run_flce(hb, wb, y, T=w.softcap, chunk=w.chunk)
    rng = np.random.default_rng(99)
    tok = np.sort(rng.choice(w.n, 24, replace=False))
    lab = y[tok][y[tok] >= 0]
    voc = np.unique(np.concatenate([rng.choice(w.V, 40, replace=False), lab]))
    o = oracle.flce_sampled(oracle.default(), hb, wb, y, tok, voc, softcap=w.softcap)
    print("  oracle done", flush=True)
    assert res.counts.cpu().tolist() == [int(o["counts"][0]), 0, int(o["counts"][2])]
    # the reduced loss against the exact logits: the bf16 rounding of single logits averages out
    got = float(res.loss_out.cpu()[0])
    assert abs(got - o["loss_out"]) <= 1e-4 * max(1.0, abs(o["loss_out"])), f"loss_out {got!r} vs {o['loss_out']!r}"
    # sampled tokens' losses against the oracle on their bf16-rounded logits
    sel = np.sort(rng.choice(w.n, 48, replace=False))
    ob, worst = bf16_logit_reference(hb[sel], wb, y[sel], T=w.softcap, red="sum")
    e_max, n_off = check_loss_tok(res.loss_tok.cpu().numpy()[sel], ob["loss_tok"], o["loss_tok"][sel], worst)
    print(f"  loss_out err {abs(got - o['loss_out']):.2e}, sampled loss_tok max err {e_max:.2e} "
          f"({n_off} on the worst-case bound)", flush=True)
    dh = res.grad_hidden[torch.from_numpy(tok).to(DEV)].view(torch.int16).cpu().numpy().view(np.uint16)
    e_h = rel_l2(bits_to_f64(dh), o["grad_hidden"])
    e_w = rel_l2(res.grad_weight[torch.from_numpy(voc).to(DEV)].cpu().numpy().astype(np.float64), o["grad_weight"])
    print(f"  rel L2 dH {e_h:.2e} dW {e_w:.2e}", flush=True)
    assert e_h <= REL_L2 and e_w <= REL_L2
