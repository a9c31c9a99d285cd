"""GPU parity: the HIP path through the C ABI against the fp64 oracle, element by element.

Every case is seeded and synthetic.  Small cases compare every output; the full-size
workloads compare sampled rows (the oracle regenerates them) plus the reduced loss over all
rows and properties that hold at any size.
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


def make_logits(rng, n, V, ld, dtype, sigma=2.0):
    x = (rng.standard_normal((n, ld)) * sigma).astype(np.float32)
    return synth.f32_to_bf16_bits(x) if dtype == "bf16" else x


def run_and_check(x: np.ndarray, y: np.ndarray, V: int, *, eps=0.0, T=0.0, red="mean", grad_out=None,
                  want_argmax=False, rows=None, full_loss=True):
    """Run the GPU op on a copy of x ([n, ld]) and compare with the oracle."""
    n, ld = x.shape
    dt = "bf16" if x.dtype == np.uint16 else "f32"
    buf = to_dev(x)
    view = buf[:, :V]
    lab = torch.from_numpy(y.astype(np.int64)).to(DEV)
    g_dev = None
    if grad_out is not None:
        g_dev = torch.from_numpy(np.asarray(grad_out, dtype=np.float32).reshape(-1)).to(DEV)
    res = lce.lce_ce_fwd_bwd(view, lab, label_smoothing=eps, softcap=T, reduction=red, grad_out=g_dev,
                             want_argmax=want_argmax)
    torch.cuda.synchronize()
    out = from_dev(buf)
    loss_tok = res.loss_tok.cpu().numpy()
    loss_out = float(res.loss_out.cpu().numpy()[0])
    counts = res.counts.cpu().numpy()
    amax = res.argmax.cpu().numpy() if want_argmax else None

    orc = oracle.default()
    o = orc.ce(x, y, V=V, label_smoothing=eps, softcap=T, reduction=red, grad_out=grad_out, rows=rows,
               want_grad=True)
    idx = np.arange(n) if rows is None else np.asarray(rows)
    check_loss(loss_tok[idx], o["loss_tok"], "loss_tok")
    nv, nb = orc.count(y, V)
    assert counts[0] == nv and counts[2] == nb, f"counts {counts} vs n_valid={nv} n_bad={nb}"
    if full_loss:
        full = o if rows is None else orc.ce(x, y, V=V, label_smoothing=eps, softcap=T, reduction=red,
                                             grad_out=grad_out, want_grad=False)
        want = full["loss_out"] if red != "none" else 0.0
        check_loss(loss_out, want, "loss_out")
    if want_argmax:
        assert np.array_equal(amax[idx], o["argmax"]), "argmax differs"
        if rows is None:
            assert counts[1] == o["counts"][1], f"n_correct {counts[1]} vs {o['counts'][1]}"
    else:
        assert counts[1] == 0
    g = out[idx, :V]
    if dt == "bf16":
        allow = smoothing_allowance(row_scales(red, grad_out, y, V)[idx], eps, V)
        n_allow = check_bf16_grad(g, o["grad"], orc, allow=allow)
        # the cancellation allowance is for isolated elements with p_j ~ eps/V only
        assert n_allow <= max(4, g.size // 1000), f"{n_allow} of {g.size} entries needed the allowance"
    else:
        check_f32_grad(g, o["grad"], row_scales(red, grad_out, y, V)[idx])
    if ld > V:   # padding columns are never touched
        assert np.array_equal(out[:, V:].view(np.uint8), x[:, V:].view(np.uint8)), "padding modified"
    return res, out


# ----------------------------------------------------------------------------- small matrix

def _labels(rng, n, V, ignore_frac=0.1, bad=0):
    y = rng.integers(0, V, n).astype(np.int64)
    k = int(round(ignore_frac * n))
    y[rng.permutation(n)[:k]] = -100
    if bad:
        pos = rng.permutation(n)[:bad]
        y[pos[::2]] = V + 3
        y[pos[1::2]] = -7
    return y


SHAPES = [  # (n, V, ld, dtype): register path with full / partial last round, K > 16, generic path
    (64, 4096, 4096, "f32"),
    (64, 4096, 4096, "bf16"),
    (32, 8 * 1024 + 8 * 37, 8 * 1024 + 8 * 37, "bf16"),
    (16, 32768, 32768 + 64, "bf16"),
    (8, 131072, 131072, "bf16"),
    (24, 65536, 65536, "bf16"),                                     # half rows of 5 rounds
    (16, 61448, 61448 + 8, "bf16"),                                 # 5 rounds, the last of one vector
    (24, 36000, 36000, "f32"),                                      # f32 half rows of 5 rounds
    (16, 92160, 92160, "bf16"),                                     # half rows of 6 rounds, exactly full
    (12, 100352, 100352 + 8, "bf16"),                               # 7 rounds
    (8, 115200, 115200, "bf16"),                                    # 8 rounds
    (12, 50000, 50000, "f32"),                                      # f32, 7 rounds
    (6, 8 * 1024 * 18 + 8 * 5, 8 * 1024 * 18 + 8 * 5, "bf16"),    # K=19 (template 20)
    (4, 202048, 202048, "bf16"),                                    # K=25 (template 26)
    (16, 4099, 4099, "bf16"),                                       # generic (V odd)
    (16, 4096, 4100, "f32"),                                        # fast: ld multiple of 4
    (16, 4096, 4098, "bf16"),                                       # generic (ld not a multiple of 8)
    (16, 1000, 1000, "f32"),
    (8, 60000, 60000, "f32"),                                       # f32 half rows of 8 rounds
    (6, 80000, 80000, "f32"),                                       # f32 resident row, K=20
    (4, 120000, 120000, "f32"),                                     # f32 too wide -> generic
    (2, 204800, 204800, "bf16"),                                    # widest resident bf16 row (K=25)
    (2, 204808, 204808, "bf16"),                                    # one vector more -> generic
    (2, 102400, 102400, "f32"),                                     # widest resident f32 row
    (2, 102404, 102404, "f32"),                                     # one vector more -> generic
]


@pytest.mark.parametrize("n,V,ld,dt", SHAPES, ids=[f"{s[0]}x{s[1]}ld{s[2]}{s[3]}" for s in SHAPES])
@pytest.mark.parametrize("feat", ["plain", "smooth_sum", "cap_argmax_none", "all"])
def test_small_matrix(n, V, ld, dt, feat):
    rng = np.random.default_rng([n, V, ld, len(feat)])
    x = make_logits(rng, n, V, ld, dt, sigma=4.0 if "cap" in feat or feat == "all" else 2.0)
    if ld > V:
        x[:, V:] = np.uint16(0x7FC1) if dt == "bf16" else np.float32(np.nan)
    y = _labels(rng, n, V, bad=2 if feat == "all" else 0)
    kw = dict(plain=dict(), smooth_sum=dict(eps=0.1, red="sum", grad_out=[0.5]),
              cap_argmax_none=dict(T=5.0, red="none", grad_out=rng.normal(size=n), want_argmax=True),
              all=dict(eps=0.2, T=30.0, red="mean", grad_out=[1.5], want_argmax=True))[feat]
    run_and_check(x, y, V, **kw)


# (n, V, dtype): the short-row kernel's families at their capacity and one vector past it, where the
# next family (or the long-row kernel) takes over; 300 rows leave a partial last row set
SHORT_ROWS = [
    (300, 2048, "bf16"), (300, 4096, "bf16"), (300, 4104, "bf16"), (300, 8192, "bf16"), (300, 8200, "bf16"),
    (300, 16384, "bf16"), (300, 16392, "bf16"), (300, 2048, "f32"), (300, 4096, "f32"), (300, 8192, "f32"),
    (300, 8196, "f32"), (1000, 64, "bf16"), (37, 520, "f32"),
    # four waves of 16 vectors a lane (calls of at most 4096 rows): full, partial, two row sets
    (300, 32768, "bf16"), (300, 24000, "bf16"), (1300, 32768, "bf16"), (300, 16384, "f32"), (300, 12000, "f32"),
]


@pytest.mark.parametrize("n,V,dt", SHORT_ROWS, ids=[f"{s[0]}x{s[1]}{s[2]}" for s in SHORT_ROWS])
@pytest.mark.parametrize("feat", ["plain", "all"])
def test_short_row_families(n, V, dt, feat):
    rng = np.random.default_rng([n, V, len(dt), len(feat)])
    x = make_logits(rng, n, V, V, dt, sigma=4.0)
    y = _labels(rng, n, V, bad=2 if feat == "all" else 0)
    kw = dict(plain=dict(), all=dict(eps=0.2, T=30.0, red="none", grad_out=rng.normal(size=n), want_argmax=True))[feat]
    run_and_check(x, y, V, **kw)


# ----------------------------------------------------------------------------- edge cases

def test_c1_full():
    w = synth.C1
    y = synth.labels(w)
    x = synth.logits(w, y)
    run_and_check(x, y, w.V)


def test_n_zero():
    x = torch.zeros((0, 64), dtype=torch.bfloat16, device=DEV)
    lab = torch.zeros(0, dtype=torch.int64, device=DEV)
    res = lce.lce_ce_fwd_bwd(x, lab)
    torch.cuda.synchronize()
    assert res.counts.cpu().tolist() == [0, 0, 0]
    assert float(res.loss_out.cpu()[0]) == 0.0


def test_single_row_and_v1_v2():
    rng = np.random.default_rng(5)
    for V in (1, 2, 3, 8, 16):
        for dt in ("f32", "bf16"):
            x = make_logits(rng, 1, V, V, dt)
            run_and_check(x, np.array([V - 1]), V, want_argmax=True)
            run_and_check(x, np.array([0]), V, eps=0.3, T=2.0, red="sum")


def test_all_ignored_mean_is_zero():
    rng = np.random.default_rng(6)
    x = make_logits(rng, 8, 4096, 4096, "bf16")
    res, out = run_and_check(x, np.full(8, -100), 4096, want_argmax=True)
    assert np.all(out.view(np.int16) & 0x7FFF == 0)


def test_label_dominated_rows():
    """p_y -> 1: the target gradient -(1 - p_y) s must keep its relative precision."""
    rng = np.random.default_rng(7)
    V = 8192
    x = rng.standard_normal((6, V)).astype(np.float32)
    y = np.array([5, 100, 4000, 8191, 0, 77])
    for i, m in enumerate((20.0, 35.0, 50.0, 60.0, 70.0, 80.0)):
        x[i, y[i]] = m
    for dt in ("f32", "bf16"):
        xx = x if dt == "f32" else synth.f32_to_bf16_bits(x)
        run_and_check(xx, y, V, red="sum")
        run_and_check(xx, y, V, red="sum", eps=0.05)


@pytest.mark.parametrize("n,V,ld,dt", [(24, 4096, 4096, "bf16"), (8, 131072, 131072, "bf16"), (16, 4099, 4099, "bf16"),
                                        (16, 4096, 4096, "f32")], ids=["bf16-4096", "bf16-131072", "generic-4099", "f32-4096"])
@pytest.mark.parametrize("eps,T", [(1.0, 0.0), (0.0, 0.5), (1.0, 1.0), (0.3, 0.25)],
                         ids=["eps1", "cap0.5", "eps1-cap1", "eps0.3-cap0.25"])
def test_full_smoothing_and_strong_cap(n, V, ld, dt, eps, T):
    """eps = 1 (a uniform target: the label only selects the row) and strong softcaps
    (T <= 1, where most logits sit in the flat part of tanh), for every reduction."""
    rng = np.random.default_rng([n, V, int(eps * 10), int(T * 100)])
    x = make_logits(rng, n, V, ld, dt, sigma=3.0)
    y = _labels(rng, n, V)
    for red, go in (("mean", [1.0]), ("sum", [0.5]), ("none", rng.normal(size=n))):
        run_and_check(x, y, V, eps=eps, T=T, red=red, grad_out=go, want_argmax=T > 0)


@pytest.mark.parametrize("dt,V", [("bf16", 131072), ("bf16", 4096), ("f32", 4096)], ids=["bf16-131072", "bf16-4096", "f32-4096"])
def test_large_magnitudes(dt, V):
    """Logits of magnitude ~1e3 (the running max jumps by hundreds, so the rescale factors
    underflow to zero), rows with one +1e4 spike at a random column (a one-hot softmax,
    the target on or off the spike), and a softcap over the same rows (tanh fully saturated)."""
    rng = np.random.default_rng([V, 41])
    n = 12
    x = (rng.standard_normal((n, V)) * 1000.0).astype(np.float32)
    y = rng.integers(0, V, n).astype(np.int64)
    spikes = rng.integers(0, V, n)
    for i in range(6, n):
        x[i, spikes[i]] = 1.0e4
    y[6:9] = spikes[6:9]          # target on the spike: loss ~ 0, gradient ~ 0
    xx = synth.f32_to_bf16_bits(x) if dt == "bf16" else x
    run_and_check(xx, y, V, want_argmax=True)
    run_and_check(xx, y, V, eps=0.1, red="sum", grad_out=[0.5])
    run_and_check(xx, y, V, T=30.0, want_argmax=True)


@pytest.mark.parametrize("n,V", [(20000, 64), (257, 4096), (513, 8192)], ids=["20000x64", "257x4096", "513x8192"])
@pytest.mark.parametrize("feat", ["plain", "argmax_smooth_cap"])
def test_schedule_many_rows_and_edges(n, V, feat):
    """The dynamic row schedule with many short rows (~80 draws per workgroup, hundreds of
    zeroing chunks) and with one or two rows past the grid; 15 % ignored rows."""
    rng = np.random.default_rng([n, V, len(feat)])
    x = make_logits(rng, n, V, V, "bf16")
    y = _labels(rng, n, V, ignore_frac=0.15)
    if feat == "plain":
        run_and_check(x, y, V)
    else:
        run_and_check(x, y, V, eps=0.1, T=20.0, red="sum", grad_out=[0.7], want_argmax=True)


@pytest.mark.parametrize("V,ld", [(30000, 30000), (60000, 60000), (90000, 90000), (110000, 110000),
                                  (155000, 155000), (170000, 170000), (202048, 202048), (60001, 60003),
                                  (110001, 110005)])
def test_softcap_families_many_rows(V, ld):
    """Softcap rows of every resident family (aligned and unaligned), more rows than workgroups: each
    round's load for a workgroup's next row goes out right after the round's gradient store, so every
    row after a workgroup's first is checked element by element."""
    rng = np.random.default_rng([V, ld, 7])
    n = 520
    x = make_logits(rng, n, V, ld, "bf16", sigma=6.0)
    y = _labels(rng, n, V, ignore_frac=0.05)
    run_and_check(x, y, V, eps=0.05, T=30.0, red="mean", want_argmax=True)


@pytest.mark.parametrize("V,dt", [(8 * 1024 * 18 + 8 * 5, "bf16"), (131072, "bf16"), (60000, "f32")],
                         ids=["bf16-147496", "bf16-131072", "f32-60000"])
def test_labels_at_round_boundaries(V, dt):
    """Targets on the first and last element of a row, of a 16-byte vector, of a round of
    1024 vectors (the LDS / register boundary included) and of a partial last round: the
    owner thread and element of the target are computed, not looked up."""
    E = 8 if dt == "bf16" else 4
    R = 1024 * E
    cand = {0, 1, E - 1, E, R - 1, R, 2 * R - 1, 2 * R, 8 * R - 1, 8 * R, 9 * R - 1, 9 * R, V - E, V - 1}
    y = np.array(sorted(c for c in cand if 0 <= c < V), dtype=np.int64)
    n = len(y)
    rng = np.random.default_rng([V, 51])
    x = make_logits(rng, n, V, V, dt)
    run_and_check(x, y, V, want_argmax=True)
    run_and_check(x, y, V, eps=0.2, T=10.0, red="none", grad_out=rng.normal(size=n))


def test_subnormal_gradients_flush_to_zero():
    """Rows where some p_j fall just below the smallest normal number (z_j - LSE ~ -90, so
    p_j ~ 8e-40, a bf16 subnormal in the oracle) next to elements just above it (z_j - LSE ~ -85):
    the former are stored as 0 (flush to zero), the latter within 2 ulps."""
    V = 4096
    x = np.full((4, V), -1000.0, dtype=np.float32)
    x[:, 0] = 0.0
    x[:, 1:9] = -90.0
    x[:, 9:17] = -85.0
    x[:, 17:25] = -87.0
    y = np.array([0, 5, 12, 3000])
    xb = synth.f32_to_bf16_bits(x)
    res, out = run_and_check(xb, y, V, red="sum")
    bits = out.view(np.uint16)
    # (row 1's target, column 5, and row 2's, column 12, sit inside the blocks: left out below)
    assert np.all(bits[[0, 2, 3]][:, 1:9] & 0x7FFF == 0)    # e^-90 < 2^-126: flushed to (+/-)0
    assert np.all(bits[[0, 1, 3]][:, 9:17] & 0x7F80 != 0)   # e^-85 > 2^-126: stored as a normal number
    assert np.all(bits[:, 17:25] & 0x7F80 != 0)              # e^-87 = 1.6e-38, just above 2^-126: stored


def test_uniform_rows_give_log_v():
    V = 131072
    x = np.zeros((4, V), dtype=np.uint16)
    x[1] = synth.f32_to_bf16_bits(np.full(V, 3.0, np.float32))
    y = np.array([0, 5, V - 1, -100])
    res, _ = run_and_check(x, y, V, eps=0.1, want_argmax=True)
    lt = res.loss_tok.cpu().numpy()
    assert np.allclose(lt[:3], np.log(V), rtol=1e-6)


def test_bad_labels_counted():
    rng = np.random.default_rng(8)
    x = make_logits(rng, 32, 2048, 2048, "bf16")
    y = _labels(rng, 32, 2048, bad=6)
    res, _ = run_and_check(x, y, 2048, want_argmax=True)
    assert int(res.counts.cpu()[2]) == 6


def test_argmax_ties_quantised():
    rng = np.random.default_rng(9)
    V = 202048
    x = np.clip(np.rint(rng.normal(0, 10, size=(6, V))), -4, 4).astype(np.float32)
    y = np.argmax(x, axis=1)
    y[1] = 5
    xb = synth.f32_to_bf16_bits(x)
    run_and_check(xb, y, V, T=30.0, want_argmax=True)
    am, counts = lce.lce_ce_argmax(to_dev(xb), torch.from_numpy(y).to(DEV))
    torch.cuda.synchronize()
    want = np.array([np.flatnonzero(r == r.max())[0] for r in x])
    assert np.array_equal(am.cpu().numpy(), want)
    assert counts.cpu().tolist() == [6, 5, 0]


@pytest.mark.parametrize("dt,V,ld", [("bf16", 131072, 131072), ("bf16", 4099, 4101), ("f32", 4096, 4096),
                                     ("f32", 1001, 1003)])
def test_argmax_entry_point(dt, V, ld):
    rng = np.random.default_rng([V, ld])
    x = make_logits(rng, 24, V, ld, dt)
    x[3, :V] = x[3, 0]   # a constant row: index 0
    y = _labels(rng, 24, V, bad=2)
    buf = to_dev(x)
    am, counts = lce.lce_ce_argmax(buf[:, :V], torch.from_numpy(y).to(DEV))
    torch.cuda.synchronize()
    o = oracle.ce(x, y, V=V, want_grad=False)
    assert np.array_equal(am.cpu().numpy(), o["argmax"])
    assert counts.cpu().tolist() == o["counts"].tolist()
    assert np.array_equal(from_dev(buf).view(np.uint8), x.view(np.uint8)), "argmax must not write the logits"


@pytest.mark.parametrize("want_argmax", [True, False], ids=["argmax", "plain"])
@pytest.mark.parametrize("n,V", [(1024, 32768), (8192, 4096), (2048, 16384)], ids=["rows", "short1", "short4"])
def test_deterministic_replay(want_argmax, n, V):
    """Rows go to workgroups dynamically (first come, first served) in the long-row kernel, so which
    workgroup handles a row changes from call to call, and in every kernel the last workgroup to
    finish does the fold; every output must still be bitwise the same.  1024 rows of 32768 keep every
    long-row workgroup drawing rows; 8192 x 4096 and 2048 x 16384 run the short-row kernel (one and
    four waves per row); 10 % ignored rows exercise the skip."""
    rng = np.random.default_rng(10)
    x = make_logits(rng, n, V, V, "bf16")
    y = _labels(rng, n, V)
    ws = torch.zeros(lce.lce_ce_workspace_bytes(n, V), dtype=torch.uint8, device=DEV)
    outs = []
    for _ in range(3):
        buf = to_dev(x)
        res = lce.lce_ce_fwd_bwd(buf, torch.from_numpy(y).to(DEV), want_argmax=want_argmax, workspace=ws)
        torch.cuda.synchronize()
        o = [from_dev(buf), res.loss_tok.cpu().numpy(), res.loss_out.cpu().numpy(), res.counts.cpu().numpy()]
        if want_argmax:
            o.append(res.argmax.cpu().numpy())
        outs.append(o)
    for other in outs[1:]:
        for a, b in zip(outs[0], other):
            assert np.array_equal(np.asarray(a).view(np.uint8), np.asarray(b).view(np.uint8))
    # a finished call leaves its three counter words clear
    assert ws[:256].view(torch.int64)[[0, 8, 16]].cpu().tolist() == [0, 0, 0]
    run_and_check(x, y, V, want_argmax=want_argmax, rows=np.arange(0, n, 97))


# a counter word that another launch left behind: tag 0xFEDCBA98 (no launch of a test process reaches
# that dispatch index) and a count part-way through a schedule
STALE_WORD = (0xFEDCBA98 << 32) | 700


@pytest.mark.parametrize("want_argmax", [False, True], ids=["plain", "argmax"])
@pytest.mark.parametrize("V", [32768, 4096], ids=["long-rows", "short-rows"])
def test_workspace_contents_do_not_matter(want_argmax, V):
    """The workspace's counters carry the tag of the launch that set them, so a workspace full of
    0xFF bytes, of random bytes, or holding the counters of a call that never finished gives
    bitwise the results of a zeroed one (1024 rows: every workgroup of the long-row kernel draws
    rows, and 10 % ignored rows make the zeroing chunks run; at V = 4096 the short-row kernel)."""
    rng = np.random.default_rng(12)
    n = 1024
    x = make_logits(rng, n, V, V, "bf16")
    y = _labels(rng, n, V)
    wsb = lce.lce_ce_workspace_bytes(n, V)
    stale = torch.zeros(wsb, dtype=torch.uint8, device=DEV)
    words = np.zeros(32, dtype=np.uint64)
    words[[0, 8, 16]] = [STALE_WORD - 690, STALE_WORD, STALE_WORD + 5]   # completion, row, zeroing counters
    stale[:256].view(torch.int64).copy_(torch.from_numpy(words.view(np.int64)).to(DEV))
    fills = {"zero": torch.zeros(wsb, dtype=torch.uint8, device=DEV),
             "ff": torch.full((wsb,), 0xFF, dtype=torch.uint8, device=DEV),
             "random": torch.from_numpy(rng.integers(0, 256, wsb, dtype=np.uint8)).to(DEV),
             "stale": stale}
    outs = {}
    for name, ws in fills.items():
        buf = to_dev(x)
        res = lce.lce_ce_fwd_bwd(buf, torch.from_numpy(y).to(DEV), want_argmax=want_argmax, workspace=ws)
        torch.cuda.synchronize()
        outs[name] = [from_dev(buf), res.loss_tok.cpu().numpy(), res.loss_out.cpu().numpy(), res.counts.cpu().numpy()]
        if want_argmax:
            outs[name].append(res.argmax.cpu().numpy())
        assert ws[:256].view(torch.int64)[[0, 8, 16]].cpu().tolist() == [0, 0, 0], name
    for name, o in outs.items():
        for a, b in zip(outs["zero"], o):
            assert np.array_equal(np.asarray(a).view(np.uint8), np.asarray(b).view(np.uint8)), name
    run_and_check(x, y, V, want_argmax=want_argmax, rows=np.arange(0, n, 101))


def test_call_on_another_stream():
    """A call on a stream other than the current one: the binding creates the upstream gradient and
    the workspace with that stream current, so nothing the kernel reads is still pending on the
    current stream (which is kept busy meanwhile); the outputs match the oracle."""
    rng = np.random.default_rng(14)
    n, V = 512, 32768
    x = make_logits(rng, n, V, V, "bf16")
    y = _labels(rng, n, V)
    buf, lab = to_dev(x), torch.from_numpy(y).to(DEV)
    big = torch.randn(4096, 4096, device=DEV)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())   # buf and lab are ready
    for _ in range(8):
        big = big @ big.T / 64.0                 # the current stream stays busy
    res = lce.lce_ce_fwd_bwd(buf, lab, label_smoothing=0.1, grad_out=0.5, reduction="sum", stream=s)
    s.synchronize()
    o = oracle.ce(x, y, V=V, label_smoothing=0.1, reduction="sum", grad_out=[0.5])
    check_loss(res.loss_tok.cpu().numpy(), o["loss_tok"], "loss_tok")
    check_loss(float(res.loss_out.cpu()[0]), o["loss_out"], "loss_out")
    allow = smoothing_allowance(row_scales("sum", [0.5], y, V), 0.1, V)
    check_bf16_grad(from_dev(buf), o["grad"], oracle.default(), allow=allow)
    torch.cuda.synchronize()


def test_graph_replay():
    """The call captured in a HIP graph (torch's stream capture): every replay is a new dispatch
    with its own counter tag, so every replay, with eager work and host syncs in between, gives
    bitwise the eager result.  1024 rows make the replays draw rows dynamically."""
    rng = np.random.default_rng(31)
    n, V = 1024, 32768
    x = make_logits(rng, n, V, V, "bf16")
    y = _labels(rng, n, V)
    pristine = to_dev(x)
    lab = torch.from_numpy(y).to(DEV)
    buf = torch.empty_like(pristine)
    loss_tok = torch.empty(n, dtype=torch.float32, device=DEV)
    loss_out = torch.empty(1, dtype=torch.float32, device=DEV)
    counts = torch.empty(3, dtype=torch.int64, device=DEV)
    go = torch.full((1,), 0.5, dtype=torch.float32, device=DEV)
    ws = torch.zeros(lce.lce_ce_workspace_bytes(n, V), dtype=torch.uint8, device=DEV)

    def call():
        lce.lce_ce_fwd_bwd(buf, lab, label_smoothing=0.1, grad_out=go, loss_tok=loss_tok, loss_out=loss_out,
                           counts=counts, workspace=ws, stream=torch.cuda.current_stream())

    buf.copy_(pristine)
    call()
    torch.cuda.synchronize()
    want = [from_dev(buf), loss_tok.cpu().numpy(), loss_out.cpu().numpy(), counts.cpu().numpy()]

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        buf.copy_(pristine)
        call()   # warm-up on the side stream before capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for _ in range(3):
        buf.copy_(pristine)
        loss_tok.fill_(-1.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [from_dev(buf), loss_tok.cpu().numpy(), loss_out.cpu().numpy(), counts.cpu().numpy()]
        for a, b in zip(want, got):
            assert np.array_equal(np.asarray(a).view(np.uint8), np.asarray(b).view(np.uint8))
    assert ws[:256].view(torch.int64)[[0, 8, 16]].cpu().tolist() == [0, 0, 0]


@pytest.mark.parametrize("pattern", ["long_ignored_runs", "all_ignored"])
@pytest.mark.parametrize("want_argmax", [False, True], ids=["plain", "argmax"])
def test_dynamic_schedule_ignored_runs(pattern, want_argmax):
    """More rows than workgroups, so rows are drawn from the workspace counter.  Long runs of
    ignored rows make one draw step over more ignored rows than its queue holds (those
    rows are then processed with scale 0); every output must still match the oracle."""
    rng = np.random.default_rng(21)
    n, V = 2048, 4096
    x = make_logits(rng, n, V, V, "bf16")
    y = rng.integers(0, V, n).astype(np.int64)
    if pattern == "all_ignored":
        y[:] = -100
    else:
        y[300:] = -100
        y[300::97] = rng.integers(0, V, len(y[300::97]))
    res, out = run_and_check(x, y, V, want_argmax=want_argmax)
    ign = y == -100
    assert np.all(out[ign].view(np.int16) & 0x7FFF == 0)
    assert np.all(res.loss_tok.cpu().numpy()[ign] == 0.0)


@pytest.mark.parametrize("n,V,ld", [(16, 32768, 32768 + 64), (8, 131072, 131072)], ids=["16x32768ld32832", "8x131072"])
def test_repeated_calls_store_the_same_bytes(n, V, ld):
    """Regression: with the round offset of the 16-byte gradient stores in soffset, the
    compiler let the next instruction overwrite a store's data register before the store read
    it, and lanes 12-15 of each 16-lane group stored that value instead (a few calls in ten).
    Repeated calls must store identical bytes, and the first must match the oracle."""
    rng = np.random.default_rng([n, V, 77])
    x = make_logits(rng, n, V, ld, "bf16")
    y = _labels(rng, n, V)
    first = None
    for _ in range(8):
        buf = to_dev(x)
        lce.lce_ce_fwd_bwd(buf[:, :V], torch.from_numpy(y).to(DEV))
        torch.cuda.synchronize()
        out = from_dev(buf)
        if first is None:
            first = out
        assert np.array_equal(out, first), f"{int(np.sum(out != first))} gradient entries differ between calls"
    run_and_check(x, y, V)


# ----------------------------------------------------------------------------- full-size workloads

def _sample_rows(w, y, k=24, seed=0):
    rng = np.random.default_rng(seed)
    ign = np.flatnonzero(y == -100)
    rows = set(rng.choice(w.n, size=k, replace=False).tolist())
    rows.update(ign[:2].tolist())
    rows.update([0, w.n - 1])
    return np.array(sorted(rows))


@pytest.mark.parametrize("w", [synth.C2, synth.C3, synth.C4], ids=lambda w: w.name)
def test_full_size_workload(w):
    """The full workload in the launch configuration the bench times; sampled rows compared
    element by element, the reduced loss over every row, and the accuracy counts exactly."""
    y = synth.labels(w)
    x = synth.logits(w, y)
    rows = _sample_rows(w, y)
    res, out = run_and_check(x, y, w.V, eps=w.label_smoothing, T=w.softcap, red=w.reduction,
                             grad_out=[w.grad_out], want_argmax=w.want_argmax, rows=rows)
    if w.want_argmax:
        o = oracle.ce(x, y, V=w.V, label_smoothing=w.label_smoothing, softcap=w.softcap, want_grad=False)
        assert np.array_equal(res.argmax.cpu().numpy(), o["argmax"])
        assert int(res.counts.cpu()[1]) == int(o["counts"][1])
        # the read-only entry point on the same logits, at the same size
        buf = to_dev(x)
        am, counts = lce.lce_ce_argmax(buf, torch.from_numpy(y).to(DEV))
        torch.cuda.synchronize()
        assert np.array_equal(am.cpu().numpy(), o["argmax"])
        assert counts.cpu().tolist() == o["counts"].tolist()
        del buf
    if w.softcap == 0:
        # property at any size: every valid row's gradient sums to ~0 (no cap)
        g = torch.from_numpy(out.view(np.int16)).view(torch.bfloat16).to(DEV).float()
        rs = g.sum(dim=1).abs().max().item()
        assert rs < 1e-5, rs
