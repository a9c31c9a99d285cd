"""lce_ce_fwd_bwd_noalloc, the entry point for callers that cannot allocate, through the C ABI: two
calls in a row, the second with a smaller input, each checked against lce_ce_fwd_bwd (with a
workspace of its own) on the same inputs -- bitwise equal outputs, integers included -- and against
the fp64 oracle on sampled rows."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import synth
from parity import check_bf16_grad, check_loss, row_scales, smoothing_allowance

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU visible to torch", allow_module_level=True)

import vocabulary_cross_entropy_row_amd as lce  # noqa: E402

DEV = torch.device("cuda:0")


def _bf16(rng, n, V, sigma):
    return synth.f32_to_bf16_bits((rng.standard_normal((n, V)) * sigma).astype(np.float32))


def _outputs(n, want_argmax):
    return dict(loss_tok=torch.empty(n, dtype=torch.float32, device=DEV),
                loss_out=torch.empty(1, dtype=torch.float32, device=DEV),
                argmax=torch.empty(n, dtype=torch.int64, device=DEV) if want_argmax else None,
                counts=torch.empty(3, dtype=torch.int64, device=DEV))


def _call(entry, x, lab, o, *, eps, T, red, grad_out, ws=None):
    """One call of the named C entry point on a fresh device copy of x; returns the gradient bits."""
    n, V = x.shape
    buf = torch.from_numpy(x.view(np.int16)).to(DEV)
    p = lambda t: None if t is None else t.data_ptr()  # noqa: E731
    st = torch.cuda.current_stream().cuda_stream
    args = [buf.data_ptr(), V, lce.LCE_BF16, lab.data_ptr(), n, V, -100, eps, T, lce.REDUCTIONS[red], p(grad_out),
            p(o["loss_tok"]), p(o["loss_out"]), p(o["argmax"]), p(o["counts"])]
    if entry == "lce_ce_fwd_bwd":
        args += [ws.data_ptr(), ws.numel()]
    status = getattr(lce.lib(), entry)(*args, st)
    assert status == lce.LCE_OK, lce.lce_last_error()
    torch.cuda.synchronize()
    return buf.cpu().numpy().view(np.uint16)


CASES = [
    # n, V, sigma, eps, T, red, argmax -- the second is smaller than the first
    (1024, 32768, 2.0, 0.0, 0.0, "mean", False),
    (300, 8192, 4.0, 0.1, 30.0, "sum", True),
]


def test_noalloc_matches_the_workspace_entry_point():
    rng = np.random.default_rng(2024)
    for n, V, sigma, eps, T, red, want_argmax in CASES:
        x = _bf16(rng, n, V, sigma)
        y = rng.integers(0, V, n).astype(np.int64)
        y[rng.permutation(n)[: n // 10]] = -100
        lab = torch.from_numpy(y).to(DEV)
        g = torch.full((1,), 0.75, dtype=torch.float32, device=DEV)
        ws = torch.empty(lce.lce_ce_workspace_bytes(n, V), dtype=torch.uint8, device=DEV)
        want_o, got_o = _outputs(n, want_argmax), _outputs(n, want_argmax)
        want_g = _call("lce_ce_fwd_bwd", x, lab, want_o, eps=eps, T=T, red=red, grad_out=g, ws=ws)
        got_g = _call("lce_ce_fwd_bwd_noalloc", x, lab, got_o, eps=eps, T=T, red=red, grad_out=g)
        assert np.array_equal(got_g, want_g), f"n={n}: gradients differ"
        for k in ("loss_tok", "loss_out", "argmax", "counts"):
            if want_o[k] is not None:
                assert torch.equal(got_o[k], want_o[k]), f"n={n}: {k} differs"
        # and both against the oracle on sampled rows
        rows = np.unique(np.concatenate([np.arange(0, n, 37), [n - 1]]))
        orc = oracle.default()
        o = orc.ce(x, y, label_smoothing=eps, softcap=T, reduction=red, grad_out=[0.75], rows=rows)
        check_loss(got_o["loss_tok"].cpu().numpy()[rows], o["loss_tok"], "loss_tok")
        full = orc.ce(x, y, label_smoothing=eps, softcap=T, reduction=red, grad_out=[0.75], want_grad=False)
        check_loss(float(got_o["loss_out"].cpu()[0]), full["loss_out"], "loss_out")
        assert got_o["counts"].cpu().tolist()[0::2] == [int(full["counts"][0]), int(full["counts"][2])]
        if want_argmax:
            assert np.array_equal(got_o["argmax"].cpu().numpy(), full["argmax"])
            assert int(got_o["counts"].cpu()[1]) == int(full["counts"][1])
        allow = smoothing_allowance(row_scales(red, [0.75], y, V)[rows], eps, V)
        check_bf16_grad(got_g[rows], o["grad"], orc, allow=allow)


def test_noalloc_rejects_bad_arguments_without_a_device_call():
    st = lce.lib().lce_ce_fwd_bwd_noalloc(0x10000, 8, lce.LCE_BF16, 0x10000, 4, 8, -100, 0.0, 0.0, 7, None, 0x10000,
                                         None, None, 0x10000, None)
    assert st == lce.LCE_ERR_INVALID_ARG and "lce_ce_fwd_bwd_noalloc: unknown reduction" in lce.lce_last_error()
