"""The oracle against its pins (CPU only)."""
import pytest

import oracle
from oracle_pins import PINS


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin):
    pin(oracle.default())


@pytest.mark.parametrize("eps,T,red", [(0.0, 30.0, "mean"), (0.1, 0.0, "sum"), (0.2, 5.0, "mean")])
def test_flce_sampled_matches_the_definition(eps, T, red):
    """The sampled fused-linear oracle (library matmuls around the row routine, for full-size checks)
    against the plain-loop definition on shapes the latter runs in full; several 16-token blocks."""
    import numpy as np
    import synth
    rng = np.random.default_rng(7)
    n, H, V = 70, 24, 56
    hb = synth.f32_to_bf16_bits(rng.standard_normal((n, H)).astype(np.float32))
    wb = synth.f32_to_bf16_bits((rng.standard_normal((V, H)) * 0.3).astype(np.float32))
    y = rng.integers(0, V, n)
    y[rng.permutation(n)[:7]] = -100
    orc = oracle.default()
    full = orc.flce(hb, wb, y, label_smoothing=eps, softcap=T, reduction=red, grad_out=[0.75])
    tok = np.array([0, 5, 16, 33, 69])
    voc = np.array([0, 3, int(y[1]), V - 1])
    smp = oracle.flce_sampled(orc, hb, wb, y, tok, voc, label_smoothing=eps, softcap=T, reduction=red,
                              grad_out=0.75, block=16)
    np.testing.assert_allclose(smp["loss_tok"], full["loss_tok"], rtol=1e-12, atol=1e-12)
    assert abs(smp["loss_out"] - full["loss_out"]) <= 1e-12 * max(1.0, abs(full["loss_out"]))
    assert list(smp["counts"]) == [int(full["counts"][0]), 0, int(full["counts"][2])]
    np.testing.assert_allclose(smp["grad_hidden"], full["grad_hidden"][tok], rtol=1e-10, atol=1e-14)
    np.testing.assert_allclose(smp["grad_weight"], full["grad_weight"][voc], rtol=1e-10, atol=1e-14)


@pytest.mark.parametrize("T", [0.0, 4.0])
def test_flce_rows_brute_force(T):
    """The fused-linear row outputs against brute force on a tiny input: logits by explicit loops over
    H, then log-sum-exp, log p_y, entropy, the first argmax, the top-2 gap and the plain loss, each
    written from its definition; the loss also against the plain-loop fused definition."""
    import math

    import numpy as np
    import synth
    rng = np.random.default_rng(11)
    n, H, V = 6, 5, 9
    hb = synth.f32_to_bf16_bits(rng.standard_normal((n, H)).astype(np.float32))
    wb = synth.f32_to_bf16_bits(rng.standard_normal((V, H)).astype(np.float32))
    wb[4] = wb[2]                      # an exact tie: the first index must win
    y = np.array([0, 8, -100, 3, 2, 4])
    h = [[float(synth.bf16_bits_to_f32(np.array([b]))[0]) for b in row] for row in hb]
    w = [[float(synth.bf16_bits_to_f32(np.array([b]))[0]) for b in row] for row in wb]
    got = oracle.flce_rows(oracle.default(), hb, wb, y, softcap=T, block=4)
    for i in range(n):
        x = [sum(h[i][k] * w[j][k] for k in range(H)) for j in range(V)]
        z = [T * math.tanh(v / T) for v in x] if T > 0 else x
        m = max(z)
        lse = m + math.log(sum(math.exp(v - m) for v in z))
        p = [math.exp(v - lse) for v in z]
        am = x.index(max(x))
        second = max(v for j, v in enumerate(x) if j != am)
        assert abs(got["lse"][i] - lse) <= 1e-12 * max(1.0, abs(lse))
        assert abs(got["entropy"][i] + sum(pj * math.log(pj) for pj in p)) <= 1e-12 * max(1.0, abs(lse))
        logp = z[y[i]] - lse if y[i] >= 0 else 0.0
        assert abs(got["logp"][i] - logp) <= 1e-12 * max(1.0, abs(lse))
        assert abs(got["loss_tok"][i] - (-logp)) <= 1e-12 * max(1.0, abs(lse))
        assert got["argmax"][i] == am
        assert abs(got["gap"][i] - (max(x) - second)) <= 1e-12
    full = oracle.default().flce(hb, wb, y, softcap=T, reduction="none")
    np.testing.assert_allclose(got["loss_tok"], full["loss_tok"], rtol=1e-12, atol=1e-12)
    # smoothing and the gradient rows against the plain-loop fused definition (mean over valid labels)
    full = oracle.default().flce(hb, wb, y, label_smoothing=0.1, softcap=T, reduction="mean", grad_out=[0.5])
    nv = int(np.sum(y >= 0))
    got = oracle.flce_rows(oracle.default(), hb, wb, y, tokens=[1, 3, 5], label_smoothing=0.1, softcap=T,
                           grad_scale=0.5 / nv, block=2)
    np.testing.assert_allclose(got["loss_tok"], full["loss_tok"][[1, 3, 5]], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(got["grad_hidden"], full["grad_hidden"][[1, 3, 5]], rtol=1e-10, atol=1e-14)
