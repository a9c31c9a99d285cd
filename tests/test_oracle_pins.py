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
