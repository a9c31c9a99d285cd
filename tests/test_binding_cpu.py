"""The Python binding's argument checks, on the CPU: tensors reach the library as raw device pointers,
so host tensors, wrong dtypes, non-contiguous or short buffers and ill-sized upstream gradients must be
refused in Python before any library call."""
import pytest

torch = pytest.importorskip("torch")

import vocabulary_cross_entropy_row_amd as lce  # noqa: E402

CPU = torch.device("cpu")


def test_host_tensors_are_refused_before_any_call():
    x = torch.zeros((4, 16), dtype=torch.bfloat16)
    y = torch.zeros(4, dtype=torch.int64)
    h = torch.zeros((4, 8), dtype=torch.bfloat16)
    w = torch.zeros((16, 8), dtype=torch.bfloat16)
    for call in (lambda: lce.lce_ce_fwd_bwd(x, y), lambda: lce.lce_ce_argmax(x, y),
                 lambda: lce.lce_ce_stats(x, y), lambda: lce.lce_ce_combine(torch.zeros((1, 4, 8)), y, 16),
                 lambda: lce.lce_flce_fwd_bwd(h, w, y), lambda: lce.lce_flce_forward(h, w, y),
                 lambda: lce.cross_entropy(x, y), lambda: lce.linear_cross_entropy(h, w, y)):
        with pytest.raises(ValueError, match="GPU tensor"):
            call()


def test_flce_operands():
    h = torch.zeros((4, 8), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="bfloat16"):
        lce.lce_flce_forward(h.float(), torch.zeros((16, 8), dtype=torch.bfloat16), torch.zeros(4, dtype=torch.int64))
    with pytest.raises(ValueError, match="contiguous 2-D"):
        lce.lce_flce_forward(h.t(), torch.zeros((16, 8), dtype=torch.bfloat16), torch.zeros(4, dtype=torch.int64))


@pytest.mark.parametrize("t,dtype,numel,needle", [
    (torch.zeros(4, dtype=torch.int32), torch.int64, 4, "must be torch.int64"),
    (torch.zeros(3, dtype=torch.int64), torch.int64, 4, "at least 4"),
    (torch.zeros((4, 2), dtype=torch.int64)[:, 0], torch.int64, 4, "contiguous"),
    ([0, 1, 2, 3], torch.int64, 4, "torch tensor"),
])
def test_buffer_checks(t, dtype, numel, needle):
    with pytest.raises((ValueError, TypeError), match=needle):
        lce._buf(t, "labels", dtype, numel, CPU, required=True)


def test_buffer_checks_pass_and_optional():
    lce._buf(torch.zeros(5, dtype=torch.int64), "labels", torch.int64, 4, CPU, required=True)
    lce._buf(None, "argmax_out", torch.int64, 4, CPU)
    with pytest.raises(ValueError, match="required"):
        lce._buf(None, "labels", torch.int64, 4, CPU, required=True)


def test_upstream_gradient_forms():
    g = lce._grad_out(0.5, "mean", 7, CPU)
    assert g.dtype == torch.float32 and g.tolist() == [0.5]
    g = lce._grad_out(2.0, "none", 3, CPU)           # a number is broadcast to one value per token
    assert g.tolist() == [2.0, 2.0, 2.0]
    g = lce._grad_out(torch.arange(6, dtype=torch.float64).reshape(2, 3)[:, ::2], "none", 4, CPU)
    assert g.is_contiguous() and g.dtype == torch.float32 and g.tolist() == [0.0, 2.0, 3.0, 5.0]
    with pytest.raises(ValueError, match="needs 5"):
        lce._grad_out(torch.ones(4), "none", 5, CPU)
    assert lce._grad_out(None, "mean", 3, CPU) is None
