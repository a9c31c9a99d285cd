"""The C-ABI library on the CPU: it loads, exports every symbol include/lce.h declares, and
rejects bad arguments before making any HIP call (so these run without a GPU)."""
import ctypes
import os
import re

import pytest

import vocabulary_cross_entropy_row_amd as lce

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lce.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(lce_[a-z0-9_]+)\s*\(", src)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for want in ("lce_ce_fwd_bwd", "lce_ce_argmax", "lce_ce_workspace_bytes", "lce_last_error"):
        assert want in names


def test_library_exports_every_declared_symbol():
    L = ctypes.CDLL(lce.LIB_PATH)
    missing = [n for n in declared_functions() if not hasattr(L, n)]
    assert not missing, f"liblce.so lacks {missing}"


def test_abi_version_and_workspace():
    assert lce.lib().lce_abi_version() == 1
    assert lce.lce_ce_workspace_bytes(2048, 131072) > 0


# A fake, never-dereferenced device address: validation must reject the call before any use.
FAKE = 0x10000
ALIGNED_WS = 0x20000


def call_fwd_bwd(**over):
    args = dict(logits=FAKE, ld=8, dtype=lce.LCE_BF16, labels=FAKE, n=4, V=8, ignore_index=-100,
                eps=0.0, softcap=0.0, red=lce.LCE_RED_MEAN, grad_out=None, loss_tok=FAKE, loss_out=None,
                argmax=None, counts=FAKE, ws=ALIGNED_WS, wsb=4096, stream=None)
    args.update(over)
    a = args
    st = lce.lib().lce_ce_fwd_bwd(a["logits"], a["ld"], a["dtype"], a["labels"], a["n"], a["V"], a["ignore_index"],
                                  a["eps"], a["softcap"], a["red"], a["grad_out"], a["loss_tok"], a["loss_out"],
                                  a["argmax"], a["counts"], a["ws"], a["wsb"], a["stream"])
    return st, lce.lce_last_error()


@pytest.mark.parametrize("over,needle", [
    (dict(n=-1), "n must be"),
    (dict(V=0), "V must be"),
    (dict(ld=7), "ld"),
    (dict(dtype=7), "dtype"),
    (dict(red=9), "reduction"),
    (dict(eps=-0.1), "label_smoothing"),
    (dict(eps=1.5), "label_smoothing"),
    (dict(eps=float("nan")), "label_smoothing"),
    (dict(softcap=-1.0), "softcap"),
    (dict(softcap=float("nan")), "softcap"),
    (dict(softcap=float("inf")), "softcap"),
    (dict(counts=None), "counts"),
    (dict(ws=None), "workspace"),
    (dict(wsb=8), "workspace_bytes"),
    (dict(ws=ALIGNED_WS + 4), "aligned"),
    (dict(logits=None), "logits"),
    (dict(labels=None), "labels"),
    (dict(loss_tok=None), "loss_tok"),
    (dict(logits=FAKE + 1), "aligned"),
])
def test_fwd_bwd_rejects_bad_arguments(over, needle):
    st, msg = call_fwd_bwd(**over)
    assert st == lce.LCE_ERR_INVALID_ARG
    assert needle in msg


def test_fwd_bwd_unsupported_sizes():
    st, msg = call_fwd_bwd(n=2 ** 31, ld=8, wsb=1 << 20)
    assert st == lce.LCE_ERR_UNSUPPORTED and "n > 2^31-1" in msg


@pytest.mark.parametrize("over,needle", [
    (dict(n=-1), "n must be"),
    (dict(V=0), "V must be"),
    (dict(ld=3), "ld"),
    (dict(dtype=5), "dtype"),
    (dict(counts=None), "counts"),
    (dict(argmax=None), "argmax_out"),
    (dict(logits=None), "logits"),
])
def test_argmax_rejects_bad_arguments(over, needle):
    a = dict(logits=FAKE, ld=8, dtype=lce.LCE_F32, labels=None, n=4, V=8, ignore_index=-100, argmax=FAKE,
             counts=FAKE, stream=None)
    a.update(over)
    st = lce.lib().lce_ce_argmax(a["logits"], a["ld"], a["dtype"], a["labels"], a["n"], a["V"], a["ignore_index"],
                                 a["argmax"], a["counts"], a["stream"])
    assert st == lce.LCE_ERR_INVALID_ARG
    assert needle in lce.lce_last_error()
