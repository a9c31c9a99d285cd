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
    assert lce.lib().lce_abi_version() == lce.ABI_VERSION == 3
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


def call_flce(**over):
    wsb_default = lce.lce_flce_workspace_bytes(64, 64, 512, 32)
    args = dict(hidden=FAKE, weight=FAKE, labels=FAKE, n=64, H=64, V=512, ignore_index=-100, eps=0.0, softcap=0.0,
                red=lce.LCE_RED_MEAN, grad_out=None, chunk=32, loss_tok=FAKE, loss_out=None, grad_hidden=FAKE,
                grad_weight=FAKE, counts=FAKE, ws=ALIGNED_WS, wsb=wsb_default, stream=None, aux=None)
    args.update(over)
    a = args
    st = lce.lib().lce_flce_fwd_bwd(a["hidden"], a["weight"], a["labels"], a["n"], a["H"], a["V"], a["ignore_index"],
                                    a["eps"], a["softcap"], a["red"], a["grad_out"], a["chunk"], a["loss_tok"],
                                    a["loss_out"], a["grad_hidden"], a["grad_weight"], a["counts"], a["ws"], a["wsb"],
                                    a["stream"], a["aux"])
    return st, lce.lce_last_error()


@pytest.mark.parametrize("over,needle,status", [
    (dict(n=-1), "n must be", lce.LCE_ERR_INVALID_ARG),
    (dict(H=0), "H must be", lce.LCE_ERR_INVALID_ARG),
    (dict(V=0), "V must be", lce.LCE_ERR_INVALID_ARG),
    (dict(chunk=0), "chunk_tokens", lce.LCE_ERR_INVALID_ARG),
    (dict(red=7), "reduction", lce.LCE_ERR_INVALID_ARG),
    (dict(eps=2.0), "label_smoothing", lce.LCE_ERR_INVALID_ARG),
    (dict(softcap=float("nan")), "softcap", lce.LCE_ERR_INVALID_ARG),
    (dict(weight=None), "weight", lce.LCE_ERR_INVALID_ARG),
    (dict(grad_weight=None), "grad_weight", lce.LCE_ERR_INVALID_ARG),
    (dict(hidden=None), "hidden", lce.LCE_ERR_INVALID_ARG),
    (dict(wsb=1024), "minimum", lce.LCE_ERR_INVALID_ARG),
    (dict(ws=ALIGNED_WS + 16), "aligned", lce.LCE_ERR_INVALID_ARG),
    (dict(H=60, wsb=1 << 26), "multiples of 8", lce.LCE_ERR_UNSUPPORTED),
    (dict(V=1004, wsb=1 << 26), "multiples of 8", lce.LCE_ERR_UNSUPPORTED),
    (dict(hidden=FAKE + 8), "aligned", lce.LCE_ERR_UNSUPPORTED),
])
def test_flce_rejects_bad_arguments(over, needle, status):
    st, msg = call_flce(**over)
    assert st == status, msg
    assert needle in msg
    # with a second stream named, the same rejection comes before any HIP call touches it
    st2, msg2 = call_flce(aux=FAKE + 0x100, **over)
    assert (st2, msg2) == (st, msg)


@pytest.mark.parametrize("fn", ["fwd_bwd", "backward"])
def test_flce_weight_in_place_limit(fn):
    """Without room for W^T the grad_hidden GEMM reads the weight in place, which needs
    V * H * 2 < 4 GiB: a one-chunk-group workspace at V = 202048, H = 16384 is refused up front
    (the default workspace, which holds W^T, is not limited by it)."""
    n, H, V, C = 2048, 16384, 202048, 1024
    one = lce.lce_flce_workspace_bytes_grouped(n, H, V, C, 1)
    if fn == "fwd_bwd":
        st, msg = call_flce(n=n, H=H, V=V, chunk=C, wsb=one, aux=FAKE + 0x100)
    else:
        st, msg = call_flce_backward(n=n, H=H, V=V, chunk=C, wsb=one, aux=FAKE + 0x100)
    assert st == lce.LCE_ERR_UNSUPPORTED and "4 GiB" in msg and "W^T" in msg, msg


def test_header_documents_the_second_stream():
    src = open(HEADER).read()
    for fn in ("lce_flce_fwd_bwd", "lce_flce_backward"):
        decl = re.search(fn + r"\(([^;]*)\);", src).group(1)
        assert decl.rstrip().endswith("hipStream_t stream, hipStream_t aux_stream"), fn
    assert "The only\n * state kept between calls is the thread-local error text" in src


def test_flce_workspace_groups():
    """The default workspace holds every chunk's transposed gradient at this size (one grad_weight
    pass) and no W^T; with one-chunk groups less is needed, and any size between is accepted."""
    n, H, V, C = 4096, 6656, 202048, 1024
    full = lce.lce_flce_workspace_bytes(n, H, V, C)
    one = lce.lce_flce_workspace_bytes_grouped(n, H, V, C, 1)
    all_groups = lce.lce_flce_workspace_bytes_grouped(n, H, V, C, 4)
    assert all_groups == lce.lce_flce_workspace_bytes_grouped(n, H, V, C, 9)
    assert full == all_groups
    assert one < lce.lce_flce_workspace_bytes_grouped(n, H, V, C, 2) < all_groups
    # the transposed group buffers: (V + H) x tokens x 2 bytes
    assert all_groups - one == pytest.approx((V + H) * (n - C) * 2, rel=1e-3)
    assert lce.lce_flce_workspace_bytes_grouped(n, H, V, C, 0) == 0
    # one byte short of the one-chunk layout is rejected before any device work
    st, msg = call_flce(n=n, H=H, V=V, chunk=C, wsb=one - 1)
    assert st == lce.LCE_ERR_INVALID_ARG and "minimum" in msg


def call_stats(**over):
    a = dict(logits=FAKE, ld=64, dtype=lce.LCE_BF16, labels=FAKE, n=4, Vs=64, v0=0, ignore_index=-100, softcap=0.0,
             stats=FAKE, stream=None)
    a.update(over)
    st = lce.lib().lce_ce_stats(a["logits"], a["ld"], a["dtype"], a["labels"], a["n"], a["Vs"], a["v0"],
                                a["ignore_index"], a["softcap"], a["stats"], a["stream"])
    return st, lce.lce_last_error()


@pytest.mark.parametrize("over,needle,status", [
    (dict(n=-1), "n must be", lce.LCE_ERR_INVALID_ARG),
    (dict(Vs=0), "shard width", lce.LCE_ERR_INVALID_ARG),
    (dict(v0=-8), "v_offset", lce.LCE_ERR_INVALID_ARG),
    (dict(ld=32), "ld", lce.LCE_ERR_INVALID_ARG),
    (dict(dtype=3), "dtype", lce.LCE_ERR_INVALID_ARG),
    (dict(stats=None), "stats", lce.LCE_ERR_INVALID_ARG),
    (dict(labels=None), "labels", lce.LCE_ERR_INVALID_ARG),
    (dict(softcap=-2.0), "softcap", lce.LCE_ERR_INVALID_ARG),
    (dict(Vs=60, ld=64), "16-byte rows", lce.LCE_ERR_UNSUPPORTED),
    (dict(logits=FAKE + 8), "16-byte rows", lce.LCE_ERR_UNSUPPORTED),
    (dict(v0=2 ** 31 - 8), "31 bits", lce.LCE_ERR_UNSUPPORTED),
])
def test_stats_rejects_bad_arguments(over, needle, status):
    st, msg = call_stats(**over)
    assert st == status, msg
    assert needle in msg


def test_combine_and_grad_reject_bad_arguments():
    L = lce.lib()
    st = L.lce_ce_combine(FAKE, 0, FAKE, 4, 64, -100, 0.0, lce.LCE_RED_MEAN, FAKE, None, FAKE, None, None, None, None,
                          FAKE, None)
    assert st == lce.LCE_ERR_INVALID_ARG and "shards" in lce.lce_last_error()
    st = L.lce_ce_combine(FAKE, 2, FAKE, 4, 64, -100, 0.0, 9, FAKE, None, FAKE, None, None, None, None, FAKE, None)
    assert st == lce.LCE_ERR_INVALID_ARG and "reduction" in lce.lce_last_error()
    st = L.lce_ce_combine(FAKE, 2, FAKE, 4, 64, -100, 0.0, lce.LCE_RED_MEAN, None, None, FAKE, None, None, None, None,
                          FAKE, None)
    assert st == lce.LCE_ERR_INVALID_ARG and "lse" in lce.lce_last_error()
    # the shard must lie inside [0, V)
    st = L.lce_ce_grad(FAKE, 64, lce.LCE_BF16, FAKE, 4, 64, 32, 64, -100, 0.0, 0.0, lce.LCE_RED_MEAN, None, FAKE, FAKE,
                       FAKE, None)
    assert st == lce.LCE_ERR_INVALID_ARG and "inside" in lce.lce_last_error()
    st = L.lce_ce_grad(FAKE, 64, lce.LCE_BF16, FAKE, 4, 64, 0, 64, -100, 0.0, 0.0, lce.LCE_RED_MEAN, None, None, FAKE,
                       FAKE, None)
    assert st == lce.LCE_ERR_INVALID_ARG and "lse" in lce.lce_last_error()
    assert lce.lib().lce_ce_stats_bytes(10) == 320


def call_flce_forward(**over):
    a = dict(hidden=FAKE, weight=FAKE, labels=FAKE, n=4, H=8, V=16, ignore_index=-100, eps=0.0, softcap=0.0,
             red=lce.LCE_RED_MEAN, loss_tok=FAKE, loss_out=None, lse=FAKE, q=FAKE, logp=None, ent=None, argmax=None,
             counts=FAKE, ws=ALIGNED_WS, wsb=1 << 20, stream=None)
    a.update(over)
    st = lce.lib().lce_flce_forward(a["hidden"], a["weight"], a["labels"], a["n"], a["H"], a["V"], a["ignore_index"],
                                    a["eps"], a["softcap"], a["red"], a["loss_tok"], a["loss_out"], a["lse"], a["q"],
                                    a["logp"], a["ent"], a["argmax"], a["counts"], a["ws"], a["wsb"], a["stream"])
    return st, lce.lce_last_error()


def call_flce_backward(**over):
    a = dict(hidden=FAKE, weight=FAKE, labels=FAKE, n=4, H=8, V=16, ignore_index=-100, eps=0.0, softcap=0.0,
             red=lce.LCE_RED_MEAN, grad_out=None, chunk=4, lse=FAKE, q=FAKE, counts=FAKE, gh=FAKE, gw=FAKE,
             ws=ALIGNED_WS, wsb=1 << 30, stream=None, aux=None)
    a.update(over)
    st = lce.lib().lce_flce_backward(a["hidden"], a["weight"], a["labels"], a["n"], a["H"], a["V"],
                                     a["ignore_index"], a["eps"], a["softcap"], a["red"], a["grad_out"], a["chunk"],
                                     a["lse"], a["q"], a["counts"], a["gh"], a["gw"], a["ws"], a["wsb"], a["stream"],
                                     a["aux"])
    return st, lce.lce_last_error()


@pytest.mark.parametrize("over,needle,status", [
    (dict(n=-1), "n must be", lce.LCE_ERR_INVALID_ARG),
    (dict(H=0), "H must be", lce.LCE_ERR_INVALID_ARG),
    (dict(V=0), "V must be", lce.LCE_ERR_INVALID_ARG),
    (dict(red=5), "reduction", lce.LCE_ERR_INVALID_ARG),
    (dict(eps=1.5), "label_smoothing", lce.LCE_ERR_INVALID_ARG),
    (dict(softcap=-1.0), "softcap", lce.LCE_ERR_INVALID_ARG),
    (dict(weight=None), "weight", lce.LCE_ERR_INVALID_ARG),
    (dict(hidden=None), "hidden", lce.LCE_ERR_INVALID_ARG),
    (dict(counts=None), "counts", lce.LCE_ERR_INVALID_ARG),
    (dict(lse=None), "lse", lce.LCE_ERR_INVALID_ARG),
    (dict(wsb=100), "workspace_bytes", lce.LCE_ERR_INVALID_ARG),
    (dict(ws=ALIGNED_WS + 16), "256-byte", lce.LCE_ERR_INVALID_ARG),
    (dict(H=12), "multiples of 8", lce.LCE_ERR_UNSUPPORTED),
    (dict(hidden=FAKE + 8), "16-byte", lce.LCE_ERR_UNSUPPORTED),
])
def test_flce_forward_rejects_bad_arguments(over, needle, status):
    st, msg = call_flce_forward(**over)
    assert st == status and needle in msg and "lce_flce_forward" in msg


@pytest.mark.parametrize("over,needle,status", [
    (dict(n=-1), "n must be", lce.LCE_ERR_INVALID_ARG),
    (dict(chunk=0), "chunk_tokens", lce.LCE_ERR_INVALID_ARG),
    (dict(gw=None), "grad_weight", lce.LCE_ERR_INVALID_ARG),
    (dict(q=None), "one_minus_py", lce.LCE_ERR_INVALID_ARG),
    (dict(wsb=100), "workspace_bytes", lce.LCE_ERR_INVALID_ARG),
    (dict(V=20), "multiples of 8", lce.LCE_ERR_UNSUPPORTED),
    (dict(gh=FAKE + 2), "16-byte", lce.LCE_ERR_UNSUPPORTED),
])
def test_flce_backward_rejects_bad_arguments(over, needle, status):
    st, msg = call_flce_backward(**over)
    assert st == status and needle in msg and "lce_flce_backward" in msg


def test_flce_stats_bytes():
    assert lce.lce_flce_stats_bytes(4096, 202048) == 4096 * 790 * 32
    assert lce.lce_flce_stats_bytes(3, 8) == 3 * 32
    assert lce.lce_flce_stats_bytes(-1, 8) == 0


def test_build_families_match_the_kernel_table():
    """The (register rounds, LDS rounds) families the build instantiates are the ones the launcher picks from."""
    from vocabulary_cross_entropy_row_amd import build
    src = open(os.path.join(ROOT, "vocabulary_cross_entropy_row_amd", "csrc", "ce_kernels.hip")).read()
    line = re.search(r"#define LCE_FAMILIES\(X\)(.*)", src).group(1)
    fams = [tuple(int(v) for v in m) for m in re.findall(r"X\((\d+),\s*(\d+)\)", line)]
    assert fams == [tuple(f) for f in build.FAMILIES]
    assert [a + b for a, b in fams] == sorted(a + b for a, b in fams)
