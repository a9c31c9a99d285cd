"""Python binding of liblce.so, the MI355X vocabulary cross-entropy library.

The functions carry the names of the C entry points in include/lce.h and only
marshal arguments: every step of the computation runs in the HIP kernels of
liblce.so.  PyTorch supplies device memory and streams: every function runs
on ``stream`` (default: the current stream) and allocates its temporaries and
default outputs with that stream current.  There
is no CPU fallback: if the library is missing this module raises on import of
the function table (``lib()``), and every call goes to the GPU.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liblce.so")

LCE_OK, LCE_ERR_INVALID_ARG, LCE_ERR_UNSUPPORTED, LCE_ERR_HIP = 0, 1, 2, 3
LCE_F32, LCE_BF16 = 0, 1
LCE_RED_NONE, LCE_RED_MEAN, LCE_RED_SUM = 0, 1, 2
REDUCTIONS = {"none": LCE_RED_NONE, "mean": LCE_RED_MEAN, "sum": LCE_RED_SUM}
ABI_VERSION = 3

_lib = None


class LCEError(RuntimeError):
    """A nonzero lce_status; the message is lce_last_error()."""

    def __init__(self, status: int, msg: str):
        super().__init__(msg)
        self.status = status


def lib() -> ctypes.CDLL:
    """The loaded liblce.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python -m vocabulary_cross_entropy_row_amd.build` (there is no CPU fallback)")
    L = ctypes.CDLL(LIB_PATH)
    p, i64, f32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_float
    L.lce_abi_version.restype = ctypes.c_int
    L.lce_abi_version.argtypes = []
    L.lce_last_error.restype = ctypes.c_char_p
    L.lce_last_error.argtypes = []
    L.lce_ce_workspace_bytes.restype = ctypes.c_size_t
    L.lce_ce_workspace_bytes.argtypes = [i64, i64]
    L.lce_ce_fwd_bwd.restype = ctypes.c_int
    L.lce_ce_fwd_bwd.argtypes = [p, i64, ctypes.c_int, p, i64, i64, i64, f32, f32, ctypes.c_int, p, p, p, p, p,
                                 p, ctypes.c_size_t, p]
    L.lce_ce_fwd_bwd_noalloc.restype = ctypes.c_int
    L.lce_ce_fwd_bwd_noalloc.argtypes = [p, i64, ctypes.c_int, p, i64, i64, i64, f32, f32, ctypes.c_int, p, p, p, p,
                                         p, p]
    L.lce_ce_argmax.restype = ctypes.c_int
    L.lce_ce_argmax.argtypes = [p, i64, ctypes.c_int, p, i64, i64, i64, p, p, p]
    L.lce_flce_workspace_bytes.restype = ctypes.c_size_t
    L.lce_flce_workspace_bytes.argtypes = [i64, i64, i64, i64]
    L.lce_ce_stats_bytes.restype = ctypes.c_size_t
    L.lce_ce_stats_bytes.argtypes = [i64]
    L.lce_ce_stats.restype = ctypes.c_int
    L.lce_ce_stats.argtypes = [p, i64, ctypes.c_int, p, i64, i64, i64, i64, f32, p, p]
    L.lce_ce_combine.restype = ctypes.c_int
    L.lce_ce_combine.argtypes = [p, i64, p, i64, i64, i64, f32, ctypes.c_int, p, p, p, p, p, p, p, p, p]
    L.lce_ce_grad.restype = ctypes.c_int
    L.lce_ce_grad.argtypes = [p, i64, ctypes.c_int, p, i64, i64, i64, i64, i64, f32, f32, ctypes.c_int, p, p, p, p,
                              p]
    L.lce_flce_workspace_bytes_grouped.restype = ctypes.c_size_t
    L.lce_flce_workspace_bytes_grouped.argtypes = [i64, i64, i64, i64, i64]
    L.lce_flce_fwd_bwd.restype = ctypes.c_int
    L.lce_flce_fwd_bwd.argtypes = [p, p, p, i64, i64, i64, i64, f32, f32, ctypes.c_int, p, i64, p, p, p, p, p, p,
                                   ctypes.c_size_t, p, p]
    L.lce_flce_stats_bytes.restype = ctypes.c_size_t
    L.lce_flce_stats_bytes.argtypes = [i64, i64]
    L.lce_flce_forward.restype = ctypes.c_int
    L.lce_flce_forward.argtypes = [p, p, p, i64, i64, i64, i64, f32, f32, ctypes.c_int, p, p, p, p, p, p, p, p, p,
                                   ctypes.c_size_t, p]
    L.lce_flce_backward.restype = ctypes.c_int
    L.lce_flce_backward.argtypes = [p, p, p, i64, i64, i64, i64, f32, f32, ctypes.c_int, p, i64, p, p, p, p, p, p,
                                    ctypes.c_size_t, p, p]
    if L.lce_abi_version() != ABI_VERSION:
        raise ImportError("liblce.so ABI version mismatch; rebuild it")
    _lib = L
    return L


def lce_last_error() -> str:
    return lib().lce_last_error().decode()


def lce_ce_workspace_bytes(n: int, V: int) -> int:
    return int(lib().lce_ce_workspace_bytes(int(n), int(V)))


def _check(status: int) -> None:
    if status != LCE_OK:
        raise LCEError(status, lce_last_error())


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _torch_stream(stream, device):
    """The stream a call runs on, as a torch stream: ``stream`` (a torch stream or a raw HIP stream
    handle) or the current stream of ``device``.  Each function allocates its temporaries and
    default outputs with this stream current, so they are ordered before the launch and go back to
    the caching allocator against the stream that uses them."""
    import torch
    if stream is None:
        return torch.cuda.current_stream(device)
    if isinstance(stream, torch.cuda.Stream):
        return stream
    return torch.cuda.ExternalStream(int(stream), device=device)


def _on_call_stream(fn):
    """Runs a binding function with its call stream current (see _torch_stream): the function
    receives that stream as ``stream``."""
    import functools

    @functools.wraps(fn)
    def wrapper(*args, stream=None, **kw):
        import torch
        first = args[0] if args else None
        if not (torch.is_tensor(first) and first.device.type == "cuda"):
            return fn(*args, stream=stream, **kw)   # the function's own checks raise
        st = _torch_stream(stream, first.device)
        with torch.cuda.stream(st):
            return fn(*args, stream=st, **kw)
    return wrapper


def _stream(stream) -> int:
    return stream.cuda_stream


_aux_streams = None   # per host thread: device index -> second stream of the fused linear calls


def _aux_stream(aux_stream, device):
    """The fused linear calls' second stream: "auto" gives this host thread's own stream on
    ``device`` (created on first use, default priority), None gives none (one stream), anything
    else is taken as given."""
    import threading
    import torch
    global _aux_streams
    if aux_stream is None:
        return None
    if not (isinstance(aux_stream, str) and aux_stream == "auto"):
        return aux_stream.cuda_stream if hasattr(aux_stream, "cuda_stream") else int(aux_stream)
    if _aux_streams is None:
        _aux_streams = threading.local()
    table = getattr(_aux_streams, "by_device", None)
    if table is None:
        table = _aux_streams.by_device = {}
    idx = device.index if device.index is not None else torch.cuda.current_device()
    if idx not in table:
        table[idx] = torch.cuda.Stream(device=idx)
    return table[idx].cuda_stream


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return LCE_BF16
    if t.dtype == torch.float32:
        return LCE_F32
    raise TypeError(f"logits must be bfloat16 or float32, not {t.dtype}")


# Every tensor reaches the library as a raw device pointer, so its device, dtype, layout and size are
# checked here: a host tensor or a short buffer would otherwise be read by a kernel.

def _on_gpu(t, name: str):
    import torch
    if not torch.is_tensor(t):
        raise TypeError(f"{name} must be a torch tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor (got {t.device}): the library takes device pointers")
    return t.device


def _buf(t, name: str, dtype, numel: int, device, required: bool = False) -> None:
    import torch
    if t is None:
        if required:
            raise ValueError(f"{name} is required")
        return
    if not torch.is_tensor(t):
        raise TypeError(f"{name} must be a torch tensor")
    if t.device != device:
        raise ValueError(f"{name} must be on {device} (got {t.device})")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype} (got {t.dtype})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.numel() < numel:
        raise ValueError(f"{name} needs at least {numel} elements (got {t.numel()})")


def _grad_out(grad_out, reduction: str, n: int, device):
    """The upstream gradient as the library reads it: fp32, contiguous, one value per token for
    reduction 'none' (a Python number is broadcast), else one value."""
    import torch
    if grad_out is None:
        return None
    need = n if reduction == "none" else 1
    if not torch.is_tensor(grad_out):
        return torch.full((max(need, 1),), float(grad_out), dtype=torch.float32, device=device)
    if grad_out.device != device:
        raise ValueError(f"grad_out must be on {device} (got {grad_out.device})")
    g = grad_out.to(torch.float32).reshape(-1).contiguous()
    if g.numel() < need:
        raise ValueError(f"grad_out needs {need} value(s) for reduction {reduction!r} (got {g.numel()})")
    return g


def _ws(workspace, need: int, device) -> None:
    import torch
    _buf(workspace, "workspace", torch.uint8, need, device, required=True)


@dataclass
class CEResult:
    loss_tok: object      # fp32 [n]
    loss_out: object      # fp32 [1]
    argmax: object        # int64 [n] or None
    counts: object        # int64 [3] {n_valid, n_correct, n_bad}


@_on_call_stream
def lce_ce_fwd_bwd(logits, labels, *, ignore_index: int = -100, label_smoothing: float = 0.0,
                   softcap: float = 0.0, reduction: str = "mean", grad_out=None, want_argmax: bool = False,
                   loss_tok=None, loss_out=None, argmax_out=None, counts=None, workspace=None,
                   stream=None) -> CEResult:
    """Cross-entropy forward + backward; ``logits`` ([n, V] view, unit column stride, row
    stride ld >= V) is overwritten with the gradient.  Outputs not passed in are allocated."""
    import torch
    if logits.dim() != 2 or (logits.size(1) > 1 and logits.stride(1) != 1):
        raise ValueError("logits must be a 2-D view with unit column stride")
    n, V = logits.shape
    ld = logits.stride(0) if n > 1 else V
    dev = _on_gpu(logits, "logits")
    _buf(labels, "labels", torch.int64, n, dev, required=True)
    grad_out = _grad_out(grad_out, reduction, n, dev)
    if loss_tok is None:
        loss_tok = torch.empty(n, dtype=torch.float32, device=dev)
    if loss_out is None:
        loss_out = torch.empty(1, dtype=torch.float32, device=dev)
    if argmax_out is None and want_argmax:
        argmax_out = torch.empty(n, dtype=torch.int64, device=dev)
    if counts is None:
        counts = torch.empty(3, dtype=torch.int64, device=dev)
    wsb = lce_ce_workspace_bytes(n, V)
    if workspace is None:   # needs no initialisation (tagged counters)
        workspace = torch.empty(wsb, dtype=torch.uint8, device=dev)
    _buf(loss_tok, "loss_tok", torch.float32, n, dev)
    _buf(loss_out, "loss_out", torch.float32, 1, dev)
    _buf(argmax_out, "argmax_out", torch.int64, n, dev)
    _buf(counts, "counts", torch.int64, 3, dev)
    _ws(workspace, wsb, dev)
    st = lib().lce_ce_fwd_bwd(_ptr(logits), ld, _dtype_code(logits), _ptr(labels), n, V, int(ignore_index),
                              float(label_smoothing), float(softcap), REDUCTIONS[reduction], _ptr(grad_out),
                              _ptr(loss_tok), _ptr(loss_out), _ptr(argmax_out), _ptr(counts), _ptr(workspace),
                              workspace.numel() * workspace.element_size(), _stream(stream))
    _check(st)
    return CEResult(loss_tok, loss_out, argmax_out, counts)


@_on_call_stream
def lce_ce_fwd_bwd_noalloc(logits, labels, *, ignore_index: int = -100, label_smoothing: float = 0.0,
                           softcap: float = 0.0, reduction: str = "mean", grad_out=None, loss_tok=None, loss_out=None,
                           argmax_out=None, counts=None, stream=None) -> CEResult:
    """lce_ce_fwd_bwd with the library's own per-device scratch instead of a workspace (for callers
    that cannot allocate: pass every output, and grad_out as an fp32 device tensor or None, and
    nothing is allocated here either).  Calls overlapping on one device race on that scratch."""
    import torch
    if logits.dim() != 2 or (logits.size(1) > 1 and logits.stride(1) != 1):
        raise ValueError("logits must be a 2-D view with unit column stride")
    n, V = logits.shape
    ld = logits.stride(0) if n > 1 else V
    dev = _on_gpu(logits, "logits")
    _buf(labels, "labels", torch.int64, n, dev, required=True)
    grad_out = _grad_out(grad_out, reduction, n, dev)
    if loss_tok is None:
        loss_tok = torch.empty(n, dtype=torch.float32, device=dev)
    if loss_out is None:
        loss_out = torch.empty(1, dtype=torch.float32, device=dev)
    if counts is None:
        counts = torch.empty(3, dtype=torch.int64, device=dev)
    _buf(loss_tok, "loss_tok", torch.float32, n, dev)
    _buf(loss_out, "loss_out", torch.float32, 1, dev)
    _buf(argmax_out, "argmax_out", torch.int64, n, dev)
    _buf(counts, "counts", torch.int64, 3, dev)
    st = lib().lce_ce_fwd_bwd_noalloc(_ptr(logits), ld, _dtype_code(logits), _ptr(labels), n, V, int(ignore_index),
                                      float(label_smoothing), float(softcap), REDUCTIONS[reduction], _ptr(grad_out),
                                      _ptr(loss_tok), _ptr(loss_out), _ptr(argmax_out), _ptr(counts), _stream(stream))
    _check(st)
    return CEResult(loss_tok, loss_out, argmax_out, counts)


@_on_call_stream
def lce_ce_argmax(logits, labels=None, *, ignore_index: int = -100, argmax_out=None, counts=None,
                  stream=None):
    """Read-only argmax sweep.  Returns (argmax int64 [n], counts int64 [3])."""
    import torch
    if logits.dim() != 2 or (logits.size(1) > 1 and logits.stride(1) != 1):
        raise ValueError("logits must be a 2-D view with unit column stride")
    n, V = logits.shape
    ld = logits.stride(0) if n > 1 else V
    dev = _on_gpu(logits, "logits")
    _buf(labels, "labels", torch.int64, n, dev)
    if argmax_out is None:
        argmax_out = torch.empty(n, dtype=torch.int64, device=dev)
    if counts is None:
        counts = torch.empty(3, dtype=torch.int64, device=dev)
    _buf(argmax_out, "argmax_out", torch.int64, n, dev)
    _buf(counts, "counts", torch.int64, 3, dev)
    st = lib().lce_ce_argmax(_ptr(logits), ld, _dtype_code(logits), _ptr(labels), n, V, int(ignore_index),
                             _ptr(argmax_out), _ptr(counts), _stream(stream))
    _check(st)
    return argmax_out, counts


# ---- split cross-entropy: shard statistics, combine, gradient --------------------------------

STATS_FLOATS = 8


def _shard_view(shard):
    if shard.dim() != 2 or (shard.size(1) > 1 and shard.stride(1) != 1):
        raise ValueError("a shard must be a 2-D view with unit column stride")
    n, Vs = shard.shape
    return n, Vs, (shard.stride(0) if n > 1 else Vs)


@_on_call_stream
def lce_ce_stats(shard, labels, *, v_offset: int = 0, ignore_index: int = -100, softcap: float = 0.0,
                 stats=None, stream=None):
    """One read-only sweep of a vocabulary shard (global columns [v_offset, v_offset + width));
    returns its stats records, fp32 [n, 8]."""
    import torch
    n, Vs, ld = _shard_view(shard)
    dev = _on_gpu(shard, "shard")
    _buf(labels, "labels", torch.int64, n, dev, required=True)
    if stats is None:
        stats = torch.empty((n, STATS_FLOATS), dtype=torch.float32, device=dev)
    _buf(stats, "stats", torch.float32, n * STATS_FLOATS, dev)
    _check(lib().lce_ce_stats(_ptr(shard), ld, _dtype_code(shard), _ptr(labels), n, Vs, int(v_offset),
                              int(ignore_index), float(softcap), _ptr(stats), _stream(stream)))
    return stats


@dataclass
class SplitRows:
    lse: object            # fp32 [n]
    one_minus_py: object   # fp32 [n]
    loss_tok: object       # fp32 [n]
    loss_out: object       # fp32 [1]
    logprob: object        # fp32 [n]
    entropy: object        # fp32 [n]
    argmax: object         # int64 [n]
    counts: object         # int64 [3]


@_on_call_stream
def lce_ce_combine(stats, labels, V: int, *, ignore_index: int = -100, label_smoothing: float = 0.0,
                   reduction: str = "mean", out: SplitRows | None = None, stream=None) -> SplitRows:
    """Row results from the stats of all shards: ``stats`` is fp32 [shards, n, 8] (or [n, 8] for one),
    shards in ascending vocabulary order.  ``out`` (optional) supplies the output tensors."""
    import torch
    if stats.dim() == 2:
        stats = stats.unsqueeze(0)
    if not stats.is_contiguous() or stats.dim() != 3 or stats.size(2) != STATS_FLOATS or stats.dtype != torch.float32:
        raise ValueError("stats must be a contiguous [shards, n, 8] fp32 tensor")
    shards, n = stats.shape[0], stats.shape[1]
    dev = _on_gpu(stats, "stats")
    _buf(labels, "labels", torch.int64, n, dev, required=True)
    if out is None:
        f = lambda: torch.empty(n, dtype=torch.float32, device=dev)  # noqa: E731
        out = SplitRows(f(), f(), f(), torch.empty(1, dtype=torch.float32, device=dev), f(), f(),
                        torch.empty(n, dtype=torch.int64, device=dev), torch.empty(3, dtype=torch.int64, device=dev))
    for name in ("lse", "one_minus_py", "loss_tok", "logprob", "entropy"):
        _buf(getattr(out, name), f"out.{name}", torch.float32, n, dev)
    _buf(out.lse, "out.lse", torch.float32, n, dev, required=True)
    _buf(out.loss_out, "out.loss_out", torch.float32, 1, dev)
    _buf(out.argmax, "out.argmax", torch.int64, n, dev)
    _buf(out.counts, "out.counts", torch.int64, 3, dev, required=True)
    _check(lib().lce_ce_combine(_ptr(stats), shards, _ptr(labels), n, int(V), int(ignore_index),
                                float(label_smoothing), REDUCTIONS[reduction], _ptr(out.lse), _ptr(out.one_minus_py),
                                _ptr(out.loss_tok), _ptr(out.loss_out), _ptr(out.logprob), _ptr(out.entropy),
                                _ptr(out.argmax), _ptr(out.counts), _stream(stream)))
    return out


@_on_call_stream
def lce_ce_grad(shard, labels, V: int, rows: SplitRows, *, v_offset: int = 0, ignore_index: int = -100,
                label_smoothing: float = 0.0, softcap: float = 0.0, reduction: str = "mean", grad_out=None,
                stream=None) -> None:
    """Write the gradient of one shard in place, from the combined row results."""
    import torch
    n, Vs, ld = _shard_view(shard)
    dev = _on_gpu(shard, "shard")
    _buf(labels, "labels", torch.int64, n, dev, required=True)
    grad_out = _grad_out(grad_out, reduction, n, dev)
    _buf(rows.lse, "rows.lse", torch.float32, n, dev, required=True)
    _buf(rows.one_minus_py, "rows.one_minus_py", torch.float32, n, dev, required=True)
    _buf(rows.counts, "rows.counts", torch.int64, 3, dev, required=True)
    _check(lib().lce_ce_grad(_ptr(shard), ld, _dtype_code(shard), _ptr(labels), n, Vs, int(v_offset), int(V),
                             int(ignore_index), float(label_smoothing), float(softcap), REDUCTIONS[reduction],
                             _ptr(grad_out), _ptr(rows.lse), _ptr(rows.one_minus_py), _ptr(rows.counts),
                             _stream(stream)))


def cross_entropy(logits, labels, *, ignore_index: int = -100, label_smoothing: float = 0.0, softcap: float = 0.0,
                  reduction: str = "mean"):
    """Autograd form of the split path with the gradient deferred to backward.

    The forward is one read-only sweep (lce_ce_stats, lce_ce_combine); backward
    writes the gradient over ``logits`` in place with the upstream gradient it
    receives (lce_ce_grad) and returns that buffer, so the gradient has the
    logits' dtype and ``logits`` must not be used after backward.  A second
    backward through the same graph raises, since the logits are gone.
    Returns (loss, logprob, entropy, argmax, counts): loss is the reduced fp32
    scalar, or fp32 [n] for reduction "none"; the rest carry no gradient.
    """
    return _DeferredCE.apply(logits, labels, int(ignore_index), float(label_smoothing), float(softcap),
                             reduction)


def _deferred_ce_class():
    import torch

    class DeferredCE(torch.autograd.Function):
        @staticmethod
        def forward(ctx, logits, labels, ignore_index, eps, softcap, reduction):
            if reduction not in REDUCTIONS:
                raise ValueError(f"unknown reduction {reduction!r}")
            V = logits.shape[-1]
            stats = lce_ce_stats(logits, labels, ignore_index=ignore_index, softcap=softcap)
            rows = lce_ce_combine(stats, labels, V, ignore_index=ignore_index, label_smoothing=eps,
                                  reduction=reduction)
            ctx.save_for_backward(logits, labels)
            ctx.rows = rows
            ctx.args = (V, ignore_index, eps, softcap, reduction)
            ctx.consumed = False
            loss = rows.loss_tok if reduction == "none" else rows.loss_out.view(())
            ctx.mark_non_differentiable(rows.logprob, rows.entropy, rows.argmax, rows.counts)
            return loss, rows.logprob, rows.entropy, rows.argmax, rows.counts

        @staticmethod
        def backward(ctx, g, *_unused):
            if ctx.consumed:
                raise RuntimeError("cross_entropy: the logits buffer already holds its gradient; "
                                   "backward through this graph a second time is not supported")
            logits, labels = ctx.saved_tensors
            V, ignore_index, eps, softcap, reduction = ctx.args
            grad_out = g.detach().to(torch.float32).reshape(-1).contiguous()
            lce_ce_grad(logits, labels, V, ctx.rows, ignore_index=ignore_index, label_smoothing=eps,
                        softcap=softcap, reduction=reduction, grad_out=grad_out)
            ctx.consumed = True
            return logits, None, None, None, None, None

    return DeferredCE


class _LazyFunction:
    """Builds the autograd class on first use, so importing this module does not import torch."""

    def __init__(self, make):
        self._make, self._cls = make, None

    def apply(self, *args):
        if self._cls is None:
            self._cls = self._make()
        return self._cls.apply(*args)


_DeferredCE = _LazyFunction(_deferred_ce_class)


def lce_flce_workspace_bytes(n: int, H: int, V: int, chunk_tokens: int) -> int:
    return int(lib().lce_flce_workspace_bytes(int(n), int(H), int(V), int(chunk_tokens)))


def lce_flce_workspace_bytes_grouped(n: int, H: int, V: int, chunk_tokens: int, group_chunks: int) -> int:
    return int(lib().lce_flce_workspace_bytes_grouped(int(n), int(H), int(V), int(chunk_tokens), int(group_chunks)))


@dataclass
class FLCEResult:
    loss_tok: object      # fp32 [n]
    loss_out: object      # fp32 [1]
    grad_hidden: object   # bf16 [n, H]
    grad_weight: object   # fp32 [V, H]
    counts: object        # int64 [3]


@_on_call_stream
def lce_flce_fwd_bwd(hidden, weight, labels, *, ignore_index: int = -100, label_smoothing: float = 0.0,
                     softcap: float = 0.0, reduction: str = "mean", grad_out=None, chunk_tokens: int = 1024,
                     loss_tok=None, loss_out=None, grad_hidden=None, grad_weight=None, counts=None, workspace=None,
                     stream=None, aux_stream="auto") -> FLCEResult:
    """Fused linear cross-entropy of hidden [n, H] (bf16) and weight [V, H] (bf16), chunked over
    tokens.  Outputs not passed in are allocated.  ``aux_stream``: the second stream the transposes
    may run on ("auto": this host thread's own stream on the device; None: one stream)."""
    import torch
    dev = _check_flce_operands(hidden, weight)
    n, H = hidden.shape
    V = weight.shape[0]
    _buf(labels, "labels", torch.int64, n, dev, required=True)
    grad_out = _grad_out(grad_out, reduction, n, dev)
    if loss_tok is None:
        loss_tok = torch.empty(n, dtype=torch.float32, device=dev)
    if loss_out is None:
        loss_out = torch.empty(1, dtype=torch.float32, device=dev)
    if grad_hidden is None:
        grad_hidden = torch.empty((n, H), dtype=torch.bfloat16, device=dev)
    if grad_weight is None:
        grad_weight = torch.empty((V, H), dtype=torch.float32, device=dev)
    if counts is None:
        counts = torch.empty(3, dtype=torch.int64, device=dev)
    wsb = lce_flce_workspace_bytes(n, H, V, chunk_tokens)
    if workspace is None:   # clobbered by the call; its contents do not matter
        workspace = torch.empty(wsb, dtype=torch.uint8, device=dev)
    _buf(loss_tok, "loss_tok", torch.float32, n, dev)
    _buf(loss_out, "loss_out", torch.float32, 1, dev)
    _buf(grad_hidden, "grad_hidden", torch.bfloat16, n * H, dev)
    _buf(grad_weight, "grad_weight", torch.float32, V * H, dev)
    _buf(counts, "counts", torch.int64, 3, dev)
    _ws(workspace, 1, dev)   # the library checks the size against the layout it needs
    st = lib().lce_flce_fwd_bwd(_ptr(hidden), _ptr(weight), _ptr(labels), n, H, V, int(ignore_index),
                                float(label_smoothing), float(softcap), REDUCTIONS[reduction], _ptr(grad_out),
                                int(chunk_tokens), _ptr(loss_tok), _ptr(loss_out), _ptr(grad_hidden),
                                _ptr(grad_weight), _ptr(counts), _ptr(workspace),
                                workspace.numel() * workspace.element_size(), _stream(stream),
                                _aux_stream(aux_stream, dev))
    _check(st)
    return FLCEResult(loss_tok, loss_out, grad_hidden, grad_weight, counts)


# ---- tile-resident fused linear cross-entropy: forward stats, deferred backward ---------------

def lce_flce_stats_bytes(n: int, V: int) -> int:
    return int(lib().lce_flce_stats_bytes(int(n), int(V)))


def _check_flce_operands(hidden, weight):
    """Both operands contiguous 2-D bf16 on one GPU, sharing H; returns that device."""
    import torch
    for t, nm in ((hidden, "hidden"), (weight, "weight")):
        if not torch.is_tensor(t) or t.dtype != torch.bfloat16 or t.dim() != 2 or not t.is_contiguous():
            raise ValueError(f"{nm} must be a contiguous 2-D bfloat16 tensor")
    dev = _on_gpu(hidden, "hidden")
    if weight.device != dev:
        raise ValueError(f"weight must be on {dev} (got {weight.device})")
    if weight.shape[1] != hidden.shape[1]:
        raise ValueError(f"hidden [n, {hidden.shape[1]}] and weight [V, {weight.shape[1]}] disagree on H")
    return dev


@_on_call_stream
def lce_flce_forward(hidden, weight, labels, *, ignore_index: int = -100, label_smoothing: float = 0.0,
                     softcap: float = 0.0, reduction: str = "mean", workspace=None, out: SplitRows | None = None,
                     stream=None) -> SplitRows:
    """Loss, log-sum-exp, 1 - p_y, log p_y, entropy, argmax and counts of the logits hidden weight^T,
    formed tile by tile and never stored.  ``out`` (optional) supplies the output tensors."""
    import torch
    dev = _check_flce_operands(hidden, weight)
    n, H = hidden.shape
    V = weight.shape[0]
    _buf(labels, "labels", torch.int64, n, dev, required=True)
    if out is None:
        f = lambda: torch.empty(n, dtype=torch.float32, device=dev)  # noqa: E731
        out = SplitRows(f(), f(), f(), torch.empty(1, dtype=torch.float32, device=dev), f(), f(),
                        torch.empty(n, dtype=torch.int64, device=dev), torch.empty(3, dtype=torch.int64, device=dev))
    if workspace is None:
        workspace = torch.empty(max(lce_flce_stats_bytes(n, V), 1), dtype=torch.uint8, device=dev)
    for name in ("lse", "one_minus_py", "loss_tok", "logprob", "entropy"):
        _buf(getattr(out, name), f"out.{name}", torch.float32, n, dev)
    _buf(out.loss_out, "out.loss_out", torch.float32, 1, dev)
    _buf(out.argmax, "out.argmax", torch.int64, n, dev)
    _buf(out.counts, "out.counts", torch.int64, 3, dev, required=True)
    _ws(workspace, lce_flce_stats_bytes(n, V), dev)
    _check(lib().lce_flce_forward(_ptr(hidden), _ptr(weight), _ptr(labels), n, H, V, int(ignore_index),
                                  float(label_smoothing), float(softcap), REDUCTIONS[reduction], _ptr(out.loss_tok),
                                  _ptr(out.loss_out), _ptr(out.lse), _ptr(out.one_minus_py), _ptr(out.logprob),
                                  _ptr(out.entropy), _ptr(out.argmax), _ptr(out.counts), _ptr(workspace),
                                  workspace.numel() * workspace.element_size(), _stream(stream)))
    return out


@_on_call_stream
def lce_flce_backward(hidden, weight, labels, rows: SplitRows, *, ignore_index: int = -100,
                      label_smoothing: float = 0.0, softcap: float = 0.0, reduction: str = "mean", grad_out=None,
                      chunk_tokens: int = 1024, grad_hidden=None, grad_weight=None, workspace=None, stream=None,
                      aux_stream="auto"):
    """grad_hidden (bf16 [n, H]) and grad_weight (fp32 [V, H]) from the forward's rows; ``aux_stream`` as
    for lce_flce_fwd_bwd."""
    import torch
    dev = _check_flce_operands(hidden, weight)
    n, H = hidden.shape
    V = weight.shape[0]
    _buf(labels, "labels", torch.int64, n, dev, required=True)
    grad_out = _grad_out(grad_out, reduction, n, dev)
    _buf(rows.lse, "rows.lse", torch.float32, n, dev, required=True)
    _buf(rows.one_minus_py, "rows.one_minus_py", torch.float32, n, dev, required=True)
    _buf(rows.counts, "rows.counts", torch.int64, 3, dev, required=True)
    if grad_hidden is None:
        grad_hidden = torch.empty((n, H), dtype=torch.bfloat16, device=dev)
    if grad_weight is None:
        grad_weight = torch.empty((V, H), dtype=torch.float32, device=dev)
    if workspace is None:
        workspace = torch.empty(lce_flce_workspace_bytes(n, H, V, chunk_tokens), dtype=torch.uint8, device=dev)
    _buf(grad_hidden, "grad_hidden", torch.bfloat16, n * H, dev)
    _buf(grad_weight, "grad_weight", torch.float32, V * H, dev)
    _ws(workspace, 1, dev)   # the library checks the size against the layout it needs
    _check(lib().lce_flce_backward(_ptr(hidden), _ptr(weight), _ptr(labels), n, H, V, int(ignore_index),
                                   float(label_smoothing), float(softcap), REDUCTIONS[reduction], _ptr(grad_out),
                                   int(chunk_tokens), _ptr(rows.lse), _ptr(rows.one_minus_py), _ptr(rows.counts),
                                   _ptr(grad_hidden), _ptr(grad_weight), _ptr(workspace),
                                   workspace.numel() * workspace.element_size(), _stream(stream),
                                   _aux_stream(aux_stream, dev)))
    return grad_hidden, grad_weight


def linear_cross_entropy(hidden, weight, labels, *, ignore_index: int = -100, label_smoothing: float = 0.0,
                         softcap: float = 0.0, reduction: str = "mean", chunk_tokens: int = 1024):
    """Autograd form of the tile-resident fused linear cross-entropy.

    Forward: lce_flce_forward (no logits stored).  Backward: lce_flce_backward with the upstream
    gradient it receives; grad_weight is accumulated in fp32 and handed to autograd, which casts it
    to the weight's dtype.  Returns (loss, logprob, entropy, argmax, counts); loss is the reduced fp32
    scalar, or fp32 [n] for reduction "none"; the rest carry no gradient.
    """
    return _DeferredFLCE.apply(hidden, weight, labels, int(ignore_index), float(label_smoothing), float(softcap),
                               reduction, int(chunk_tokens))


def _deferred_flce_class():
    import torch

    class DeferredFLCE(torch.autograd.Function):
        @staticmethod
        def forward(ctx, hidden, weight, labels, ignore_index, eps, softcap, reduction, chunk_tokens):
            if reduction not in REDUCTIONS:
                raise ValueError(f"unknown reduction {reduction!r}")
            rows = lce_flce_forward(hidden, weight, labels, ignore_index=ignore_index, label_smoothing=eps,
                                    softcap=softcap, reduction=reduction)
            ctx.save_for_backward(hidden, weight, labels)
            ctx.rows = rows
            ctx.args = (ignore_index, eps, softcap, reduction, chunk_tokens)
            loss = rows.loss_tok if reduction == "none" else rows.loss_out.view(())
            ctx.mark_non_differentiable(rows.logprob, rows.entropy, rows.argmax, rows.counts)
            return loss, rows.logprob, rows.entropy, rows.argmax, rows.counts

        @staticmethod
        def backward(ctx, g, *_unused):
            hidden, weight, labels = ctx.saved_tensors
            ignore_index, eps, softcap, reduction, chunk_tokens = ctx.args
            grad_out = g.detach().to(torch.float32).reshape(-1).contiguous()
            gh, gw = lce_flce_backward(hidden, weight, labels, ctx.rows, ignore_index=ignore_index,
                                       label_smoothing=eps, softcap=softcap, reduction=reduction, grad_out=grad_out,
                                       chunk_tokens=chunk_tokens)
            return gh, gw, None, None, None, None, None, None

    return DeferredFLCE


_DeferredFLCE = _LazyFunction(_deferred_flce_class)
