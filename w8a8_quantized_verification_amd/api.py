"""Python binding of libw8a8.so on torch tensors.

Every function checks dtype, device, contiguity and shape, then passes raw
device pointers and torch's current HIP stream to the C ABI (include/w8a8.h);
all arithmetic happens in the library's kernels.  Outputs are allocated with
torch unless passed in.  Tensors must live on a ROCm device: there is no CPU
path.
"""
from __future__ import annotations

import torch

from ._lib import W8A8Error, check, lib

__all__ = [
    "W8A8Error", "quantize_act", "quantize_weight", "tile_weight", "tiled_shape", "linear",
    "linear_workspace_bytes",
    "verify_accept", "verify_accept_workspace_bytes", "lm_head_verify", "lm_head_argmax",
    "accept_from_keys", "bf16_linear", "bf16_tiled_shape", "tile_weight_bf16", "Workspace",
    "verify_sample",
    "verify_sample_workspace_bytes", "sample_weights", "w4_shape", "quantize_weight_w4",
    "linear_w4", "lm_head_argmax_w4", "residual_rmsnorm_quant", "silu_mul_quant",
    "quantize_act_tiled", "linear_tiled_act", "linear_tiled_act_workspace_bytes",
    "verify_attention", "qk_norm_rope_append",
    "pack_v_cache", "hbm_read_probe", "HBM_PROBE_SINK_WORDS", "lm_head_verify_noalloc",
    "NOALLOC_MAX_ROWS",
]

NOALLOC_MAX_ROWS = 288        # W8A8_NOALLOC_MAX_ROWS

HBM_PROBE_SINK_WORDS = 1      # W8A8_HBM_PROBE_SINK_WORDS


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _need(t: torch.Tensor, name: str, dtype, ndim: int, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise TypeError(f"{name} must be on a ROCm device (got {t.device}); there is no CPU path")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype} (got {t.dtype})")
    if t.dim() != ndim:
        raise ValueError(f"{name} must be {ndim}-D (got shape {tuple(t.shape)})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _out(t, shape, dtype, device, name):
    if t is None:
        return torch.empty(shape, dtype=dtype, device=device)
    _need(t, name, dtype, len(shape), device)
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)} (got {tuple(t.shape)})")
    return t


class Workspace:
    """Per-device scratch buffers, one per device and use:

    * ``"zeroed"`` (allocated zero-filled): w8a8_linear's split-K partials
      and arrival counters, which every completed call leaves zero again;
    * ``"keys"`` (allocated zero-filled): the LM-head argmax keys.
      lm_head_argmax (phase 1) leaves non-zero keys behind until the
      accept_from_keys that follows it reads and resets them, so they get a
      buffer of their own: a split-K linear between the two phases would
      otherwise add its partials onto the keys;
    * ``"verify"``: per-chunk results of verify_accept, verify_sample and
      the attention split, overwritten by each call and left non-zero.

    Calls that use one Workspace must run in order on one stream (the
    default use)."""

    USES = ("zeroed", "keys", "verify")

    def __init__(self):
        self._buf = {}

    def get(self, nbytes: int, device: torch.device, use: str) -> torch.Tensor | None:
        if use not in self.USES:
            raise ValueError(f"unknown workspace use {use!r} (one of {self.USES})")
        if nbytes == 0:
            return None
        if device.index is not None:
            idx = device.index
        else:
            idx = torch.cuda.current_device() if device.type == "cuda" else -1
        key = (idx, use)
        b = self._buf.get(key)
        if b is None or b.numel() < nbytes:
            b = torch.zeros(max(nbytes, 1 << 20), dtype=torch.uint8, device=device)
            self._buf[key] = b
        return b


_default_ws = Workspace()


def quantize_act(x: torch.Tensor, smooth: torch.Tensor | None = None, *, xq=None, x_scale=None):
    """Per-token symmetric int8 quantization of bf16 ``x[M][K]``; returns
    ``(xq int8[M][K], x_scale float32[M])``."""
    _need(x, "x", torch.bfloat16, 2)
    M, K = x.shape
    if smooth is not None:
        _need(smooth, "smooth", torch.float32, 1, x.device)
    xq = _out(xq, (M, K), torch.int8, x.device, "xq")
    x_scale = _out(x_scale, (M,), torch.float32, x.device, "x_scale")
    check(lib().w8a8_quantize_act(_ptr(x), _ptr(smooth), M, K, _ptr(xq), _ptr(x_scale),
                                  _stream(x.device)))
    return xq, x_scale


def tiled_shape(N: int, K: int) -> tuple:
    """Shape of the tiled weight layout as an int8 tensor: [ceil(N/16),
    ceil(K/64), 64 lanes, 16 bytes] (see include/w8a8.h)."""
    return ((N + 15) // 16, (K + 63) // 64, 64, 16)


def quantize_weight(w: torch.Tensor, smooth: torch.Tensor | None = None, *, tiled: bool = False,
                    wq=None, w_scale=None):
    """Per-output-channel symmetric int8 quantization of fp32 ``w[N][K]``;
    returns ``(wq, w_scale float32[N])`` with ``wq`` int8 ``[N][K]`` or, with
    ``tiled=True``, in the tiled layout (shape :func:`tiled_shape`)."""
    _need(w, "w", torch.float32, 2)
    N, K = w.shape
    if smooth is not None:
        _need(smooth, "smooth", torch.float32, 1, w.device)
    shape = tiled_shape(N, K) if tiled else (N, K)
    wq = _out(wq, shape, torch.int8, w.device, "wq")
    w_scale = _out(w_scale, (N,), torch.float32, w.device, "w_scale")
    f = lib().w8a8_quantize_weight_tiled if tiled else lib().w8a8_quantize_weight
    check(f(_ptr(w), _ptr(smooth), N, K, _ptr(wq), _ptr(w_scale), _stream(w.device)))
    return wq, w_scale


def tile_weight(wq: torch.Tensor, *, out=None) -> torch.Tensor:
    """Rearrange row-major int8 ``wq[N][K]`` into the tiled layout."""
    _need(wq, "wq", torch.int8, 2)
    N, K = wq.shape
    out = _out(out, tiled_shape(N, K), torch.int8, wq.device, "out")
    check(lib().w8a8_tile_weight(_ptr(wq), N, K, _ptr(out), _stream(wq.device)))
    return out


def linear_workspace_bytes(M: int, N: int, K: int) -> int:
    return int(lib().w8a8_linear_workspace_bytes(M, N, K))


def linear(xq, x_scale, wq, w_scale, *, want_bf16=True, want_f32=False, want_acc=False,
           y_bf16=None, y_f32=None, acc=None, workspace: Workspace | None = None):
    """One W8A8 linear.  ``wq`` is int8 ``[N][K]`` or the tiled layout (4-D,
    shape :func:`tiled_shape`).  Returns ``(y_bf16, y_f32, acc)``, each None
    unless requested (``want_*``) or passed in."""
    _need(xq, "xq", torch.int8, 2)
    dev = xq.device
    _need(x_scale, "x_scale", torch.float32, 1, dev)
    _need(w_scale, "w_scale", torch.float32, 1, dev)
    M, K = xq.shape
    N = w_scale.shape[0]
    tiled = isinstance(wq, torch.Tensor) and wq.dim() == 4
    _need(wq, "wq", torch.int8, 4 if tiled else 2, dev)
    if tiled:
        if tuple(wq.shape) != tiled_shape(N, K):
            raise ValueError(f"tiled wq must have shape {tiled_shape(N, K)} (got {tuple(wq.shape)})")
    elif tuple(wq.shape) != (N, K):
        raise ValueError("shape mismatch between xq[M][K], wq[N][K], w_scale[N]")
    if x_scale.shape[0] != M:
        raise ValueError("x_scale must have M entries")
    if want_bf16 or y_bf16 is not None:
        y_bf16 = _out(y_bf16, (M, N), torch.bfloat16, dev, "y_bf16")
    if want_f32 or y_f32 is not None:
        y_f32 = _out(y_f32, (M, N), torch.float32, dev, "y_f32")
    if want_acc or acc is not None:
        acc = _out(acc, (M, N), torch.int32, dev, "acc")
    need = linear_workspace_bytes(M, N, K)
    ws = (workspace or _default_ws).get(need, dev, use="zeroed")
    f = lib().w8a8_linear_tiled if tiled else lib().w8a8_linear
    check(f(_ptr(xq), _ptr(x_scale), _ptr(wq), _ptr(w_scale), M, N, K,
            _ptr(y_bf16), _ptr(y_f32), _ptr(acc), _ptr(ws),
            0 if ws is None else ws.numel(), _stream(dev)))
    return y_bf16, y_f32, acc


def verify_accept_workspace_bytes(B: int, G: int, V: int) -> int:
    return int(lib().w8a8_verify_accept_workspace_bytes(B, G, V))


def verify_accept(logits, draft, *, want_argmax=True, argmax=None, accept_len=None,
                  next_token=None, workspace: Workspace | None = None):
    """Argmax of every row of fp32 ``logits[B*(G+1)][V]`` and greedy
    acceptance of int32 ``draft[B][G]``.  Returns ``(argmax or None,
    accept_len, next_token)``."""
    _need(logits, "logits", torch.float32, 2)
    dev = logits.device
    _need(draft, "draft", torch.int32, 2, dev)
    B, G = draft.shape
    R, V = logits.shape
    if R != B * (G + 1):
        raise ValueError(f"logits must have B*(G+1) = {B * (G + 1)} rows (got {R})")
    if want_argmax or argmax is not None:
        argmax = _out(argmax, (R,), torch.int32, dev, "argmax")
    accept_len = _out(accept_len, (B,), torch.int32, dev, "accept_len")
    next_token = _out(next_token, (B,), torch.int32, dev, "next_token")
    need = verify_accept_workspace_bytes(B, G, V)
    ws = (workspace or _default_ws).get(need, dev, use="verify")
    check(lib().w8a8_verify_accept(_ptr(logits), V, _ptr(draft), B, G, _ptr(argmax),
                                   _ptr(accept_len), _ptr(next_token), _ptr(ws),
                                   0 if ws is None else ws.numel(), _stream(dev)))
    return argmax, accept_len, next_token


def lm_head_verify(xq, x_scale, wq_tiled, w_scale, draft, *, want_logits=False,
                   want_argmax=True, logits=None, argmax=None, accept_len=None, next_token=None,
                   workspace: Workspace | None = None):
    """LM-head W8A8 linear with the argmax's first pass fused into its
    epilogue, then greedy acceptance.  ``xq[B*(G+1)][K]``, tiled ``wq_tiled``
    for ``[V][K]``, ``draft[B][G]``.  Returns ``(logits or None, argmax or
    None, accept_len, next_token)``."""
    _need(xq, "xq", torch.int8, 2)
    dev = xq.device
    _need(x_scale, "x_scale", torch.float32, 1, dev)
    _need(w_scale, "w_scale", torch.float32, 1, dev)
    _need(draft, "draft", torch.int32, 2, dev)
    R, K = xq.shape
    V = w_scale.shape[0]
    B, G = draft.shape
    if R != B * (G + 1) or x_scale.shape[0] != R:
        raise ValueError(f"xq and x_scale must have B*(G+1) = {B * (G + 1)} rows")
    _need(wq_tiled, "wq_tiled", torch.int8, 4, dev)
    if tuple(wq_tiled.shape) != tiled_shape(V, K):
        raise ValueError(f"wq_tiled must have shape {tiled_shape(V, K)}")
    if want_logits or logits is not None:
        logits = _out(logits, (R, V), torch.float32, dev, "logits")
    if want_argmax or argmax is not None:
        argmax = _out(argmax, (R,), torch.int32, dev, "argmax")
    accept_len = _out(accept_len, (B,), torch.int32, dev, "accept_len")
    next_token = _out(next_token, (B,), torch.int32, dev, "next_token")
    need = int(lib().w8a8_lm_head_verify_workspace_bytes(B, G, V, K))
    ws = (workspace or _default_ws).get(need, dev, use="keys")
    check(lib().w8a8_lm_head_verify(_ptr(xq), _ptr(x_scale), _ptr(wq_tiled), _ptr(w_scale), V, K,
                                    _ptr(draft), B, G, _ptr(logits), _ptr(argmax),
                                    _ptr(accept_len), _ptr(next_token), _ptr(ws),
                                    0 if ws is None else ws.numel(), _stream(dev)))
    return logits, argmax, accept_len, next_token



def lm_head_verify_noalloc(xq, x_scale, wq_tiled, w_scale, draft, *, logits=None, argmax=None,
                           accept_len=None, next_token=None):
    """:func:`lm_head_verify` through the entry point that takes no workspace
    (the argmax keys live in the library's per-GPU scratch array; at most
    ``NOALLOC_MAX_ROWS`` verified rows).  Outputs that are not passed are
    allocated here with torch before the call; pass them all to keep the
    call allocation-free.  Returns ``(logits or None, argmax or None,
    accept_len, next_token)``."""
    _need(xq, "xq", torch.int8, 2)
    dev = xq.device
    _need(x_scale, "x_scale", torch.float32, 1, dev)
    _need(w_scale, "w_scale", torch.float32, 1, dev)
    _need(draft, "draft", torch.int32, 2, dev)
    R, K = xq.shape
    V = w_scale.shape[0]
    B, G = draft.shape
    if R != B * (G + 1) or x_scale.shape[0] != R:
        raise ValueError(f"xq and x_scale must have B*(G+1) = {B * (G + 1)} rows")
    _need(wq_tiled, "wq_tiled", torch.int8, 4, dev)
    if tuple(wq_tiled.shape) != tiled_shape(V, K):
        raise ValueError(f"wq_tiled must have shape {tiled_shape(V, K)}")
    if logits is not None:
        logits = _out(logits, (R, V), torch.float32, dev, "logits")
    if argmax is not None:
        argmax = _out(argmax, (R,), torch.int32, dev, "argmax")
    accept_len = _out(accept_len, (B,), torch.int32, dev, "accept_len")
    next_token = _out(next_token, (B,), torch.int32, dev, "next_token")
    check(lib().w8a8_lm_head_verify_noalloc(_ptr(xq), _ptr(x_scale), _ptr(wq_tiled), _ptr(w_scale),
                                            V, K, _ptr(draft), B, G, _ptr(logits), _ptr(argmax),
                                            _ptr(accept_len), _ptr(next_token), _stream(dev)))
    return logits, argmax, accept_len, next_token

def lm_head_argmax(xq, x_scale, wq_tiled, w_scale, *, logits=None,
                   workspace: Workspace | None = None, events=None):
    """Phase 1 of :func:`lm_head_verify`: the LM-head linear with the row
    maxima folded into the workspace keys (and the logits written if
    ``logits`` is given).  ``events=(start, stop)``: two timing-enabled
    ``torch.cuda.Event`` objects, each recorded at least once before (torch
    creates the underlying event lazily), that receive the kernel's own start
    and end timestamps (``start.elapsed_time(stop)`` is its duration)."""
    _need(xq, "xq", torch.int8, 2)
    dev = xq.device
    _need(x_scale, "x_scale", torch.float32, 1, dev)
    _need(w_scale, "w_scale", torch.float32, 1, dev)
    M, K = xq.shape
    V = w_scale.shape[0]
    _need(wq_tiled, "wq_tiled", torch.int8, 4, dev)
    if tuple(wq_tiled.shape) != tiled_shape(V, K):
        raise ValueError(f"wq_tiled must have shape {tiled_shape(V, K)}")
    if logits is not None:
        logits = _out(logits, (M, V), torch.float32, dev, "logits")
    ws = (workspace or _default_ws).get(int(lib().w8a8_lm_head_verify_workspace_bytes(M, 0, V, K)),
                                        dev, use="keys")
    if events is not None:
        start, stop = events
        if not (start.cuda_event and stop.cuda_event):
            raise ValueError("record each timing event once before passing it (torch creates "
                             "the underlying event lazily)")
        check(lib().w8a8_lm_head_argmax_timed(_ptr(xq), _ptr(x_scale), _ptr(wq_tiled),
                                              _ptr(w_scale), M, V, K, _ptr(logits), _ptr(ws),
                                              0 if ws is None else ws.numel(), start.cuda_event,
                                              stop.cuda_event, _stream(dev)))
        return logits
    check(lib().w8a8_lm_head_argmax(_ptr(xq), _ptr(x_scale), _ptr(wq_tiled), _ptr(w_scale), M, V,
                                    K, _ptr(logits), _ptr(ws), 0 if ws is None else ws.numel(),
                                    _stream(dev)))
    return logits


def lm_head_argmax_tiled_act(xq_tiled, x_scale, wq_tiled, w_scale, *, K: int, logits=None,
                             workspace: Workspace | None = None):
    """:func:`lm_head_argmax` with the activations in the tiled layout of
    :func:`quantize_act_tiled` (for many rows, e.g. 32 sequences x 9).
    Follow with :func:`accept_from_keys` on the same workspace."""
    _need(xq_tiled, "xq_tiled", torch.int8, 4)
    dev = xq_tiled.device
    _need(x_scale, "x_scale", torch.float32, 1, dev)
    _need(w_scale, "w_scale", torch.float32, 1, dev)
    M = x_scale.shape[0]
    V = w_scale.shape[0]
    if tuple(xq_tiled.shape) != tiled_shape(M, K):
        raise ValueError(f"xq_tiled must have shape {tiled_shape(M, K)}")
    _need(wq_tiled, "wq_tiled", torch.int8, 4, dev)
    if tuple(wq_tiled.shape) != tiled_shape(V, K):
        raise ValueError(f"wq_tiled must have shape {tiled_shape(V, K)}")
    if logits is not None:
        logits = _out(logits, (M, V), torch.float32, dev, "logits")
    ws = (workspace or _default_ws).get(int(lib().w8a8_lm_head_verify_workspace_bytes(M, 0, V, K)),
                                        dev, use="keys")
    check(lib().w8a8_lm_head_argmax_tiled_act(_ptr(xq_tiled), _ptr(x_scale), _ptr(wq_tiled),
                                              _ptr(w_scale), M, V, K, _ptr(logits), _ptr(ws),
                                              0 if ws is None else ws.numel(), _stream(dev)))
    return logits


def accept_from_keys(draft, *, want_argmax=True, argmax=None, accept_len=None, next_token=None,
                     workspace: Workspace | None = None):
    """Phase 2 of :func:`lm_head_verify`: read and reset the keys a preceding
    :func:`lm_head_argmax` left in the same workspace, then accept."""
    _need(draft, "draft", torch.int32, 2)
    dev = draft.device
    B, G = draft.shape
    R = B * (G + 1)
    if want_argmax or argmax is not None:
        argmax = _out(argmax, (R,), torch.int32, dev, "argmax")
    accept_len = _out(accept_len, (B,), torch.int32, dev, "accept_len")
    next_token = _out(next_token, (B,), torch.int32, dev, "next_token")
    ws = (workspace or _default_ws).get(int(lib().w8a8_lm_head_verify_workspace_bytes(R, 0, 1, 0)),
                                        dev, use="keys")
    check(lib().w8a8_accept_from_keys(_ptr(ws), 0 if ws is None else ws.numel(), _ptr(draft), B, G,
                                      _ptr(argmax), _ptr(accept_len), _ptr(next_token),
                                      _stream(dev)))
    return argmax, accept_len, next_token


def bf16_tiled_shape(N: int, K: int) -> tuple:
    """Shape of the tiled bf16 weight layout as a bfloat16 tensor:
    [ceil(N/16), ceil(K/32), 64 lanes, 8 values] (see include/w8a8.h)."""
    return ((N + 15) // 16, (K + 31) // 32, 64, 8)


def tile_weight_bf16(w: torch.Tensor, *, out=None) -> torch.Tensor:
    """Rearrange a row-major bf16 ``w[N][K]`` into the tiled layout of
    :func:`bf16_linear` (shape :func:`bf16_tiled_shape`)."""
    _need(w, "w", torch.bfloat16, 2)
    N, K = w.shape
    out = _out(out, bf16_tiled_shape(N, K), torch.bfloat16, w.device, "out")
    check(lib().w8a8_tile_weight_bf16(_ptr(w), N, K, _ptr(out), _stream(w.device)))
    return out


def bf16_linear(x, w, *, N: int | None = None, want_bf16=True, want_f32=False, y_bf16=None,
                y_f32=None):
    """The bf16 reference linear ``x[M][K] @ w[N][K]^T`` (M <= 16), fp32
    accumulation.  ``w`` is row-major bf16 ``[N][K]`` or the tiled layout
    (4-D, from :func:`tile_weight_bf16`; then ``N`` is required).  Returns
    ``(y_bf16, y_f32)``."""
    _need(x, "x", torch.bfloat16, 2)
    dev = x.device
    M, K = x.shape
    tiled = isinstance(w, torch.Tensor) and w.dim() == 4
    _need(w, "w", torch.bfloat16, 4 if tiled else 2, dev)
    if tiled:
        if N is None:
            raise ValueError("N is required with tiled weights")
        if tuple(w.shape) != bf16_tiled_shape(N, K):
            raise ValueError(f"tiled w must have shape {bf16_tiled_shape(N, K)} (got {tuple(w.shape)})")
    else:
        N, K2 = w.shape
        if K2 != K:
            raise ValueError("x and w must share K")
    if want_bf16 or y_bf16 is not None:
        y_bf16 = _out(y_bf16, (M, N), torch.bfloat16, dev, "y_bf16")
    if want_f32 or y_f32 is not None:
        y_f32 = _out(y_f32, (M, N), torch.float32, dev, "y_f32")
    f = lib().w8a8_bf16_linear_tiled if tiled else lib().w8a8_bf16_linear
    check(f(_ptr(x), _ptr(w), M, N, K, _ptr(y_bf16), _ptr(y_f32), _stream(dev)))
    return y_bf16, y_f32


def _need_bits(t, name, dtypes, ndim, device):
    """A tensor of random words: any of the given dtypes (same bits), on
    ``device``, contiguous, ``ndim`` dimensions."""
    if not isinstance(t, torch.Tensor) or t.dtype not in dtypes:
        raise TypeError(f"{name} must be a tensor of dtype {' or '.join(map(str, dtypes))}")
    if t.device != device:
        raise ValueError(f"{name} must be on {device}")
    if t.dim() != ndim or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous {ndim}-D tensor")


def verify_sample_workspace_bytes(B: int, G: int, V: int) -> int:
    return int(lib().w8a8_verify_sample_workspace_bytes(B, G, V))


def verify_sample(logits, draft, temperature: float, u_accept, u_sample, *, accept_len=None,
                  next_token=None, workspace: Workspace | None = None):
    """Stochastic verification at temperature ``T > 0`` of int32
    ``draft[B][G]`` on fp32 ``logits[B*(G+1)][V]``: each draft is accepted
    with its softmax probability (decided by the uint32 words
    ``u_accept[B][G]``), the next token is drawn from the residual or the
    bonus row (decided by the uint64 words ``u_sample[B]``).  int32/int64
    tensors holding the same bits are accepted for the random words.
    Returns ``(accept_len, next_token)``."""
    _need(logits, "logits", torch.float32, 2)
    dev = logits.device
    _need(draft, "draft", torch.int32, 2, dev)
    B, G = draft.shape
    R, V = logits.shape
    if R != B * (G + 1):
        raise ValueError(f"logits must have B*(G+1) = {B * (G + 1)} rows (got {R})")
    _need_bits(u_accept, "u_accept", (torch.uint32, torch.int32), 2, dev)
    _need_bits(u_sample, "u_sample", (torch.uint64, torch.int64), 1, dev)
    if tuple(u_accept.shape) != (B, G) or tuple(u_sample.shape) != (B,):
        raise ValueError("u_accept must be [B][G] and u_sample [B]")
    accept_len = _out(accept_len, (B,), torch.int32, dev, "accept_len")
    next_token = _out(next_token, (B,), torch.int32, dev, "next_token")
    need = verify_sample_workspace_bytes(B, G, V)
    ws = (workspace or _default_ws).get(need, dev, use="verify")
    check(lib().w8a8_verify_sample(_ptr(logits), V, _ptr(draft), B, G, float(temperature),
                                   _ptr(u_accept), _ptr(u_sample), _ptr(accept_len),
                                   _ptr(next_token), _ptr(ws), 0 if ws is None else ws.numel(),
                                   _stream(dev)))
    return accept_len, next_token


def sample_weights(logits, temperature: float, *, weights=None, workspace: Workspace | None = None):
    """The fixed-point softmax numerators (uint64 bits in an int64 tensor
    ``[R][V]``) that :func:`verify_sample` draws from."""
    _need(logits, "logits", torch.float32, 2)
    dev = logits.device
    R, V = logits.shape
    weights = _out(weights, (R, V), torch.int64, dev, "weights")
    need = int(lib().w8a8_sample_weights_workspace_bytes(R, V))
    ws = (workspace or _default_ws).get(need, dev, use="verify")
    check(lib().w8a8_sample_weights(_ptr(logits), R, V, float(temperature), _ptr(weights),
                                    _ptr(ws), 0 if ws is None else ws.numel(), _stream(dev)))
    return weights


def w4_shape(N: int, K: int) -> tuple:
    """Shape of the int4 tiled weight layout as an int8 tensor: [ceil(N/16),
    ceil(K/128), 64 lanes, 16 bytes] (two int4 codes per byte; see
    include/w8a8.h)."""
    return ((N + 15) // 16, (K + 127) // 128, 64, 16)


def quantize_weight_w4(w: torch.Tensor, smooth: torch.Tensor | None = None, *, wq4=None,
                       w_scale=None):
    """Per-output-channel symmetric int4 quantization of fp32 ``w[N][K]``
    into the int4 tiled layout; returns ``(wq4, w_scale float32[N])``."""
    _need(w, "w", torch.float32, 2)
    N, K = w.shape
    if smooth is not None:
        _need(smooth, "smooth", torch.float32, 1, w.device)
    wq4 = _out(wq4, w4_shape(N, K), torch.int8, w.device, "wq4")
    w_scale = _out(w_scale, (N,), torch.float32, w.device, "w_scale")
    check(lib().w8a8_quantize_weight_w4(_ptr(w), _ptr(smooth), N, K, _ptr(wq4), _ptr(w_scale),
                                        _stream(w.device)))
    return wq4, w_scale


def _need_w4(wq4, w_scale, K, dev):
    _need(w_scale, "w_scale", torch.float32, 1, dev)
    N = w_scale.shape[0]
    _need(wq4, "wq4", torch.int8, 4, dev)
    if tuple(wq4.shape) != w4_shape(N, K):
        raise ValueError(f"wq4 must have shape {w4_shape(N, K)} (got {tuple(wq4.shape)})")
    return N


def linear_w4(xq, x_scale, wq4, w_scale, *, want_bf16=True, want_f32=False, want_acc=False,
              y_bf16=None, y_f32=None, acc=None):
    """The W4A8 linear (int4 tiled weights); outputs as :func:`linear`."""
    _need(xq, "xq", torch.int8, 2)
    dev = xq.device
    _need(x_scale, "x_scale", torch.float32, 1, dev)
    M, K = xq.shape
    N = _need_w4(wq4, w_scale, K, dev)
    if want_bf16 or y_bf16 is not None:
        y_bf16 = _out(y_bf16, (M, N), torch.bfloat16, dev, "y_bf16")
    if want_f32 or y_f32 is not None:
        y_f32 = _out(y_f32, (M, N), torch.float32, dev, "y_f32")
    if want_acc or acc is not None:
        acc = _out(acc, (M, N), torch.int32, dev, "acc")
    check(lib().w8a8_linear_w4(_ptr(xq), _ptr(x_scale), _ptr(wq4), _ptr(w_scale), M, N, K,
                               _ptr(y_bf16), _ptr(y_f32), _ptr(acc), _stream(dev)))
    return y_bf16, y_f32, acc


def lm_head_argmax_w4(xq, x_scale, wq4, w_scale, *, logits=None,
                      workspace: Workspace | None = None):
    """:func:`lm_head_argmax` with int4 weights; follow with
    :func:`accept_from_keys` on the same workspace."""
    _need(xq, "xq", torch.int8, 2)
    dev = xq.device
    _need(x_scale, "x_scale", torch.float32, 1, dev)
    M, K = xq.shape
    V = _need_w4(wq4, w_scale, K, dev)
    if logits is not None:
        logits = _out(logits, (M, V), torch.float32, dev, "logits")
    ws = (workspace or _default_ws).get(int(lib().w8a8_lm_head_verify_workspace_bytes(M, 0, V, K)),
                                        dev, use="keys")
    check(lib().w8a8_lm_head_argmax_w4(_ptr(xq), _ptr(x_scale), _ptr(wq4), _ptr(w_scale), M, V, K,
                                       _ptr(logits), _ptr(ws), 0 if ws is None else ws.numel(),
                                       _stream(dev)))
    return logits


def residual_rmsnorm_quant(h, gamma, eps: float, *, delta=None, smooth=None, h_out=None,
                           want_normed=False, normed=None, xq=None, x_scale=None):
    """Residual add (when ``delta`` is given; the sum goes to ``h_out``, which
    may be ``h``), RMSNorm with bf16 ``gamma[D]``, then the per-token int8
    quantization of the normed row.  ``h``, ``delta``: bf16 ``[M][D]``.
    Returns ``(xq, x_scale, normed or None, h_out or None)``."""
    _need(h, "h", torch.bfloat16, 2)
    dev = h.device
    M, D = h.shape
    _need(gamma, "gamma", torch.bfloat16, 1, dev)
    if gamma.shape[0] != D:
        raise ValueError("gamma must have length D")
    if delta is not None:
        _need(delta, "delta", torch.bfloat16, 2, dev)
        if tuple(delta.shape) != (M, D):
            raise ValueError("delta must have h's shape")
        h_out = _out(h_out, (M, D), torch.bfloat16, dev, "h_out")
    elif h_out is not None:
        raise ValueError("h_out is written only with delta")
    if smooth is not None:
        _need(smooth, "smooth", torch.float32, 1, dev)
    if want_normed or normed is not None:
        normed = _out(normed, (M, D), torch.bfloat16, dev, "normed")
    xq = _out(xq, (M, D), torch.int8, dev, "xq")
    x_scale = _out(x_scale, (M,), torch.float32, dev, "x_scale")
    check(lib().w8a8_residual_rmsnorm_quant(_ptr(h), _ptr(delta), _ptr(gamma), float(eps),
                                            _ptr(smooth), M, D, _ptr(h_out), _ptr(normed),
                                            _ptr(xq), _ptr(x_scale), _stream(dev)))
    return xq, x_scale, normed, h_out


def silu_mul_quant(gate, up, *, smooth=None, want_act=False, act=None, xq=None, x_scale=None):
    """SwiGLU product ``bf16(bf16(silu(gate)) * up)`` then the per-token int8
    quantization.  ``gate`` and ``up`` are bf16 ``[M][F]`` views with the same
    row stride (e.g. the two column halves of a fused [gate;up] output).
    Returns ``(xq, x_scale, act or None)``."""
    for t, n in ((gate, "gate"), (up, "up")):
        if not isinstance(t, torch.Tensor) or t.dtype != torch.bfloat16 or t.dim() != 2:
            raise TypeError(f"{n} must be a 2-D bfloat16 tensor")
        if t.device.type != "cuda":
            raise TypeError(f"{n} must be on a ROCm device; there is no CPU path")
        if t.stride(1) != 1:
            raise ValueError(f"{n} rows must be contiguous")
    if gate.shape != up.shape or gate.stride(0) != up.stride(0) or gate.device != up.device:
        raise ValueError("gate and up must have the same shape, row stride and device")
    dev = gate.device
    M, F = gate.shape
    if smooth is not None:
        _need(smooth, "smooth", torch.float32, 1, dev)
    if want_act or act is not None:
        act = _out(act, (M, F), torch.bfloat16, dev, "act")
    xq = _out(xq, (M, F), torch.int8, dev, "xq")
    x_scale = _out(x_scale, (M,), torch.float32, dev, "x_scale")
    check(lib().w8a8_silu_mul_quant(_ptr(gate), _ptr(up), gate.stride(0), _ptr(smooth), M, F,
                                    _ptr(act), _ptr(xq), _ptr(x_scale), _stream(dev)))
    return xq, x_scale, act


def quantize_act_tiled(x: torch.Tensor, smooth: torch.Tensor | None = None, *, xq_tiled=None,
                       x_scale=None):
    """:func:`quantize_act` with the codes written in the tiled layout (token
    rows in place of channels, shape ``tiled_shape(M, K)``), for
    :func:`linear_tiled_act`.  Returns ``(xq_tiled, x_scale float32[M])``."""
    _need(x, "x", torch.bfloat16, 2)
    M, K = x.shape
    if smooth is not None:
        _need(smooth, "smooth", torch.float32, 1, x.device)
    xq_tiled = _out(xq_tiled, tiled_shape(M, K), torch.int8, x.device, "xq_tiled")
    x_scale = _out(x_scale, (M,), torch.float32, x.device, "x_scale")
    check(lib().w8a8_quantize_act_tiled(_ptr(x), _ptr(smooth), M, K, _ptr(xq_tiled),
                                        _ptr(x_scale), _stream(x.device)))
    return xq_tiled, x_scale


def linear_tiled_act(xq_tiled, x_scale, wq_tiled, w_scale, *, K: int | None = None,
                     want_bf16=True, want_f32=False, want_acc=False, y_bf16=None, y_f32=None,
                     acc=None, workspace: Workspace | None = None):
    """The batched W8A8 linear with tiled activations (from
    :func:`quantize_act_tiled`) and tiled weights; same outputs as
    :func:`linear`.  ``K`` defaults to the padded width of the layout (the
    result is the same for any K with the same 64-wide step count).  Long
    reductions on mid-size grids split k across workgroups through the
    ``"zeroed"`` workspace (see :func:`linear_tiled_act_workspace_bytes`)."""
    _need(xq_tiled, "xq_tiled", torch.int8, 4)
    dev = xq_tiled.device
    _need(x_scale, "x_scale", torch.float32, 1, dev)
    _need(w_scale, "w_scale", torch.float32, 1, dev)
    _need(wq_tiled, "wq_tiled", torch.int8, 4, dev)
    M, N = x_scale.shape[0], w_scale.shape[0]
    if K is None:
        K = xq_tiled.shape[1] * 64
    if tuple(xq_tiled.shape) != tiled_shape(M, K) or tuple(wq_tiled.shape) != tiled_shape(N, K):
        raise ValueError("xq_tiled / wq_tiled shapes do not match M, N, K")
    if want_bf16 or y_bf16 is not None:
        y_bf16 = _out(y_bf16, (M, N), torch.bfloat16, dev, "y_bf16")
    if want_f32 or y_f32 is not None:
        y_f32 = _out(y_f32, (M, N), torch.float32, dev, "y_f32")
    if want_acc or acc is not None:
        acc = _out(acc, (M, N), torch.int32, dev, "acc")
    need = linear_tiled_act_workspace_bytes(M, N, K)
    ws = (workspace or _default_ws).get(need, dev, use="zeroed")
    check(lib().w8a8_linear_tiled_act(_ptr(xq_tiled), _ptr(x_scale), _ptr(wq_tiled),
                                      _ptr(w_scale), M, N, K, _ptr(y_bf16), _ptr(y_f32),
                                      _ptr(acc), _ptr(ws), 0 if ws is None else ws.numel(),
                                      _stream(dev)))
    return y_bf16, y_f32, acc


def linear_tiled_act_workspace_bytes(M: int, N: int, K: int) -> int:
    """Bytes of the ``"zeroed"`` workspace :func:`linear_tiled_act` needs
    (0 when the reduction is not split across workgroups)."""
    return int(lib().w8a8_linear_tiled_act_workspace_bytes(M, N, K))


def pack_v_cache(v, *, out=None):
    """A row-major V cache bf16 ``[B][Hkv][Lmax][128]`` in the blocked layout
    that ``verify_attention`` reads (same shape and dtype, values permuted
    within each 16-position block)."""
    _need(v, "v", torch.bfloat16, 4)
    B, Hkv, Lmax, Dh = v.shape
    out = _out(out, (B, Hkv, Lmax, Dh), torch.bfloat16, v.device, "out")
    check(lib().w8a8_pack_v_cache(_ptr(v), B, Hkv, Lmax, Dh, _ptr(out), _stream(v.device)))
    return out


def verify_attention(q, k_cache, v_cache, lengths, *, out=None, workspace: Workspace | None = None):
    """Causal grouped-query attention of the verified block: ``q`` bf16
    ``[B][T][Hq][128]``, ``k_cache`` bf16 ``[B][Hkv][Lmax][128]``,
    ``v_cache`` bf16 of the same shape in the blocked layout (see
    ``pack_v_cache``), ``lengths`` int32 ``[B]`` (valid cache positions, the
    block's own T included).  Returns ``out`` bf16 ``[B][T][Hq][128]``."""
    _need(q, "q", torch.bfloat16, 4)
    dev = q.device
    _need(k_cache, "k_cache", torch.bfloat16, 4, dev)
    _need(v_cache, "v_cache", torch.bfloat16, 4, dev)
    _need(lengths, "lengths", torch.int32, 1, dev)
    B, T, Hq, Dh = q.shape
    _, Hkv, Lmax, _ = k_cache.shape
    if tuple(k_cache.shape) != (B, Hkv, Lmax, Dh) or v_cache.shape != k_cache.shape:
        raise ValueError("k_cache and v_cache must be [B][Hkv][Lmax][Dh]")
    if lengths.shape[0] != B:
        raise ValueError("lengths must have B entries")
    out = _out(out, (B, T, Hq, Dh), torch.bfloat16, dev, "out")
    need = int(lib().w8a8_verify_attention_workspace_bytes(B, Hkv, Lmax))
    ws = (workspace or _default_ws).get(need, dev, use="verify")
    check(lib().w8a8_verify_attention(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(lengths), B, T,
                                      Hq, Hkv, Dh, Lmax, _ptr(out), _ptr(ws),
                                      0 if ws is None else ws.numel(), _stream(dev)))
    return out


def qk_norm_rope_append(qkv, q_gamma, k_gamma, lengths, k_cache, v_cache, *, T: int, Hq: int,
                        Hkv: int, eps: float = 1e-6, rope_base: float = 1e6, q_out=None):
    """Per-head q/k RMSNorm, rotary embedding at position L_b - T + i, and the
    append of k, v into the caches (v in the blocked layout).  ``qkv`` bf16 ``[B*T][(Hq + 2 Hkv) * 128]``
    (e.g. a fused [q;k;v] linear's output), ``lengths`` int32 ``[B]`` (valid
    positions after the append).  Returns ``q_out`` bf16 ``[B][T][Hq][128]``."""
    _need(qkv, "qkv", torch.bfloat16, 2)
    dev = qkv.device
    R, W = qkv.shape
    if W != (Hq + 2 * Hkv) * 128 or R % T != 0:
        raise ValueError("qkv must be [B*T][(Hq + 2*Hkv) * 128]")
    B = R // T
    _need(q_gamma, "q_gamma", torch.bfloat16, 1, dev)
    _need(k_gamma, "k_gamma", torch.bfloat16, 1, dev)
    _need(lengths, "lengths", torch.int32, 1, dev)
    _need(k_cache, "k_cache", torch.bfloat16, 4, dev)
    _need(v_cache, "v_cache", torch.bfloat16, 4, dev)
    Lmax = k_cache.shape[2]
    if tuple(k_cache.shape) != (B, Hkv, Lmax, 128) or v_cache.shape != k_cache.shape:
        raise ValueError("caches must be [B][Hkv][Lmax][128]")
    q_out = _out(q_out, (B, T, Hq, 128), torch.bfloat16, dev, "q_out")
    check(lib().w8a8_qk_norm_rope_append(_ptr(qkv), B, T, Hq, Hkv, 128, _ptr(q_gamma),
                                         _ptr(k_gamma), float(eps), float(rope_base),
                                         _ptr(lengths), Lmax, _ptr(q_out), _ptr(k_cache),
                                         _ptr(v_cache), _stream(dev)))
    return q_out


def hbm_read_probe(buf: torch.Tensor, *, sink=None, events=None) -> torch.Tensor:
    """Read every byte of the contiguous device tensor ``buf`` once with the
    library's streaming-read probe (a measurement of the sustained read
    bandwidth).  ``sink``: int32 ``[HBM_PROBE_SINK_WORDS]`` scratch output.
    ``events=(start, stop)`` as for :func:`lm_head_argmax` (the kernel's own
    timestamps).  Returns ``sink``."""
    if not isinstance(buf, torch.Tensor) or buf.device.type != "cuda":
        raise TypeError("buf must be a torch.Tensor on a ROCm device; there is no CPU path")
    if not buf.is_contiguous():
        raise ValueError("buf must be contiguous")
    nbytes = buf.numel() * buf.element_size()
    sink = _out(sink, (HBM_PROBE_SINK_WORDS,), torch.int32, buf.device, "sink")
    ev0 = ev1 = None
    if events is not None:
        start, stop = events
        if not (start.cuda_event and stop.cuda_event):
            raise ValueError("record each timing event once before passing it (torch creates "
                             "the underlying event lazily)")
        ev0, ev1 = start.cuda_event, stop.cuda_event
    check(lib().w8a8_hbm_read_probe(_ptr(buf), nbytes, _ptr(sink), ev0, ev1, _stream(buf.device)))
    return sink

