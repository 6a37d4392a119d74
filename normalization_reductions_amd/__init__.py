"""normalization_reductions_amd -- per-slice normalization on AMD MI355X (gfx950).

A thin binding over libnormred.so. Functions take torch tensors only as device memory: the
binding reads shapes and pointers, allocates outputs and workspaces with torch, and calls the
C ABI on torch's current stream. Every step of the computation runs in the library's HIP
kernels; there is no fallback path, and a missing library or a non-GPU tensor raises.

Entry points (names as in include/normred.h):
  inorm_forward(x, ...)               instance norm over the spatial extent of x[N, C, ...]
  bn_train_forward(x, ...)            training-mode batch norm (batch statistics), then a scale
  conv_norm_epilogue_forward(x, w, b, ...)  k=3 conv -> normalize -> fused epilogue
"""
from __future__ import annotations

import ctypes
import math

from . import _lib
from ._lib import (NR_NORM_BATCH_TRAIN, NR_NORM_INSTANCE, NR_VARIANT_AUTO, NR_VARIANT_RESIDENT,
                   NR_VARIANT_SPLIT, NormredError, check)

__all__ = [
    "inorm_forward", "bn_train_forward", "conv_norm_epilogue_forward", "conv_bn_eval_forward",
    "inorm_workspace_size",
    "bn_train_workspace_size", "conv_norm_epilogue_workspace_size", "workspace_clear",
    "workspace_check", "stream_copy", "version", "NormredError", "NR_VARIANT_AUTO",
    "NR_VARIANT_RESIDENT", "NR_VARIANT_SPLIT", "NR_NORM_BATCH_TRAIN", "NR_NORM_INSTANCE",
]


def _torch():
    import torch

    return torch


def version() -> str:
    return _lib.load().nr_version().decode()


def _dev_f32(t, name):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.device.type != "cuda":
        raise ValueError("%s must be in GPU memory (got %s)" % (name, t.device))
    if t.dtype != torch.float32:
        raise TypeError("%s must be float32 (got %s)" % (name, t.dtype))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    return t


def _opt_ptr(t, name, numel=None, device=None):
    if t is None:
        return None
    _dev_f32(t, name)
    if numel is not None and t.numel() != numel:
        raise ValueError("%s must have %d elements (got %d)" % (name, numel, t.numel()))
    if device is not None and t.device != device:
        raise ValueError("%s is on %s, expected %s" % (name, t.device, device))
    return t.data_ptr()


def _stream(device, stream=None):
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream(device)
    return ctypes.c_void_p(s.cuda_stream)


# ---------------------------------------------------------------------------------------------
# Workspaces: one zero-filled buffer per (device, stream), grown on demand. The library leaves
# a workspace valid after each call, so it is zero-filled only when (re)allocated.
# ---------------------------------------------------------------------------------------------
_ws_cache: dict = {}


def get_workspace(nbytes: int, device, stream=None):
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream(device)
    key = (str(device), s.cuda_stream)
    buf = _ws_cache.get(key)
    if buf is None or buf.numel() < nbytes:
        buf = torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)
        workspace_clear(buf, stream=s)
        _ws_cache[key] = buf
    return buf


def workspace_clear(ws, stream=None):
    lib = _lib.load()
    check(lib.nr_workspace_clear(ctypes.c_void_p(ws.data_ptr()), ws.numel() * ws.element_size(),
                                 _stream(ws.device, stream)), "nr_workspace_clear")


def workspace_check(ws, stream=None) -> int:
    """Synchronizes, returns and clears the workspace's sticky error flags (0 = healthy)."""
    lib = _lib.load()
    flags = ctypes.c_uint32(0)
    check(lib.nr_workspace_check(ctypes.c_void_p(ws.data_ptr()), ws.numel() * ws.element_size(),
                                 _stream(ws.device, stream), ctypes.byref(flags)),
          "nr_workspace_check")
    return int(flags.value)


def _nc_s(x):
    if x.dim() < 2:
        raise ValueError("x must have at least 2 dimensions [N, C, ...]")
    N, C = int(x.shape[0]), int(x.shape[1])
    S = int(math.prod(x.shape[2:])) if x.dim() > 2 else 1
    return N, C, S


# ---------------------------------------------------------------------------------------------
# Instance norm
# ---------------------------------------------------------------------------------------------
def inorm_workspace_size(N: int, C: int, S: int) -> int:
    return int(_lib.load().inorm_workspace_size(N, C, S))


def inorm_forward(x, y=None, *, eps: float = 1e-5, gamma=None, beta=None, save_mean=None,
                  save_invstd=None, workspace=None, variant: int = NR_VARIANT_AUTO, stream=None):
    """Instance norm of x[N, C, *spatial] over the spatial extent (see normred.h). Returns y
    (allocated if not given; pass y=x for in place)."""
    lib = _lib.load()
    torch = _torch()
    _dev_f32(x, "x")
    N, C, S = _nc_s(x)
    if y is None:
        y = torch.empty_like(x)
    _dev_f32(y, "y")
    if y.shape != x.shape or y.device != x.device:
        raise ValueError("y must match x in shape and device")
    g = _opt_ptr(gamma, "gamma", C, x.device)
    b = _opt_ptr(beta, "beta", C, x.device)
    sm = _opt_ptr(save_mean, "save_mean", N * C, x.device)
    si = _opt_ptr(save_invstd, "save_invstd", N * C, x.device)
    need = inorm_workspace_size(N, C, S)
    ws = workspace if workspace is not None else get_workspace(need, x.device, stream)
    check(lib.inorm_forward_ex(x.data_ptr(), y.data_ptr(), N, C, S, float(eps), g, b, sm, si,
                               ctypes.c_void_p(ws.data_ptr()), ws.numel() * ws.element_size(),
                               int(variant), _stream(x.device, stream)), "inorm_forward")
    return y


def inorm_forward_noalloc(x, y, *, eps: float = 1e-5, gamma=None, beta=None, save_mean=None,
                          save_invstd=None, stream=None):
    """inorm_forward with the library's own 8 MiB device workspace: the call allocates nothing
    (y must be given). Calls that overlap on one GPU race (see normred.h)."""
    lib = _lib.load()
    _dev_f32(x, "x")
    N, C, S = _nc_s(x)
    _dev_f32(y, "y")
    if y.shape != x.shape or y.device != x.device:
        raise ValueError("y must match x in shape and device")
    g = _opt_ptr(gamma, "gamma", C, x.device)
    b = _opt_ptr(beta, "beta", C, x.device)
    sm = _opt_ptr(save_mean, "save_mean", N * C, x.device)
    si = _opt_ptr(save_invstd, "save_invstd", N * C, x.device)
    check(lib.inorm_forward_noalloc(x.data_ptr(), y.data_ptr(), N, C, S, float(eps), g, b, sm, si,
                                    _stream(x.device, stream)), "inorm_forward_noalloc")
    return y


# ---------------------------------------------------------------------------------------------
# Batch norm (training mode)
# ---------------------------------------------------------------------------------------------
def bn_train_workspace_size(N: int, C: int, S: int) -> int:
    return int(_lib.load().bn_train_workspace_size(N, C, S))


def bn_train_forward(x, y=None, *, eps: float = 1e-5, gamma=None, beta=None,
                     out_scale: float = 1.0, save_mean=None, save_invstd=None, running_mean=None,
                     running_var=None, momentum: float = 0.1, workspace=None, stream=None):
    """Training-mode batch norm of x[N, C, *spatial] with batch statistics, then * out_scale;
    running_mean / running_var ([C], both or neither) are updated in place with `momentum`."""
    lib = _lib.load()
    torch = _torch()
    _dev_f32(x, "x")
    N, C, S = _nc_s(x)
    if y is None:
        y = torch.empty_like(x)
    _dev_f32(y, "y")
    if y.shape != x.shape or y.device != x.device:
        raise ValueError("y must match x in shape and device")
    g = _opt_ptr(gamma, "gamma", C, x.device)
    b = _opt_ptr(beta, "beta", C, x.device)
    sm = _opt_ptr(save_mean, "save_mean", C, x.device)
    si = _opt_ptr(save_invstd, "save_invstd", C, x.device)
    rm = _opt_ptr(running_mean, "running_mean", C, x.device)
    rv = _opt_ptr(running_var, "running_var", C, x.device)
    need = bn_train_workspace_size(N, C, S)
    ws = workspace if workspace is not None else get_workspace(need, x.device, stream)
    check(lib.bn_train_forward_ex(x.data_ptr(), y.data_ptr(), N, C, S, float(eps), g, b,
                                  float(out_scale), sm, si, float(momentum), rm, rv,
                                  ctypes.c_void_p(ws.data_ptr()), ws.numel() * ws.element_size(),
                                  _stream(x.device, stream)),
          "bn_train_forward")
    return y


# ---------------------------------------------------------------------------------------------
# Conv -> normalize -> epilogue
# ---------------------------------------------------------------------------------------------
def _desc(x, w, *, norm, eps, pre_mul, gamma, beta, out_scale, clamp, post_mul, reduce_max_c,
          running_mean=None, running_var=None, momentum=0.1, channels_last=False):
    dims = x.dim() - 2
    if dims not in (2, 3):
        raise ValueError("x must be [N, C, H, W] or [N, C, D, H, W] (channels last: "
                         "[N, H, W, C] or [N, D, H, W, C])")
    cin = int(x.shape[-1]) if channels_last else int(x.shape[1])
    if w.dim() != x.dim() or int(w.shape[1]) != cin:
        raise ValueError("w must be [C_out, C_in, 3, ...] matching x")
    d = _lib.ConvNormDesc()
    d.spatial_dims = dims
    d.ksize = int(w.shape[-1])
    d.N, d.C_in, d.C_out = int(x.shape[0]), cin, int(w.shape[0])
    d.channels_last = 1 if channels_last else 0
    sp = [int(s) for s in (x.shape[1:-1] if channels_last else x.shape[2:])]
    d.in_d, d.in_h, d.in_w = (sp[0], sp[1], sp[2]) if dims == 3 else (1, sp[0], sp[1])
    d.norm = norm
    d.eps = float(eps)
    cout = int(w.shape[0])
    d.pre_mul = _opt_ptr(pre_mul, "pre_mul", cout, x.device)
    d.gamma = _opt_ptr(gamma, "gamma", cout, x.device)
    d.beta = _opt_ptr(beta, "beta", cout, x.device)
    d.out_scale = float(out_scale)
    d.clamp = 0 if clamp is None else 1
    d.clamp_lo, d.clamp_hi = (0.0, 0.0) if clamp is None else (float(clamp[0]), float(clamp[1]))
    d.post_mul = _opt_ptr(post_mul, "post_mul", cout, x.device)
    d.reduce_max_c = 1 if reduce_max_c else 0
    d.momentum = float(momentum)
    d.running_mean = _opt_ptr(running_mean, "running_mean", cout, x.device)
    d.running_var = _opt_ptr(running_var, "running_var", cout, x.device)
    osp = tuple(s - 2 for s in sp)
    if reduce_max_c:
        oshape = (d.N,) + osp
    else:
        oshape = (d.N,) + osp + (cout,) if channels_last else (d.N, cout) + osp
    return d, oshape


def conv_norm_epilogue_workspace_size(desc) -> int:
    return int(_lib.load().conv_norm_epilogue_workspace_size(ctypes.byref(desc)))


def conv_norm_epilogue_forward(x, w, b=None, out=None, *, norm=NR_NORM_BATCH_TRAIN, eps=1e-5,
                               pre_mul=None, gamma=None, beta=None, out_scale=1.0, clamp=None,
                               post_mul=None, reduce_max_c=False, running_mean=None,
                               running_var=None, momentum=0.1, channels_last=False,
                               workspace=None, stream=None):
    """k=3 valid conv (+bias) -> pre_mul -> batch/instance norm -> gamma, beta -> out_scale ->
    clamp -> post_mul -> optional max over channels (see normred.h). channels_last: x is
    [N, (D,) H, W, C_in] and the output [N, (D-2,) H-2, W-2, C_out] (or the channel max)."""
    lib = _lib.load()
    torch = _torch()
    _dev_f32(x, "x")
    _dev_f32(w, "w")
    d, oshape = _desc(x, w, norm=norm, eps=eps, pre_mul=pre_mul, gamma=gamma, beta=beta,
                      out_scale=out_scale, clamp=clamp, post_mul=post_mul,
                      reduce_max_c=reduce_max_c, running_mean=running_mean,
                      running_var=running_var, momentum=momentum, channels_last=channels_last)
    bp = _opt_ptr(b, "b", d.C_out, x.device)
    if out is None:
        out = torch.empty(oshape, dtype=torch.float32, device=x.device)
    _dev_f32(out, "out")
    if tuple(out.shape) != tuple(oshape):
        raise ValueError("out must have shape %s" % (oshape,))
    need = conv_norm_epilogue_workspace_size(d)
    if need == 0:
        # no workspace (an empty batch) -- or a descriptor the size query rejects, which this
        # call then reports
        check(lib.conv_norm_epilogue_forward(ctypes.byref(d), x.data_ptr(), w.data_ptr(), bp,
                                             out.data_ptr(), None, 0, _stream(x.device, stream)),
              "conv_norm_epilogue_forward")
        return out
    ws = workspace if workspace is not None else get_workspace(need, x.device, stream)
    check(lib.conv_norm_epilogue_forward(ctypes.byref(d), x.data_ptr(), w.data_ptr(), bp,
                                         out.data_ptr(), ctypes.c_void_p(ws.data_ptr()),
                                         ws.numel() * ws.element_size(),
                                         _stream(x.device, stream)),
          "conv_norm_epilogue_forward")
    return out


def conv_bn_eval_forward(x, w, b, running_mean, running_var, out=None, *, eps=1e-5, gamma=None,
                         beta=None, out_scale=1.0, channels_last=False, workspace=None,
                         stream=None):
    """k=3 valid conv (+bias) -> eval-mode batch norm with running statistics -> * out_scale,
    folded into the conv weights (see normred.h)."""
    lib = _lib.load()
    torch = _torch()
    _dev_f32(x, "x")
    _dev_f32(w, "w")
    d, oshape = _desc(x, w, norm=NR_NORM_BATCH_TRAIN, eps=eps, pre_mul=None, gamma=gamma, beta=beta,
                      out_scale=out_scale, clamp=None, post_mul=None, reduce_max_c=False,
                      channels_last=channels_last)
    bp = _opt_ptr(b, "b", d.C_out, x.device)
    rm = _opt_ptr(running_mean, "running_mean", d.C_out, x.device)
    rv = _opt_ptr(running_var, "running_var", d.C_out, x.device)
    if out is None:
        out = torch.empty(oshape, dtype=torch.float32, device=x.device)
    _dev_f32(out, "out")
    if tuple(out.shape) != tuple(oshape):
        raise ValueError("out must have shape %s" % (oshape,))
    need = int(lib.conv_bn_eval_workspace_size(ctypes.byref(d)))
    ws = workspace if workspace is not None else get_workspace(max(need, 256), x.device, stream)
    check(lib.conv_bn_eval_forward(ctypes.byref(d), x.data_ptr(), w.data_ptr(), bp, rm, rv,
                                   out.data_ptr(), ctypes.c_void_p(ws.data_ptr()),
                                   ws.numel() * ws.element_size(), _stream(x.device, stream)),
          "conv_bn_eval_forward")
    return out


def stream_copy(src, dst, stream=None, workspace=None):
    """dst <- src with the library's streaming copy; with a workspace (>= 256 bytes), the
    persistent copy that takes its units from a counter there."""
    lib = _lib.load()
    _dev_f32(src, "src")
    _dev_f32(dst, "dst")
    if src.numel() != dst.numel():
        raise ValueError("src and dst sizes differ")
    if workspace is None:
        check(lib.nr_stream_copy(src.data_ptr(), dst.data_ptr(), src.numel(),
                                 _stream(src.device, stream)), "nr_stream_copy")
    else:
        check(lib.nr_stream_copy_ws(src.data_ptr(), dst.data_ptr(), src.numel(),
                                    ctypes.c_void_p(workspace.data_ptr()),
                                    workspace.numel() * workspace.element_size(),
                                    _stream(src.device, stream)), "nr_stream_copy_ws")
    return dst
