"""fp64 CPU oracle for the per-slice normalization path -- TEST INFRASTRUCTURE.

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may
import this package. The HIP library and its Python binding never import it, and it imports
nothing from them.

The arithmetic lives in ``oracle.c`` (plain C, fp64, sequential sums, two-pass variance).
This module only marshals numpy arrays into it. Each wrapper names the page passage its C
function follows; the pages are the "Kimi-K2.6" kernel-task traces:

* IN2d page: task l1_p34, InstanceNorm2d on x[112,64,512,512];
* BN page:   task l2_p73, Conv2d(8->64,k=3) -> BatchNorm2d -> x2.0;
* IN3d page: task l2_p79, Conv3d(3->16,k=3) -> xmultiplier -> InstanceNorm3d -> clamp ->
  xmultiplier -> max over channels.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
# NORMRED_ORACLE_LIB selects another build of oracle.c (the host-sanitizer test's)
_LIB = os.environ.get("NORMRED_ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")

_lib = None


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so with gcc (no fast-math: fp64 stays IEEE)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.run(
            ["gcc", "-O2", "-std=c11", "-Wall", "-fPIC", "-shared", "-pthread",
             "-o", tmp, _SRC, "-lm"],
            check=True,
        )
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB):
        build(force=True)
    lib = ctypes.CDLL(_LIB)
    i64, dbl, vp, ci = ctypes.c_int64, ctypes.c_double, ctypes.c_void_p, ctypes.c_int
    lib.or_default_threads.restype = ci
    lib.or_instance_norm.argtypes = [vp, vp, i64, i64, i64, dbl, vp, vp, vp, vp, ci]
    lib.or_instance_norm.restype = ci
    lib.or_conv_k3.argtypes = [vp, vp, vp, vp, ci, i64, i64, i64, i64, i64, i64, ci]
    lib.or_conv_k3.restype = ci
    lib.or_batch_norm_train.argtypes = [vp, vp, i64, i64, i64, dbl, vp, vp, dbl, vp, vp, ci]
    lib.or_batch_norm_train.restype = ci
    lib.or_conv_bn_eval.argtypes = [vp, vp, vp, vp, vp, vp, vp, dbl, dbl, vp, ci, i64, i64, i64,
                                    i64, i64, i64, ci]
    lib.or_conv_bn_eval.restype = ci
    lib.or_bn_running_update.argtypes = [vp, vp, i64, i64, dbl, vp, vp]
    lib.or_bn_running_update.restype = ci
    lib.or_conv_norm_epilogue.argtypes = [
        vp, vp, vp, vp, ci, i64, i64, i64, i64, i64, i64,
        ci, dbl, vp, vp, vp, dbl, ci, dbl, dbl, vp, ci, vp, vp, ci]
    lib.or_conv_norm_epilogue.restype = ci
    _lib = lib
    return lib


def _ptr(a):
    return None if a is None else a.ctypes.data


def _f32(a):
    return None if a is None else np.ascontiguousarray(a, dtype=np.float32)


def default_threads() -> int:
    return int(_load().or_default_threads())


def instance_norm(x, eps=1e-5, gamma=None, beta=None, nthreads=0, with_stats=False):
    """Instance norm of x[N, C, *spatial] (IN2d page, statement of the op; IN3d page, its
    InstanceNorm3d reading): per (n, c) mean and biased variance over the spatial extent,
    y = (x - mean)/sqrt(var + eps) (* gamma[c] + beta[c] when given). Returns fp32 y, and
    with ``with_stats`` also the fp64 per-slice mean and variance, shaped [N, C]."""
    x = _f32(x)
    N, C = x.shape[0], x.shape[1]
    S = int(np.prod(x.shape[2:])) if x.ndim > 2 else 1
    y = np.empty_like(x)
    mean = np.empty((N, C), np.float64)
    var = np.empty((N, C), np.float64)
    g, b = _f32(gamma), _f32(beta)
    rc = _load().or_instance_norm(_ptr(x), _ptr(y), N * C, C, S, float(eps), _ptr(g), _ptr(b),
                                  _ptr(mean), _ptr(var), int(nthreads))
    if rc != 0:
        raise ValueError("or_instance_norm rejected its arguments")
    return (y, mean, var) if with_stats else y


def instance_norm_slices(slices, eps=1e-5, nthreads=0, with_stats=False):
    """Instance norm of independent slices given as a 2-D array [count, S] (no affine)."""
    s = _f32(slices)
    y = np.empty_like(s)
    mean = np.empty(s.shape[0], np.float64)
    var = np.empty(s.shape[0], np.float64)
    rc = _load().or_instance_norm(_ptr(s), _ptr(y), s.shape[0], 1, s.shape[1], float(eps), None,
                                  None, _ptr(mean), _ptr(var), int(nthreads))
    if rc != 0:
        raise ValueError("or_instance_norm rejected its arguments")
    return (y, mean, var) if with_stats else y


def conv_k3(x, w, b=None, nthreads=0):
    """Valid, stride-1, k=3 cross-correlation with bias, in fp64 (BN page, its direct-conv
    indexing; IN3d page, output extent = input - 2). x: [N, Cin, (D,) H, W]."""
    x, w, b = _f32(x), _f32(w), _f32(b)
    dims = x.ndim - 2
    N, Cin = x.shape[0], x.shape[1]
    Cout = w.shape[0]
    if dims == 2:
        D, (H, W) = 1, x.shape[2:]
        oshape = (N, Cout, H - 2, W - 2)
    elif dims == 3:
        D, H, W = x.shape[2:]
        oshape = (N, Cout, D - 2, H - 2, W - 2)
    else:
        raise ValueError("conv_k3 takes a 4-D or 5-D input")
    out = np.empty(oshape, np.float64)
    rc = _load().or_conv_k3(_ptr(x), _ptr(w), _ptr(b), _ptr(out), dims, N, Cin, Cout, D, H, W,
                            int(nthreads))
    if rc != 0:
        raise ValueError("or_conv_k3 rejected its arguments")
    return out


def batch_norm_train(x, eps=1e-5, gamma=None, beta=None, scale=1.0, nthreads=0, with_stats=False):
    """Training-mode batch norm (BN page, opening analysis): per channel mean and biased
    variance over (N, spatial), y = ((x - mean)/sqrt(var+eps)*gamma + beta)*scale. x is used
    in fp64 (a float32 input is widened exactly)."""
    x64 = np.ascontiguousarray(x, dtype=np.float64)
    N, C = x64.shape[0], x64.shape[1]
    S = int(np.prod(x64.shape[2:])) if x64.ndim > 2 else 1
    y = np.empty(x64.shape, np.float32)
    mean = np.empty(C, np.float64)
    var = np.empty(C, np.float64)
    g, b = _f32(gamma), _f32(beta)
    rc = _load().or_batch_norm_train(_ptr(x64), _ptr(y), N, C, S, float(eps), _ptr(g), _ptr(b),
                                     float(scale), _ptr(mean), _ptr(var), int(nthreads))
    if rc != 0:
        raise ValueError("or_batch_norm_train rejected its arguments")
    return (y, mean, var) if with_stats else y


def bn_running_update(mean, var, count, running_mean, running_var, momentum=0.1):
    """Running-statistics step of training-mode batch norm (BN page, opening analysis):
    running = (1 - momentum) * running + momentum * batch, with the unbiased batch variance
    var * count / (count - 1). mean/var are the fp64 batch statistics (var biased). Returns the
    updated fp32 running mean and variance (new arrays)."""
    mean = np.ascontiguousarray(mean, dtype=np.float64)
    var = np.ascontiguousarray(var, dtype=np.float64)
    rm = np.array(running_mean, dtype=np.float32, copy=True)
    rv = np.array(running_var, dtype=np.float32, copy=True)
    rc = _load().or_bn_running_update(_ptr(mean), _ptr(var), mean.size, int(count), float(momentum),
                                      _ptr(rm), _ptr(rv))
    if rc != 0:
        raise ValueError("or_bn_running_update rejected its arguments")
    return rm, rv


def conv_norm_epilogue(x, w, b, *, batch, eps=1e-5, pre_mul=None, gamma=None, beta=None,
                       out_scale=1.0, clamp=None, post_mul=None, reduce_max_c=False, nthreads=0,
                       with_stats=False):
    """The conv -> normalize -> epilogue chain, in the order both model pages state it:
    conv+bias, x pre_mul[k], normalize (batch: per channel over (N, space), BN page;
    instance: per (n, k) over space, IN3d page), x gamma + beta, x out_scale, clamp(lo, hi),
    x post_mul[k], optional max over channels (IN3d page). All fp64, one final rounding."""
    x, w, b = _f32(x), _f32(w), _f32(b)
    dims = x.ndim - 2
    N, Cin = x.shape[0], x.shape[1]
    Cout = w.shape[0]
    if dims == 2:
        D, (H, W) = 1, x.shape[2:]
        sp = (H - 2, W - 2)
    else:
        D, H, W = x.shape[2:]
        sp = (D - 2, H - 2, W - 2)
    oshape = (N,) + sp if reduce_max_c else (N, Cout) + sp
    out = np.empty(oshape, np.float32)
    nstat = Cout if batch else N * Cout
    mean = np.empty(nstat, np.float64)
    inv = np.empty(nstat, np.float64)
    lo, hi = (clamp if clamp is not None else (0.0, 0.0))
    # keep every converted array bound to a name until the call returns
    pm, g, be, qm = _f32(pre_mul), _f32(gamma), _f32(beta), _f32(post_mul)
    rc = _load().or_conv_norm_epilogue(
        _ptr(x), _ptr(w), _ptr(b), _ptr(out), dims, N, Cin, Cout, D, H, W,
        1 if batch else 0, float(eps), _ptr(pm), _ptr(g), _ptr(be),
        float(out_scale), 1 if clamp is not None else 0, float(lo), float(hi),
        _ptr(qm), 1 if reduce_max_c else 0, _ptr(mean), _ptr(inv), int(nthreads))
    if rc != 0:
        raise ValueError("or_conv_norm_epilogue rejected its arguments")
    return (out, mean, inv) if with_stats else out


def conv_bn_eval(x, w, b, running_mean, running_var, *, gamma=None, beta=None, eps=1e-5,
                 scale=1.0, nthreads=0):
    """Conv k=3 then eval-mode batch norm with running statistics, then * scale (BN page, its
    eval-mode discussion), unfolded: ((conv(x) - rm)/sqrt(rv + eps) * gamma + beta) * scale."""
    x, w, b = _f32(x), _f32(w), _f32(b)
    rm, rv, g, bt = _f32(running_mean), _f32(running_var), _f32(gamma), _f32(beta)
    dims = x.ndim - 2
    N, Cin = x.shape[0], x.shape[1]
    Cout = w.shape[0]
    if dims == 2:
        D, (H, W) = 1, x.shape[2:]
        oshape = (N, Cout, H - 2, W - 2)
    else:
        D, H, W = x.shape[2:]
        oshape = (N, Cout, D - 2, H - 2, W - 2)
    out = np.empty(oshape, np.float32)
    rc = _load().or_conv_bn_eval(_ptr(x), _ptr(w), _ptr(b), _ptr(rm), _ptr(rv), _ptr(g), _ptr(bt),
                                 float(eps), float(scale), _ptr(out), dims, N, Cin, Cout, D, H, W,
                                 int(nthreads))
    if rc != 0:
        raise ValueError("or_conv_bn_eval rejected its arguments")
    return out
