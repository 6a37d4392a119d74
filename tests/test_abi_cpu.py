"""The C ABI without a GPU: the library loads, exports every function normred.h declares, and
rejects bad arguments on the host before touching the HIP runtime."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "normred.h")


@pytest.fixture(scope="module")
def lib():
    from normalization_reductions_amd import _lib

    return _lib.load()


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][\w\s\*]*?\b([a-z_][a-z0-9_]*)\s*\(", text, re.M)
    return sorted(set(n for n in names if not n.startswith("__")))


def test_header_declares_the_boundary():
    names = _declared_functions()
    for must in ("inorm_forward", "bn_train_forward", "conv_norm_epilogue_forward",
                 "inorm_workspace_size", "bn_train_workspace_size",
                 "conv_norm_epilogue_workspace_size", "nr_last_error"):
        assert must in names


def test_library_exports_every_declared_symbol(lib):
    from normalization_reductions_amd import _lib

    for name in _declared_functions():
        assert hasattr(lib, name), name
        assert name in _lib.SIGNATURES, name


def test_version(lib):
    assert b"gfx950" in lib.nr_version()


def test_desc_struct_layout_matches_header():
    # offsets the C compiler gives nr_conv_norm_desc (x86-64 SysV): ints 4, int64/pointers 8
    from normalization_reductions_amd._lib import ConvNormDesc as D

    assert D.spatial_dims.offset == 0 and D.ksize.offset == 4 and D.N.offset == 8
    assert D.in_w.offset == 48 and D.norm.offset == 56 and D.eps.offset == 60
    assert D.pre_mul.offset == 64 and D.beta.offset == 80 and D.out_scale.offset == 88
    assert D.clamp.offset == 92 and D.clamp_hi.offset == 100 and D.post_mul.offset == 104
    assert D.reduce_max_c.offset == 112 and ctypes.sizeof(D) == 120


def test_workspace_sizes(lib):
    # config-3 shape: exchange regions + split partials fit in a few MB
    n = lib.inorm_workspace_size(112, 64, 512 * 512)
    assert 256 < n < 8 << 20
    assert lib.inorm_workspace_size(0, 1, 1) >= 256  # empty batch: a valid (header-only) size
    assert lib.inorm_workspace_size(1, 1, 0) == 0
    assert lib.inorm_workspace_size(1, 1, -3) == 0
    assert lib.inorm_workspace_size(1 << 40, 1 << 40, 1) == 0  # overflow
    assert lib.bn_train_workspace_size(128, 64, 3844) > 256


FAKE = 0x10000  # a 256-aligned address never dereferenced: every call below fails validation


def _inorm(lib, x=FAKE, y=FAKE + (1 << 36), N=1, C=1, S=16, eps=1e-5, gamma=None, beta=None,
           sm=None, si=None, ws=FAKE + (1 << 37), wsb=1 << 20, variant=0):
    return lib.inorm_forward_ex(x, y, N, C, S, eps, gamma, beta, sm, si, ws, wsb, variant, None)


@pytest.mark.parametrize("kw,status", [
    (dict(x=None), 1), (dict(y=None), 1), (dict(N=-1), 1), (dict(C=-1), 1), (dict(S=0), 1),
    (dict(N=1 << 40, C=1 << 30), 1), (dict(x=FAKE + 2), 2), (dict(y=FAKE + 6), 2),
    (dict(gamma=FAKE), 1), (dict(beta=FAKE), 1), (dict(gamma=FAKE + 2, beta=FAKE + 8), 2),
    (dict(eps=-1.0), 1), (dict(eps=float("nan")), 1), (dict(eps=float("inf")), 1),
    (dict(variant=7), 1), (dict(ws=None), 4), (dict(wsb=16), 4), (dict(ws=FAKE + (1 << 37) + 16), 2),
    (dict(y=FAKE + 8, S=64), 1),  # partial overlap of x and y
    (dict(variant=1, S=18), 3),  # resident variant needs S % 4 == 0
    (dict(variant=1, x=FAKE + 4, y=FAKE + (1 << 36) + 4), 3),  # ... and 16-byte alignment
    (dict(variant=1, S=16 * 65536 * 2), 3),  # ... and a slice that fits 16 parts
])
def test_inorm_rejects(lib, kw, status):
    if "wsb" not in kw and kw.get("S", 16) > 1 << 16:
        kw["wsb"] = 1 << 30
    assert _inorm(lib, **kw) == status
    assert lib.nr_last_error().decode().startswith("inorm_forward")


def test_empty_batches_are_noops_without_workspace(lib):
    assert lib.inorm_forward(FAKE, FAKE, 0, 5, 16, 1e-5, None, None, None, None, None, 0, None) == 0
    assert lib.inorm_forward(None, None, 0, 5, 16, 1e-5, None, None, None, None, None, 0, None) == 0
    assert lib.inorm_forward(None, None, 0, 5, 0, 1e-5, None, None, None, None, None, 0, None) == 1
    assert lib.inorm_forward(FAKE, FAKE, 3, 0, 16, 1e-5, None, None, None, None, None, 0, None) == 0
    assert lib.bn_train_forward(FAKE, FAKE, 2, 0, 4, 1e-5, None, None, 1.0, None, None, None, 0,
                                None) == 0
    assert lib.bn_train_forward(FAKE, FAKE, 0, 2, 4, 1e-5, None, None, 1.0, None, None, None, 0,
                                None) == 1  # batch statistics over no samples
    assert lib.bn_train_workspace_size(2, 0, 4) >= 256
    d = _desc(N=0)
    assert lib.conv_norm_epilogue_workspace_size(ctypes.byref(d)) >= 256
    assert lib.conv_norm_epilogue_forward(ctypes.byref(d), FAKE, FAKE, None, FAKE, None, 0, None) == 0


def test_bn_rejects(lib):
    f = lib.bn_train_forward
    assert f(None, FAKE, 1, 1, 4, 1e-5, None, None, 1.0, None, None, FAKE, 1 << 20, None) == 1
    assert f(FAKE, FAKE, 1, 1, 4, 1e-5, FAKE, None, 1.0, None, None, FAKE, 1 << 20, None) == 1
    assert f(FAKE, FAKE, 1, 1, 4, 1e-5, None, None, float("nan"), None, None, FAKE, 1 << 20, None) == 1
    assert f(FAKE, FAKE, 1, 1, 4, 1e-5, None, None, 1.0, None, None, FAKE, 8, None) == 4
    assert f(FAKE + 1, FAKE + 1, 1, 1, 4, 1e-5, None, None, 1.0, None, None, FAKE, 1 << 20, None) == 2


def _desc(**over):
    from normalization_reductions_amd._lib import ConvNormDesc

    d = ConvNormDesc()
    d.spatial_dims, d.ksize, d.N, d.C_in, d.C_out = 2, 3, 2, 3, 4
    d.in_d, d.in_h, d.in_w = 1, 8, 9
    d.norm, d.eps, d.out_scale = 1, 1e-5, 1.0
    d.clamp, d.clamp_lo, d.clamp_hi, d.reduce_max_c = 0, 0.0, 0.0, 0
    for k, v in over.items():
        setattr(d, k, v)
    return d


@pytest.mark.parametrize("over,status", [
    (dict(spatial_dims=1), 1), (dict(ksize=5), 3), (dict(N=-1), 1), (dict(C_out=0), 1),
    (dict(in_h=2), 1), (dict(spatial_dims=3, in_d=2), 1), (dict(norm=0), 1), (dict(eps=-1.0), 1),
    (dict(clamp=1, clamp_lo=1.0, clamp_hi=-1.0), 1), (dict(clamp=2), 1), (dict(reduce_max_c=3), 1),
    (dict(pre_mul=FAKE + 2), 2), (dict(N=70000), 3),
])
def test_conv_rejects(lib, over, status):
    d = _desc(**over)
    r = lib.conv_norm_epilogue_forward(ctypes.byref(d), FAKE, FAKE, None, FAKE, FAKE, 1 << 30, None)
    assert r == status
    assert lib.conv_norm_epilogue_workspace_size(ctypes.byref(d)) == 0


def test_conv_rejects_pointers_and_workspace(lib):
    d = _desc()
    need = lib.conv_norm_epilogue_workspace_size(ctypes.byref(d))
    assert need > 0
    f = lib.conv_norm_epilogue_forward
    assert f(None, FAKE, FAKE, None, FAKE, FAKE, need, None) == 1
    assert f(ctypes.byref(d), None, FAKE, None, FAKE, FAKE, need, None) == 1
    assert f(ctypes.byref(d), FAKE, FAKE, None, FAKE, FAKE, need - 1, None) == 4
    assert f(ctypes.byref(d), FAKE, FAKE, FAKE + 1, FAKE, FAKE, need, None) == 2


def test_helpers_reject(lib):
    assert lib.nr_workspace_clear(None, 16, None) == 1
    flags = ctypes.c_uint32()
    assert lib.nr_workspace_check(None, 256, None, ctypes.byref(flags)) == 1
    assert lib.nr_workspace_check(FAKE, 16, None, ctypes.byref(flags)) == 4
    assert lib.nr_stream_copy(None, FAKE, 4, None) == 1
    assert lib.nr_stream_copy(FAKE, FAKE, 4, None) == 1
    assert lib.nr_stream_copy(FAKE + 1, FAKE + 64, 4, None) == 2


def test_binding_refuses_cpu_tensors():
    import torch

    import normalization_reductions_amd as nra

    with pytest.raises(ValueError):
        nra.inorm_forward(torch.zeros(1, 1, 4))
