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


def test_desc_struct_layout_matches_header(tmp_path):
    # the ctypes mirror must give every field of nr_conv_norm_desc the offset the C compiler does
    import shutil
    import subprocess

    from normalization_reductions_amd._lib import ConvNormDesc as D

    if shutil.which("gcc") is None or not os.path.isdir("/opt/rocm/include"):
        pytest.skip("needs gcc and the ROCm headers")
    names = [f[0] for f in D._fields_]
    src = tmp_path / "layout.c"
    src.write_text("#include <stdio.h>\n#include <stddef.h>\n#include \"normred.h\"\nint main(void) {\n"
                   + "".join('printf("%%zu\\n", offsetof(nr_conv_norm_desc, %s));\n' % n for n in names)
                   + 'printf("%zu\\n", sizeof(nr_conv_norm_desc));\nreturn 0;\n}\n')
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
                    "-I", "/opt/rocm/include", str(src), "-o", str(exe)], check=True)
    got = [int(v) for v in subprocess.run([str(exe)], check=True, capture_output=True,
                                          text=True).stdout.split()]
    assert got[:-1] == [getattr(D, n).offset for n in names]
    assert got[-1] == ctypes.sizeof(D)


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
    (dict(variant=1, S=65531), 3),  # resident variant: S % 4 != 0 only up to 65,530
    (dict(variant=1, S=3), 3),  # ... and in a tensor of at least 4 values
    (dict(variant=1, x=FAKE + 4, y=FAKE + (1 << 36) + 4), 3),  # ... and 16-byte alignment
    (dict(variant=1, S=18, x=FAKE + 4, y=FAKE + (1 << 36) + 4), 3),  # ... for any S
    (dict(variant=1, S=32 * 32768 + 4), 3),  # ... and a slice that fits 32 parts
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


def _bn_ex(lib, momentum=0.1, rm=FAKE + (1 << 38), rv=FAKE + (1 << 39), N=2, S=4):
    return lib.bn_train_forward_ex(FAKE, FAKE + (1 << 36), N, 3, S, 1e-5, None, None, 1.0, None,
                                   None, momentum, rm, rv, FAKE + (1 << 37), 1 << 20, None)


@pytest.mark.parametrize("kw,status", [
    (dict(momentum=-0.1), 1), (dict(momentum=1.5), 1), (dict(momentum=float("nan")), 1),
    (dict(rm=None), 1), (dict(rv=None), 1), (dict(rm=FAKE + (1 << 38) + 2), 2),
    (dict(N=1, S=1), 1),  # one value per channel: no unbiased variance
])
def test_bn_running_stats_rejects(lib, kw, status):
    assert _bn_ex(lib, **kw) == status
    assert "bn_train_forward" in lib.nr_last_error().decode()


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
    (dict(channels_last=2), 1), (dict(channels_last=1, C_out=300), 3),
])
def test_conv_rejects(lib, over, status):
    d = _desc(**over)
    r = lib.conv_norm_epilogue_forward(ctypes.byref(d), FAKE, FAKE, None, FAKE, FAKE, 1 << 30, None)
    assert r == status
    assert lib.conv_norm_epilogue_workspace_size(ctypes.byref(d)) == 0


@pytest.mark.parametrize("over,status", [
    (dict(norm=2, running_mean=FAKE, running_var=FAKE + 64), 1),  # instance norm keeps none
    (dict(running_mean=FAKE), 1), (dict(running_mean=FAKE, running_var=FAKE + 64, momentum=2.0), 1),
    (dict(running_mean=FAKE + 1, running_var=FAKE + 64), 2),
    (dict(N=1, in_h=3, in_w=3, running_mean=FAKE, running_var=FAKE + 64), 1),  # 1 value/channel
])
def test_conv_running_stats_rejects(lib, over, status):
    d = _desc(**over)
    r = lib.conv_norm_epilogue_forward(ctypes.byref(d), FAKE, FAKE, None, FAKE, FAKE, 1 << 30, None)
    assert r == status


@pytest.mark.parametrize("over,status", [
    (dict(norm=2), 1), (dict(pre_mul=FAKE), 3), (dict(post_mul=FAKE), 3), (dict(clamp=1), 3),
    (dict(reduce_max_c=1), 3), (dict(running_mean=FAKE, running_var=FAKE + 64), 3),
    (dict(ksize=5), 3), (dict(eps=float("nan")), 1),
])
def test_conv_bn_eval_rejects(lib, over, status):
    d = _desc(**over)
    f = lib.conv_bn_eval_forward
    assert f(ctypes.byref(d), FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, 1 << 30, None) == status
    assert lib.conv_bn_eval_workspace_size(ctypes.byref(d)) == 0
    assert lib.nr_last_error().decode().startswith("conv_bn_eval")


def test_conv_bn_eval_rejects_pointers_and_workspace(lib):
    d = _desc()
    need = lib.conv_bn_eval_workspace_size(ctypes.byref(d))
    assert need >= 256 + 4 * (4 * 3 * 9 + 4)
    f = lib.conv_bn_eval_forward
    assert f(ctypes.byref(d), FAKE, FAKE, None, None, FAKE, FAKE, FAKE, need, None) == 1
    assert f(ctypes.byref(d), FAKE, FAKE, None, FAKE, None, FAKE, FAKE, need, None) == 1
    assert f(ctypes.byref(d), FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, need - 1, None) == 4
    assert f(ctypes.byref(d), FAKE, FAKE, FAKE + 2, FAKE, FAKE, FAKE, FAKE, need, None) == 2
    d0 = _desc(N=0)
    assert f(ctypes.byref(d0), None, None, None, None, None, None, None, 0, None) == 0


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
    assert lib.nr_stream_copy_ws(None, FAKE, 4, FAKE, 256, None) == 1
    assert lib.nr_stream_copy_ws(FAKE, FAKE + 8, 4, FAKE + 4096, 256, None) == 1   # overlap
    assert lib.nr_stream_copy_ws(FAKE, FAKE + 4096, 4, None, 256, None) == 4        # no workspace
    assert lib.nr_stream_copy_ws(FAKE, FAKE + 4096, 4, FAKE + 8192, 255, None) == 4  # too small
    assert lib.nr_stream_copy_ws(FAKE, FAKE + 4096, 4, FAKE + 8200, 256, None) == 4  # misaligned


def test_binding_refuses_cpu_tensors():
    import torch

    import normalization_reductions_amd as nra

    with pytest.raises(ValueError):
        nra.inorm_forward(torch.zeros(1, 1, 4))
