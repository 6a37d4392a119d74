"""inorm_forward_noalloc (the entry point that allocates nothing) against inorm_forward, through
the C ABI (needs an MI355X: run with -m gpu).

Two calls in a row share the library's device array: the first on a workload of 4-part slices
(the exchange counter and slots in the array), the second on a smaller input. Each output must
match inorm_forward's on the same input within the parity gate (the same kernels run, so
bitwise), and the oracle's. A shape whose workspace exceeds the array is rejected on the host.
"""
import ctypes

import numpy as np
import pytest

pytestmark = pytest.mark.gpu
TOL = 1e-4


@pytest.fixture(scope="module")
def dev():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    return torch.device("cuda:0")


def _maxerr(a, b):
    return float(np.max(np.abs(np.asarray(a, np.float64) - np.asarray(b, np.float64))))


def test_noalloc_matches_inorm_forward(dev):
    import torch

    import normalization_reductions_amd as nra
    import oracle

    g = np.random.Generator(np.random.PCG64(0x5EED0A11))
    # each call smaller than the one before: 4, then 3 exchanging parts per slice, then slices
    # off 16-byte boundaries (one workgroup each, no exchange)
    shapes = [(16, 64, 65536), (2, 3, 40000), (3, 5, 1001)]
    for shape in shapes:
        print("case inorm_forward_noalloc %s" % (shape,), flush=True)
        x = (g.standard_normal(shape) * 3 + 5).astype(np.float32)
        xt = torch.from_numpy(x).to(dev)
        y_ref = nra.inorm_forward(xt)
        y = torch.full_like(xt, float("nan"))
        sm = torch.empty(shape[0] * shape[1], device=dev)
        si = torch.empty(shape[0] * shape[1], device=dev)
        nra.inorm_forward_noalloc(xt, y, save_mean=sm, save_invstd=si)
        torch.cuda.synchronize()
        yh = y.cpu().numpy()
        err_ref = _maxerr(yh, y_ref.cpu().numpy())
        ref, mean, var = oracle.instance_norm_slices(x.reshape(-1, shape[-1]), with_stats=True)
        err_or = _maxerr(yh.reshape(-1, shape[-1]), ref)
        print("inorm_forward_noalloc %s: vs inorm_forward %.3e, vs oracle %.3e"
              % (shape, err_ref, err_or), flush=True)
        assert err_ref <= TOL and err_or <= TOL
        assert torch.equal(y, y_ref)
        np.testing.assert_allclose(sm.cpu().numpy(), mean, rtol=1e-6, atol=1e-6)
        np.testing.assert_allclose(si.cpu().numpy(), 1.0 / np.sqrt(var + 1e-5), rtol=1e-5)


def test_noalloc_rejects_shapes_beyond_its_array(dev):
    import normalization_reductions_amd as nra
    from normalization_reductions_amd import _lib

    lib = _lib.load()
    N, C, S = 1 << 20, 16, 1024  # 16M slices: workspace far beyond 8 MiB
    assert lib.inorm_workspace_size(N, C, S) > (8 << 20)
    dummy = ctypes.c_void_p(256)  # never dereferenced: the host check rejects the call first
    st = lib.inorm_forward_noalloc(dummy, dummy, N, C, S, 1e-5, None, None, None, None, None)
    assert st == _lib.NR_ERR_WORKSPACE
    assert "no-allocation" in _lib.last_error()
    assert nra is not None
