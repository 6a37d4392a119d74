"""Parity of the HIP path against the fp64 oracle (needs an MI355X: run with -m gpu).

Bar: max |gpu - oracle| <= 1e-4 over every compared output element (fp32 outputs), the
tolerance the workloads state; bit-identical results across repeated runs; the workspace's
error flags stay clear. Inputs are seeded and synthetic: synth/'s generators, torch's seeded
device generator for the tensors beyond 2^31 elements, and the native client's counter-based
generator (SplitMix64).
"""
import os

import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu
TOL = 1e-4


@pytest.fixture(scope="module")
def dev():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    return torch.device("cuda:0")


@pytest.fixture(scope="module")
def nra(dev):
    import normalization_reductions_amd as m

    m._lib.load()
    return m


@pytest.fixture(scope="module")
def orc():
    import oracle

    oracle._load()
    return oracle


def T(a, dev):
    import torch

    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def H(t):
    import torch

    torch.cuda.synchronize()
    return t.detach().cpu().numpy()


def maxerr(a, b):
    return float(np.max(np.abs(np.asarray(a, np.float64) - np.asarray(b, np.float64)))) if np.size(a) else 0.0


def _log(msg):
    print(msg, flush=True)


# ------------------------------------------------------------------------------------------
# Instance norm: the three InstanceNorm2d workloads
# ------------------------------------------------------------------------------------------
@pytest.mark.parametrize("variant", [0, 1, 2])
def test_inorm_workload1(dev, nra, orc, variant):
    inp = synth.host_inputs(1)
    y = nra.inorm_forward(T(inp["x"], dev), eps=inp["eps"], variant=variant)
    err = maxerr(H(y), orc.instance_norm(inp["x"], eps=inp["eps"]))
    _log("inorm x[2,4,32,32] variant %d: max_abs_err %.3e" % (variant, err))
    assert err <= TOL


@pytest.mark.parametrize("variant", [0, 2])
def test_inorm_workload2_full(dev, nra, orc, variant):
    inp = synth.host_inputs(2)
    x = T(inp["x"], dev)
    n, c = x.shape[:2]
    import torch

    sm = torch.empty(n * c, device=dev)
    si = torch.empty(n * c, device=dev)
    y = nra.inorm_forward(x, eps=inp["eps"], save_mean=sm, save_invstd=si, variant=variant)
    ref, mean, var = orc.instance_norm(inp["x"], eps=inp["eps"], with_stats=True)
    err = maxerr(H(y), ref)
    _log("inorm x[16,64,256,256] (offsets +-100) variant %d: max_abs_err %.3e" % (variant, err))
    assert err <= TOL
    np.testing.assert_allclose(H(sm), mean.ravel(), rtol=2e-7, atol=2e-5)
    np.testing.assert_allclose(H(si), 1.0 / np.sqrt(var.ravel() + 1e-5), rtol=1e-5)
    y2 = nra.inorm_forward(x, eps=inp["eps"], variant=variant)
    assert torch.equal(y, y2)


@pytest.fixture(scope="module")
def w3(dev):
    import torch

    x = synth.device_inputs_cfg3(dev)["x"]
    yield x
    del x
    torch.cuda.empty_cache()


def _sample_slices(total, k, seed):
    g = np.random.Generator(np.random.PCG64(seed))
    fixed = [0, 1, 63, 64, 511, 512, total // 2, total - 2, total - 1]
    rest = g.choice(total, size=k, replace=False).tolist()
    return sorted(set(fixed + rest))


@pytest.mark.parametrize("variant", [0, 2])
def test_inorm_workload3_full_size(dev, nra, orc, w3, variant):
    import torch

    x = w3
    N, C = x.shape[:2]
    S = x.shape[2] * x.shape[3]
    sm = torch.empty(N * C, device=dev)
    si = torch.empty(N * C, device=dev)
    ws = torch.zeros(nra.inorm_workspace_size(N, C, S), dtype=torch.uint8, device=dev)
    y = nra.inorm_forward(x, eps=1e-5, save_mean=sm, save_invstd=si, workspace=ws, variant=variant)
    torch.cuda.synchronize()
    assert nra.workspace_check(ws) == 0

    # every slice against the oracle, element by element, 512 slices (512 MiB) at a time
    xv, yv = x.view(N * C, S), y.view(N * C, S)
    smh, sih = H(sm), H(si)
    err = 0.0
    for lo in range(0, N * C, 512):
        hi = min(lo + 512, N * C)
        ref, mean, var = orc.instance_norm_slices(xv[lo:hi].cpu().numpy(), eps=1e-5, with_stats=True)
        yb = yv[lo:hi].cpu().numpy()
        err = max(err, maxerr(yb, ref))
        np.testing.assert_allclose(smh[lo:hi], mean, rtol=1e-6, atol=1e-6)
        np.testing.assert_allclose(sih[lo:hi], 1.0 / np.sqrt(var + 1e-5), rtol=1e-5)
        # closed form of the op: per slice output mean 0 and variance var / (var + eps), with
        # the oracle's variances (moments taken on the device in fp64)
        blk = yv[lo:hi].double()
        assert float(blk.mean(dim=1).abs().max()) < 1e-5
        vy = blk.var(dim=1, unbiased=False).cpu().numpy()
        assert float(np.max(np.abs(vy - var / (var + 1e-5)))) < 2e-5
        del blk
    _log("inorm x[112,64,512,512] variant %d: all %d slices, max_abs_err %.3e" % (variant, N * C, err))
    assert err <= TOL

    y2 = nra.inorm_forward(x, eps=1e-5, workspace=ws, variant=variant)
    assert torch.equal(y, y2)
    assert nra.workspace_check(ws) == 0
    del y, y2


# ------------------------------------------------------------------------------------------
# Instance norm: every compiled read-once configuration, ragged parts, edge shapes
# ------------------------------------------------------------------------------------------
RESIDENT_CASES = [
    # (block, vec, S). S <= block*4*vec: one workgroup per slice (full and ragged);
    # larger S: the pipelined kernel with P = ceil(S / (block*4*vec)) parts -- 2, ragged,
    # a 4-element last part, and the 32-part maximum.
    (256, 1, 1024), (256, 1, 1000), (256, 2, 2048), (256, 4, 4096), (256, 8, 8192),
    (256, 16, 16384), (256, 16, 12600), (512, 16, 32768), (512, 16, 20000),
    (1024, 16, 65536), (1024, 16, 50000),
    (256, 8, 16384), (256, 8, 20000), (256, 8, 262144),
    (256, 16, 262144), (256, 16, 65540), (256, 16, 524288), (256, 16, 40000),
    (512, 16, 65536), (512, 16, 1048576), (512, 16, 200004),
]


@pytest.mark.parametrize("block,vec,S", RESIDENT_CASES)
def test_inorm_resident_configurations(dev, nra, orc, monkeypatch, block, vec, S):
    import torch

    monkeypatch.setenv("NORMRED_RESIDENT_CFG", "%d,%d" % (block, vec))
    nc = max(2, min(24, (8 << 20) // S))
    x = synth.per_slice_affine_normal((nc, 1, S), 1000 + S, (0.1, 10.0), (-100.0, 100.0))
    xt = T(x, dev)
    ws = torch.zeros(nra.inorm_workspace_size(nc, 1, S), dtype=torch.uint8, device=dev)
    y = nra.inorm_forward(xt, variant=nra.NR_VARIANT_RESIDENT, workspace=ws)
    err = maxerr(H(y), orc.instance_norm(x))
    _log("resident block %d vec %d S %d slices %d: max_abs_err %.3e" % (block, vec, S, nc, err))
    assert err <= TOL
    assert nra.workspace_check(ws) == 0
    y2 = nra.inorm_forward(xt, variant=nra.NR_VARIANT_RESIDENT, workspace=ws)
    assert torch.equal(y, y2)


EDGE_SHAPES = [(1, 1, 1), (3, 2, 5), (2, 3, 1023), (1, 1, 4), (2, 2, 65540), (1, 3, 262148),
               (4, 2, 100000), (1, 1, 1048576), (2, 1, 1048580), (5, 7, 12600), (1, 1, 7),
               # S % 4 != 0 in aligned tensors (flat 16-byte path): several chunks per slice,
               # and many one-chunk slices
               (2, 3, 70001), (256, 64, 961)]


@pytest.fixture(scope="module")
def shared_ws(dev):
    """One workspace reused by calls of every shape and variant (sized for the largest)."""
    import torch

    ws = torch.zeros(64 << 20, dtype=torch.uint8, device=dev)
    return ws


@pytest.mark.parametrize("shape", EDGE_SHAPES)
@pytest.mark.parametrize("variant", [0, 2])
def test_inorm_edge_shapes(dev, nra, orc, shared_ws, shape, variant):
    x = synth.per_slice_affine_normal(shape, 7 + shape[2], (0.1, 10.0), (-100.0, 100.0))
    y = nra.inorm_forward(T(x, dev), variant=variant, workspace=shared_ws)
    err = maxerr(H(y), orc.instance_norm(x))
    _log("inorm edge %s variant %d: max_abs_err %.3e" % (shape, variant, err))
    assert err <= TOL
    assert nra.workspace_check(shared_ws) == 0


def test_inorm_workspace_carries_no_state(dev, nra, orc):
    # A workspace full of arbitrary bytes, reused across shapes whose regions overlap
    # differently (split partials over the exchange slots of another shape, 3 then 9 then 2
    # parts), must not change any result.
    import torch

    ws = torch.randint(0, 256, (64 << 20,), dtype=torch.uint8, device=dev)
    ws[:256] = 0  # the sticky error word is the one thing read across calls
    seq = [((2, 2, 65540), 0), ((3, 2, 5), 2), ((1, 3, 262148), 0), ((2, 3, 1023), 2),
           ((1, 3, 262148), 0), ((16, 4, 65536), 0), ((2, 2, 65540), 2), ((1, 3, 262148), 1)]
    for i, (shape, variant) in enumerate(seq):
        x = synth.per_slice_affine_normal(shape, 300 + i, (0.1, 10.0), (-100.0, 100.0))
        y = nra.inorm_forward(T(x, dev), variant=variant, workspace=ws)
        err = maxerr(H(y), orc.instance_norm(x))
        _log("shared dirty workspace step %d %s variant %d: max_abs_err %.3e"
             % (i, shape, variant, err))
        assert err <= TOL
        assert nra.workspace_check(ws) == 0


def test_exchange_wait_gives_up_and_raises_flag(dev, nra, orc, monkeypatch):
    """The failure path of the bounded waits (the read-once kernels' exchange, and the
    recomputing batch-norm chain's wait for its published statistics), forced from the host:
    under NORMRED_TEST_WAIT_GIVEUP=1 every wait looks for a tag no part publishes and gives up
    after 64 polls. The call must still finish (every kernel exits normally) and raise the
    sticky timeout flag, which nr_workspace_check reports once and clears; the next call
    without the switch is correct again with the flag clear."""
    import torch

    g = np.random.Generator(np.random.PCG64(91))
    x = g.standard_normal((4, 8, 65536)).astype(np.float32)  # 4 parts per slice
    xb = g.standard_normal((128, 16, 62, 62)).astype(np.float32)  # batch groups, 31 parts
    xt, xbt = T(x, dev), T(xb, dev)
    ws = torch.zeros(max(nra.inorm_workspace_size(4, 8, 65536),
                         nra.bn_train_workspace_size(128, 16, 62 * 62)), dtype=torch.uint8, device=dev)
    monkeypatch.setenv("NORMRED_TEST_WAIT_GIVEUP", "1")
    nra.inorm_forward(xt, workspace=ws)
    torch.cuda.synchronize()
    assert nra.workspace_check(ws) & 1
    assert nra.workspace_check(ws) == 0  # reported once, then cleared
    nra.bn_train_forward(xbt, workspace=ws)
    torch.cuda.synchronize()
    assert nra.workspace_check(ws) & 1
    # the recomputing Conv2d -> batch norm chain: its apply pass waits for the statistics its
    # first workgroups publish
    xc = g.standard_normal((4, 8, 18, 64)).astype(np.float32)
    wc = (g.standard_normal((64, 8, 3, 3)) * 0.2).astype(np.float32)
    bc = g.standard_normal(64).astype(np.float32)
    rm, rv = T(np.zeros(64, np.float32), dev), T(np.ones(64, np.float32), dev)
    cargs = (T(xc, dev), T(wc, dev), T(bc, dev))
    wsc = torch.zeros(64 << 20, dtype=torch.uint8, device=dev)
    nra.conv_norm_epilogue_forward(*cargs, norm=nra.NR_NORM_BATCH_TRAIN, workspace=wsc)
    torch.cuda.synchronize()
    assert nra.workspace_check(wsc) & 1
    monkeypatch.delenv("NORMRED_TEST_WAIT_GIVEUP")
    y = nra.inorm_forward(xt, workspace=ws)
    yb = nra.bn_train_forward(xbt, workspace=ws)
    yc = nra.conv_norm_epilogue_forward(*cargs, norm=nra.NR_NORM_BATCH_TRAIN, running_mean=rm,
                                        running_var=rv, momentum=0.5, workspace=wsc)
    torch.cuda.synchronize()
    assert nra.workspace_check(ws) == 0
    assert nra.workspace_check(wsc) == 0
    assert maxerr(H(y), orc.instance_norm(x)) <= TOL
    assert maxerr(H(yb), orc.batch_norm_train(xb)) <= TOL
    assert maxerr(H(yc), orc.conv_norm_epilogue(xc, wc, bc, batch=True)) <= TOL
    c = orc.conv_k3(xc, wc, bc)
    _, mean, var = orc.batch_norm_train(c, with_stats=True)
    n = c.size // 64
    rm_ref, rv_ref = orc.bn_running_update(mean, var, n, np.zeros(64, np.float32),
                                           np.ones(64, np.float32), momentum=0.5)
    np.testing.assert_allclose(H(rm), rm_ref, rtol=1e-5, atol=1e-6)
    np.testing.assert_allclose(H(rv), rv_ref, rtol=1e-5, atol=1e-6)


def test_inorm_two_streams_concurrently(dev, nra, orc):
    # two persistent read-once launches in flight on different streams, each with its own
    # workspace: both must finish with correct results and clean workspace flags
    import torch

    g = np.random.Generator(np.random.PCG64(91))
    xs = [(g.standard_normal((4, 64, 131072)) * s + o).astype(np.float32) for s, o in ((1, 0), (3, -2))]
    xt = [T(x, dev) for x in xs]
    ys = [torch.empty_like(x) for x in xt]
    streams = [torch.cuda.Stream(device=dev) for _ in range(2)]
    wss = [torch.zeros(nra.inorm_workspace_size(4, 64, 131072), dtype=torch.uint8, device=dev)
           for _ in range(2)]
    torch.cuda.synchronize()
    for _ in range(3):
        for i in range(2):
            with torch.cuda.stream(streams[i]):
                nra.inorm_forward(xt[i], ys[i], workspace=wss[i], stream=streams[i])
    torch.cuda.synchronize()
    for i in range(2):
        assert nra.workspace_check(wss[i]) == 0
        assert maxerr(H(ys[i]), orc.instance_norm(xs[i])) <= TOL


# ------------------------------------------------------------------------------------------
# Beyond 2^31 elements (64-bit offsets everywhere): ~8.6 GB inputs, sampled parity
# ------------------------------------------------------------------------------------------
def _big_normal(shape, seed, dev):
    import torch

    gen = torch.Generator(device=dev)
    gen.manual_seed(seed)
    return torch.randn(*shape, device=dev, generator=gen)


@pytest.mark.parametrize("variant", [0, 2])
def test_inorm_beyond_2pow31_elements(dev, nra, orc, variant):
    import torch

    N, C, S = 2, 4100, 262144  # 2,149,580,800 elements: read-once (auto) and split variants
    x = _big_normal((N, C, S), 0x5EED0101, dev)
    ws = torch.zeros(nra.inorm_workspace_size(N, C, S), dtype=torch.uint8, device=dev)
    y = nra.inorm_forward(x, eps=1e-5, workspace=ws, variant=variant)
    assert nra.workspace_check(ws) == 0
    pick = _sample_slices(N * C, 5, 17 + variant)
    xs = x.view(N * C, S)[pick].cpu().numpy()
    ys = y.view(N * C, S)[pick].cpu().numpy()
    err = maxerr(ys, orc.instance_norm_slices(xs))
    _log("inorm beyond 2^31 elements, variant %d: max_abs_err %.3e over %d slices" % (variant, err, len(pick)))
    del x, y, ws
    torch.cuda.empty_cache()
    assert err <= TOL


def test_inorm_huge_slices_split_path(dev, nra, orc):
    import torch

    N, C, S = 1, 130, (1 << 24) + 4  # 16.8M values per slice: beyond any read-once part count
    x = _big_normal((N, C, S), 0x5EED0102, dev)
    x.mul_(3.0).add_(-7.0)
    y = nra.inorm_forward(x)
    pick = [0, 64, 129]
    xs = x.view(C, S)[pick].cpu().numpy()
    ys = y.view(C, S)[pick].cpu().numpy()
    err = maxerr(ys, orc.instance_norm_slices(xs))
    _log("inorm 130 slices of 2^24+4: max_abs_err %.3e" % err)
    del x, y
    torch.cuda.empty_cache()
    assert err <= TOL


def test_bn_train_beyond_2pow31_elements(dev, nra, orc):
    import torch

    N, C, S = 128, 64, 262148  # 2.15e9 elements; 33.6M values per channel (split path)
    x = _big_normal((N, C, S), 0x5EED0103, dev)
    y = nra.bn_train_forward(x, out_scale=2.0)
    chans = [0, 63]
    xs = x[:, chans].cpu().numpy()
    ys = y[:, chans].cpu().numpy()
    err = maxerr(ys, orc.batch_norm_train(xs, scale=2.0))
    _log("bn_train beyond 2^31 elements: max_abs_err %.3e on channels %s" % (err, chans))
    del x, y
    torch.cuda.empty_cache()
    assert err <= TOL


def test_inorm_empty_batch(dev, nra):
    import torch

    x = torch.empty((0, 4, 16, 16), device=dev)
    y = nra.inorm_forward(x)
    assert y.shape == x.shape


@pytest.mark.parametrize("variant", [0, 1, 2])
def test_inorm_constant_slices_are_exactly_zero(dev, nra, variant):
    import torch

    vals = torch.tensor([0.0, 3.25, -1234.5, 1e6, 7.0, -0.5], device=dev)
    x = vals.view(2, 3, 1).expand(2, 3, 65536).contiguous()
    y = nra.inorm_forward(x, variant=variant)
    torch.cuda.synchronize()
    assert bool((y == 0).all())


def test_inorm_large_offset_small_spread(dev, nra, orc):
    x = synth.per_slice_affine_normal((2, 4, 256, 256), 5, (0.01, 0.01), (1e4, 1e4))
    y = nra.inorm_forward(T(x, dev))
    err = maxerr(H(y), orc.instance_norm(x))
    _log("inorm offset 1e4, spread 1e-2: max_abs_err %.3e" % err)
    assert err <= TOL


@pytest.mark.parametrize("S", [1024, 65536, 262144, 1000])
def test_inorm_affine_inplace_stats(dev, nra, orc, S):
    import torch

    g = np.random.Generator(np.random.PCG64(S))
    N, C = 3, 5
    x = synth.per_slice_affine_normal((N, C, S), 99, (0.5, 2.0), (-3.0, 3.0))
    gamma = g.uniform(0.5, 1.5, C).astype(np.float32)
    beta = g.uniform(-1, 1, C).astype(np.float32)
    xt = T(x, dev)
    sm = torch.empty(N * C, device=dev)
    si = torch.empty(N * C, device=dev)
    nra.inorm_forward(xt, xt, gamma=T(gamma, dev), beta=T(beta, dev), save_mean=sm,
                      save_invstd=si)  # in place
    ref, mean, var = orc.instance_norm(x, gamma=gamma, beta=beta, with_stats=True)
    err = maxerr(H(xt), ref)
    _log("inorm affine in-place S=%d: max_abs_err %.3e" % (S, err))
    assert err <= TOL
    np.testing.assert_allclose(H(sm), mean.ravel(), rtol=1e-6, atol=2e-6)
    np.testing.assert_allclose(H(si), 1.0 / np.sqrt(var.ravel() + 1e-5), rtol=1e-5)


@pytest.mark.parametrize("shape", [(3, 5, 961), (2, 2, 70003), (7, 3, 2)])
def test_odd_slices_in_place(dev, nra, orc, shape):
    # S % 4 != 0, y == x. Instance norm: one workgroup per slice touching only its own values
    # (S <= 65,530), else the split path; batch norm: the split path, whose flat apply step
    # reads and writes each 16-byte block in one thread after the statistics pass has read x
    g = np.random.Generator(np.random.PCG64(shape[2] * 3 + shape[0]))
    x = (g.standard_normal(shape) * 2.0 + 3.0).astype(np.float32)
    xt = T(x, dev)
    yt = nra.inorm_forward(xt, xt)
    err_i = maxerr(H(yt), orc.instance_norm(x))
    xt = T(x, dev)
    yt = nra.bn_train_forward(xt, xt, out_scale=1.5)
    err_b = maxerr(H(yt), orc.batch_norm_train(x, scale=1.5))
    _log("odd slices in place %s: inorm %.3e, bn %.3e" % (shape, err_i, err_b))
    assert max(err_i, err_b) <= TOL


# S % 4 != 0 (and S < 1024) through the read-once kernel that gives each slice one workgroup:
# every configuration (one wave up to 1024 threads) at the edges of its range, the largest slice
# it takes, and a full-size tensor of 31 x 31 and of 255 x 255 slices
FLAT_SHAPES = [(5, 3, 3), (4, 5, 250), (3, 3, 1019), (2, 3, 1023), (2, 2, 4093), (2, 2, 4095),
               (1, 3, 16381), (1, 3, 16383), (1, 2, 32767), (1, 2, 65530), (256, 64, 961),
               (16, 64, 65025),
               # short aligned slices take the same kernel
               (7, 5, 4), (1024, 64, 8), (300, 64, 256), (3, 3, 512), (5, 3, 1020),
               # slices of up to 1018 values share workgroups in groups of 4..64 lanes (a
               # partly filled last workgroup included): 7 x 7 at full size, each group shape
               # at the edges of its range, a single slice, and S = 1
               (128, 512, 49), (1000, 3, 3), (9, 7, 13), (33, 3, 19), (7, 5, 35), (5, 5, 67),
               (3, 7, 131), (1, 1, 5), (2, 2, 1), (3, 3, 10), (3, 3, 11), (5, 3, 26),
               (5, 3, 27), (3, 3, 58), (3, 3, 59), (3, 3, 122), (3, 3, 123), (3, 3, 251),
               (3, 3, 506), (3, 3, 507), (3, 3, 1018), (128, 1024, 196)]


@pytest.mark.parametrize("shape", FLAT_SHAPES)
def test_inorm_flat_read_once(dev, nra, orc, shape):
    import torch

    N, C, S = shape
    x = synth.per_slice_affine_normal(shape, 11 + S, (0.1, 10.0), (-100.0, 100.0))
    g = np.random.Generator(np.random.PCG64(S))
    gamma = g.uniform(0.5, 2.0, C).astype(np.float32)
    beta = g.uniform(-1, 1, C).astype(np.float32)
    ref, mean, var = orc.instance_norm(x, gamma=gamma, beta=beta, with_stats=True)
    xt = T(x, dev)
    gt, bt = T(gamma, dev), T(beta, dev)
    sm = torch.empty(N * C, device=dev)
    si = torch.empty(N * C, device=dev)
    y = nra.inorm_forward(xt, gamma=gt, beta=bt, save_mean=sm, save_invstd=si,
                          variant=nra.NR_VARIANT_RESIDENT)
    err = maxerr(H(y), ref)
    y_auto = nra.inorm_forward(xt, gamma=gt, beta=bt)
    # in place; then the same call repeated must give the same bits
    x2 = T(x, dev)
    nra.inorm_forward(x2, x2, gamma=gt, beta=bt, variant=nra.NR_VARIANT_RESIDENT)
    err_in = maxerr(H(x2), ref)
    y2 = nra.inorm_forward(xt, gamma=gt, beta=bt, variant=nra.NR_VARIANT_RESIDENT)
    _log("inorm flat read-once %s: max_abs_err %.3e, in place %.3e" % (shape, err, err_in))
    assert max(err, err_in, maxerr(H(y_auto), ref)) <= TOL
    assert torch.equal(y, y2)
    np.testing.assert_allclose(H(sm), mean.ravel(), rtol=1e-6, atol=TOL)
    np.testing.assert_allclose(H(si), 1.0 / np.sqrt(var.ravel() + 1e-5), rtol=1e-5)


def test_inorm_unaligned_and_side_stream(dev, nra, orc):
    import torch

    N, C, S = 2, 3, 4096
    x = synth.per_slice_affine_normal((N, C, S), 123, (0.5, 2.0), (-3.0, 3.0))
    buf = torch.empty(N * C * S + 1, device=dev)
    buf[1:] = T(x, dev).view(-1)
    xu = buf[1:].view(N, C, S)  # 4-byte offset: not 16-byte aligned
    assert xu.data_ptr() % 16 != 0
    s = torch.cuda.Stream(device=dev)
    with torch.cuda.stream(s):
        y = nra.inorm_forward(xu)
    s.synchronize()
    err = maxerr(y.cpu().numpy(), orc.instance_norm(x))
    assert err <= TOL
    with pytest.raises(nra.NormredError):
        nra.inorm_forward(xu, variant=nra.NR_VARIANT_RESIDENT)


# ------------------------------------------------------------------------------------------
# Training-mode batch norm
# ------------------------------------------------------------------------------------------
BN_SHAPES = [
    (128, 64, 3844),   # the Conv2d->BN workload's activation: 31 parts per channel (read-once)
    (1, 3, 1), (5, 2, 7), (64, 16, 1),  # S % 4 != 0: split path
    # ... or, where one workgroup holds a channel, read once in lane groups (each group
    # shape, with live and empty groups); the split statistics step in lane groups of 4 to 64
    (128, 512, 49), (9, 7, 115), (5, 3, 250), (4, 5, 500), (3, 3, 1017), (512, 3, 9),
    (513, 3, 9), (129, 3, 49), (17, 3, 250), (1024, 64, 3), (33, 3, 500), (256, 4, 121),
    (8, 2048, 49),  # more channels than resident workgroups: the split path
    (256, 8, 49), (257, 3, 49),  # more slices per channel than a workgroup holds: split path
    (2, 4, 4100), (7, 3, 1000),          # one workgroup per channel
    (128, 8, 196), (2, 3, 16384), (3, 2, 5464),  # ... of 512 threads (16K-32K values)
    (3, 1, 100000), (33, 2, 16000), (1, 5, 65536),  # pipelined: ragged, 17 and 4 parts
    (65, 2, 32768),    # 2.1M values per channel: beyond the read-once index range -> split
    (9, 5, 20003), (256, 64, 961),      # S % 4 != 0, flat 16-byte split path: several chunks
]


@pytest.mark.parametrize("shape", BN_SHAPES)
def test_bn_train(dev, nra, orc, shape):
    import torch

    N, C, S = shape
    g = np.random.Generator(np.random.PCG64(N * 1000 + C))
    z = g.standard_normal(shape).astype(np.float32)
    x = (z * g.uniform(0.1, 3, (1, C, 1)) + g.uniform(-5, 5, (1, C, 1))).astype(np.float32)
    gamma = g.uniform(0.5, 1.5, C).astype(np.float32)
    beta = g.uniform(-0.5, 0.5, C).astype(np.float32)
    sm = torch.empty(C, device=dev)
    si = torch.empty(C, device=dev)
    xt = T(x, dev)
    y = nra.bn_train_forward(xt, gamma=T(gamma, dev), beta=T(beta, dev), out_scale=2.0,
                             save_mean=sm, save_invstd=si)
    ref, mean, var = orc.batch_norm_train(x, gamma=gamma, beta=beta, scale=2.0, with_stats=True)
    err = maxerr(H(y), ref)
    _log("bn_train %s: max_abs_err %.3e" % (shape, err))
    assert err <= TOL
    np.testing.assert_allclose(H(sm), mean, rtol=1e-6, atol=2e-6)
    np.testing.assert_allclose(H(si), 1.0 / np.sqrt(var + 1e-5), rtol=1e-5)
    y2 = nra.bn_train_forward(xt, gamma=T(gamma, dev), beta=T(beta, dev), out_scale=2.0)
    assert torch.equal(y, y2)
    nra.bn_train_forward(xt, xt, gamma=T(gamma, dev), beta=T(beta, dev), out_scale=2.0)  # in place
    assert torch.equal(xt, y)


@pytest.mark.parametrize("shape", [(8, 4, 4096), (16, 2, 65536), (4, 3, 1001)])
def test_bn_train_large_offset_small_spread(dev, nra, orc, shape):
    # mean ~1000, spread ~0.01: the statistics must not lose the spread to the offset
    # (single-workgroup, pipelined and split paths)
    N, C, S = shape
    g = np.random.Generator(np.random.PCG64(N * 31 + S))
    x = (1000.0 + 0.01 * g.standard_normal(shape) + g.uniform(-1, 1, (1, C, 1))).astype(np.float32)
    y = nra.bn_train_forward(T(x, dev))
    err = maxerr(H(y), orc.batch_norm_train(x))
    _log("bn_train offset 1000, spread 0.01 %s: max_abs_err %.3e" % (shape, err))
    assert err <= TOL


# running statistics: resident single-workgroup, pipelined, split (S % 4 != 0) and the
# beyond-index-range split path; two steps in a row so the update compounds
BN_RUNNING_SHAPES = [(128, 64, 3844), (5, 2, 7), (2, 4, 4100), (33, 2, 16000), (65, 2, 32768),
                     (9, 5, 20003), (128, 32, 49), (3, 3, 1017)]


def _check_running(rm_gpu, rv_gpu, rm_ref, rv_ref, what):
    em = float(np.max(np.abs(H(rm_gpu) - rm_ref)))
    ev = float(np.max(np.abs(H(rv_gpu) - rv_ref) / np.maximum(np.abs(rv_ref), 1e-30)))
    _log("%s: running_mean max_abs_err %.3e, running_var max_rel_err %.3e" % (what, em, ev))
    assert em <= 1e-5
    assert ev <= 1e-5


@pytest.mark.parametrize("shape", BN_RUNNING_SHAPES)
def test_bn_running_statistics(dev, nra, orc, shape):
    N, C, S = shape
    g = np.random.Generator(np.random.PCG64(N * 7919 + C * 31 + S))
    z = g.standard_normal(shape).astype(np.float32)
    x = (z * g.uniform(0.1, 3, (1, C, 1)) + g.uniform(-5, 5, (1, C, 1))).astype(np.float32)
    rm0 = g.uniform(-1, 1, C).astype(np.float32)
    rv0 = g.uniform(0.5, 2, C).astype(np.float32)
    rm, rv = T(rm0, dev), T(rv0, dev)
    xt = T(x, dev)
    _, mean, var = orc.batch_norm_train(x, with_stats=True)
    rm_ref, rv_ref = rm0, rv0
    for step in range(2):
        y = nra.bn_train_forward(xt, running_mean=rm, running_var=rv, momentum=0.3)
        rm_ref, rv_ref = orc.bn_running_update(mean, var, N * S, rm_ref, rv_ref, momentum=0.3)
        _check_running(rm, rv, rm_ref, rv_ref, "bn_train %s step %d" % (shape, step))
    assert maxerr(H(y), orc.batch_norm_train(x)) <= TOL


# ------------------------------------------------------------------------------------------
# Conv -> normalize -> epilogue
# ------------------------------------------------------------------------------------------
def test_conv_bn_workload4_full(dev, nra, orc):
    import torch

    inp = synth.host_inputs(4)
    t = lambda a: T(a, dev)
    args = (t(inp["x"]), t(inp["w"]), t(inp["b"]))
    kw = dict(norm=nra.NR_NORM_BATCH_TRAIN, eps=inp["eps"], gamma=t(inp["gamma"]),
              beta=t(inp["beta"]), out_scale=inp["scale"])
    # the output starts as NaN, so a position left unwritten fails the comparison
    out = torch.full((128, 64, 62, 62), float("nan"), device=dev)
    nra.conv_norm_epilogue_forward(*args, out, **kw)
    ref = orc.conv_norm_epilogue(inp["x"], inp["w"], inp["b"], batch=True, gamma=inp["gamma"],
                                 beta=inp["beta"], out_scale=inp["scale"])
    err = maxerr(H(out), ref)
    _log("conv2d(8->64) + bn_train + x2 on x[128,8,64,64]: max_abs_err %.3e" % err)
    assert err <= TOL
    assert torch.equal(out, nra.conv_norm_epilogue_forward(*args, **kw))


def test_conv_in3d_workload5_full(dev, nra, orc):
    import torch

    inp = synth.host_inputs(5)
    t = lambda a: T(a, dev)
    args = (t(inp["x"]), t(inp["w"]), t(inp["b"]))
    kw = dict(norm=nra.NR_NORM_INSTANCE, eps=inp["eps"], pre_mul=t(inp["mult"]),
              clamp=inp["clamp"], post_mul=t(inp["mult"]), reduce_max_c=True)
    out = nra.conv_norm_epilogue_forward(*args, **kw)
    ref = orc.conv_norm_epilogue(inp["x"], inp["w"], inp["b"], batch=False, pre_mul=inp["mult"],
                                 clamp=inp["clamp"], post_mul=inp["mult"], reduce_max_c=True)
    err = maxerr(H(out), ref)
    _log("conv3d(3->16) + IN3d + clamp + max_c on x[128,3,16,32,32]: max_abs_err %.3e" % err)
    assert out.shape == (128, 14, 30, 30)
    assert err <= TOL
    assert torch.equal(out, nra.conv_norm_epilogue_forward(*args, **kw))


CHAIN_CASES = [
    # (x shape, Cout, batch, reduce_max_c, use every optional parameter)
    ((2, 3, 9, 11), 5, True, False, True),
    ((2, 3, 9, 11), 5, False, True, True),
    ((3, 1, 5, 6, 7), 20, False, False, True),
    ((3, 1, 5, 6, 7), 20, True, True, True),
    ((1, 4, 3, 3), 16, True, False, False),
    ((4, 2, 6, 7, 9), 17, False, True, False),
    ((2, 8, 34, 35), 64, True, False, True),
    ((1, 2, 260, 260), 3, False, False, True),   # in place, pipelined instance chain (5 parts)
    ((40, 2, 42, 42), 4, True, False, True),     # in place, pipelined batch chain (4 parts)
    ((9, 2, 40, 42), 6, True, False, False),     # in place, one workgroup per channel
    # shapes of the matrix-core producers (2-D C_in 8 -> 64, 3-D C_in 3 -> 16), ragged tails
    ((2, 8, 15, 13), 64, True, False, True),     # 143 positions: scalar stores, split path
    ((3, 8, 20, 22), 64, True, False, True),     # 360 positions: 16-byte stores, in place
    ((2, 3, 6, 9, 11), 16, False, True, True),   # 252 positions, max over channels
    ((2, 3, 5, 7, 8), 16, False, True, True),    # 90 positions: scalar stores
    # the 2-D 64-wide producer (32-position tiles taken from a counter): one row, odd heights
    # (rows starting at position 2 mod 4), split path, max over channels
    ((1, 8, 3, 64), 64, True, False, True),
    ((3, 8, 9, 64), 64, True, False, True),
    ((5, 8, 17, 64), 64, False, False, True),
    ((2, 8, 6, 64), 64, True, True, True),
    # the 2-D matrix producer with whole boxes of 4 output rows (even output heights): boxes of
    # 4, 4, 2 rows; instance statistics with the max over channels
    ((3, 8, 12, 64), 64, True, False, True),
    ((2, 8, 10, 64), 64, False, True, True),
    # instance statistics and the max over 16 channels on 2-D shapes: 1596 and 16384 positions
    ((3, 4, 40, 44), 16, False, True, True),
    ((2, 2, 130, 130), 16, False, True, False),
    # instance statistics taken by the ring producer itself: without the max (90 positions),
    # one tile per workgroup (an item over 2 workgroups), workgroups spanning many items, and
    # the 2-D ring shape
    ((2, 3, 5, 7, 8), 16, False, False, True),
    ((64, 3, 4, 5, 6), 16, False, True, True),
    ((1000, 3, 3, 4, 5), 16, False, True, False),
    ((900, 3, 3, 6, 7), 16, False, False, True),
    ((3, 8, 9, 30), 64, False, True, True),
    # 97 statistics slots per item (several per slot lane), and one item over 512 workgroups:
    # past 128 slots the statistics come from a pass over the conv output instead
    ((8, 3, 8, 34, 34), 16, False, True, True),
    ((1, 3, 10, 34, 34), 16, False, True, True),
]


@pytest.mark.parametrize("shape,cout,batch,red,full", CHAIN_CASES)
def test_conv_chain_general(dev, nra, orc, shape, cout, batch, red, full):
    g = np.random.Generator(np.random.PCG64(len(shape) * 100 + cout))
    x = g.standard_normal(shape).astype(np.float32)
    dims = len(shape) - 2
    w = (g.standard_normal((cout, shape[1]) + (3,) * dims) * 0.3).astype(np.float32)
    b = g.standard_normal(cout).astype(np.float32) if full else None
    opt = lambda a: a if full else None
    pm = opt(g.standard_normal(cout).astype(np.float32))
    gm = opt(g.uniform(0.5, 1.5, cout).astype(np.float32))
    bt = opt(g.uniform(-0.5, 0.5, cout).astype(np.float32))
    qm = opt(g.standard_normal(cout).astype(np.float32))
    clamp = (-0.8, 1.1) if full else None
    t = lambda a: None if a is None else T(a, dev)
    out = nra.conv_norm_epilogue_forward(
        t(x), t(w), t(b), norm=nra.NR_NORM_BATCH_TRAIN if batch else nra.NR_NORM_INSTANCE,
        pre_mul=t(pm), gamma=t(gm), beta=t(bt), out_scale=1.5 if full else 1.0, clamp=clamp,
        post_mul=t(qm), reduce_max_c=red)
    ref = orc.conv_norm_epilogue(x, w, b, batch=batch, pre_mul=pm, gamma=gm, beta=bt,
                                 out_scale=1.5 if full else 1.0, clamp=clamp, post_mul=qm,
                                 reduce_max_c=red)
    err = maxerr(H(out), ref)
    _log("chain %s Cout %d batch %s max_c %s: max_abs_err %.3e" % (shape, cout, batch, red, err))
    assert err <= TOL


@pytest.mark.parametrize("cl", [False, True])
@pytest.mark.parametrize("red", [False, True])
def test_conv_chain_ring_statistics_offset_inputs(dev, nra, orc, cl, red):
    """Instance statistics taken inside the 3-D ring producer on inputs with a large common
    offset: the conv output's mean is ~20 standard deviations from zero, which a sum-of-squares
    shortcut without a shift would not survive."""
    g = np.random.Generator(np.random.PCG64(4242 + 2 * cl + red))
    shape = (6, 3, 7, 12, 13)
    x = (10.0 + 0.5 * g.standard_normal(shape)).astype(np.float32)
    w = (g.standard_normal((16, 3, 3, 3, 3)) * 0.3).astype(np.float32)
    b = g.standard_normal(16).astype(np.float32)
    pm = g.uniform(0.5, 1.5, 16).astype(np.float32)
    xin = _to_cl(x) if cl else x
    out = nra.conv_norm_epilogue_forward(T(xin, dev), T(w, dev), T(b, dev), norm=nra.NR_NORM_INSTANCE,
                                         pre_mul=T(pm, dev), clamp=(-3.0, 3.0), reduce_max_c=red,
                                         channels_last=cl)
    ref = orc.conv_norm_epilogue(x, w, b, batch=False, pre_mul=pm, clamp=(-3.0, 3.0),
                                 reduce_max_c=red)
    got = H(out) if (red or not cl) else np.moveaxis(H(out), -1, 1)
    err = maxerr(got, ref)
    _log("ring statistics, offset inputs, cl %s max_c %s: max_abs_err %.3e" % (cl, red, err))
    assert err <= TOL


CHAIN_RUNNING_CASES = [
    # (x shape, Cout, reduce_max_c): split path, pipelined in place, one workgroup per channel,
    # max over channels, the 2-D ring producer shape, and the 64-wide matrix producer
    ((2, 8, 15, 13), 64, False), ((40, 2, 42, 42), 4, False), ((9, 2, 40, 42), 6, False),
    ((3, 1, 5, 6, 7), 20, True), ((3, 8, 20, 22), 64, False),
    # the 2-D 64-wide matrix producer with even output height: batch norm by recomputation
    ((3, 8, 12, 64), 64, False),
]


@pytest.mark.parametrize("shape,cout,red", CHAIN_RUNNING_CASES)
def test_conv_chain_running_statistics(dev, nra, orc, shape, cout, red):
    g = np.random.Generator(np.random.PCG64(len(shape) * 1000 + cout * 3 + shape[0]))
    x = g.standard_normal(shape).astype(np.float32)
    dims = len(shape) - 2
    w = (g.standard_normal((cout, shape[1]) + (3,) * dims) * 0.3).astype(np.float32)
    b = g.standard_normal(cout).astype(np.float32)
    pm = g.uniform(0.5, 2, cout).astype(np.float32)
    rm0 = g.uniform(-1, 1, cout).astype(np.float32)
    rv0 = g.uniform(0.5, 2, cout).astype(np.float32)
    t = lambda a: T(a, dev)
    rm, rv = t(rm0), t(rv0)
    out = nra.conv_norm_epilogue_forward(t(x), t(w), t(b), norm=nra.NR_NORM_BATCH_TRAIN,
                                         pre_mul=t(pm), reduce_max_c=red, running_mean=rm,
                                         running_var=rv, momentum=0.25)
    # the statistics are those of the normalized input: conv + bias, times pre_mul
    c = orc.conv_k3(x, w, b) * pm.astype(np.float64).reshape((1, cout) + (1,) * dims)
    _, mean, var = orc.batch_norm_train(c, with_stats=True)
    count = c.size // cout
    rm_ref, rv_ref = orc.bn_running_update(mean, var, count, rm0, rv0, momentum=0.25)
    _check_running(rm, rv, rm_ref, rv_ref, "chain %s Cout %d max_c %s" % (shape, cout, red))
    ref = orc.conv_norm_epilogue(x, w, b, batch=True, pre_mul=pm, reduce_max_c=red)
    assert maxerr(H(out), ref) <= TOL


# eval-mode batch norm folded into the conv: the two model shapes, plus ragged small cases
# ((3, 8, 10, 64): the 2-D matrix producer with an even output height)
CONV_EVAL_CASES = [((128, 8, 64, 64), 64), ((128, 3, 16, 32, 32), 16), ((2, 3, 9, 11), 5),
                   ((3, 2, 5, 6, 7), 17), ((1, 8, 15, 13), 64), ((7, 8, 13, 64), 64),
                   ((3, 8, 10, 64), 64)]


@pytest.mark.parametrize("shape,cout", CONV_EVAL_CASES)
def test_conv_bn_eval(dev, nra, orc, shape, cout):
    import torch

    g = np.random.Generator(np.random.PCG64(cout * 77 + len(shape)))
    x = g.standard_normal(shape).astype(np.float32)
    dims = len(shape) - 2
    w = (g.standard_normal((cout, shape[1]) + (3,) * dims) * 0.3).astype(np.float32)
    b = g.standard_normal(cout).astype(np.float32)
    rm = g.uniform(-1, 1, cout).astype(np.float32)
    rv = g.uniform(0.3, 3, cout).astype(np.float32)
    gm = g.uniform(0.5, 1.5, cout).astype(np.float32)
    bt = g.uniform(-0.5, 0.5, cout).astype(np.float32)
    t = lambda a: T(a, dev)
    out = nra.conv_bn_eval_forward(t(x), t(w), t(b), t(rm), t(rv), gamma=t(gm), beta=t(bt),
                                   out_scale=2.0)
    ref = orc.conv_bn_eval(x, w, b, rm, rv, gamma=gm, beta=bt, scale=2.0)
    err = maxerr(H(out), ref)
    _log("conv_bn_eval %s Cout %d: max_abs_err %.3e" % (shape, cout, err))
    assert err <= TOL
    out2 = nra.conv_bn_eval_forward(t(x), t(w), None, t(rm), t(rv))  # no bias, no affine
    assert maxerr(H(out2), orc.conv_bn_eval(x, w, None, rm, rv)) <= TOL
    assert torch.equal(out, nra.conv_bn_eval_forward(t(x), t(w), t(b), t(rm), t(rv), gamma=t(gm),
                                                     beta=t(bt), out_scale=2.0))


# channels last: x [N, spatial, C_in], out [N, spatial, C_out] (or the channel max); the oracle
# runs on the planar transpose of the same values
CL_CASES = [
    # (planar x shape, Cout, batch, reduce_max_c, every optional parameter)
    ((128, 3, 16, 32, 32), 16, False, True, True),   # the IN3d model's shape, full size
    ((128, 8, 64, 64), 64, True, False, True),       # the batch-norm model's shape, full size
    ((2, 3, 9, 11), 5, True, False, True),           # vector-ALU producer
    ((4, 2, 6, 7, 9), 17, False, True, False),
    ((3, 1, 5, 6, 7), 20, False, True, True),
    ((2, 8, 15, 13), 64, False, False, True),        # 2-D matrix-core ring, ragged rows
    ((1, 8, 3, 64), 64, True, False, True),
    ((2, 3, 6, 9, 11), 16, False, True, True),       # 3-D matrix-core ring, scalar staging
    ((3, 3, 5, 7, 8), 16, True, False, True),
    ((2, 3, 5, 6, 7), 8, False, True, True),         # two lanes per position
    ((3, 2, 9, 10), 4, False, False, True),          # one lane per position, in place
    ((2, 2, 7, 9), 128, True, False, False),         # 32 lanes per position
    ((64, 3, 4, 5, 6), 16, False, True, True),       # ring statistics: one tile per workgroup
    ((1000, 3, 3, 4, 5), 16, False, False, True),    # workgroups spanning many items, in place
    ((8, 3, 8, 34, 34), 16, False, True, True),      # 97 slots: several per chunk lane
    ((1, 3, 10, 34, 34), 16, False, True, False),    # over 128 slots: statistics pass instead
]


def _to_cl(a):
    return np.ascontiguousarray(np.moveaxis(a, 1, -1))


@pytest.mark.parametrize("shape,cout,batch,red,full", CL_CASES)
def test_conv_chain_channels_last(dev, nra, orc, shape, cout, batch, red, full):
    g = np.random.Generator(np.random.PCG64(len(shape) * 10000 + cout * 7 + shape[0]))
    x = g.standard_normal(shape).astype(np.float32)
    dims = len(shape) - 2
    w = (g.standard_normal((cout, shape[1]) + (3,) * dims) * 0.3).astype(np.float32)
    b = g.standard_normal(cout).astype(np.float32) if full else None
    opt = lambda a: a if full else None
    pm = opt(g.standard_normal(cout).astype(np.float32))
    gm = opt(g.uniform(0.5, 1.5, cout).astype(np.float32))
    bt = opt(g.uniform(-0.5, 0.5, cout).astype(np.float32))
    qm = opt(g.standard_normal(cout).astype(np.float32))
    clamp = (-0.8, 1.1) if full else None
    import torch

    t = lambda a: None if a is None else T(a, dev)
    args = (t(_to_cl(x)), t(w), t(b))
    kw = dict(norm=nra.NR_NORM_BATCH_TRAIN if batch else nra.NR_NORM_INSTANCE, pre_mul=t(pm),
              gamma=t(gm), beta=t(bt), out_scale=1.5 if full else 1.0, clamp=clamp,
              post_mul=t(qm), reduce_max_c=red, channels_last=True)
    out = nra.conv_norm_epilogue_forward(*args, **kw)
    # fixed merge orders everywhere: a second call gives the same bits
    assert torch.equal(out, nra.conv_norm_epilogue_forward(*args, **kw))
    ref = orc.conv_norm_epilogue(x, w, b, batch=batch, pre_mul=pm, gamma=gm, beta=bt,
                                 out_scale=1.5 if full else 1.0, clamp=clamp, post_mul=qm,
                                 reduce_max_c=red)
    got = H(out) if red else np.moveaxis(H(out), -1, 1)
    err = maxerr(got, ref)
    _log("channels-last chain %s Cout %d batch %s max_c %s: max_abs_err %.3e"
         % (shape, cout, batch, red, err))
    assert err <= TOL


@pytest.mark.parametrize("red", [False, True])
def test_conv_chain_channels_last_misaligned_out(dev, nra, orc, red):
    # `out` four bytes off 16-byte alignment: without the max the conv writes it directly
    # (scalar stores) and the epilogue normalizes it in place with one thread per position,
    # merging the producer's statistics slots itself; with the max only the maxima move
    import torch

    g = np.random.Generator(np.random.PCG64(909 + red))
    shape = (2, 3, 6, 9, 11)
    x = g.standard_normal(shape).astype(np.float32)
    w = (g.standard_normal((16, 3, 3, 3, 3)) * 0.3).astype(np.float32)
    b = g.standard_normal(16).astype(np.float32)
    pm = g.standard_normal(16).astype(np.float32)
    osh = (2, 4, 7, 9) if red else (2, 4, 7, 9, 16)
    n = int(np.prod(osh))
    buf = torch.empty(n + 1, dtype=torch.float32, device=dev)
    out = buf[1:].view(osh)
    assert out.data_ptr() % 16 != 0
    nra.conv_norm_epilogue_forward(T(_to_cl(x), dev), T(w, dev), T(b, dev), out=out,
                                   norm=nra.NR_NORM_INSTANCE, pre_mul=T(pm, dev),
                                   clamp=(-1.0, 1.0), post_mul=T(pm, dev), reduce_max_c=red,
                                   channels_last=True)
    ref = orc.conv_norm_epilogue(x, w, b, batch=False, pre_mul=pm, clamp=(-1.0, 1.0),
                                 post_mul=pm, reduce_max_c=red)
    got = H(out) if red else np.moveaxis(H(out), -1, 1)
    err = maxerr(got, ref)
    _log("channels-last chain, misaligned out, max_c %s: max_abs_err %.3e" % (red, err))
    assert err <= TOL


def test_conv_chain_channels_last_running_statistics(dev, nra, orc):
    g = np.random.Generator(np.random.PCG64(4242))
    x = g.standard_normal((4, 3, 6, 10, 12)).astype(np.float32)
    w = (g.standard_normal((16, 3, 3, 3, 3)) * 0.3).astype(np.float32)
    b = g.standard_normal(16).astype(np.float32)
    rm0 = g.uniform(-1, 1, 16).astype(np.float32)
    rv0 = g.uniform(0.5, 2, 16).astype(np.float32)
    t = lambda a: T(a, dev)
    rm, rv = t(rm0), t(rv0)
    out = nra.conv_norm_epilogue_forward(t(_to_cl(x)), t(w), t(b), norm=nra.NR_NORM_BATCH_TRAIN,
                                         running_mean=rm, running_var=rv, momentum=0.2,
                                         channels_last=True)
    c = orc.conv_k3(x, w, b)
    _, mean, var = orc.batch_norm_train(c, with_stats=True)
    rm_ref, rv_ref = orc.bn_running_update(mean, var, c.size // 16, rm0, rv0, momentum=0.2)
    _check_running(rm, rv, rm_ref, rv_ref, "channels-last chain running statistics")
    ref = orc.conv_norm_epilogue(x, w, b, batch=True)
    assert maxerr(np.moveaxis(H(out), -1, 1), ref) <= TOL


@pytest.mark.parametrize("shape,cout", [((128, 8, 64, 64), 64), ((128, 3, 16, 32, 32), 16),
                                        ((2, 3, 9, 11), 5), ((1, 8, 15, 13), 64)])
def test_conv_bn_eval_channels_last(dev, nra, orc, shape, cout):
    g = np.random.Generator(np.random.PCG64(cout * 31 + len(shape)))
    x = g.standard_normal(shape).astype(np.float32)
    dims = len(shape) - 2
    w = (g.standard_normal((cout, shape[1]) + (3,) * dims) * 0.3).astype(np.float32)
    b = g.standard_normal(cout).astype(np.float32)
    rm = g.uniform(-1, 1, cout).astype(np.float32)
    rv = g.uniform(0.3, 3, cout).astype(np.float32)
    t = lambda a: T(a, dev)
    out = nra.conv_bn_eval_forward(t(_to_cl(x)), t(w), t(b), t(rm), t(rv), out_scale=2.0,
                                   channels_last=True)
    ref = orc.conv_bn_eval(x, w, b, rm, rv, scale=2.0)
    err = maxerr(np.moveaxis(H(out), -1, 1), ref)
    _log("channels-last conv_bn_eval %s Cout %d: max_abs_err %.3e" % (shape, cout, err))
    assert err <= TOL


def test_conv_vector_alu_producer(dev, nra, orc, monkeypatch):
    # the vector-ALU conv producer (used for shapes without a matrix-core instantiation),
    # forced on the IN3d workload
    monkeypatch.setenv("NORMRED_CONV", "valu")
    inp = synth.host_inputs(5)
    t = lambda a: T(a, dev)
    out = nra.conv_norm_epilogue_forward(t(inp["x"][:16]), t(inp["w"]), t(inp["b"]),
                                         norm=nra.NR_NORM_INSTANCE, pre_mul=t(inp["mult"]),
                                         clamp=inp["clamp"], post_mul=t(inp["mult"]),
                                         reduce_max_c=True)
    ref = orc.conv_norm_epilogue(inp["x"][:16], inp["w"], inp["b"], batch=False,
                                 pre_mul=inp["mult"], clamp=inp["clamp"], post_mul=inp["mult"],
                                 reduce_max_c=True)
    assert maxerr(H(out), ref) <= TOL


@pytest.mark.parametrize("mode", ["bf16x6", "fp32"])
def test_conv2d_matrix_producer_fp32_accuracy(dev, nra, orc, monkeypatch, mode):
    # The 2-D C_in 8 -> C_out 64 producer read through the eval entry point with an identity
    # fold (running mean 0, running variance 1, eps 0, no affine: W and b pass unchanged), so
    # the output is the conv itself. Both matrix forms must be fp32-accurate element by
    # element: |conv - fp64 conv| <= 2^-20 (sum |x||w| + |b|). The default splits every value
    # into three bf16 parts (six partial products); a two-part split would leave errors near
    # 4e-6 of that sum and fail. "fp32" selects the fp32 matrix instruction.
    if mode == "fp32":
        monkeypatch.setenv("NORMRED_CONV", "fp32")
    g = np.random.Generator(np.random.PCG64(7272))
    x = (g.standard_normal((3, 8, 20, 64)) * 3).astype(np.float32)  # 18 output rows: last box of 2
    bound = 1 / np.sqrt(72)
    w = g.uniform(-bound, bound, (64, 8, 3, 3)).astype(np.float32)
    b = g.uniform(-bound, bound, 64).astype(np.float32)
    t = lambda a: T(a, dev)
    out = nra.conv_bn_eval_forward(t(x), t(w), t(b), t(np.zeros(64, np.float32)),
                                   t(np.ones(64, np.float32)), eps=0.0)
    ref = orc.conv_k3(x, w, b)
    den = orc.conv_k3(np.abs(x), np.abs(w), np.abs(b))
    ratio = float(np.max(np.abs(H(out).astype(np.float64) - ref) / den))
    _log("conv2d producer %s: max |err| / (sum|x||w| + |b|) = %.3e" % (mode, ratio))
    assert ratio <= 2.0 ** -20


def test_conv2d_fp32_matrix_producer_chain(dev, nra, orc, monkeypatch):
    # the fp32-instruction form of the 2-D producer through the batch-norm chain
    monkeypatch.setenv("NORMRED_CONV", "fp32")
    inp = synth.host_inputs(4)
    t = lambda a: T(a, dev)
    x = np.ascontiguousarray(inp["x"][:8])
    out = nra.conv_norm_epilogue_forward(t(x), t(inp["w"]), t(inp["b"]),
                                         norm=nra.NR_NORM_BATCH_TRAIN, gamma=t(inp["gamma"]),
                                         beta=t(inp["beta"]), out_scale=2.0)
    ref = orc.conv_norm_epilogue(x, inp["w"], inp["b"], batch=True, gamma=inp["gamma"],
                                 beta=inp["beta"], out_scale=2.0)
    assert maxerr(H(out), ref) <= TOL


@pytest.mark.parametrize("shape,misalign", [((1, 8, 4, 64), False), ((3, 8, 18, 64), True)])
def test_conv2d_bn_recompute_edges(dev, nra, orc, shape, misalign):
    # batch norm on the 2-D matrix producer's shape: a single box of two output rows (waves
    # repeat the last tile, whose positions must count once in the statistics), and an x four
    # bytes off 16-byte alignment, which the producer cannot take (the in-place plan runs)
    import torch

    g = np.random.Generator(np.random.PCG64(4242 + shape[2]))
    x = (g.standard_normal(shape) * 2 + 0.5).astype(np.float32)
    w = (g.standard_normal((64, 8, 3, 3)) * 0.2).astype(np.float32)
    b = g.standard_normal(64).astype(np.float32)
    rm0 = g.uniform(-1, 1, 64).astype(np.float32)
    rv0 = g.uniform(0.5, 2, 64).astype(np.float32)
    if misalign:
        buf = torch.empty(x.size + 1, dtype=torch.float32, device=dev)
        xt = buf[1:].view(shape)
        xt.copy_(torch.from_numpy(x))
        assert xt.data_ptr() % 16 != 0
    else:
        xt = T(x, dev)
    rm, rv = T(rm0, dev), T(rv0, dev)
    out = nra.conv_norm_epilogue_forward(xt, T(w, dev), T(b, dev), norm=nra.NR_NORM_BATCH_TRAIN,
                                         running_mean=rm, running_var=rv, momentum=0.5)
    ref = orc.conv_norm_epilogue(x, w, b, batch=True)
    err = maxerr(H(out), ref)
    _log("conv2d bn %s misaligned %s: max_abs_err %.3e" % (shape, misalign, err))
    assert err <= TOL
    c = orc.conv_k3(x, w, b)
    _, mean, var = orc.batch_norm_train(c, with_stats=True)
    rm_ref, rv_ref = orc.bn_running_update(mean, var, c.size // 64, rm0, rv0, momentum=0.5)
    _check_running(rm, rv, rm_ref, rv_ref, "conv2d bn %s" % (shape,))


@pytest.mark.parametrize("n,h", [(1, 6), (1, 66), (3, 10), (7, 34), (2, 36), (5, 20)])
def test_conv2d_64wide_box_geometry(dev, nra, orc, n, h):
    # the 2-D 64-wide producer over boxes of 4 output rows: output heights 4, 64, 8, 32 fill
    # every box, 34 and 18 end each batch item on a box of 2 rows (4 tiles for 8 tile slots:
    # overlapping and repeated tiles, whose positions the statistics must count once); 1-7
    # items put from one to a few boxes in each workgroup. Batch norm by recomputation (with
    # running statistics) and the eval chain, both against the oracle.
    g = np.random.Generator(np.random.PCG64(6000 + 97 * n + h))
    x = (g.standard_normal((n, 8, h, 64)) * 1.5 - 0.25).astype(np.float32)
    bound = 1 / np.sqrt(72)
    w = g.uniform(-bound, bound, (64, 8, 3, 3)).astype(np.float32)
    b = g.uniform(-bound, bound, 64).astype(np.float32)
    gm = g.uniform(0.5, 1.5, 64).astype(np.float32)
    bt = g.uniform(-0.5, 0.5, 64).astype(np.float32)
    rm0 = g.uniform(-0.2, 0.2, 64).astype(np.float32)
    rv0 = g.uniform(0.5, 1.5, 64).astype(np.float32)
    rm, rv = T(rm0, dev), T(rv0, dev)
    import torch

    # outputs start as NaN: every position must be written (the producer drops the stores of
    # positions an earlier tile of the same box wrote)
    nan_out = lambda: torch.full((n, 64, h - 2, 62), float("nan"), device=dev)
    out = nra.conv_norm_epilogue_forward(T(x, dev), T(w, dev), T(b, dev), nan_out(), norm=nra.NR_NORM_BATCH_TRAIN,
                                         gamma=T(gm, dev), beta=T(bt, dev), out_scale=2.0,
                                         running_mean=rm, running_var=rv, momentum=0.3)
    err = maxerr(H(out), orc.conv_norm_epilogue(x, w, b, batch=True, gamma=gm, beta=bt, out_scale=2.0))
    c = orc.conv_k3(x, w, b)
    _, mean, var = orc.batch_norm_train(c, with_stats=True)
    rm_ref, rv_ref = orc.bn_running_update(mean, var, c.size // 64, rm0, rv0, momentum=0.3)
    _check_running(rm, rv, rm_ref, rv_ref, "conv2d 64-wide n %d h %d" % (n, h))
    ev = nra.conv_bn_eval_forward(T(x, dev), T(w, dev), T(b, dev), T(rm0, dev), T(rv0, dev), nan_out(),
                                  gamma=T(gm, dev), beta=T(bt, dev), out_scale=2.0)
    err_ev = maxerr(H(ev), orc.conv_bn_eval(x, w, b, rm0, rv0, gamma=gm, beta=bt, scale=2.0))
    _log("conv2d 64-wide n %d h %d: bn max_abs_err %.3e, eval %.3e" % (n, h, err, err_ev))
    assert err <= TOL
    assert err_ev <= TOL


# The 3-D bf16 producer's shape (C_in 3 -> C_out 16 over 32 x 32 input planes) at sizes that
# give workgroups ranges of one tile (one output row) up to several output slices, ranges
# crossing batch items, a single output slice (D = 3), and the many statistics slots of small
# batches; every plan on top of it: instance norm with and without the channel max, batch
# norm, and the eval fold
C3_CASES = [(1, 3), (2, 5), (3, 4), (5, 7), (16, 4), (8, 16),
            (64, 3),   # one output slice per item: ranges of 3-4 rows cross items at every turn
            (40, 5)]   # ranges spanning a few items, each restaging its window


@pytest.mark.parametrize("cl", [False, True])
@pytest.mark.parametrize("n,d", C3_CASES)
def test_conv3d_32x32_planes(dev, nra, orc, n, d, cl):
    g = np.random.Generator(np.random.PCG64(7000 + 31 * n + d))
    x = (g.standard_normal((n, 3, d, 32, 32)) * 1.3 + 0.4).astype(np.float32)
    w = (g.standard_normal((16, 3, 3, 3, 3)) / 9).astype(np.float32)
    b = (g.standard_normal(16) * 0.3).astype(np.float32)
    gm = g.uniform(0.5, 1.5, 16).astype(np.float32)
    bt = g.uniform(-0.5, 0.5, 16).astype(np.float32)
    pm = g.uniform(0.5, 1.5, 16).astype(np.float32)
    xin = np.moveaxis(x, 1, -1) if cl else x
    for batch, red in ((False, True), (False, False), (True, False)):
        out = nra.conv_norm_epilogue_forward(
            T(xin, dev), T(w, dev), T(b, dev), norm=nra.NR_NORM_BATCH_TRAIN if batch else nra.NR_NORM_INSTANCE,
            pre_mul=None if batch else T(pm, dev), gamma=T(gm, dev), beta=T(bt, dev), out_scale=1.5,
            clamp=None if batch else (-1.0, 1.0), post_mul=None if batch else T(pm, dev),
            reduce_max_c=red, channels_last=cl)
        ref = orc.conv_norm_epilogue(x, w, b, batch=batch, pre_mul=None if batch else pm, gamma=gm,
                                     beta=bt, out_scale=1.5, clamp=None if batch else (-1.0, 1.0),
                                     post_mul=None if batch else pm, reduce_max_c=red)
        got = H(out) if (red or not cl) else np.moveaxis(H(out), -1, 1)
        err = maxerr(got, ref)
        _log("conv3d 32x32 N %d D %d cl %d batch %d max_c %d: %.3e" % (n, d, cl, batch, red, err))
        assert err <= TOL
    rm = g.uniform(-0.3, 0.3, 16).astype(np.float32)
    rv = g.uniform(0.5, 2.0, 16).astype(np.float32)
    ev = nra.conv_bn_eval_forward(T(xin, dev), T(w, dev), T(b, dev), T(rm, dev), T(rv, dev),
                                  gamma=T(gm, dev), beta=T(bt, dev), out_scale=2.0, channels_last=cl)
    gev = H(ev) if not cl else np.moveaxis(H(ev), -1, 1)
    err = maxerr(gev, orc.conv_bn_eval(x, w, b, rm, rv, gamma=gm, beta=bt, scale=2.0))
    _log("conv3d 32x32 N %d D %d cl %d eval: %.3e" % (n, d, cl, err))
    assert err <= TOL


def test_conv3d_32x32_matches_fp32_ring(dev, nra, orc, monkeypatch):
    # the bf16-split producer and the fp32 ring (NORMRED_CONV=fp32) on the IN3d model's shape:
    # both within the tolerance of the oracle on sampled batch items, and of each other everywhere
    import synth

    i5 = synth.host_inputs(5)
    x, w, b = T(i5["x"], dev), T(i5["w"], dev), T(i5["b"], dev)
    rm = T(np.linspace(-0.2, 0.2, 16).astype(np.float32), dev)
    rv = T(np.linspace(0.5, 1.5, 16).astype(np.float32), dev)
    got = H(nra.conv_bn_eval_forward(x, w, b, rm, rv))
    monkeypatch.setenv("NORMRED_CONV", "fp32")
    ring = H(nra.conv_bn_eval_forward(x, w, b, rm, rv))
    monkeypatch.delenv("NORMRED_CONV")
    assert maxerr(got, ring) <= TOL
    for n in (0, 77, 127):
        ref = orc.conv_bn_eval(i5["x"][n:n + 1], i5["w"], i5["b"], H(rm), H(rv))
        assert maxerr(got[n:n + 1], ref) <= TOL


def _random_chain_cases(count, seed):
    g = np.random.Generator(np.random.PCG64(seed))
    cases = []
    for i in range(count):
        kind = i % 3
        if kind == 0:    # 2-D C_in 8 -> 64: the 64-wide matrix producer or the ring (other widths)
            shape, cout = (int(g.integers(1, 6)), 8, int(g.integers(3, 30)), int(g.choice([64, int(g.integers(3, 80))]))), 64
        elif kind == 1:  # 3-D C_in 3 -> 16: the ring
            shape, cout = (int(g.integers(1, 4)), 3, int(g.integers(3, 10)), int(g.integers(3, 30)), int(g.integers(3, 30))), 16
        else:            # other channel counts: the vector-ALU producer
            shape, cout = (int(g.integers(1, 4)), int(g.integers(1, 5)), int(g.integers(3, 20)), int(g.integers(3, 20))), int(g.choice([4, 8, 32]))
        batch = bool(g.integers(0, 2))
        cases.append((i, shape, cout, batch, bool(g.integers(0, 2)), (not batch) and bool(g.integers(0, 2)),
                      (not batch) and bool(g.integers(0, 2))))
    return cases


@pytest.mark.parametrize("i,shape,cout,batch,cl,red,clamp", _random_chain_cases(24, 9090))
def test_conv_chain_random_cases(dev, nra, orc, i, shape, cout, batch, cl, red, clamp):
    # seeded random shapes and flags through the conv -> normalize -> epilogue chain and the
    # eval fold, every producer, both layouts, against the oracle
    g = np.random.Generator(np.random.PCG64(4000 + i))
    x = (g.standard_normal(shape) * g.uniform(0.5, 2) + g.uniform(-1, 1)).astype(np.float32)
    cin = shape[1]
    k = (3,) * (len(shape) - 2)
    w = (g.standard_normal((cout, cin) + k) / np.sqrt(cin * 3 ** len(k))).astype(np.float32)
    b = (g.standard_normal(cout) * 0.3).astype(np.float32)
    gm = g.uniform(0.5, 1.5, cout).astype(np.float32)
    bt = g.uniform(-0.5, 0.5, cout).astype(np.float32)
    pm = None if batch else g.uniform(0.5, 1.5, cout).astype(np.float32)
    cl_rng = (-1.0, 1.0) if clamp else None
    xin = np.moveaxis(x, 1, -1) if cl else x
    out = nra.conv_norm_epilogue_forward(
        T(xin, dev), T(w, dev), T(b, dev), norm=nra.NR_NORM_BATCH_TRAIN if batch else nra.NR_NORM_INSTANCE,
        pre_mul=None if pm is None else T(pm, dev), gamma=T(gm, dev), beta=T(bt, dev), out_scale=1.5,
        clamp=cl_rng, post_mul=None if pm is None else T(pm, dev), reduce_max_c=red, channels_last=cl)
    ref = orc.conv_norm_epilogue(x, w, b, batch=batch, pre_mul=pm, gamma=gm, beta=bt, out_scale=1.5,
                                 clamp=cl_rng, post_mul=pm, reduce_max_c=red)
    got = H(out) if (red or not cl) else np.moveaxis(H(out), -1, 1)
    rm = g.uniform(-0.3, 0.3, cout).astype(np.float32)
    rv = g.uniform(0.5, 2.0, cout).astype(np.float32)
    ev = nra.conv_bn_eval_forward(T(xin, dev), T(w, dev), T(b, dev), T(rm, dev), T(rv, dev),
                                  gamma=T(gm, dev), beta=T(bt, dev), out_scale=2.0, channels_last=cl)
    gev = H(ev) if not cl else np.moveaxis(H(ev), -1, 1)
    err, err_ev = maxerr(got, ref), maxerr(gev, orc.conv_bn_eval(x, w, b, rm, rv, gamma=gm, beta=bt, scale=2.0))
    _log("random chain %d %s cout %d batch %d cl %d max_c %d clamp %d: %.3e, eval %.3e"
         % (i, shape, cout, batch, cl, red, clamp, err, err_ev))
    assert err <= TOL
    assert err_ev <= TOL


def test_conv2d_bn_recompute_statistics_accuracy(dev, nra, orc):
    # The recomputing batch-norm chain's statistics pass forms the apply pass's six bf16
    # products and sums each lane's values shifted by its first one. With momentum 1 the
    # running buffers receive the batch mean and unbiased variance themselves; they must match
    # the fp64 oracle to 1e-6 (of the channel's std for the mean, relative for the variance).
    # A conv from fewer products misses this: W in two parts biases the variance by ~1.9e-6
    # (measured), a one-product conv by ~4e-6.
    g = np.random.Generator(np.random.PCG64(8080))
    x = g.standard_normal((16, 8, 64, 64)).astype(np.float32)
    bound = 1 / np.sqrt(72)
    w = g.uniform(-bound, bound, (64, 8, 3, 3)).astype(np.float32)
    b = g.uniform(-bound, bound, 64).astype(np.float32)
    rm = T(np.zeros(64, np.float32), dev)
    rv = T(np.ones(64, np.float32), dev)
    nra.conv_norm_epilogue_forward(T(x, dev), T(w, dev), T(b, dev), norm=nra.NR_NORM_BATCH_TRAIN,
                                   running_mean=rm, running_var=rv, momentum=1.0)
    c = orc.conv_k3(x, w, b)
    _, mean, var = orc.batch_norm_train(c, with_stats=True)
    count = c.size // 64
    var_u = var * count / (count - 1)
    em = float(np.max(np.abs(H(rm) - mean) / np.sqrt(var)))
    ev = float(np.max(np.abs(H(rv) - var_u) / var_u))
    _log("recompute statistics: mean err / std %.3e, var rel err %.3e" % (em, ev))
    assert em <= 1e-6
    assert ev <= 1e-6


def test_conv2d_bn_recompute_offset_inputs(dev, nra, orc):
    # x = 1 + 0.1 N(0,1) puts each channel's conv output up to 25 (median 6) standard
    # deviations from zero (mean sum(w) + b, std 0.1 |w| ~ 0.06). The statistics pass sums each
    # lane's values shifted by its first one, so the sums stay at the spread's scale; unshifted
    # fp32 sums of squares over a lane's ~128 values would put the variance ~128 x 6e-8 x 25^2
    # ~ 5e-3 off, and the outputs ~1e-3. The outputs must meet the 1e-4 gate (at larger offsets
    # the conv's own fp32 accumulation, ~6e-8 of |y| per rounding, reaches the gate after the
    # division by the std, whatever the statistics). With momentum 1 the running buffers receive
    # the batch mean and unbiased variance: the mean must lie within the conv's error bound of
    # the fp64 oracle's (2^-20 (sum |x||w| + |b|) per value, tested for the producer alone), the
    # variance within 1e-5 relative.
    g = np.random.Generator(np.random.PCG64(8181))
    x = (1.0 + 0.1 * g.standard_normal((16, 8, 64, 64))).astype(np.float32)
    bound = 1 / np.sqrt(72)
    w = g.uniform(-bound, bound, (64, 8, 3, 3)).astype(np.float32)
    b = g.uniform(-bound, bound, 64).astype(np.float32)
    gm = g.uniform(0.5, 1.0, 64).astype(np.float32)
    bt = g.uniform(-0.5, 0.5, 64).astype(np.float32)
    rm = T(np.zeros(64, np.float32), dev)
    rv = T(np.ones(64, np.float32), dev)
    out = nra.conv_norm_epilogue_forward(T(x, dev), T(w, dev), T(b, dev), norm=nra.NR_NORM_BATCH_TRAIN,
                                         gamma=T(gm, dev), beta=T(bt, dev),
                                         running_mean=rm, running_var=rv, momentum=1.0)
    ref = orc.conv_norm_epilogue(x, w, b, batch=True, gamma=gm, beta=bt)
    err = maxerr(H(out), ref)
    c = orc.conv_k3(x, w, b)
    _, mean, var = orc.batch_norm_train(c, with_stats=True)
    std = np.sqrt(var)
    ratio = float(np.max(np.abs(mean) / std))
    conv_bound = 2.0 ** -20 * (np.abs(w).reshape(64, -1).sum(1) * float(np.abs(x).max()) + np.abs(b))
    count = c.size // 64
    var_u = var * count / (count - 1)
    em = np.abs(H(rm) - mean)
    ev = float(np.max(np.abs(H(rv) - var_u) / var_u))
    _log("recompute, offset inputs (|mean|/std up to %.1f): max_abs_err %.3e, mean err / std %.3e "
         "(bound %.3e), var rel err %.3e" % (ratio, err, float(np.max(em / std)),
                                             float(np.min(conv_bound / std)), ev))
    assert ratio > 20
    assert err <= TOL
    assert np.all(em <= conv_bound + 1e-6 * std)
    assert ev <= 1e-5


def test_conv_chain_max_c_misaligned_out(dev, nra, orc):
    # an `out` four bytes off 16-byte alignment: the epilogue takes its scalar path
    import torch

    i5 = synth.host_inputs(5)
    x = np.ascontiguousarray(i5["x"][:2])
    t = lambda a: T(a, dev)
    buf = torch.empty(2 * 14 * 30 * 30 + 1, dtype=torch.float32, device=dev)
    out = buf[1:].view(2, 14, 30, 30)
    assert out.data_ptr() % 16 != 0
    nra.conv_norm_epilogue_forward(t(x), t(i5["w"]), t(i5["b"]), out=out, norm=nra.NR_NORM_INSTANCE,
                                   pre_mul=t(i5["mult"]), clamp=(-1.0, 1.0), post_mul=t(i5["mult"]),
                                   reduce_max_c=True)
    ref = orc.conv_norm_epilogue(x, i5["w"], i5["b"], batch=False, pre_mul=i5["mult"],
                                 clamp=(-1.0, 1.0), post_mul=i5["mult"], reduce_max_c=True)
    assert maxerr(H(out), ref) <= TOL


def test_graph_capture_and_replay(dev, nra, orc):
    # every launch of these entry points can be captured: no hipMemsetAsync (fill kernels
    # instead), no synchronization, regular launches. Capture instance norm (read-once
    # pipelined), batch norm, the IN3d conv chain (4 items: statistics from a pass over the
    # conv output; 32 items, planar and channels last: statistics taken by the producer) and
    # the 2-D 64-wide producer's two chains (batch norm by recomputation, whose statistics pass
    # clears the tagged words the apply pass publishes; eval mode folded into W) and the 3-D
    # producer's eval conv once, then replay three times with eager changes of the inputs in
    # between, checking every replay against the oracle.
    import torch

    g = np.random.Generator(np.random.PCG64(5150))
    xi = T(g.standard_normal((2, 8, 100000)).astype(np.float32), dev)
    xb = T(g.standard_normal((16, 8, 3000)).astype(np.float32), dev)
    i5 = synth.host_inputs(5)
    xc = T(np.ascontiguousarray(i5["x"][:4]), dev)
    wc, bc, mc = T(i5["w"], dev), T(i5["b"], dev), T(i5["mult"], dev)
    yi, yb = torch.empty_like(xi), torch.empty_like(xb)
    yc = torch.empty((4, 14, 30, 30), device=dev)
    xd = T(np.ascontiguousarray(i5["x"][:32]), dev)
    xdl = torch.empty((32, 16, 32, 32, 3), device=dev)
    yd, ydl = torch.empty((32, 14, 30, 30), device=dev), torch.empty((32, 14, 30, 30), device=dev)
    i4 = synth.host_inputs(4)
    xe = T(np.ascontiguousarray(i4["x"][:12]), dev)
    we, be, ge, bte = T(i4["w"], dev), T(i4["b"], dev), T(i4["gamma"], dev), T(i4["beta"], dev)
    rme = T(g.uniform(-0.5, 0.5, 64).astype(np.float32), dev)
    rve = T(g.uniform(0.5, 2.0, 64).astype(np.float32), dev)
    ye, yev = torch.empty((12, 64, 62, 62), device=dev), torch.empty((12, 64, 62, 62), device=dev)
    rm3 = T(g.uniform(-0.3, 0.3, 16).astype(np.float32), dev)
    rv3 = T(g.uniform(0.5, 2.0, 16).astype(np.float32), dev)
    y3 = torch.empty((32, 16, 14, 30, 30), device=dev)
    s = torch.cuda.Stream(device=dev)
    ws = [torch.zeros(1 << 26, dtype=torch.uint8, device=dev) for _ in range(8)]
    chain = dict(norm=nra.NR_NORM_INSTANCE, pre_mul=mc, clamp=(-1.0, 1.0), post_mul=mc,
                 reduce_max_c=True)

    def work():
        nra.inorm_forward(xi, yi, workspace=ws[0], stream=s)
        nra.bn_train_forward(xb, yb, out_scale=2.0, workspace=ws[1], stream=s)
        nra.conv_norm_epilogue_forward(xc, wc, bc, yc, workspace=ws[2], stream=s, **chain)
        nra.conv_norm_epilogue_forward(xd, wc, bc, yd, workspace=ws[3], stream=s, **chain)
        nra.conv_norm_epilogue_forward(xdl, wc, bc, ydl, workspace=ws[4], stream=s,
                                       channels_last=True, **chain)
        nra.conv_norm_epilogue_forward(xe, we, be, ye, norm=nra.NR_NORM_BATCH_TRAIN, gamma=ge,
                                       beta=bte, out_scale=2.0, workspace=ws[5], stream=s)
        nra.conv_bn_eval_forward(xe, we, be, rme, rve, yev, gamma=ge, beta=bte, out_scale=2.0,
                                 workspace=ws[6], stream=s)
        nra.conv_bn_eval_forward(xd, wc, bc, rm3, rv3, y3, out_scale=0.5, workspace=ws[7], stream=s)

    s.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(s):
        work()  # warm-up outside the capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        work()
    torch.cuda.synchronize()
    for rep in range(3):
        with torch.no_grad():
            xi.mul_(1.5).add_(0.25)
            xb.mul_(0.5).sub_(1.0)
            xc.mul_(-1.0)
            xd.mul_(-0.5).add_(0.125)
            xdl.copy_(xd.permute(0, 2, 3, 4, 1))
            xe.mul_(0.75).add_(0.5)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for w in ws:
            assert nra.workspace_check(w) == 0
        e1 = maxerr(H(yi), orc.instance_norm(H(xi)))
        e2 = maxerr(H(yb), orc.batch_norm_train(H(xb), scale=2.0))
        e3 = maxerr(H(yc), orc.conv_norm_epilogue(H(xc), i5["w"], i5["b"], batch=False,
                                                  pre_mul=i5["mult"], clamp=(-1.0, 1.0),
                                                  post_mul=i5["mult"], reduce_max_c=True))
        rd = orc.conv_norm_epilogue(H(xd), i5["w"], i5["b"], batch=False, pre_mul=i5["mult"],
                                    clamp=(-1.0, 1.0), post_mul=i5["mult"], reduce_max_c=True)
        e4, e5 = maxerr(H(yd), rd), maxerr(H(ydl), rd)
        e6 = maxerr(H(ye), orc.conv_norm_epilogue(H(xe), i4["w"], i4["b"], batch=True,
                                                  gamma=i4["gamma"], beta=i4["beta"], out_scale=2.0))
        e7 = maxerr(H(yev), orc.conv_bn_eval(H(xe), i4["w"], i4["b"], H(rme), H(rve),
                                             gamma=i4["gamma"], beta=i4["beta"], scale=2.0))
        e8 = maxerr(H(y3), orc.conv_bn_eval(H(xd), i5["w"], i5["b"], H(rm3), H(rv3), scale=0.5))
        _log("graph replay %d: max_abs_err %.3e %.3e %.3e %.3e %.3e %.3e %.3e %.3e"
             % (rep, e1, e2, e3, e4, e5, e6, e7, e8))
        assert max(e1, e2, e3, e4, e5, e6, e7, e8) <= TOL


def test_concurrent_streams(dev, nra, orc):
    # The persistent kernels wait only on workgroups that have started (units handed out in
    # order; the Conv2d->BN apply pass waits on its lowest-numbered workgroups), so they need no
    # co-residency of their whole grid. Two streams run them at once, three rounds with no
    # synchronization between the launches: pipelined instance norm (4 parts per slice), batch
    # norm on channels of 16 parts, and the Conv2d->BN chain, each with its own workspace.
    # Every result must match the oracle and no exchange wait may have given up.
    import torch

    g = np.random.Generator(np.random.PCG64(7070))
    xi = T(g.standard_normal((8, 64, 256, 256)).astype(np.float32), dev)
    xb = T((g.standard_normal((64, 64, 62, 62)) * 2 + 1).astype(np.float32), dev)
    i4 = synth.host_inputs(4)
    xc = T(np.ascontiguousarray(i4["x"][:32]), dev)
    wc, bc, gc, btc = (T(i4[k], dev) for k in ("w", "b", "gamma", "beta"))
    s1, s2 = torch.cuda.Stream(device=dev), torch.cuda.Stream(device=dev)
    rounds = 3
    outs = []
    ws = []
    torch.cuda.synchronize()
    for r in range(rounds):
        yi, yb = torch.empty_like(xi), torch.empty_like(xb)
        yc = torch.empty((32, 64, 62, 62), device=dev)
        w3 = [torch.zeros(1 << 26, dtype=torch.uint8, device=dev) for _ in range(3)]
        torch.cuda.synchronize()
        nra.inorm_forward(xi, yi, workspace=w3[0], stream=s1)
        nra.bn_train_forward(xb, yb, workspace=w3[1], stream=s2)
        nra.conv_norm_epilogue_forward(xc, wc, bc, yc, norm=nra.NR_NORM_BATCH_TRAIN, gamma=gc,
                                       beta=btc, out_scale=2.0, workspace=w3[2], stream=s1 if r % 2 else s2)
        outs.append((yi, yb, yc))
        ws += w3
    torch.cuda.synchronize()
    for w in ws:
        assert nra.workspace_check(w) == 0
    ri = orc.instance_norm(H(xi))
    rb = orc.batch_norm_train(H(xb))
    rc = orc.conv_norm_epilogue(i4["x"][:32], i4["w"], i4["b"], batch=True, gamma=i4["gamma"],
                                beta=i4["beta"], out_scale=2.0)
    for r, (yi, yb, yc) in enumerate(outs):
        e1, e2, e3 = maxerr(H(yi), ri), maxerr(H(yb), rb), maxerr(H(yc), rc)
        _log("concurrent streams round %d: max_abs_err %.3e %.3e %.3e" % (r, e1, e2, e3))
        assert max(e1, e2, e3) <= TOL


def test_native_c_abi_roundtrip(dev, orc, tmp_path):
    # a plain C++ program (tests/native/abi_roundtrip.cpp, built by build()) drives the C ABI
    # with hipMalloc'd buffers and its own stream; its outputs must match the oracle
    import subprocess

    exe = os.path.join(os.path.dirname(os.path.abspath(__file__)), "native", "abi_roundtrip")
    assert os.path.exists(exe), "build the native client first (__graft_entry__.build())"
    r = subprocess.run([exe, str(tmp_path)], capture_output=True, text=True, timeout=120)
    _log("native client: rc %d, stdout %r, stderr %r" % (r.returncode, r.stdout[-200:], r.stderr[-400:]))
    assert r.returncode == 0
    shape = (3, 5, 100004)
    x = np.fromfile(tmp_path / "x.bin", np.float32).reshape(shape)
    y = np.fromfile(tmp_path / "inorm.bin", np.float32).reshape(shape)
    z = np.fromfile(tmp_path / "bn.bin", np.float32).reshape(shape)
    assert maxerr(y, orc.instance_norm(x)) <= TOL
    assert maxerr(z, orc.batch_norm_train(x, scale=2.0)) <= TOL
    u = np.fromfile(tmp_path / "noalloc.bin", np.float32).reshape(shape)
    assert np.array_equal(u, y)  # the same kernels in the library's own workspace
    x5 = np.fromfile(tmp_path / "x5.bin", np.float32).reshape(2, 3, 6, 9, 11)
    w5 = np.fromfile(tmp_path / "w5.bin", np.float32).reshape(16, 3, 3, 3, 3)
    b5 = np.fromfile(tmp_path / "b5.bin", np.float32)
    m5 = np.fromfile(tmp_path / "m5.bin", np.float32)
    out5 = np.fromfile(tmp_path / "chain.bin", np.float32).reshape(2, 4, 7, 9)
    ref5 = orc.conv_norm_epilogue(x5, w5, b5, batch=False, pre_mul=m5, clamp=(-1.0, 1.0),
                                  post_mul=m5, reduce_max_c=True)
    assert maxerr(out5, ref5) <= TOL


def test_stream_copy(dev, nra):
    import torch

    a = torch.randn(1 << 20, device=dev)
    b = torch.empty_like(a)
    nra.stream_copy(a, b)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    c = torch.randn(1001, device=dev)
    d = torch.empty_like(c)
    nra.stream_copy(c, d)
    torch.cuda.synchronize()
    assert torch.equal(c, d)
    # the persistent copy: whole 64 KiB units, a ragged last unit, fewer units than CUs, and
    # two calls in a row on one workspace (its counter is zeroed by every call)
    ws = torch.empty(256, dtype=torch.uint8, device=dev)
    for n in (1 << 24, (1 << 22) + 4 * 37, 4096 * 3 + 8, 1001):
        a = torch.randn(n, device=dev)
        b = torch.full_like(a, float("nan"))
        nra.stream_copy(a, b, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(a, b), n
