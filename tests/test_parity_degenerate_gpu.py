"""Degenerate and quantized inputs through the conv chains and batch norm, at full size (needs an
MI355X: run with -m gpu).

A constant input gives every output channel of a valid convolution one value, so its variance is
0 and the normalize step multiplies any difference between the statistics' mean and the values
it normalizes by 1/sqrt(eps) ~ 316. The formulas fix the result: training-mode batch norm then
x2 gives exactly 2 * beta_k (BN page, opening training-mode analysis), instance norm gives 0
before the clamp, so the max over channels of 0 * m_k is 0 (IN3d page, its step list). The GPU
must give exactly those values, and the oracle must be within the gate of them.

Quantized inputs (k / 255, the values of an 8-bit image scaled to [0, 1]) repeat few distinct
values, so per-value rounding errors do not average out of the statistics.
"""
import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu
TOL = 1e-4
VALUES = [1.0 / 3.0, 0.7, 10.0, "q255"]


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
    return float(np.max(np.abs(np.asarray(a, np.float64) - np.asarray(b, np.float64))))


def _log(msg):
    print(msg, flush=True)


def _input(shape, value, seed):
    if value == "q255":
        g = np.random.Generator(np.random.PCG64(seed))
        return (g.integers(0, 256, size=shape) / 255.0).astype(np.float32)
    return np.full(shape, np.float32(value), dtype=np.float32)


def _to_cl(a):
    return np.ascontiguousarray(np.moveaxis(a, 1, -1))


@pytest.mark.parametrize("cl", [False, True])
@pytest.mark.parametrize("value", VALUES)
def test_conv_bn_workload4_degenerate(dev, nra, orc, value, cl):
    inp = synth.host_inputs(4)
    x = _input(inp["x"].shape, value, 0x5EED0404)
    _log("case conv2d+bn x[128,8,64,64] value %s channels_last %s" % (value, cl))
    kw = dict(norm=nra.NR_NORM_BATCH_TRAIN, eps=inp["eps"], gamma=T(inp["gamma"], dev),
              beta=T(inp["beta"], dev), out_scale=inp["scale"], channels_last=cl)
    out = nra.conv_norm_epilogue_forward(T(_to_cl(x) if cl else x, dev), T(inp["w"], dev),
                                         T(inp["b"], dev), **kw)
    got = np.moveaxis(H(out), -1, 1) if cl else H(out)
    ref = orc.conv_norm_epilogue(x, inp["w"], inp["b"], batch=True, gamma=inp["gamma"],
                                 beta=inp["beta"], out_scale=inp["scale"])
    err = maxerr(got, ref)
    _log("conv2d+bn x[128,8,64,64] value %s channels_last %s: max_abs_err %.3e" % (value, cl, err))
    assert err <= TOL
    if value != "q255":
        two_beta = (inp["beta"] * np.float32(inp["scale"])).astype(np.float32)[None, :, None, None]
        # the oracle: 2 beta up to its own rounding. It sums a channel's n = 492032 equal fp64
        # conv values one after another, so its mean is off the value by up to
        # (n - 1) * 2^-53 * |c| (~6e-10 for |c| <= 10), which the normalize step multiplies by
        # gamma * scale / sqrt(eps) (<= 950): at most ~6e-7
        assert maxerr(ref, np.broadcast_to(two_beta, ref.shape)) <= 1e-6
        assert np.array_equal(got, np.broadcast_to(two_beta, got.shape))  # the GPU: exactly


@pytest.mark.parametrize("cl", [False, True])
@pytest.mark.parametrize("value", VALUES)
def test_conv_in3d_workload5_degenerate(dev, nra, orc, value, cl):
    inp = synth.host_inputs(5)
    x = _input(inp["x"].shape, value, 0x5EED0505)
    _log("case conv3d+in3d x[128,3,16,32,32] value %s channels_last %s" % (value, cl))
    out = nra.conv_norm_epilogue_forward(
        T(_to_cl(x) if cl else x, dev), T(inp["w"], dev), T(inp["b"], dev),
        norm=nra.NR_NORM_INSTANCE, eps=inp["eps"], pre_mul=T(inp["mult"], dev), clamp=inp["clamp"],
        post_mul=T(inp["mult"], dev), reduce_max_c=True, channels_last=cl)
    got = H(out)
    ref = orc.conv_norm_epilogue(x, inp["w"], inp["b"], batch=False, pre_mul=inp["mult"],
                                 clamp=inp["clamp"], post_mul=inp["mult"], reduce_max_c=True)
    err = maxerr(got, ref)
    _log("conv3d+in3d x[128,3,16,32,32] value %s channels_last %s: max_abs_err %.3e"
         % (value, cl, err))
    assert got.shape == (128, 14, 30, 30)
    assert err <= TOL
    if value != "q255":
        # the oracle: 0 up to its sequential fp64 mean over 12600 values (see above): <= 1e-7
        assert float(np.max(np.abs(ref))) <= 1e-7
        assert np.all(got == 0.0)  # the GPU: exactly


@pytest.mark.parametrize("cl", [False, True])
def test_conv_in3d_constant_per_item_channel(dev, nra, orc, cl):
    # x constant over space within each (n, c_in) but different across them: every instance
    # group (n, k) is constant, while batch items and input channels differ
    inp = synth.host_inputs(5)
    g = np.random.Generator(np.random.PCG64(0x5EED0506))
    lv = g.uniform(-12.0, 12.0, size=(128, 3, 1, 1, 1)).astype(np.float32)
    x = np.ascontiguousarray(np.broadcast_to(lv, inp["x"].shape)).astype(np.float32)
    out = nra.conv_norm_epilogue_forward(
        T(_to_cl(x) if cl else x, dev), T(inp["w"], dev), T(inp["b"], dev),
        norm=nra.NR_NORM_INSTANCE, eps=inp["eps"], pre_mul=T(inp["mult"], dev), clamp=inp["clamp"],
        post_mul=T(inp["mult"], dev), reduce_max_c=True, channels_last=cl)
    got = H(out)
    ref = orc.conv_norm_epilogue(x, inp["w"], inp["b"], batch=False, pre_mul=inp["mult"],
                                 clamp=inp["clamp"], post_mul=inp["mult"], reduce_max_c=True)
    err = maxerr(got, ref)
    _log("conv3d+in3d constant per (n, c_in), channels_last %s: max_abs_err %.3e" % (cl, err))
    assert err <= TOL
    assert np.all(got == 0.0)


BN_CONST_SHAPES = [(128, 64, 62, 62), (16, 64, 256, 256), (128, 512, 7, 7), (64, 32, 9, 9),
                   (4, 3, 1001, 1)]


@pytest.mark.parametrize("shape", BN_CONST_SHAPES)
def test_bn_train_constant_channels(dev, nra, orc, shape):
    # every channel constant at its own value: y = beta * out_scale exactly
    g = np.random.Generator(np.random.PCG64(0x5EED0507 + shape[1]))
    C = shape[1]
    lv = g.uniform(-20.0, 20.0, size=(1, C, 1, 1)).astype(np.float32)
    x = np.ascontiguousarray(np.broadcast_to(lv, shape)).astype(np.float32)
    gm = g.uniform(0.5, 1.5, C).astype(np.float32)
    bt = g.uniform(-0.5, 0.5, C).astype(np.float32)
    _log("case bn_train constant channels %s" % (shape,))
    y = nra.bn_train_forward(T(x, dev), gamma=T(gm, dev), beta=T(bt, dev), out_scale=2.0)
    got = H(y)
    ref = orc.batch_norm_train(x, gamma=gm, beta=bt, scale=2.0)
    err = maxerr(got, ref)
    _log("bn_train constant channels %s: max_abs_err %.3e" % (shape, err))
    assert err <= TOL
    expect = np.broadcast_to((bt * np.float32(2.0)).astype(np.float32)[None, :, None, None], shape)
    assert maxerr(ref, expect) <= 1e-6  # the oracle's sequential fp64 mean, as above
    assert np.array_equal(got, expect)


@pytest.mark.parametrize("shape", [(128, 64, 62, 62), (16, 64, 256, 256)])
def test_bn_train_quantized(dev, nra, orc, shape):
    g = np.random.Generator(np.random.PCG64(0x5EED0508 + shape[0]))
    x = (g.integers(0, 256, size=shape) / 255.0).astype(np.float32)
    y = nra.bn_train_forward(T(x, dev), out_scale=2.0)
    err = maxerr(H(y), orc.batch_norm_train(x, scale=2.0))
    _log("bn_train quantized %s: max_abs_err %.3e" % (shape, err))
    assert err <= TOL


@pytest.mark.parametrize("shape", [(16, 64, 256, 256), (8, 16, 12600), (4, 8, 1001)])
def test_inorm_quantized(dev, nra, orc, shape):
    g = np.random.Generator(np.random.PCG64(0x5EED0509 + shape[0]))
    x = (g.integers(0, 256, size=shape) / 255.0).astype(np.float32)
    y = nra.inorm_forward(T(x, dev))
    err = maxerr(H(y), orc.instance_norm(x))
    _log("inorm quantized %s: max_abs_err %.3e" % (shape, err))
    assert err <= TOL


# Other plans of the conv chains with a constant input: the conv writes c into `out` and a
# read-once kernel normalizes it in place (instance and batch groups, pipelined or one
# workgroup), the split statistics path, the vector-ALU producer's shapes, channels last.
PLAN_CASES = [
    # (x shape, C_out, batch, reduce_max_c, channels_last)
    ((1, 2, 260, 260), 3, False, False, False),   # in place, pipelined instance groups
    ((40, 2, 42, 42), 4, True, False, False),     # in place, pipelined batch groups
    ((9, 2, 40, 42), 6, True, False, False),      # in place, one workgroup per channel
    ((2, 8, 15, 13), 64, True, False, False),     # split path (143 positions)
    ((2, 3, 9, 11), 5, False, True, False),       # max over channels, statistics pass over c
    ((3, 1, 5, 6, 7), 20, True, True, False),     # 3-D, batch norm, max over channels
    ((3, 2, 9, 10), 4, True, False, True),        # channels last, batch norm, in place
    ((2, 3, 6, 9, 11), 16, False, False, True),   # channels last, 3-D, ring statistics
]


@pytest.mark.parametrize("shape,cout,batch,red,cl", PLAN_CASES)
@pytest.mark.parametrize("value", [0.7, -9.5])
def test_conv_chain_plans_constant_input(dev, nra, orc, shape, cout, batch, red, cl, value):
    g = np.random.Generator(np.random.PCG64(0x5EED050A + cout))
    dims = len(shape) - 2
    x = np.full(shape, np.float32(value), dtype=np.float32)
    w = (g.standard_normal((cout, shape[1]) + (3,) * dims) * 0.3).astype(np.float32)
    b = g.standard_normal(cout).astype(np.float32)
    pm = g.uniform(0.5, 2.0, cout).astype(np.float32) * np.where(g.random(cout) < 0.5, -1, 1).astype(np.float32)
    gm = g.uniform(0.5, 1.5, cout).astype(np.float32)
    bt = g.uniform(-0.5, 0.5, cout).astype(np.float32)
    qm = g.standard_normal(cout).astype(np.float32)
    _log("case chain plan %s Cout %d batch %s max_c %s cl %s value %s" % (shape, cout, batch, red, cl, value))
    xin = _to_cl(x) if cl else x
    out = nra.conv_norm_epilogue_forward(
        T(xin, dev), T(w, dev), T(b, dev), norm=nra.NR_NORM_BATCH_TRAIN if batch else nra.NR_NORM_INSTANCE,
        pre_mul=T(pm, dev), gamma=T(gm, dev), beta=T(bt, dev), out_scale=1.5, clamp=(-0.8, 1.1),
        post_mul=T(qm, dev), reduce_max_c=red, channels_last=cl)
    got = H(out) if (red or not cl) else np.moveaxis(H(out), -1, 1)
    ref = orc.conv_norm_epilogue(x, w, b, batch=batch, pre_mul=pm, gamma=gm, beta=bt, out_scale=1.5,
                                 clamp=(-0.8, 1.1), post_mul=qm, reduce_max_c=red)
    err = maxerr(got, ref)
    _log("chain plan %s value %s: max_abs_err %.3e" % (shape, value, err))
    assert err <= TOL
    # the closed form: every channel is constant, so the normalized value is 0 and each output
    # is clamp(beta * 1.5) * post_mul (max over the channels of that with the max)
    z = np.clip(bt * np.float32(1.5), -0.8, 1.1) * qm
    expect = np.max(z) if red else z.reshape((1, cout) + (1,) * dims)
    assert maxerr(got, np.broadcast_to(expect, got.shape)) <= 1e-6
