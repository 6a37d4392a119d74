"""Pins of the fp64 oracle to things other than itself (CPU only).

Each test fixes one part of the oracle against hand-derived values, a closed form, exact
rational brute force, an invariance, or an independent library routine (torch CPU float64).
Between them they fail on the plausible mistakes: a dropped eps, a wrong sign, the unbiased
variance, a transposed operand or index in the conv, statistics over the wrong axes, a wrong
channel for gamma/beta or a multiplier, a misplaced clamp or scale, min instead of max.
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append([float(t) for t in line.split()])
    return np.array(rows)


# ------------------------------------------------------------------------------------------
# Instance norm
# ------------------------------------------------------------------------------------------
def test_in_hand_example(oracle_mod):
    g = _golden("in_hand_example.txt")
    x = g[:, 0].astype(np.float32).reshape(1, 1, 4)
    y = oracle_mod.instance_norm(x, eps=1e-5)
    np.testing.assert_allclose(y.ravel(), g[:, 1], rtol=0, atol=2e-7)


@pytest.mark.parametrize("a,b", [(1.0, 0.0), (0.01, 1000.0), (3.0, -7.5), (1e-3, 0.0), (100.0, 4.0)])
def test_in_alternating_closed_form(oracle_mod, a, b):
    # x_i = b + a*(-1)^i has mean b and biased variance a^2 exactly (even length), so
    # y_i = (-1)^i * a / sqrt(a^2 + eps). A dropped eps, the unbiased variance (a^2*S/(S-1))
    # or a sign error each move y away from this.
    S = 256
    sign = np.where(np.arange(S) % 2 == 0, 1.0, -1.0)
    x = (b + a * sign).astype(np.float32)
    a32 = float(np.float32(b + a) - np.float32(b))  # the spread actually representable
    y = oracle_mod.instance_norm(x.reshape(1, 1, S), eps=1e-5).ravel()
    expect = sign * a32 / math.sqrt(a32 * a32 + 1e-5)
    np.testing.assert_allclose(y, expect, rtol=1e-6, atol=1e-7)


def test_in_constant_slice_is_zero(oracle_mod):
    for c in (0.0, 3.25, -1234.5, 1e6):
        x = np.full((1, 2, 7, 9), c, np.float32)
        y = oracle_mod.instance_norm(x)
        assert np.all(y == 0.0)


def test_in_single_element_is_zero(oracle_mod):
    x = np.array([[[5.5]], [[-2.0]]], np.float32)  # N=2, C=1, S=1
    y = oracle_mod.instance_norm(x)
    assert np.all(y == 0.0)


def test_in_exact_rational_brute_force(oracle_mod):
    # Mean and variance computed exactly with Fractions from the fp32 values, then one
    # rounding; the oracle's fp64 result must agree to a few fp32 ulps.
    g = np.random.Generator(np.random.PCG64(11))
    for S in (2, 3, 5, 17, 64):
        x = (g.standard_normal(S) * g.uniform(0.1, 10) + g.uniform(-50, 50)).astype(np.float32)
        fx = [Fraction(float(v)) for v in x]
        mu = sum(fx) / S
        var = sum((v - mu) ** 2 for v in fx) / S
        inv = 1.0 / math.sqrt(float(var) + 1e-5)
        expect = np.array([float(v - mu) * inv for v in fx])
        y = oracle_mod.instance_norm(x.reshape(1, 1, S)).ravel()
        np.testing.assert_allclose(y, expect, rtol=0, atol=3e-7)


def test_in_shift_invariance_bitwise(oracle_mod):
    # x on a 2^-10 grid and S a power of two: the mean of x+256 is exactly mean(x)+256 and
    # every deviation is unchanged, so y must match bit for bit.
    g = np.random.Generator(np.random.PCG64(12))
    x = (np.round(g.standard_normal((2, 3, 1024)) * 1024) / 1024).astype(np.float32)
    y0 = oracle_mod.instance_norm(x)
    y1 = oracle_mod.instance_norm((x + np.float32(256)).astype(np.float32))
    assert np.array_equal(y0, y1)


def test_in_power_of_two_scale(oracle_mod):
    # y(a*x) = (x - mean) * a / sqrt(a^2 var + eps); with a = 2^k the scaled input is exact.
    g = np.random.Generator(np.random.PCG64(13))
    x = g.standard_normal((1, 1, 4096)).astype(np.float32)
    _, _, var = oracle_mod.instance_norm(x, with_stats=True)
    var = float(var.ravel()[0])
    mean = float(np.mean(x.astype(np.float64)))
    for a in (2.0 ** -6, 2.0 ** -3, 8.0):
        y = oracle_mod.instance_norm((x * np.float32(a)).astype(np.float32)).ravel()
        expect = (x.ravel().astype(np.float64) - mean) * a / math.sqrt(a * a * var + 1e-5)
        np.testing.assert_allclose(y, expect, rtol=0, atol=1e-6)


def test_in_output_moments_closed_form(oracle_mod):
    # per slice: mean(y) = 0 and var_biased(y) = var/(var + eps) (not exactly 1).
    g = np.random.Generator(np.random.PCG64(14))
    x = (g.standard_normal((3, 4, 1000)) * 0.1 + 5.0).astype(np.float32)
    y, _, var = oracle_mod.instance_norm(x, with_stats=True)
    y64 = y.astype(np.float64)
    np.testing.assert_allclose(y64.mean(axis=2), 0.0, atol=1e-6)
    np.testing.assert_allclose(y64.var(axis=2), var / (var + 1e-5), rtol=1e-5)


def test_in_matches_torch_float64(oracle_mod):
    import torch
    import torch.nn.functional as F

    import synth

    x = synth.host_inputs(1)["x"]
    g = np.random.Generator(np.random.PCG64(15))
    gamma = g.uniform(0.5, 1.5, 4).astype(np.float32)
    beta = g.uniform(-1, 1, 4).astype(np.float32)
    for gm, bt in ((None, None), (gamma, beta)):
        y = oracle_mod.instance_norm(x, gamma=gm, beta=bt)
        ref = F.instance_norm(torch.from_numpy(x).double(),
                              weight=None if gm is None else torch.from_numpy(gm).double(),
                              bias=None if bt is None else torch.from_numpy(bt).double(),
                              eps=1e-5).numpy()
        np.testing.assert_allclose(y, ref, rtol=0, atol=1e-6)


def test_in_cancellation_workload_matches_torch(oracle_mod):
    # the offset +-100 / spread 0.1..10 recipe, a few slices: fp64 must still agree.
    import torch
    import torch.nn.functional as F

    import synth

    x = synth.per_slice_affine_normal((2, 8, 64, 64), 1234, (0.1, 10.0), (-100.0, 100.0))
    y = oracle_mod.instance_norm(x)
    ref = F.instance_norm(torch.from_numpy(x).double(), eps=1e-5).numpy()
    np.testing.assert_allclose(y, ref, rtol=0, atol=2e-6)


def test_in_slices_form_matches_torch_float64(oracle_mod):
    # the [count, S] form the sampled full-size checks use: each row normalized on its own
    # (torch's float64 instance norm over a [1, count, S] view), ragged S, returned statistics
    import torch
    import torch.nn.functional as F

    g = np.random.Generator(np.random.PCG64(31))
    for S in (1, 7, 1000, 4099):
        xs = (g.standard_normal((5, S)) * g.uniform(0.1, 10, (5, 1)) + g.uniform(-50, 50, (5, 1))).astype(np.float32)
        y, mean, var = oracle_mod.instance_norm_slices(xs, with_stats=True)
        if S == 1:  # one value per slice: y = 0 (torch refuses the shape)
            ref = np.zeros_like(xs)
        else:
            ref = F.instance_norm(torch.from_numpy(xs).double()[None], eps=1e-5)[0].numpy()
        np.testing.assert_allclose(y, ref, rtol=0, atol=2e-6)
        np.testing.assert_allclose(mean, xs.astype(np.float64).mean(axis=1), rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(var, xs.astype(np.float64).var(axis=1), rtol=1e-10, atol=1e-12)


def test_in_naive_sum_of_squares_fails_on_cancellation_workload(oracle_mod):
    # IN2d page, its numerics discussion: sum and sum of squares in fp32 lose the variance to
    # cancellation. On the offset/spread workload that shortcut misses the 1e-4 bar while
    # the oracle does not: the oracle can tell the two apart.
    import synth

    x = synth.per_slice_affine_normal((1, 16, 256, 256), 2, (0.1, 10.0), (-100.0, 100.0))
    xs = x.reshape(16, -1)
    y = oracle_mod.instance_norm_slices(xs)
    n = np.float32(xs.shape[1])
    s1 = xs.sum(axis=1, dtype=np.float32)
    s2 = (xs * xs).sum(axis=1, dtype=np.float32)
    mu = s1 / n
    var = np.maximum(s2 / n - mu * mu, np.float32(0))
    naive = (xs - mu[:, None]) / np.sqrt(var[:, None] + np.float32(1e-5))
    assert np.max(np.abs(naive - y)) > 1e-4


# ------------------------------------------------------------------------------------------
# Convolution
# ------------------------------------------------------------------------------------------
@pytest.mark.parametrize("dims", [2, 3])
def test_conv_delta_input_reads_weights_unflipped(oracle_mod, dims):
    # x = unit impulse at (c0, p0): out[k, p0 - t] = W[k, c0, t] for every tap t with
    # p0 - t inside the output (cross-correlation: no kernel flip), bias 0.
    g = np.random.Generator(np.random.PCG64(21))
    Cin, Cout = 3, 4
    sp = (5, 6, 7) if dims == 3 else (6, 7)
    w = g.standard_normal((Cout, Cin) + (3,) * dims).astype(np.float32)
    c0, p0 = 1, tuple(s // 2 for s in sp)
    x = np.zeros((1, Cin) + sp, np.float32)
    x[(0, c0) + p0] = 1.0
    out = oracle_mod.conv_k3(x, w, None)
    osp = tuple(s - 2 for s in sp)
    expect = np.zeros((1, Cout) + osp)
    for t in np.ndindex(*(3,) * dims):
        o = tuple(p - ti for p, ti in zip(p0, t))
        if all(0 <= oi < si for oi, si in zip(o, osp)):
            expect[(0, slice(None)) + o] = w[(slice(None), c0) + t]
    np.testing.assert_array_equal(out, expect)


@pytest.mark.parametrize("dims", [2, 3])
def test_conv_matches_torch_float64(oracle_mod, dims):
    import torch
    import torch.nn.functional as F

    g = np.random.Generator(np.random.PCG64(22 + dims))
    sp = (6, 9, 8) if dims == 3 else (11, 13)
    x = g.standard_normal((2, 3) + sp).astype(np.float32)
    w = g.standard_normal((5, 3) + (3,) * dims).astype(np.float32)
    b = g.standard_normal(5).astype(np.float32)
    out = oracle_mod.conv_k3(x, w, b)
    fn = F.conv3d if dims == 3 else F.conv2d
    ref = fn(torch.from_numpy(x).double(), torch.from_numpy(w).double(),
             torch.from_numpy(b).double()).numpy()
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-12)


def test_conv_bias_only_and_linearity(oracle_mod):
    g = np.random.Generator(np.random.PCG64(24))
    x1 = g.standard_normal((1, 2, 5, 5)).astype(np.float32)
    x2 = g.standard_normal((1, 2, 5, 5)).astype(np.float32)
    w = g.standard_normal((3, 2, 3, 3)).astype(np.float32)
    b = np.array([1.5, -2.0, 0.25], np.float32)
    zero = oracle_mod.conv_k3(np.zeros_like(x1), w, b)
    assert np.all(zero == b[None, :, None, None])
    lhs = oracle_mod.conv_k3(x1, w) + oracle_mod.conv_k3(x2, w)
    rhs = oracle_mod.conv_k3(x1.astype(np.float64) + x2, w)  # sum rounded to fp32 on entry
    np.testing.assert_allclose(lhs, rhs, atol=1e-5)


# ------------------------------------------------------------------------------------------
# Batch norm (training mode)
# ------------------------------------------------------------------------------------------
def test_bn_hand_example(oracle_mod):
    g = _golden("bn_hand_example.txt")
    x = g[:, 2].reshape(2, 1, 2)
    y = oracle_mod.batch_norm_train(x, gamma=np.array([0.5]), beta=np.array([0.25]), scale=2.0)
    np.testing.assert_allclose(y.ravel(), g[:, 3], rtol=0, atol=2e-7)


def test_bn_alternating_closed_form(oracle_mod):
    # per channel k, values b_k + a_k*(-1)^i over all (n, s): mean b_k, variance a_k^2, so
    # y = scale * (gamma_k * (+-a_k)/sqrt(a_k^2 + eps) + beta_k). The statistics must run
    # over (n, s) per channel: per-(n, k) statistics would give the same only by accident,
    # so each n gets a different number of + and - entries.
    N, C, S = 3, 4, 10
    a = np.array([0.5, 2.0, 0.01, 7.0])
    b = np.array([1.0, -3.0, 100.0, 0.0])
    gamma = np.array([1.0, 0.5, 2.0, 1.5], np.float32)
    beta = np.array([0.0, 0.25, -1.0, 0.5], np.float32)
    sign = np.where(np.arange(N * S) % 2 == 0, 1.0, -1.0).reshape(N, S)
    x = b[None, :, None] + a[None, :, None] * sign[:, None, :]
    y = oracle_mod.batch_norm_train(x, gamma=gamma, beta=beta, scale=2.0)
    expect = 2.0 * (gamma[None, :, None] * sign[:, None, :] * (a / np.sqrt(a * a + 1e-5))[None, :, None]
                    + beta[None, :, None])
    np.testing.assert_allclose(y, expect, rtol=0, atol=2e-6)


def test_bn_matches_torch_float64(oracle_mod):
    import torch
    import torch.nn.functional as F

    g = np.random.Generator(np.random.PCG64(31))
    x = (g.standard_normal((4, 6, 7, 5)) * 2 + 3).astype(np.float32)
    gamma = g.uniform(0.5, 1.5, 6).astype(np.float32)
    beta = g.uniform(-0.5, 0.5, 6).astype(np.float32)
    y = oracle_mod.batch_norm_train(x, gamma=gamma, beta=beta, scale=2.0)
    ref = 2.0 * F.batch_norm(torch.from_numpy(x).double(), None, None,
                             torch.from_numpy(gamma).double(), torch.from_numpy(beta).double(),
                             training=True, eps=1e-5).numpy()
    np.testing.assert_allclose(y, ref, rtol=0, atol=1e-6)


def test_bn_running_update_matches_torch_float64(oracle_mod):
    import torch
    import torch.nn.functional as F

    g = np.random.Generator(np.random.PCG64(32))
    x = (g.standard_normal((5, 3, 4, 6)) * 1.5 + 2).astype(np.float32)
    rm0 = g.standard_normal(3).astype(np.float32)
    rv0 = g.uniform(0.5, 2.0, 3).astype(np.float32)
    _, mean, var = oracle_mod.batch_norm_train(x, with_stats=True)
    rm, rv = oracle_mod.bn_running_update(mean, var, 5 * 4 * 6, rm0, rv0, momentum=0.1)
    trm = torch.from_numpy(rm0).double()
    trv = torch.from_numpy(rv0).double()
    F.batch_norm(torch.from_numpy(x).double(), trm, trv, training=True, momentum=0.1, eps=1e-5)
    np.testing.assert_allclose(rm, trm.numpy(), rtol=1e-6, atol=1e-7)
    np.testing.assert_allclose(rv, trv.numpy(), rtol=1e-6, atol=1e-7)


def test_bn_running_update_closed_form(oracle_mod):
    # values b +- a over an even count: batch mean b, biased var a^2, unbiased a^2 n/(n-1)
    rm, rv = oracle_mod.bn_running_update([3.0], [4.0], 10, [1.0], [2.0], momentum=0.25)
    assert abs(rm[0] - (0.75 * 1.0 + 0.25 * 3.0)) < 1e-7
    assert abs(rv[0] - (0.75 * 2.0 + 0.25 * 4.0 * 10 / 9)) < 1e-6


# ------------------------------------------------------------------------------------------
# Conv -> normalize -> epilogue chains
# ------------------------------------------------------------------------------------------
def _torch_chain(x, w, b, *, batch, pre_mul=None, gamma=None, beta=None, out_scale=1.0,
                 clamp=None, post_mul=None, reduce_max_c=False):
    import torch
    import torch.nn.functional as F

    t = lambda a: None if a is None else torch.from_numpy(np.asarray(a)).double()
    dims = x.ndim - 2
    conv = F.conv3d if dims == 3 else F.conv2d
    c = conv(t(x), t(w), t(b))
    bshape = (1, -1) + (1,) * dims
    if pre_mul is not None:
        c = c * t(pre_mul).view(bshape)
    if batch:
        z = F.batch_norm(c, None, None, t(gamma), t(beta), training=True, eps=1e-5)
    else:
        z = F.instance_norm(c, eps=1e-5)
        if gamma is not None:
            z = z * t(gamma).view(bshape)
        if beta is not None:
            z = z + t(beta).view(bshape)
    z = z * out_scale
    if clamp is not None:
        z = torch.clamp(z, clamp[0], clamp[1])
    if post_mul is not None:
        z = z * t(post_mul).view(bshape)
    if reduce_max_c:
        z = torch.amax(z, dim=1)
    return z.numpy()


def test_chain_hand_example(oracle_mod):
    g = _golden("chain_hand_example.txt")
    # identity conv: 2 channels, x[0,k,0,0:4] = conv output row, W[k,c,0,0] = [k == c]
    x = np.zeros((1, 2, 3, 6), np.float32)
    x[0, 0, 0, 0:4] = [0, 0, 0, 4]
    x[0, 1, 0, 0:4] = [3, 1, 2, 2]
    x[0, :, 1:, :] = 9.0  # rows the identity taps never read
    w = np.zeros((2, 2, 3, 3), np.float32)
    w[0, 0, 0, 0] = w[1, 1, 0, 0] = 1.0
    m = np.array([2.0, -1.0], np.float32)
    out = oracle_mod.conv_norm_epilogue(x, w, np.zeros(2, np.float32), batch=False, pre_mul=m,
                                        clamp=(-1.0, 1.0), post_mul=m, reduce_max_c=True)
    np.testing.assert_allclose(out.ravel(), g[:, 1], rtol=0, atol=2e-7)


def test_chain_bn_workload_shape_matches_torch(oracle_mod):
    # conv2d -> training batch norm (gamma, beta) -> x2.0, on a reduced batch of the
    # Conv2d(8->64) workload recipe.
    import synth

    inp = synth.host_inputs(4)
    x = inp["x"][:4, :, :20, :24]
    out = oracle_mod.conv_norm_epilogue(x, inp["w"], inp["b"], batch=True, gamma=inp["gamma"],
                                        beta=inp["beta"], out_scale=2.0)
    ref = _torch_chain(x, inp["w"], inp["b"], batch=True, gamma=inp["gamma"], beta=inp["beta"],
                       out_scale=2.0)
    np.testing.assert_allclose(out, ref, rtol=0, atol=2e-6)


def test_chain_in3d_workload_shape_matches_torch(oracle_mod):
    import synth

    inp = synth.host_inputs(5)
    x = inp["x"][:3, :, :7, :9, :11]
    kw = dict(batch=False, pre_mul=inp["mult"], clamp=(-1.0, 1.0), post_mul=inp["mult"],
              reduce_max_c=True)
    out = oracle_mod.conv_norm_epilogue(x, inp["w"], inp["b"], **kw)
    ref = _torch_chain(x, inp["w"], inp["b"], **kw)
    np.testing.assert_allclose(out, ref, rtol=0, atol=2e-6)


def test_chain_general_flags_match_torch(oracle_mod):
    g = np.random.Generator(np.random.PCG64(41))
    x = g.standard_normal((2, 3, 8, 9)).astype(np.float32)
    w = g.standard_normal((5, 3, 3, 3)).astype(np.float32) * 0.2
    b = g.standard_normal(5).astype(np.float32)
    pm = g.standard_normal(5).astype(np.float32)
    gm = g.uniform(0.5, 2, 5).astype(np.float32)
    bt = g.uniform(-1, 1, 5).astype(np.float32)
    qm = g.standard_normal(5).astype(np.float32)
    for batch in (True, False):
        for red in (False, True):
            kw = dict(batch=batch, pre_mul=pm, gamma=gm, beta=bt, out_scale=0.75,
                      clamp=(-0.6, 0.9), post_mul=qm, reduce_max_c=red)
            out = oracle_mod.conv_norm_epilogue(x, w, b, **kw)
            ref = _torch_chain(x, w, b, **kw)
            np.testing.assert_allclose(out, ref, rtol=0, atol=2e-6)


def test_chain_invariants(oracle_mod):
    import synth

    inp = synth.host_inputs(5)
    x = inp["x"][:2, :, :6, :8, :8]
    m = inp["mult"]
    out = oracle_mod.conv_norm_epilogue(x, inp["w"], inp["b"], batch=False, pre_mul=m,
                                        clamp=(-1.0, 1.0), post_mul=m, reduce_max_c=True)
    # |out| <= max_k |m_k| because the clamp bounds every term by |m_k|
    assert np.max(np.abs(out)) <= np.max(np.abs(m)) + 1e-7
    # one channel: the max is the channel itself, m * clamp(IN(m * c))
    w1, b1 = inp["w"][:1], inp["b"][:1]
    o1 = oracle_mod.conv_norm_epilogue(x, w1, b1, batch=False, pre_mul=m[:1], clamp=(-1.0, 1.0),
                                       post_mul=m[:1], reduce_max_c=True)
    c = oracle_mod.conv_k3(x, w1, b1)
    s = c * float(m[0])
    mu = s.reshape(2, -1).mean(axis=1).reshape(2, 1, 1, 1, 1)
    var = s.reshape(2, -1).var(axis=1).reshape(2, 1, 1, 1, 1)
    ref = float(m[0]) * np.clip((s - mu) / np.sqrt(var + 1e-5), -1, 1)
    np.testing.assert_allclose(o1, ref[:, 0], rtol=0, atol=2e-7)


@pytest.mark.parametrize("dims", [2, 3])
def test_conv_bn_eval_matches_torch_float64(oracle_mod, dims):
    import torch
    import torch.nn.functional as F

    g = np.random.Generator(np.random.PCG64(51 + dims))
    sp = (5, 8, 9) if dims == 3 else (10, 12)
    x = g.standard_normal((2, 3) + sp).astype(np.float32)
    w = (g.standard_normal((6, 3) + (3,) * dims) * 0.3).astype(np.float32)
    b = g.standard_normal(6).astype(np.float32)
    rm = g.standard_normal(6).astype(np.float32)
    rv = g.uniform(0.2, 3.0, 6).astype(np.float32)
    gm = g.uniform(0.5, 1.5, 6).astype(np.float32)
    bt = g.uniform(-0.5, 0.5, 6).astype(np.float32)
    out = oracle_mod.conv_bn_eval(x, w, b, rm, rv, gamma=gm, beta=bt, scale=2.0)
    t = lambda a: torch.from_numpy(a).double()
    conv = F.conv3d if dims == 3 else F.conv2d
    ref = 2.0 * F.batch_norm(conv(t(x), t(w), t(b)), t(rm), t(rv), t(gm), t(bt), training=False,
                             eps=1e-5)
    np.testing.assert_allclose(out, ref.numpy(), rtol=0, atol=2e-6)


def test_conv_bn_eval_identity_statistics(oracle_mod):
    # running mean 0, running var 1 - eps, gamma 1, beta 0, scale 1: the conv itself
    g = np.random.Generator(np.random.PCG64(53))
    x = g.standard_normal((1, 2, 6, 7)).astype(np.float32)
    w = g.standard_normal((3, 2, 3, 3)).astype(np.float32)
    b = g.standard_normal(3).astype(np.float32)
    rv = np.full(3, 1.0 - 1e-5, np.float32)
    out = oracle_mod.conv_bn_eval(x, w, b, np.zeros(3, np.float32), rv)
    ref = oracle_mod.conv_k3(x, w, b) / np.sqrt(rv.astype(np.float64)[None, :, None, None] + 1e-5)
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-6)
