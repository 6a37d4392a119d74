"""Seeded synthetic inputs for the per-slice normalization workloads.

This module draws random numbers and nothing else: it holds none of the normalization, conv or
epilogue arithmetic. Both the oracle-side tests and the HIP-side tests/bench take their inputs
from here, so the two sides always see the same tensors.

Workloads (shapes and value distributions of the source pages' tasks, synthetic values):

====  =========================================================================================
id    recipe
====  =========================================================================================
1     InstanceNorm2d x[2,4,32,32] = z*s + o, z~N(0,1); per slice s~U(0.5,2), o~U(-3,3)
2     InstanceNorm2d x[16,64,256,256] = z*s + o; per slice s~U(0.1,10), o~U(-100,100)
      (large offsets against small spreads: stresses cancellation in the variance)
3     InstanceNorm2d x[112,64,512,512] ~ N(0,1)  (7168 slices of 262144; drawn on the device)
4     Conv2d(8->64,k3,valid,bias) x[128,8,64,64]~N(0,1), W,b~U(+-1/sqrt(72));
      BatchNorm2d (training) gamma~U(0.5,1.5), beta~U(-0.5,0.5); scale 2.0
5     Conv3d(3->16,k3,valid,bias) x[128,3,16,32,32]~N(0,1), W,b~U(+-1/sqrt(81));
      multiplier[16]~N(0,1); clamp [-1,1]; max over channels
====  =========================================================================================

Host draws use numpy's PCG64 generator seeded with ``SEED_BASE + id``; the one device draw
(workload 3, 7.5 GB) uses torch's device generator with the same seed.
"""
from __future__ import annotations

import numpy as np

SEED_BASE = 0x5EED0000
EPS = 1e-5

SHAPES = {
    1: (2, 4, 32, 32),
    2: (16, 64, 256, 256),
    3: (112, 64, 512, 512),
    4: (128, 8, 64, 64),
    5: (128, 3, 16, 32, 32),
}


def rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def per_slice_affine_normal(shape, seed, s_range, o_range) -> np.ndarray:
    """x = z*s + o with z~N(0,1) per element and s~U(s_range), o~U(o_range) per (n, c) slice."""
    g = rng(seed)
    N, C = shape[0], shape[1]
    z = g.standard_normal(shape, dtype=np.float32)
    s = g.uniform(s_range[0], s_range[1], size=(N, C)).astype(np.float32)
    o = g.uniform(o_range[0], o_range[1], size=(N, C)).astype(np.float32)
    bshape = (N, C) + (1,) * (len(shape) - 2)
    return (z * s.reshape(bshape) + o.reshape(bshape)).astype(np.float32)


def normal(shape, seed) -> np.ndarray:
    return rng(seed).standard_normal(shape, dtype=np.float32)


def conv_params(seed, cout, cin, ksz_dims, with_bias=True):
    """W [cout, cin, 3...] and b [cout] ~ U(+-1/sqrt(cin*3^dims))."""
    g = rng(seed)
    fan_in = cin * 3 ** ksz_dims
    bound = 1.0 / np.sqrt(fan_in)
    w = g.uniform(-bound, bound, size=(cout, cin) + (3,) * ksz_dims).astype(np.float32)
    b = g.uniform(-bound, bound, size=(cout,)).astype(np.float32) if with_bias else None
    return w, b


def host_inputs(cfg: int) -> dict:
    """Numpy inputs for workloads 1, 2, 4, 5 (host memory)."""
    seed = SEED_BASE + cfg
    if cfg == 1:
        return {"x": per_slice_affine_normal(SHAPES[1], seed, (0.5, 2.0), (-3.0, 3.0)), "eps": EPS}
    if cfg == 2:
        return {"x": per_slice_affine_normal(SHAPES[2], seed, (0.1, 10.0), (-100.0, 100.0)),
                "eps": EPS}
    if cfg == 4:
        x = normal(SHAPES[4], seed)
        w, b = conv_params(seed + 0x100, 64, 8, 2)
        g = rng(seed + 0x200)
        gamma = g.uniform(0.5, 1.5, size=64).astype(np.float32)
        beta = g.uniform(-0.5, 0.5, size=64).astype(np.float32)
        return {"x": x, "w": w, "b": b, "gamma": gamma, "beta": beta, "scale": 2.0, "eps": EPS}
    if cfg == 5:
        x = normal(SHAPES[5], seed)
        w, b = conv_params(seed + 0x100, 16, 3, 3)
        m = rng(seed + 0x200).standard_normal(16, dtype=np.float32)
        return {"x": x, "w": w, "b": b, "mult": m, "clamp": (-1.0, 1.0), "eps": EPS}
    raise ValueError("workload %d has no host recipe (workload 3 is drawn on the device)" % cfg)


def device_normal(shape, seed, device):
    """z ~ N(0,1) drawn directly in device memory with torch's seeded device generator."""
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return torch.randn(shape, generator=g, device=device, dtype=torch.float32)


def device_inputs_cfg3(device):
    return {"x": device_normal(SHAPES[3], SEED_BASE + 3, device), "eps": EPS}
