"""Seeded synthetic inputs for the submanifold 3x3x3 sparse convolution.

This module is the only code shared by the CPU oracle and the HIP path.  It
draws inputs and nothing else: voxel coordinate sets (surface shells on a
grid), feature rows, KRSC weights and biases.  It holds none of the method's
arithmetic: no neighbour lookup, no convolution, no subdivide.  Where a
workload is defined as "a shell after subdivide", this module returns the
parent shell and each side subdivides it with its own implementation.

Geometry (voxel centres p = (z, y, x) on an integer grid, u = (p - c)/|p - c|):

* thin sphere: keep p iff | |p - c| - r | < 1/2.
* solid ellipsoid: |Q^T (p - c) / a| < 1 with Q a random rotation.
* noisy sphere: |p - c| < min(r_max, R0 (1 + A sum_k c_k cos(pi f_k . u + phi_k))),
  eight terms, f_k integer vectors in [-fmax, fmax]^3, c_k ~ N(0,1)/sqrt(8),
  phi_k ~ U[0, 2 pi).
* a shell of thickness t is the solid minus its t-fold erosion by the 3x3x3
  cube, with everything outside the grid counted as exterior.

Row order is C order over (b, z, y, x) (numpy argwhere), which is also the
ascending order of the packed key; callers shuffle rows themselves when they
want another order.

Values: features ~ N(0, 1) in fp32; weights He-normal (std sqrt(2 / (27 Cin)))
unless stated; biases U(-1/sqrt(27 Cin), +1/sqrt(27 Cin)) or zero.  bf16 inputs
are the round-to-nearest-even image of the fp32 draws; `bf16_bits` and
`bf16_to_f32` below are that dtype conversion, done once here so that both
sides see the same bits.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np
from scipy import ndimage

__all__ = [
    "Workload", "WORKLOADS", "workload", "make_values", "shuffle_rows",
    "thin_sphere", "ellipsoid_union_shell", "noisy_sphere_shell",
    "bf16_bits", "bf16_to_f32", "random_coords",
]


# ----------------------------------------------------------------------------
# dtype conversion (input preparation only)
# ----------------------------------------------------------------------------

def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bfloat16 (nearest, ties to even); return uint16 bits.

    Finite inputs only (the draws here are finite)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return rounded.astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bits (uint16) to fp32."""
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


# ----------------------------------------------------------------------------
# geometry
# ----------------------------------------------------------------------------

def _grid_offsets(res: int, centre) -> tuple:
    ax = np.arange(res, dtype=np.float64)
    c = np.asarray(centre, dtype=np.float64)
    return ax - c[0], ax - c[1], ax - c[2]


def _shell(solid: np.ndarray, t: int) -> np.ndarray:
    """Voxels of `solid` within Chebyshev distance t of the exterior."""
    eroded = ndimage.binary_erosion(solid, structure=np.ones((3, 3, 3), bool),
                                    iterations=t, border_value=0)
    return solid & ~eroded


def thin_sphere(res: int, centre, radius: float) -> np.ndarray:
    """Boolean [res]^3 mask of | |p - c| - radius | < 1/2."""
    dz, dy, dx = _grid_offsets(res, centre)
    rho = np.sqrt(dz[:, None, None] ** 2 + dy[None, :, None] ** 2 + dx[None, None, :] ** 2)
    return np.abs(rho - radius) < 0.5


def ellipsoid_union_shell(res: int, count: int, seed: int, axes_lo: float, axes_hi: float,
                          centre_jitter: float, t: int) -> np.ndarray:
    """Union of `count` ellipsoid shells (thickness t), random axes/rotation/centre."""
    rng = np.random.default_rng(seed)
    mask = np.zeros((res, res, res), bool)
    mid = (res - 1) / 2.0
    for _ in range(count):
        q, _r = np.linalg.qr(rng.standard_normal((3, 3)))
        a = rng.uniform(axes_lo, axes_hi, size=3)
        c = mid + rng.uniform(-centre_jitter, centre_jitter, size=3)
        dz, dy, dx = _grid_offsets(res, c)
        d = np.stack(np.broadcast_arrays(dz[:, None, None], dy[None, :, None], dx[None, None, :]), -1)
        local = d @ q  # Q^T (p - c) for every p, as row vectors
        solid = np.sum((local / a) ** 2, axis=-1) < 1.0
        mask |= _shell(solid, t)
    return mask


def noisy_sphere_shell(res: int, seed: int, r0: float, amp: float, fmax: int, r_max: float,
                       t: int, centre=None) -> np.ndarray:
    """Shell (thickness t) of a sphere whose radius is modulated by 8 cosines."""
    rng = np.random.default_rng(seed)
    freqs = rng.integers(-fmax, fmax + 1, size=(8, 3)).astype(np.float64)
    coef = rng.standard_normal(8) / np.sqrt(8.0)
    phase = rng.uniform(0.0, 2.0 * np.pi, size=8)
    c = np.full(3, (res - 1) / 2.0) if centre is None else np.asarray(centre, np.float64)
    dz, dy, dx = _grid_offsets(res, c)
    solid = np.zeros((res, res, res), bool)
    for z in range(res):  # one slab at a time keeps memory at O(res^2)
        pz = np.full((res, res), dz[z])
        py = np.broadcast_to(dy[:, None], (res, res))
        px = np.broadcast_to(dx[None, :], (res, res))
        rho = np.sqrt(pz * pz + py * py + px * px)
        safe = np.where(rho > 0, rho, 1.0)
        u = np.stack([pz / safe, py / safe, px / safe], -1)
        mod = np.cos(np.pi * (u @ freqs.T) + phase) @ coef
        radius = np.minimum(r_max, r0 * (1.0 + amp * mod))
        solid[z] = rho < radius
    return _shell(solid, t)


def _mask_coords(masks) -> np.ndarray:
    """int32 [N,4] (b, z, y, x) of one or more grids, batch-major, C order."""
    out = []
    for b, m in enumerate(masks):
        zyx = np.argwhere(m).astype(np.int32)
        col = np.full((zyx.shape[0], 1), b, np.int32)
        out.append(np.concatenate([col, zyx], axis=1))
    return np.ascontiguousarray(np.concatenate(out, axis=0), dtype=np.int32)


def random_coords(n: int, res: int, batch: int, seed: int) -> np.ndarray:
    """n distinct uniformly random coordinates, in random row order."""
    rng = np.random.default_rng(seed)
    total = batch * res ** 3
    if n > total:
        raise ValueError("more voxels than grid cells")
    flat = rng.choice(total, size=n, replace=False)
    b, r = np.divmod(flat, res ** 3)
    z, r = np.divmod(r, res * res)
    y, x = np.divmod(r, res)
    return np.ascontiguousarray(np.stack([b, z, y, x], 1).astype(np.int32))


def shuffle_rows(n: int, seed: int) -> np.ndarray:
    """A seeded permutation of n rows."""
    return np.random.default_rng(seed).permutation(n)


# ----------------------------------------------------------------------------
# workloads
# ----------------------------------------------------------------------------

@dataclasses.dataclass(frozen=True)
class Workload:
    """One benchmark / parity configuration.

    `coords` are the coordinates the convolution runs on, except when
    `subdivide_parent` is true: then `coords` is the parent set on a grid of
    res/2 and the workload runs on its subdivision (8 children per parent).
    """
    name: str
    res: int
    batch: int
    cin: int
    cout: int
    dtypes: tuple
    weight_std: Optional[float]   # None = He-normal
    bias: str                     # "zero" | "uniform"
    value_seed: int
    subdivide_parent: bool
    build: object                 # () -> int32 [M,4]
    note: str


def _cfg1():
    return _mask_coords([thin_sphere(16, (8, 8, 8), 6.0)])


def _cfg2():
    # geometry seed 12: 20,384 voxels, inside both "~20k" and 18.9k +- 10%
    return _mask_coords([ellipsoid_union_shell(64, 3, seed=12, axes_lo=14, axes_hi=28,
                                               centre_jitter=3.5, t=1)])


def _cfg3():
    return _mask_coords([noisy_sphere_shell(128, seed=0, r0=62, amp=0.10, fmax=4, r_max=62, t=2)])


def _cfg4():
    return _mask_coords([noisy_sphere_shell(256, seed=10 + b, r0=84, amp=0.10, fmax=3,
                                            r_max=125, t=2) for b in range(4)])


def _cfg5_parent():
    return _mask_coords([noisy_sphere_shell(256, seed=5, r0=96, amp=0.10, fmax=3, r_max=125, t=2)])


WORKLOADS = {
    1: Workload("sphere16_c16_f32", 16, 1, 16, 16, ("f32",), 1.0 / np.sqrt(27 * 16), "zero", 0,
                False, _cfg1, "B=1, 16^3, thin sphere r=6 about (8,8,8)"),
    2: Workload("ellipsoids64_c64_f32", 64, 1, 64, 64, ("f32",), None, "uniform", 0,
                False, _cfg2, "B=1, 64^3, union of 3 ellipsoid shells t=1"),
    3: Workload("noisysphere128_c128", 128, 1, 128, 128, ("f32", "bf16"), None, "uniform", 0,
                False, _cfg3, "B=1, 128^3, noisy-sphere shell t=2"),
    4: Workload("noisysphere256x4_c64_bf16", 256, 4, 64, 64, ("bf16",), None, "uniform", 0,
                False, _cfg4, "B=4, 256^3 each, noisy-sphere shells t=2"),
    5: Workload("subdiv512_c32_bf16", 512, 1, 32, 32, ("bf16",), None, "uniform", 0,
                True, _cfg5_parent, "B=1, 512^3, subdivided 256^3 noisy-sphere shell t=2"),
}

_COORD_CACHE: dict = {}


# A decoder-like chain (the pages' V-VAE decoder has 18 sparse conv kernels and grows
# its set by subdivision): at each level some SubMConv3d layers share one map, then
# the set is subdivided.  Levels: (grid, channels, convolutions); the first layer of a
# level maps the previous level's channels to this level's.
CHAIN_LEVELS = ((64, 128, 4), (128, 64, 4), (256, 32, 4), (512, 32, 6))
CHAIN_SMALL = ((16, 16, 2), (32, 32, 2), (64, 32, 2))   # the same shape of chain, oracle-sized


def chain_start(res: int = 64) -> np.ndarray:
    """Start set of the chain: a noisy-sphere shell, one voxel thick (6,182 voxels at
    64^3, 3.17M after three subdivisions, the size of the 512^3 workload); the 16^3
    thin sphere for the small chain."""
    if res == 16:
        return _mask_coords([thin_sphere(16, (8, 8, 8), 6.0)])
    return _mask_coords([noisy_sphere_shell(res, seed=5, r0=res * 0.27, amp=0.10, fmax=3, r_max=res / 2 - 1,
                                            t=1)])


def chain_values(levels, n0: int, seed: int = 90):
    """Start features [n0, C0] and per layer (weight KRSC, bias), LeCun-normal weights
    (std 1/sqrt(27 Cin)) so the scale of the activations stays bounded along the chain."""
    feats, _, _ = make_values(n0, levels[0][1], 1, seed)
    layers = []
    cin = levels[0][1]
    for li, (_, ch, convs) in enumerate(levels):
        for j in range(convs):
            _, w, b = make_values(1, cin, ch, seed + 1 + 16 * li + j, 1.0 / np.sqrt(27 * cin))
            layers.append((li, w, b))
            cin = ch
    return feats, layers


def workload(idx: int) -> tuple:
    """(Workload, coords int32 [M,4]); cached per process."""
    w = WORKLOADS[idx]
    if idx not in _COORD_CACHE:
        _COORD_CACHE[idx] = w.build()
    return w, _COORD_CACHE[idx]


def device_normal(n: int, c: int, seed: int, device):
    """Standard-normal float32 [n, c] drawn on `device` by torch's seeded generator, for
    sets too large to draw on the host (the oracle then reads back only the rows it needs)."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return torch.randn((n, c), generator=g, device=device, dtype=torch.float32)


def make_values(n: int, cin: int, cout: int, seed: int, weight_std: Optional[float] = None,
                bias: str = "uniform") -> tuple:
    """fp32 feats [n,cin], KRSC weight [cout,3,3,3,cin], bias [cout].

    Each array has its own stream (seed, tag), so n does not change the weights."""
    feats = np.random.default_rng([seed, 1]).standard_normal((n, cin), dtype=np.float32)
    std = np.sqrt(2.0 / (27 * cin)) if weight_std is None else weight_std
    weight = (np.random.default_rng([seed, 2]).standard_normal((cout, 3, 3, 3, cin)) * std).astype(np.float32)
    if bias == "zero":
        b = np.zeros(cout, np.float32)
    else:
        bound = 1.0 / np.sqrt(27 * cin)
        b = np.random.default_rng([seed, 3]).uniform(-bound, bound, cout).astype(np.float32)
    return feats, weight, b
