"""Plain Python/numpy oracle for submanifold 3x3x3 sparse convolution.

TEST INFRASTRUCTURE ONLY.  Only tests, the smoke check and the benchmark's
CPU-baseline leg may import this module.  It shares no code with the HIP
library and imports nothing from it.

Everything here is the definition written out, slow and in float64:

* the neighbour table is a dict from (b, z, y, x) to row, probed once per tap;
* the forward pass is one float64 matmul per tap over the rows that have that
  neighbour, summed over taps, plus the bias.

Sources (web pages; cited by page title and section):

* lato.2_mrp_mlx working notes (CLAUDE.md), commit summary: the convolution is
  the submanifold 3x3x3 one, resolved per voxel with 27 lookups, and a flag
  builds the mirrored kernel; section "Key facts": stride 1, output set = input
  set, weights in KRSC layout [out, kz, ky, kx, in]; upsampling by subdivide
  (coords*2 + unit cube, feats replicated); section "Unresolved": correlation
  vs convolution orientation is open.
* trellis_sparse_mrp_mlx commits (branch main), the spatial2channel /
  channel2spatial commit: slot index sum_i (coord_i mod f) f^i with axis 0
  fastest, unoccupied slots zero-filled; the downsample / upsample commit:
  downsample reduces by max or mean, upsample is a 0/1-masked expansion whose
  child index decodes axis 0 fastest, the reverse of subdivide's C order.

Readings where the pages are silent (each also listed in the design notes):

* tap k <-> offset (dz, dy, dx) = (k//9 - 1, (k//3)%3 - 1, k%3 - 1), i.e.
  C order over KRSC's (kz, ky, kx); kernel axis a pairs with coords column a+1.
* default orientation is correlation (neighbour at c + d uses W[d]); flip uses
  W[-d], i.e. weight tap 26 - k.
* a neighbour outside the grid or in another batch does not exist (-1);
  missing neighbours contribute exactly zero.
* duplicate or out-of-range coordinates are errors.
* space-to-depth output rows are in ascending (b, z, y, x) order of the coarse
  voxel; slot s occupies channels [s*C, (s+1)*C).
"""
from __future__ import annotations

import numpy as np

TAPS = 27
CENTRE = 13


class OracleError(ValueError):
    """Invalid coordinate set (duplicate or out of range)."""


def tap_offset(k: int) -> tuple:
    """(dz, dy, dx) of tap k: C order over the 3x3x3 kernel, centre k = 13."""
    return (k // 9 - 1, (k // 3) % 3 - 1, k % 3 - 1)


def check_coords(coords: np.ndarray, res: int, batch: int) -> None:
    """Raise OracleError unless every row is in range and rows are distinct."""
    c = np.asarray(coords)
    if c.ndim != 2 or c.shape[1] != 4:
        raise OracleError("coords must be [N,4]")
    if c.shape[0] == 0:
        return
    if (c[:, 0] < 0).any() or (c[:, 0] >= batch).any():
        raise OracleError("batch index out of range")
    if (c[:, 1:] < 0).any() or (c[:, 1:] >= res).any():
        raise OracleError("coordinate out of range")
    seen = set()
    for row in map(tuple, c.tolist()):
        if row in seen:
            raise OracleError("duplicate coordinate %r" % (row,))
        seen.add(row)


def neighbor_table(coords: np.ndarray, res: int, batch: int = None) -> np.ndarray:
    """nbr int32 [N,27]: nbr[i,k] = row of the voxel at coords[i] + offset(k), else -1.

    (lato.2_mrp_mlx working notes, commit summary: 27 lookups per voxel.)"""
    c = np.asarray(coords, dtype=np.int64)
    if batch is None:
        batch = int(c[:, 0].max()) + 1 if len(c) else 1
    check_coords(c, res, batch)
    index = {tuple(r): i for i, r in enumerate(c.tolist())}
    offsets = [tap_offset(k) for k in range(TAPS)]
    nbr = np.full((len(c), TAPS), -1, np.int32)
    for i, (b, z, y, x) in enumerate(c.tolist()):
        for k, (dz, dy, dx) in enumerate(offsets):
            nbr[i, k] = index.get((b, z + dz, y + dy, x + dx), -1)
    return nbr


def weight_tap(weight: np.ndarray, k: int, flip: bool) -> np.ndarray:
    """W for neighbour tap k as [Cout, Cin]: KRSC W[:, kz, ky, kx, :].

    Correlation uses (kz, ky, kx) = offset(k) + 1; the mirrored kernel uses
    1 - offset(k) (lato.2_mrp_mlx working notes, "Unresolved")."""
    dz, dy, dx = tap_offset(k)
    if flip:
        return weight[:, 1 - dz, 1 - dy, 1 - dx, :]
    return weight[:, dz + 1, dy + 1, dx + 1, :]


def conv3d_to_krsc(weight: np.ndarray) -> np.ndarray:
    """A torch Conv3d weight [Cout, Cin, kz, ky, kx] as KRSC [Cout, kz, ky, kx, Cin]
    (lato.2_mrp_mlx working notes, "Key facts": both layouts are 5-D)."""
    return np.ascontiguousarray(np.transpose(np.asarray(weight), (0, 2, 3, 4, 1)))


def mirror_krsc(weight: np.ndarray) -> np.ndarray:
    """The mirrored KRSC kernel W'[o, kz, ky, kx, c] = W[o, 2-kz, 2-ky, 2-kx, c] (tap k -> 26 - k),
    the weights the flip option stands for (same page, "Unresolved")."""
    return np.ascontiguousarray(np.asarray(weight)[:, ::-1, ::-1, ::-1, :])


def forward(feats: np.ndarray, weight: np.ndarray, bias, nbr: np.ndarray, flip: bool = False) -> np.ndarray:
    """out[i] = bias + sum over present taps k of W_k @ feats[nbr[i,k]], in float64.

    feats [N,Cin], weight KRSC [Cout,3,3,3,Cin], bias [Cout] or None, nbr [M,27]
    (the table rows of the outputs wanted: all N, or a subset of them)."""
    f = np.asarray(feats, dtype=np.float64)
    w = np.asarray(weight, dtype=np.float64)
    n, cout = nbr.shape[0], w.shape[0]          # one output row per table row
    out = np.zeros((n, cout), np.float64)
    for k in range(TAPS):
        rows = nbr[:, k]
        have = rows >= 0
        if have.any():
            out[have] += f[rows[have]] @ weight_tap(w, k, flip).T
    if bias is not None:
        out += np.asarray(bias, dtype=np.float64)[None, :]
    return out


def subdivide(coords: np.ndarray, feats: np.ndarray = None) -> tuple:
    """Each voxel -> its 8 children (2z+dz, 2y+dy, 2x+dx), C order (dz slowest),
    parent-major rows, feats replicated (lato.2_mrp_mlx working notes, "Key facts")."""
    c = np.asarray(coords, dtype=np.int64)
    kids = []
    for dz in (0, 1):
        for dy in (0, 1):
            for dx in (0, 1):
                kids.append((dz, dy, dx))
    out_c = np.zeros((len(c) * 8, 4), np.int32)
    for i, (b, z, y, x) in enumerate(c.tolist()):
        for q, (dz, dy, dx) in enumerate(kids):
            out_c[8 * i + q] = (b, 2 * z + dz, 2 * y + dy, 2 * x + dx)
    out_f = None
    if feats is not None:
        out_f = np.repeat(np.asarray(feats), 8, axis=0)
    return out_c, out_f


def s2d_slot(z: int, y: int, x: int, f: int = 2) -> int:
    """Slot of a fine voxel in its coarse cell: sum_i (coord_i mod f) f^i, axis 0 (z)
    fastest (trellis_sparse_mrp_mlx commits, spatial2channel commit)."""
    return (z % f) + (y % f) * f + (x % f) * f * f


def space_to_depth(coords: np.ndarray, feats: np.ndarray, f: int = 2) -> tuple:
    """Sparse space-to-depth: coarse coords (b, z//f, y//f, x//f) in ascending order,
    feats [M, f^3 C] with slot s at channels [sC, (s+1)C), unoccupied slots zero,
    and the 0/1 occupancy mask [M, f^3]."""
    c = np.asarray(coords, dtype=np.int64)
    fe = np.asarray(feats)
    ch = fe.shape[1]
    cells = {}
    for i, (b, z, y, x) in enumerate(c.tolist()):
        cells.setdefault((b, z // f, y // f, x // f), []).append((s2d_slot(z, y, x, f), i))
    keys = sorted(cells)
    out_c = np.array(keys, dtype=np.int32).reshape(-1, 4)
    out_f = np.zeros((len(keys), f ** 3 * ch), fe.dtype)
    mask = np.zeros((len(keys), f ** 3), np.uint8)
    for m, key in enumerate(keys):
        for slot, i in cells[key]:
            out_f[m, slot * ch:(slot + 1) * ch] = fe[i]
            mask[m, slot] = 1
    return out_c, out_f, mask


def child_offset(slot: int, f: int = 2) -> tuple:
    """(dz, dy, dx) of child `slot`: slot // f^i % f for axis i, axis 0 fastest."""
    return (slot % f, (slot // f) % f, (slot // (f * f)) % f)


def depth_to_space(coarse_coords: np.ndarray, coarse_feats: np.ndarray, mask=None, f: int = 2) -> tuple:
    """Inverse of space_to_depth: every coarse voxel emits its children in slot order
    (all of them, or those whose mask entry is 1); child feats = that slot's channels."""
    c = np.asarray(coarse_coords, dtype=np.int64)
    fe = np.asarray(coarse_feats)
    ch = fe.shape[1] // f ** 3
    out_c, out_f = [], []
    for m, (b, z, y, x) in enumerate(c.tolist()):
        for slot in range(f ** 3):
            if mask is not None and not mask[m, slot]:
                continue
            dz, dy, dx = child_offset(slot, f)
            out_c.append((b, f * z + dz, f * y + dy, f * x + dx))
            out_f.append(fe[m, slot * ch:(slot + 1) * ch])
    out_c = np.array(out_c, dtype=np.int32).reshape(-1, 4)
    out_f = np.array(out_f, dtype=fe.dtype).reshape(-1, ch)
    return out_c, out_f


def upsample_masked(coords: np.ndarray, feats: np.ndarray, mask: np.ndarray, f: int = 2) -> tuple:
    """Masked expansion: voxel i emits child `slot` iff mask[i, slot] = 1, slot decoded
    axis 0 fastest, feats replicated (trellis_sparse_mrp_mlx commits, upsample commit)."""
    c = np.asarray(coords, dtype=np.int64)
    fe = np.asarray(feats)
    out_c, out_f = [], []
    for i, (b, z, y, x) in enumerate(c.tolist()):
        for slot in range(f ** 3):
            if mask[i, slot]:
                dz, dy, dx = child_offset(slot, f)
                out_c.append((b, f * z + dz, f * y + dy, f * x + dx))
                out_f.append(fe[i])
    return (np.array(out_c, dtype=np.int32).reshape(-1, 4),
            np.array(out_f, dtype=fe.dtype).reshape(-1, fe.shape[1]))


def downsample(coords: np.ndarray, feats: np.ndarray, mode: str, f: int = 2) -> tuple:
    """Pool each coarse cell (b, z//f, y//f, x//f) over its occupied children by
    max or mean, coarse rows in ascending order (trellis_sparse_mrp_mlx commits,
    downsample commit: the mode is explicit)."""
    if mode not in ("max", "mean"):
        raise ValueError("mode must be 'max' or 'mean'")
    c = np.asarray(coords, dtype=np.int64)
    fe = np.asarray(feats, dtype=np.float64)
    cells = {}
    for i, (b, z, y, x) in enumerate(c.tolist()):
        cells.setdefault((b, z // f, y // f, x // f), []).append(i)
    keys = sorted(cells)
    out = np.zeros((len(keys), fe.shape[1]), np.float64)
    for m, key in enumerate(keys):
        rows = fe[cells[key]]
        out[m] = rows.max(axis=0) if mode == "max" else rows.mean(axis=0)
    return np.array(keys, dtype=np.int32).reshape(-1, 4), out
