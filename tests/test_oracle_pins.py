"""Pins for the CPU oracle: each test checks the oracle against something other
than itself (hand-worked values, brute force, dense torch conv3d, scipy
correlation, closed forms, invariants).  CPU only."""
import json
import os

import numpy as np
import pytest
import torch
from scipy import ndimage

import synth
from oracle import dense, reference as ref, OracleError

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.fixture(autouse=True, scope="module")
def _built(oracle_built):
    return oracle_built


# ---------------------------------------------------------------- helpers

def brute_force_nbr(coords):
    """O(N^2): for every pair (i, j) in one batch with d = c_j - c_i in {-1,0,1}^3,
    column 9(dz+1) + 3(dy+1) + (dx+1) of row i is j."""
    c = coords.astype(np.int64)
    n = len(c)
    nbr = np.full((n, 27), -1, np.int32)
    d = c[None, :, :] - c[:, None, :]            # [i, j, 4]
    near = (d[..., 0] == 0) & (np.abs(d[..., 1:]) <= 1).all(-1)
    ii, jj = np.nonzero(near)
    k = 9 * (d[ii, jj, 1] + 1) + 3 * (d[ii, jj, 2] + 1) + (d[ii, jj, 3] + 1)
    nbr[ii, k] = jj
    return nbr


def dense_conv_at_sites(coords, feats, weight, bias, res, flip):
    """torch conv3d (float64, padding 1) on the scattered dense volume, read at the sites."""
    c = torch.from_numpy(coords.astype(np.int64))
    batch = int(c[:, 0].max()) + 1
    cin = feats.shape[1]
    vol = torch.zeros((batch, cin, res, res, res), dtype=torch.float64)
    vol[c[:, 0], :, c[:, 1], c[:, 2], c[:, 3]] = torch.from_numpy(feats.astype(np.float64))
    w = torch.from_numpy(weight.astype(np.float64)).permute(0, 4, 1, 2, 3).contiguous()
    if flip:
        w = torch.flip(w, dims=[2, 3, 4])
    b = None if bias is None else torch.from_numpy(bias.astype(np.float64))
    out = torch.nn.functional.conv3d(vol, w, b, padding=1)
    return out[c[:, 0], :, c[:, 1], c[:, 2], c[:, 3]].numpy()


def occupancy_counts(coords, res):
    """Per-voxel count of occupied cells in its 3x3x3 block (scipy correlate, zero border)."""
    batch = int(coords[:, 0].max()) + 1
    occ = np.zeros((batch, res, res, res), np.int32)
    occ[coords[:, 0], coords[:, 1], coords[:, 2], coords[:, 3]] = 1
    cnt = np.stack([ndimage.correlate(occ[b], np.ones((3, 3, 3), np.int32), mode="constant", cval=0)
                    for b in range(batch)])
    return cnt[coords[:, 0], coords[:, 1], coords[:, 2], coords[:, 3]]


def random_set(n, res, batch, seed):
    return synth.random_coords(n, res, batch, seed)


# ---------------------------------------------------------------- hand-worked example

def test_hand_example_both_oracles():
    g = json.load(open(os.path.join(GOLDEN, "hand_example.json")))
    coords = np.array(g["coords"], np.int32)
    feats = np.array(g["feats"], np.float64)
    w = np.zeros((1, 3, 3, 3, 1))
    for kz in range(3):
        for ky in range(3):
            for kx in range(3):
                w[0, kz, ky, kx, 0] = 9 * kz + 3 * ky + kx + 1
    bias = np.array(g["bias"])
    expect_nbr = np.full((4, 27), -1, np.int32)
    for i, taps in g["nbr_present"].items():
        for k, j in taps.items():
            expect_nbr[int(i), int(k)] = j
    for table in (ref.neighbor_table(coords, g["res"], 1), dense.neighbor_table(coords, g["res"], 1)):
        np.testing.assert_array_equal(table, expect_nbr)
    for flip, key in ((False, "out_corr"), (True, "out_flip")):
        a = ref.forward(feats, w, bias, expect_nbr, flip)[:, 0]
        b = dense.forward(feats, w, bias, expect_nbr, flip)[:, 0]
        np.testing.assert_array_equal(a, np.array(g[key]))
        np.testing.assert_array_equal(b, np.array(g[key]))


# ---------------------------------------------------------------- P1 brute force

@pytest.mark.parametrize("n,res,batch,seed", [(1, 1, 1, 0), (40, 4, 1, 1), (300, 8, 2, 2),
                                              (1500, 12, 3, 3), (1000, 10, 1, 4)])
def test_p1_brute_force(n, res, batch, seed):
    coords = random_set(n, res, batch, seed)
    bf = brute_force_nbr(coords)
    np.testing.assert_array_equal(ref.neighbor_table(coords, res, batch), bf)
    np.testing.assert_array_equal(dense.neighbor_table(coords, res, batch), bf)


def test_p1_brute_force_config1():
    _, coords = synth.workload(1)
    np.testing.assert_array_equal(dense.neighbor_table(coords, 16, 1), brute_force_nbr(coords))


# ---------------------------------------------------------------- P2 dense torch conv3d

@pytest.mark.parametrize("flip", [False, True])
@pytest.mark.parametrize("n,res,batch,cin,cout,seed", [(60, 5, 1, 3, 2, 0), (400, 10, 2, 5, 7, 1),
                                                        (900, 12, 1, 8, 4, 2), (2500, 16, 2, 4, 16, 3)])
def test_p2_dense_conv3d(flip, n, res, batch, cin, cout, seed):
    coords = random_set(n, res, batch, seed)
    feats, weight, bias = synth.make_values(n, cin, cout, seed)
    expect = dense_conv_at_sites(coords, feats, weight, bias, res, flip)
    nbr = ref.neighbor_table(coords, res, batch)
    np.testing.assert_allclose(ref.forward(feats, weight, bias, nbr, flip), expect, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dense.forward(feats, weight, bias, nbr, flip), expect, rtol=1e-12, atol=1e-12)


def test_p2_dense_conv3d_shell_no_bias():
    _, coords = synth.workload(1)
    feats, weight, _ = synth.make_values(len(coords), 6, 5, 7)
    nbr = dense.neighbor_table(coords, 16, 1)
    expect = dense_conv_at_sites(coords, feats, weight, None, 16, False)
    np.testing.assert_allclose(ref.forward(feats, weight, None, nbr), expect, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------- P3 counts

@pytest.mark.parametrize("idx", [1, 2, 3])
def test_p3_counts_match_correlation(idx):
    w, coords = synth.workload(idx)
    nbr = dense.neighbor_table(coords, w.res, w.batch)
    np.testing.assert_array_equal((nbr >= 0).sum(1), occupancy_counts(coords, w.res))


# ---------------------------------------------------------------- invariants I1-I4

def check_invariants(coords, nbr):
    n = len(coords)
    assert nbr.shape == (n, 27) and nbr.dtype == np.int32
    np.testing.assert_array_equal(nbr[:, 13], np.arange(n))                     # I1
    i, k = np.nonzero(nbr >= 0)
    j = nbr[i, k]
    np.testing.assert_array_equal(nbr[j, 26 - k], i)                            # I2 symmetry
    off = np.stack([k // 9 - 1, (k // 3) % 3 - 1, k % 3 - 1], 1)
    np.testing.assert_array_equal(coords[j, 1:] - coords[i, 1:], off)            # I3 offsets
    np.testing.assert_array_equal(coords[j, 0], coords[i, 0])                    # I3 batch


@pytest.mark.parametrize("idx", [1, 2, 3])
def test_invariants_and_o1_o2_agree(idx):
    w, coords = synth.workload(idx)
    a = dense.neighbor_table(coords, w.res, w.batch)
    check_invariants(coords, a)
    if len(coords) <= 200000:
        np.testing.assert_array_equal(ref.neighbor_table(coords, w.res, w.batch), a)


@pytest.mark.slow
def test_invariants_config4():
    w, coords = synth.workload(4)
    nbr = dense.neighbor_table(coords, w.res, w.batch)
    check_invariants(coords, nbr)
    # I4 via P3 on one grid
    sel = coords[:, 0] == 2
    cnt = occupancy_counts(coords[sel] * [0, 1, 1, 1], w.res)
    np.testing.assert_array_equal((nbr[sel] >= 0).sum(1), cnt)


# ---------------------------------------------------------------- closed forms I5-I8

def test_i5_identity_kernel_exact():
    w, coords = synth.workload(2)
    feats, _, _ = synth.make_values(len(coords), 8, 8, 0)
    weight = np.zeros((8, 3, 3, 3, 8))
    weight[:, 1, 1, 1, :] = np.eye(8)
    nbr = dense.neighbor_table(coords, w.res)
    for out in (ref.forward(feats, weight, None, nbr), dense.forward(feats, weight, None, nbr)):
        np.testing.assert_array_equal(out, feats.astype(np.float64))


def test_i6_isolated_voxel():
    coords = np.array([[0, 0, 0, 0], [0, 5, 5, 5], [0, 2, 2, 2], [0, 2, 2, 3]], np.int32)
    feats, weight, bias = synth.make_values(4, 3, 5, 11)
    nbr = ref.neighbor_table(coords, 8)
    out = ref.forward(feats, weight, bias, nbr)
    for i in (0, 1):
        assert (nbr[i] >= 0).sum() == 1
        np.testing.assert_allclose(out[i], bias + weight[:, 1, 1, 1, :].astype(np.float64) @ feats[i],
                                   rtol=1e-13)


@pytest.mark.parametrize("k", range(27))
def test_i7_single_tap(k):
    coords = random_set(500, 8, 1, 21)
    feats, _, bias = synth.make_values(500, 4, 3, 22)
    nbr = ref.neighbor_table(coords, 8)
    dz, dy, dx = k // 9 - 1, (k // 3) % 3 - 1, k % 3 - 1
    wk = np.random.default_rng(k).standard_normal((3, 4))
    weight = np.zeros((3, 3, 3, 3, 4))
    weight[:, dz + 1, dy + 1, dx + 1, :] = wk
    index = {tuple(r): i for i, r in enumerate(coords.tolist())}
    expect = np.tile(bias.astype(np.float64), (500, 1))
    for i, (b, z, y, x) in enumerate(coords.tolist()):
        j = index.get((b, z + dz, y + dy, x + dx))
        if j is not None:
            expect[i] += wk @ feats[j]
    np.testing.assert_allclose(ref.forward(feats, weight, bias, nbr), expect, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(dense.forward(feats, weight, bias, nbr), expect, rtol=1e-13, atol=1e-13)


def test_i8_all_ones():
    w, coords = synth.workload(1)
    n = len(coords)
    nbr = dense.neighbor_table(coords, w.res)
    out = dense.forward(np.ones((n, 16)), np.ones((5, 3, 3, 3, 16)), None, nbr)
    cnt = occupancy_counts(coords, w.res)
    np.testing.assert_array_equal(out, 16.0 * cnt[:, None] * np.ones((1, 5)))


# ---------------------------------------------------------------- I9-I11

def test_i9_flip_consistency():
    coords = random_set(800, 10, 2, 31)
    feats, weight, bias = synth.make_values(800, 6, 5, 32)
    nbr = dense.neighbor_table(coords, 10, 2)
    a = ref.forward(feats, weight, bias, nbr, flip=True)
    b = ref.forward(feats, weight[:, ::-1, ::-1, ::-1, :], bias, nbr, flip=False)
    np.testing.assert_allclose(a, b, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(dense.forward(feats, weight, bias, nbr, flip=True), b, rtol=1e-13, atol=1e-13)


def test_weight_layouts_against_dense_conv3d():
    """conv3d_to_krsc: a torch Conv3d weight [O, I, kz, ky, kx], converted, drives the
    oracle forward to torch's conv3d with the unconverted weight (library routine).
    mirror_krsc: tap k of the mirror is tap 26 - k, and it is torch.flip of the
    Conv3d weight over the three kernel axes, converted."""
    coords = random_set(500, 9, 1, 51)
    n = len(coords)
    rng = np.random.default_rng(51)
    feats = rng.standard_normal((n, 5))
    wc = rng.standard_normal((4, 5, 3, 3, 3))
    krsc = ref.conv3d_to_krsc(wc)
    assert krsc.shape == (4, 3, 3, 3, 5)
    c = torch.from_numpy(coords.astype(np.int64))
    vol = torch.zeros((1, 5, 9, 9, 9), dtype=torch.float64)
    vol[c[:, 0], :, c[:, 1], c[:, 2], c[:, 3]] = torch.from_numpy(feats)
    dense_out = torch.nn.functional.conv3d(vol, torch.from_numpy(wc), None, padding=1)
    expect = dense_out[c[:, 0], :, c[:, 1], c[:, 2], c[:, 3]].numpy()
    nbr = ref.neighbor_table(coords, 9, 1)
    np.testing.assert_allclose(ref.forward(feats, krsc, None, nbr), expect, rtol=1e-12, atol=1e-12)
    mirror = ref.mirror_krsc(krsc)
    for k in range(27):
        np.testing.assert_array_equal(ref.weight_tap(mirror, k, False), ref.weight_tap(krsc, 26 - k, False))
    np.testing.assert_array_equal(ref.conv3d_to_krsc(np.flip(wc, (2, 3, 4))), mirror)
    np.testing.assert_allclose(ref.forward(feats, mirror, None, nbr), ref.forward(feats, krsc, None, nbr, flip=True),
                               rtol=1e-13, atol=1e-13)


def test_i10_equivariances():
    _, coords = synth.workload(1)
    n = len(coords)
    feats, weight, bias = synth.make_values(n, 4, 4, 41)
    base = ref.forward(feats, weight, bias, ref.neighbor_table(coords, 16))
    # row permutation
    p = synth.shuffle_rows(n, 42)
    nbr_p = ref.neighbor_table(coords[p], 16)
    np.testing.assert_allclose(ref.forward(feats[p], weight, bias, nbr_p), base[p], rtol=1e-13, atol=1e-13)
    inv = np.argsort(p)
    base_nbr = ref.neighbor_table(coords, 16)
    relabel = np.where(base_nbr[p] >= 0, inv[np.maximum(base_nbr[p], 0)], -1)
    np.testing.assert_array_equal(nbr_p, relabel)
    # translation inside the grid (shell spans 2..14, grid 20)
    t = coords + np.array([0, 3, 1, 4], np.int32)
    np.testing.assert_allclose(ref.forward(feats, weight, bias, ref.neighbor_table(t, 20)), base,
                               rtol=1e-13, atol=1e-13)
    # two batches holding the same set
    two = np.concatenate([coords, coords + np.array([1, 0, 0, 0], np.int32)])
    out2 = ref.forward(np.concatenate([feats, feats]), weight, bias, ref.neighbor_table(two, 16, 2))
    np.testing.assert_array_equal(out2[:n], out2[n:])
    np.testing.assert_allclose(out2[:n], base, rtol=1e-13, atol=1e-13)


def test_i11_linearity():
    coords = random_set(600, 9, 1, 51)
    f1, w1, _ = (a.astype(np.float64) for a in synth.make_values(600, 5, 6, 52))
    f2, w2, _ = (a.astype(np.float64) for a in synth.make_values(600, 5, 6, 53))
    nbr = dense.neighbor_table(coords, 9)
    fw = lambda f, w: ref.forward(f, w, None, nbr)
    np.testing.assert_allclose(fw(2 * f1 - 3 * f2, w1), 2 * fw(f1, w1) - 3 * fw(f2, w1), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(fw(f1, w1 + w2), fw(f1, w1) + fw(f1, w2), rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------- I12 boundary

@pytest.mark.parametrize("table", ["ref", "dense"])
def test_i12_full_cube_counts(table):
    res = 4
    zyx = np.argwhere(np.ones((res,) * 3, bool)).astype(np.int32)
    coords = np.concatenate([np.zeros((len(zyx), 1), np.int32), zyx], 1)
    nbr = (ref if table == "ref" else dense).neighbor_table(coords, res, 1)
    cnt = (nbr >= 0).sum(1)
    border = ((zyx == 0) | (zyx == res - 1)).sum(1)      # number of axes on the boundary
    np.testing.assert_array_equal(cnt, np.array([27, 18, 12, 8])[border])
    # no wrap-around: a voxel at x=0 never sees x=res-1 of the previous row
    for i in np.nonzero(zyx[:, 2] == 0)[0]:
        for k in range(27):
            j = nbr[i, k]
            if j >= 0:
                assert zyx[j, 2] <= 1


# ---------------------------------------------------------------- I13-I14 helpers

def test_i13_subdivide_min_neighbours():
    _, parent = synth.workload(1)
    kids = dense.subdivide(parent)
    nbr = dense.neighbor_table(kids, 32, 1)
    assert (nbr >= 0).sum(1).min() >= 8
    ref_kids, _ = ref.subdivide(parent)
    np.testing.assert_array_equal(ref_kids, kids)


@pytest.mark.slow
def test_i13_config5_subdivided():
    w, parent = synth.workload(5)
    kids = dense.subdivide(parent)
    assert abs(len(kids) - 3.10e6) / 3.10e6 < 0.1
    nbr = dense.neighbor_table(kids, w.res, 1)
    assert (nbr >= 0).sum(1).min() >= 8
    check_invariants(kids, nbr)


def test_i14_subdivide_parent_relation():
    coords = random_set(200, 8, 2, 61)
    feats = np.arange(200 * 3, dtype=np.float32).reshape(200, 3)
    kids, kf = ref.subdivide(coords, feats)
    np.testing.assert_array_equal(kids[:, 1:] // 2, np.repeat(coords[:, 1:], 8, 0))
    np.testing.assert_array_equal(kids[:, 0], np.repeat(coords[:, 0], 8))
    np.testing.assert_array_equal(kf, np.repeat(feats, 8, 0))
    # C order of the children: dz slowest, dx fastest
    q = np.arange(len(kids)) % 8
    np.testing.assert_array_equal(kids[:, 1:] % 2, np.stack([q >> 2, (q >> 1) & 1, q & 1], 1))


def test_i14_s2d_round_trip_and_zero_fill():
    coords = random_set(700, 12, 2, 71)
    feats = np.random.default_rng(72).standard_normal((700, 3))
    cc, cf, mask = ref.space_to_depth(coords, feats)
    # every coarse cell listed once, ascending
    keys = [tuple(r) for r in cc.tolist()]
    assert keys == sorted(set(keys))
    assert mask.sum() == 700
    for m in range(len(cc)):
        for s in range(8):
            if not mask[m, s]:
                assert (cf[m, 3 * s:3 * s + 3] == 0).all()
    # slot: axis 0 (z) fastest
    for i in range(50):
        b, z, y, x = coords[i]
        m = keys.index((b, z // 2, y // 2, x // 2))
        s = (z % 2) + 2 * (y % 2) + 4 * (x % 2)
        assert mask[m, s] == 1
        np.testing.assert_array_equal(cf[m, 3 * s:3 * s + 3], feats[i])
    back_c, back_f = ref.depth_to_space(cc, cf, mask)
    order = np.lexsort(coords.T[::-1])
    border = np.lexsort(back_c.T[::-1])
    np.testing.assert_array_equal(back_c[border], coords[order])
    np.testing.assert_array_equal(back_f[border], feats[order])
    # without the mask every slot is emitted, unoccupied ones with zero features
    all_c, all_f = ref.depth_to_space(cc, cf)
    assert len(all_c) == 8 * len(cc)


def test_s2d_hand_example_golden():
    """Space-to-depth and both inverses against a hand-worked example
    (tests/golden/s2d_hand_example.json): coarse coordinates and slots, the
    channel layout, zero rows of unoccupied slots, and the children of the
    unmasked inverse in slot order."""
    g = json.load(open(os.path.join(GOLDEN, "s2d_hand_example.json")))
    coords = np.array(g["fine_coords"], np.int32)
    feats = np.array(g["fine_feats"], np.float64)
    cc, cf, mask = ref.space_to_depth(coords, feats)
    np.testing.assert_array_equal(cc, g["coarse_coords"])
    np.testing.assert_array_equal(cf, g["coarse_feats"])
    np.testing.assert_array_equal(mask, g["mask"])
    all_c, all_f = ref.depth_to_space(cc, cf)
    np.testing.assert_array_equal(all_c, g["unmasked_children_coords"])
    np.testing.assert_array_equal(all_f, g["unmasked_children_feats"])
    kc, kf = ref.depth_to_space(cc, cf, mask)
    np.testing.assert_array_equal(kc, g["masked_children_coords"])
    np.testing.assert_array_equal(kf, g["masked_children_feats"])


def test_i14_masked_upsample():
    coords = np.array([[0, 1, 2, 3], [0, 4, 4, 4], [1, 0, 0, 0]], np.int32)
    feats = np.array([[1.0], [2.0], [3.0]])
    mask = np.zeros((3, 8), np.uint8)
    mask[0, [1, 6]] = 1        # slot 1 -> (+1,0,0); slot 6 -> (0,+1,+1)
    # voxel 1 flags nothing and contributes nothing; voxel 2 flags all
    mask[2, :] = 1
    kc, kf = ref.upsample_masked(coords, feats, mask)
    assert len(kc) == 2 + 8
    np.testing.assert_array_equal(kc[0], [0, 3, 4, 6])
    np.testing.assert_array_equal(kc[1], [0, 2, 5, 7])
    np.testing.assert_array_equal(kf[:2, 0], [1.0, 1.0])
    np.testing.assert_array_equal(kf[2:, 0], 3.0)
    # axis-0-fastest decoding is the reverse of subdivide's C order
    sub, _ = ref.subdivide(coords[2:3])
    np.testing.assert_array_equal(np.sort(kc[2:], 0), np.sort(sub, 0))
    assert not (kc[2:] == sub).all()


def test_downsample_modes():
    coords = np.array([[0, 0, 0, 0], [0, 1, 1, 1], [0, 2, 0, 0], [0, 3, 1, 0]], np.int32)
    feats = np.array([[1.0, -5.0], [3.0, 1.0], [7.0, 2.0], [-1.0, 4.0]])
    cm, fmax = ref.downsample(coords, feats, "max")
    _, fmean = ref.downsample(coords, feats, "mean")
    np.testing.assert_array_equal(cm, [[0, 0, 0, 0], [0, 1, 0, 0]])
    np.testing.assert_array_equal(fmax, [[3.0, 1.0], [7.0, 4.0]])
    np.testing.assert_array_equal(fmean, [[2.0, -2.0], [3.0, 3.0]])


# ---------------------------------------------------------------- errors

@pytest.mark.parametrize("impl", ["ref", "dense"])
def test_errors(impl):
    t = ref if impl == "ref" else dense
    with pytest.raises(OracleError):
        t.neighbor_table(np.array([[0, 1, 1, 1], [0, 1, 1, 1]], np.int32), 4, 1)
    with pytest.raises(OracleError):
        t.neighbor_table(np.array([[0, 4, 1, 1]], np.int32), 4, 1)
    with pytest.raises(OracleError):
        t.neighbor_table(np.array([[0, -1, 1, 1]], np.int32), 4, 1)
    with pytest.raises(OracleError):
        t.neighbor_table(np.array([[1, 0, 0, 0]], np.int32), 4, 1)


# ---------------------------------------------------------------- workloads and bf16

def test_workload_sizes():
    expect = {1: (450, 450), 2: (17010, 20790), 3: (131000, 161000)}   # 18.9k +- 10%; 146k +- 10%
    for idx, (lo, hi) in expect.items():
        _, c = synth.workload(idx)
        assert lo <= len(c) <= hi
        assert c.dtype == np.int32 and c.flags.c_contiguous


def test_bf16_conversion_matches_torch():
    x = np.random.default_rng(5).standard_normal(100000).astype(np.float32)
    x[:4] = [1.00390625, 1.01171875, -1.00390625, 3.0]   # exact ties and an exact value
    bits = synth.bf16_bits(x)
    tb = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(bits, tb)
    np.testing.assert_array_equal(synth.bf16_to_f32(bits), torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_forward_of_row_subset_equals_rows_of_full_forward():
    coords = random_set(700, 9, 1, 81)
    feats, weight, bias = synth.make_values(700, 4, 5, 82)
    nbr = dense.neighbor_table(coords, 9)
    rows = np.array([0, 5, 17, 699, 350])
    np.testing.assert_array_equal(ref.forward(feats, weight, bias, nbr[rows]),
                                  ref.forward(feats, weight, bias, nbr)[rows])
