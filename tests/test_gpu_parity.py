"""GPU parity: the HIP library against the CPU oracle on the same seeded inputs.

Neighbour tables are compared bit-exactly; features within the stated
tolerance (1e-4 fp32, 2e-2 bf16, relative to max|out|).  Every call goes
through the C ABI via the binding."""
import numpy as np
import pytest
import torch

import synth
import submanifold_sparse_convolution_submconv3d_amd as sc
from oracle import dense, reference as ref

from gpu_common import assert_close, device_values, note, to_f64

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


@pytest.fixture(scope="module", autouse=True)
def _gpu(oracle_built):
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    sc.load_library()


def coords_dev(c):
    return torch.from_numpy(np.ascontiguousarray(c, dtype=np.int32)).to(DEV)


def build(c, res, batch):
    rb = sc.submconv_build_map(coords_dev(c), res, batch)
    torch.cuda.synchronize()
    return rb


# ---------------------------------------------------------------- map build

@pytest.mark.parametrize("n,res,batch,seed", [(1, 1, 1, 0), (2, 2, 1, 1), (40, 4, 1, 2), (300, 8, 2, 3),
                                              (2047, 16, 1, 4), (2049, 16, 1, 5), (5000, 32, 3, 6),
                                              (20000, 64, 2, 7)])
def test_map_random_sets(n, res, batch, seed):
    c = synth.random_coords(n, res, batch, seed)
    note("map random n=%d res=%d batch=%d seed=%d" % (n, res, batch, seed))
    rb = build(c, res, batch)
    got = rb.neighbors().cpu().numpy()
    np.testing.assert_array_equal(got, dense.neighbor_table(c, res, batch))
    assert rb.taps_present == int((got >= 0).sum())


# The builder picks one of four strategies by set size and key-space size:
#   small bitmap (n <= 2048, <= 16 key bits), small sort (n <= 2048, more bits),
#   occupancy bitmap + rank (dense key space), radix sort + windowed search (sparse).
@pytest.mark.parametrize("n,res,batch,seed,shift,extent", [
    (700, 16, 1, 20, 0, 12),          # small bitmap
    (1500, 64, 2, 21, 30, 12),        # small sort (19 key bits)
    (30000, 48, 3, 22, 0, 48),        # occupancy bitmap
    (6000, 1024, 1, 23, 970, 24),     # radix sort + windows (30 key bits, sparse)
    (150000, 1024, 2, 24, 976, 48),   # radix sort + windows, many blocks
])
def test_map_build_strategies(n, res, batch, seed, shift, extent):
    # a dense cluster (neighbours exist) of the given extent, `shift` voxels into the grid
    c = synth.random_coords(n, extent, batch, seed)
    c[:, 1:] += shift
    c = c[synth.shuffle_rows(len(c), seed)]
    note("map strategy n=%d res=%d batch=%d" % (n, res, batch))
    got = build(c, res, batch).neighbors().cpu().numpy()
    expect = ref.neighbor_table(c, res, batch) if res > 256 else dense.neighbor_table(c, res, batch)
    assert (expect >= 0).sum() > 2 * n
    np.testing.assert_array_equal(got, expect)


@pytest.mark.parametrize("res,n,shift", [(16, 500, 0), (64, 1500, 0), (48, 3000, 0), (1024, 3000, 970)])
def test_map_duplicate_and_range_each_strategy(res, n, shift):
    base = synth.random_coords(n, min(res, 48), 1, 30)
    base[:, 1:] += shift
    dup = np.concatenate([base, base[17:18]])
    note("map dup res=%d" % res)
    with pytest.raises(sc.SubmconvError) as e:
        build(dup, res, 1)
    assert e.value.status == -3
    bad = base.copy()
    bad[5, 3] = res
    with pytest.raises(sc.SubmconvError) as e:
        build(bad, res, 1)
    assert e.value.status == -2


def test_map_hand_example():
    c = np.array([[0, 1, 1, 1], [0, 1, 1, 2], [0, 2, 1, 1], [0, 3, 3, 3]], np.int32)
    note("map hand example")
    got = build(c, 4, 1).neighbors().cpu().numpy()
    np.testing.assert_array_equal(got, ref.neighbor_table(c, 4, 1))


@pytest.mark.parametrize("res", [4, 5, 8])
def test_map_full_cube_boundary(res):
    zyx = np.argwhere(np.ones((res,) * 3, bool)).astype(np.int32)
    c = np.concatenate([np.zeros((len(zyx), 1), np.int32), zyx], 1)
    note("map full cube res=%d" % res)
    got = build(c, res, 1).neighbors().cpu().numpy()
    np.testing.assert_array_equal(got, dense.neighbor_table(c, res, 1))


@pytest.mark.parametrize("res,batch", [(33, 2), (64, 1), (100, 3)])
def test_map_grid_faces_dense_path(res, batch):
    """A hollow box three voxels thick on all six faces of the grid (60% of its cells),
    in every batch entry: more than 2048 voxels and at least 6 key bits per axis, so the
    bitmap path forms all nine rows from one word offset.  Rows that fall off the grid
    (below 0, past res - 1 into the next row, plane or batch entry, or past the bitmap's
    end) must come out absent."""
    rng = np.random.default_rng(1000 + res)
    g = np.arange(res)
    z, y, x = np.meshgrid(g, g, g, indexing="ij")
    box = (np.minimum(np.minimum(z, y), x) < 3) | (np.maximum(np.maximum(z, y), x) >= res - 3)
    zyx = np.argwhere(box).astype(np.int32)
    parts = []
    for b in range(batch):
        keep = zyx[rng.random(len(zyx)) < 0.6]
        parts.append(np.concatenate([np.full((len(keep), 1), b, np.int32), keep], 1))
    c = np.concatenate(parts)
    c = c[synth.shuffle_rows(len(c), res)]
    assert len(c) > 2048
    note("map grid faces res=%d batch=%d n=%d" % (res, batch, len(c)))
    rb = build(c, res, batch)
    got = rb.neighbors().cpu().numpy()
    np.testing.assert_array_equal(got, dense.neighbor_table(c, res, batch))
    assert rb.taps_present == int((got >= 0).sum())


def test_map_batches_isolated():
    # the same set in batch 0 and 2, batch 1 empty: no voxel may see another batch
    base = synth.random_coords(500, 8, 1, 9)
    c = np.concatenate([base, base + np.array([2, 0, 0, 0], np.int32)])
    note("map batch isolation")
    got = build(c, 8, 3).neighbors().cpu().numpy()
    np.testing.assert_array_equal(got, dense.neighbor_table(c, 8, 3))


@pytest.mark.parametrize("idx", [1, 2, 3, 4])
@pytest.mark.parametrize("shuffled", [False, True])
def test_map_workloads(idx, shuffled):
    w, c = synth.workload(idx)
    if shuffled:
        c = c[synth.shuffle_rows(len(c), 100 + idx)]
    note("map workload %d shuffled=%s n=%d" % (idx, shuffled, len(c)))
    got = build(c, w.res, w.batch).neighbors().cpu().numpy()
    np.testing.assert_array_equal(got, dense.neighbor_table(c, w.res, w.batch))


def test_map_workload5_subdivided():
    w, parent = synth.workload(5)
    note("map workload 5 (device subdivide) n=%d" % (8 * len(parent)))
    kids, _ = sc.submconv_subdivide(coords_dev(parent))
    kids_h = kids.cpu().numpy()
    np.testing.assert_array_equal(kids_h, dense.subdivide(parent))
    rb = sc.submconv_build_map(kids, w.res, 1)
    got = rb.neighbors().cpu().numpy()
    np.testing.assert_array_equal(got, dense.neighbor_table(kids_h, w.res, 1))
    assert (got >= 0).sum(1).min() >= 8


def test_map_large_key_uses_64_bits():
    # res 2048 and 4 batches need 3*11 + 2 = 35 key bits: the 64-bit key path.
    # Dense clusters at both ends of the grid so that neighbours exist at the boundaries.
    lo = synth.random_coords(4000, 16, 4, 11)
    hi = synth.random_coords(4000, 16, 4, 12) + np.array([0, 2032, 2032, 2032], np.int32)
    c = np.concatenate([lo, hi])
    c = c[synth.shuffle_rows(len(c), 3)]
    note("map 64-bit key n=%d" % len(c))
    got = build(c, 2048, 4).neighbors().cpu().numpy()
    expect = ref.neighbor_table(c, 2048, 4)
    assert (expect >= 0).sum() > 4 * len(c)
    np.testing.assert_array_equal(got, expect)


def test_map_errors():
    note("map errors")
    dup = np.array([[0, 1, 1, 1], [0, 2, 2, 2], [0, 1, 1, 1]], np.int32)
    with pytest.raises(sc.SubmconvError) as e:
        build(dup, 4, 1)
    assert e.value.status == -3
    for bad in ([[0, 4, 1, 1]], [[0, 1, -1, 1]], [[1, 0, 0, 0]], [[-1, 0, 0, 0]]):
        with pytest.raises(sc.SubmconvError) as e:
            build(np.array(bad, np.int32), 4, 1)
        assert e.value.status == -2


def test_map_empty():
    note("map empty")
    rb = sc.submconv_build_map(torch.zeros((0, 4), dtype=torch.int32, device=DEV), 8, 1)
    assert rb.n == 0 and rb.neighbors().shape == (0, 27)
    out = sc.submconv_forward(torch.zeros((0, 16), device=DEV), torch.zeros((16, 3, 3, 3, 16), device=DEV), None, rb)
    assert out.shape == (0, 16)


def test_map_deterministic():
    w, c = synth.workload(2)
    note("map determinism")
    a = build(c, w.res, 1).neighbors().cpu().numpy()
    b = build(c, w.res, 1).neighbors().cpu().numpy()
    np.testing.assert_array_equal(a, b)


# ---------------------------------------------------------------- forward

KERNELS = {"generic": sc.KERNEL_GENERIC, "lowc": sc.KERNEL_LOWC, "mfma": sc.KERNEL_MFMA,
           "window": sc.KERNEL_WINDOW, "persistent": sc.KERNEL_PERSISTENT}


def run_forward(c, res, batch, cin, cout, dtype, kernel, flip, seed=0, bias="uniform", std=None):
    feats, weight, b = synth.make_values(len(c), cin, cout, seed, std, bias)
    tf, tw, tb, f64, w64 = device_values(feats, weight, b, dtype)
    rb = build(c, res, batch)
    note("forward n=%d %d->%d %s %s flip=%d" % (len(c), cin, cout, dtype, kernel, flip))
    out = sc.submconv_forward(tf, tw, tb, rb, flip=flip, variant=KERNELS[kernel])
    got = to_f64(out)
    nbr = dense.neighbor_table(c, res, batch)
    expect = dense.forward(f64, w64, b, nbr, flip)
    return got, expect


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("flip", [0, 1])
@pytest.mark.parametrize("kernel,cin,cout", [("generic", 16, 16), ("generic", 3, 5), ("generic", 24, 40),
                                             ("lowc", 16, 16), ("lowc", 8, 32), ("lowc", 32, 16), ("lowc", 32, 32),
                                             ("mfma", 16, 16), ("mfma", 32, 32), ("mfma", 64, 64), ("mfma", 128, 128),
                                             ("mfma", 32, 128), ("mfma", 128, 64), ("mfma", 32, 64),
                                             ("mfma", 64, 128), ("mfma", 64, 32), ("mfma", 128, 32),
                                             ("persistent", 64, 64), ("persistent", 128, 128)])
def test_forward_random_set(dtype, flip, kernel, cin, cout):
    if kernel == "persistent" and dtype == "f32":
        pytest.skip("the persistent kernel takes bf16 only")
    c = synth.random_coords(3001, 14, 2, 5)      # ragged: not a multiple of any tile
    got, expect = run_forward(c, 14, 2, cin, cout, dtype, kernel, flip)
    assert_close(got, expect, dtype, "%s %d->%d %s flip=%d" % (kernel, cin, cout, dtype, flip))


def _cube(res, batch=1):
    g = np.stack(np.meshgrid(np.arange(batch), np.arange(res), np.arange(res), np.arange(res),
                             indexing="ij"), -1).reshape(-1, 4)
    return np.ascontiguousarray(g.astype(np.int32))


# the windowed kernel (bf16, 32 -> 32): tiles of 128 sorted voxels staged in LDS,
# tiles whose neighbourhood does not fit gathered from global memory instead
@pytest.mark.parametrize("case", ["sparse", "cube16", "cube16_ragged", "shell", "mixed", "tiny1", "tiny33",
                                  "tiny129", "batches"])
@pytest.mark.parametrize("flip", [0, 1])
def test_forward_window_sets(case, flip):
    if case == "sparse":        # wide windows: every tile takes the global-gather path
        c, res, batch = synth.random_coords(3001, 64, 1, 11), 64, 1
    elif case == "cube16":      # dense: every tile staged in LDS
        c, res, batch = _cube(16), 16, 1
    elif case == "cube16_ragged":
        c, res, batch = _cube(16)[:4000], 16, 1
    elif case == "shell":
        w, c = synth.workload(3)
        res, batch = w.res, w.batch
        c = c[:30001]
    elif case == "mixed":       # a dense cube next to scattered voxels: both paths in one call
        cube = _cube(12) + np.array([0, 2, 2, 2], np.int32)
        far = synth.random_coords(700, 64, 1, 12)
        far = far[(far[:, 1:] >= 20).any(axis=1)]
        c, res, batch = np.ascontiguousarray(np.concatenate([cube, far])), 64, 1
    elif case == "tiny1":
        c, res, batch = np.array([[0, 3, 3, 3]], np.int32), 8, 1
    elif case == "tiny33":
        c, res, batch = _cube(4)[:33], 4, 1
    elif case == "tiny129":
        c, res, batch = _cube(6)[:129], 6, 1
    else:
        c, res, batch = _cube(8, 3), 8, 3
    got, expect = run_forward(c, res, batch, 32, 32, "bf16", "window", flip, seed=4)
    assert_close(got, expect, "bf16", "window %s flip=%d" % (case, flip))


# the persistent kernel: units of 512 (128 ch) or 1024 (64 ch) sorted voxels per block
@pytest.mark.parametrize("c", [64, 128])
@pytest.mark.parametrize("case", ["one", "unit_plus_one", "shell", "batches"])
def test_forward_persistent_sets(c, case):
    if case == "one":
        coords, res, batch = np.array([[0, 2, 3, 4]], np.int32), 8, 1
    elif case == "unit_plus_one":   # a ragged last unit
        coords, res, batch = _cube(11)[: (512 if c == 128 else 1024) + 1], 11, 1
    elif case == "shell":
        w, coords = synth.workload(3)
        coords, res, batch = coords[:20001], w.res, w.batch
    else:
        coords, res, batch = _cube(9, 3), 9, 3
    for flip in (0, 1):
        got, expect = run_forward(coords, res, batch, c, c, "bf16", "persistent", flip, seed=6)
        assert_close(got, expect, "bf16", "persistent %d %s flip=%d" % (c, case, flip))


def test_forward_window_shuffled_and_f32_rejected():
    w, c = synth.workload(2)
    p = synth.shuffle_rows(len(c), 5)
    got, expect = run_forward(np.ascontiguousarray(c[p]), w.res, w.batch, 32, 32, "bf16", "window", 0, seed=2)
    assert_close(got, expect, "bf16", "window shuffled")
    rb = build(c, w.res, w.batch)
    f = torch.zeros((len(c), 32), device=DEV)
    note("window f32 rejected")
    with pytest.raises(sc.SubmconvError) as e:
        sc.submconv_forward(f, torch.zeros((32, 3, 3, 3, 32), device=DEV), None, rb, variant=sc.KERNEL_WINDOW)
    assert e.value.status == -4


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("kernel,c", [("generic", 8), ("lowc", 16), ("mfma", 16), ("mfma", 32), ("mfma", 128), ("window", 32),
                                      ("persistent", 64), ("persistent", 128)])
def test_forward_identity_kernel_exact(dtype, kernel, c):
    if kernel in ("window", "persistent") and dtype == "f32":
        pytest.skip("this kernel takes bf16 only")
    _, coords = synth.workload(2)
    feats = np.random.default_rng(3).standard_normal((len(coords), c)).astype(np.float32)
    weight = np.zeros((c, 3, 3, 3, c), np.float32)
    weight[:, 1, 1, 1, :] = np.eye(c)
    tf, tw, _, f64, _ = device_values(feats, weight, None, dtype)
    rb = build(coords, 64, 1)
    note("identity %s %s c=%d" % (kernel, dtype, c))
    out = sc.submconv_forward(tf, tw, None, rb, variant=KERNELS[kernel])
    np.testing.assert_array_equal(to_f64(out), f64)


@pytest.mark.parametrize("idx,dtype", [(1, "f32"), (2, "f32"), (3, "f32"), (3, "bf16")])
def test_forward_workloads_full(idx, dtype):
    w, c = synth.workload(idx)
    got, expect = run_forward(c, w.res, w.batch, w.cin, w.cout, dtype, _auto_kernel(w.cin, w.cout, dtype), 0,
                              w.value_seed, w.bias, w.weight_std)
    assert_close(got, expect, dtype, "workload %d %s" % (idx, dtype))


def _auto_kernel(cin, cout, dtype="f32"):
    if cin == 32 and cout == 32 and dtype == "bf16":
        return "window"
    if dtype == "bf16" and (cin, cout) in ((64, 64), (128, 128)):
        return "persistent"
    if (cin in (32, 64, 128) and cout in (32, 64, 128)) or cin == cout == 16:
        return "mfma"
    return "lowc" if cin <= 32 and cout <= 32 else "generic"


def full_check(c, res, batch, cin, cout, dtype, seed, bias, std, calls=1):
    """Every output row of a full-size workload against the C oracle (OpenMP, fp64),
    the table bit-exact, and `calls` forwards on the one rulebook bit-identical to
    the first (no atomics, so reruns must agree to the bit)."""
    feats, weight, b = synth.make_values(len(c), cin, cout, seed, std, bias)
    tf, tw, tb, f64, w64 = device_values(feats, weight, b, dtype)
    rb = sc.submconv_build_map(coords_dev(c), res, batch)
    note("full forward n=%d %d->%d %s, %d call(s) on one rulebook" % (len(c), cin, cout, dtype, calls))
    out = sc.submconv_forward(tf, tw, tb, rb)
    table = rb.neighbors().cpu().numpy()
    expect_table = dense.neighbor_table(c, res, batch)
    np.testing.assert_array_equal(table, expect_table)
    assert rb.taps_present == int((expect_table >= 0).sum())
    expect = dense.forward(f64, w64, b, expect_table)
    got = to_f64(out)
    assert_close(got, expect, dtype, "all %d rows" % len(c))
    for _ in range(calls - 1):
        again = sc.submconv_forward(tf, tw, tb, rb)
        assert torch.equal(out, again)
    rb.free()


# the rows MFMA kernel's three block layouts: on small sets two waves share a
# 32-voxel column and split Cout (the random-set tests above); from 512 blocks of
# 128 voxels on, one wave per column; from 2 * 256 * 256 voxels on, two columns per
# wave.  The 16 -> 16 sets take the 16-channel kernel, whose at most 2048 waves each walk
# several 16-voxel columns at 70k voxels.  Every output row against the oracle.
@pytest.mark.parametrize("n,cin,cout,dtype", [(70001, 64, 64, "f32"), (70001, 32, 128, "bf16"),
                                              (140001, 64, 64, "bf16"), (140001, 128, 64, "f32"),
                                              (70001, 16, 16, "f32"), (70001, 16, 16, "bf16")])
def test_forward_mfma_rows_layouts(n, cin, cout, dtype):
    c = synth.random_coords(n, 64, 1, 21)
    feats, weight, b = synth.make_values(len(c), cin, cout, 5)
    tf, tw, tb, f64, w64 = device_values(feats, weight, b, dtype)
    rb = build(c, 64, 1)
    note("mfma rows layout n=%d %d->%d %s" % (n, cin, cout, dtype))
    out = sc.submconv_forward(tf, tw, tb, rb, variant=sc.KERNEL_MFMA)
    expect = dense.forward(f64, w64, b, dense.neighbor_table(c, 64, 1))
    assert_close(to_f64(out), expect, dtype, "mfma rows n=%d %d->%d %s" % (n, cin, cout, dtype))


# The persistent fp32 128 -> 128 kernel: each block of 8 waves (one per CU) walks a
# balanced run of 32-voxel columns in rounds of 8, and its last round splits Cout among
# the waves when 1 to 4 columns remain (5 to 7: idle waves).  With 256 blocks the
# columns per block are: 24576 voxels 3; 40000 voxels 4 or 5; 52000 voxels 6 or 7;
# 65536 voxels 8 (one full round, no partial one); 146279 voxels 17 or 18 (two full
# rounds, then 1 or 2).  Every output row against the oracle.
@pytest.mark.parametrize("n", [24576, 40000, 52000, 65536, 146279])
def test_forward_mfma_persistent_rounds(n):
    c = synth.random_coords(n, 64, 1, 23)
    feats, weight, b = synth.make_values(len(c), 128, 128, 7)
    tf, tw, tb, f64, w64 = device_values(feats, weight, b, "f32")
    rb = build(c, 64, 1)
    note("mfma persistent rounds n=%d" % n)
    out = sc.submconv_forward(tf, tw, tb, rb, variant=sc.KERNEL_MFMA)
    expect = dense.forward(f64, w64, b, dense.neighbor_table(c, 64, 1))
    assert_close(to_f64(out), expect, "f32", "mfma persistent n=%d" % n)


# Sets of 1 to 300 voxels through the automatic kernel choice: one voxel, one ragged
# 32-voxel column, a column and one voxel, and a few columns (the persistent fp32
# 128 -> 128 kernel then runs only its partial round, with idle waves; the rows
# kernel has blocks past the last voxel).  Every row against the oracle.
@pytest.mark.parametrize("n", [1, 31, 33, 300])
@pytest.mark.parametrize("cin,cout,dtype", [(128, 128, "f32"), (64, 64, "f32"), (32, 64, "bf16"),
                                            (64, 64, "bf16"), (128, 128, "bf16"), (16, 16, "f32"), (16, 16, "bf16")])
def test_forward_tiny_sets(n, cin, cout, dtype):
    c = synth.random_coords(n, 8, 1, 40 + n)
    feats, weight, b = synth.make_values(len(c), cin, cout, 11)
    tf, tw, tb, f64, w64 = device_values(feats, weight, b, dtype)
    rb = build(c, 8, 1)
    note("tiny set n=%d %d->%d %s" % (n, cin, cout, dtype))
    out = sc.submconv_forward(tf, tw, tb, rb)
    expect = dense.forward(f64, w64, b, dense.neighbor_table(c, 8, 1), 0)
    assert_close(to_f64(out), expect, dtype, "tiny n=%d %d->%d %s" % (n, cin, cout, dtype))


# Kernels that address bf16 feature rows by 32-bit byte offsets take N * Cin * 2 <=
# 2^31 - 1 (windowed: 32 channels; persistent: 64 and 128).  Just past the cap,
# forcing the kernel is refused and the automatic choice runs another one.  A dense
# slab (depth x 512 x 512 voxels, C order, plus 1001 of the next plane), so the
# neighbours of the sampled rows follow from their index.
@pytest.mark.parametrize("ch,kernel,depth", [(32, "window", 128), (64, "persistent", 64), (128, "persistent", 32)])
def test_forward_size_caps(ch, kernel, depth):
    plane, nslab = 512 * 512, depth * 512 * 512
    n = nslab + 1001
    assert n * ch * 2 > 2 ** 31 - 1 >= (n - 1002) * ch * 2
    i = np.arange(n, dtype=np.int64)
    c = np.zeros((n, 4), np.int32)
    c[:, 1], c[:, 2], c[:, 3] = i // plane, (i // 512) % 512, i % 512
    _, weight, b = synth.make_values(1, ch, ch, 9)
    _, tw, tb, _, w64 = device_values(np.zeros((1, ch), np.float32), weight, b, "bf16")
    tf = synth.device_normal(n, ch, 9, DEV).to(torch.bfloat16)
    rb = build(c, 512, 1)
    note("size cap: forced %s refused, n=%d, %d ch" % (kernel, n, ch))
    with pytest.raises(sc.SubmconvError) as e:
        sc.submconv_forward(tf, tw, tb, rb, variant=KERNELS[kernel])
    assert e.value.status == -4
    note("size cap: automatic choice, n=%d, %d ch" % (n, ch))
    out = sc.submconv_forward(tf, tw, tb, rb)
    pick = np.random.default_rng(5).choice(n, size=2000, replace=False)
    pick = np.unique(np.concatenate([pick, [0, n - 1, nslab - plane, nslab - 1, nslab, nslab + 511]]))
    z, y, x = pick // plane, (pick // 512) % 512, pick % 512
    table = np.full((len(pick), 27), -1, np.int64)
    for k in range(27):
        dz, dy, dx = ref.tap_offset(k)
        nz, ny, nx = z + dz, y + dy, x + dx
        j = nz * plane + ny * 512 + nx
        ok = (nz >= 0) & (ny >= 0) & (ny < 512) & (nx >= 0) & (nx < 512) & (j < n)
        table[ok, k] = j[ok]
    rows, inv = np.unique(table[table >= 0], return_inverse=True)
    compact = np.full(table.shape, -1, np.int64)
    compact[table >= 0] = inv
    f64 = to_f64(tf[torch.from_numpy(rows).to(DEV)])
    expect = ref.forward(f64, w64, b, compact)
    got = to_f64(out[torch.from_numpy(pick).to(DEV)])
    assert_close(got, expect, "bf16", "size cap %d ch, automatic kernel" % ch)
    rb.free()


# Workload 4 (4 x 256^3 shells, 1.19M voxels, 64 -> 64 bf16; the map is built once
# and the forward runs 4 times on it) and workload 5 (the 512^3 subdivision of a 256^3
# shell, 3.24M voxels, 32 -> 32 bf16): every output row against the oracle.
def test_forward_workload4_full():
    w, c = synth.workload(4)
    full_check(c, w.res, w.batch, w.cin, w.cout, "bf16", w.value_seed, w.bias, w.weight_std, calls=4)


def test_forward_workload5_full():
    w, parent = synth.workload(5)
    kids = dense.subdivide(parent)
    full_check(kids, w.res, 1, w.cin, w.cout, "bf16", w.value_seed, w.bias, w.weight_std, calls=2)


@pytest.mark.parametrize("idx", [4, 5])
def test_forward_workload_shuffled_full(idx):
    """The same workloads in a seeded random row order (every row against the oracle)."""
    w, c = synth.workload(idx)
    if idx == 5:
        c = dense.subdivide(c)
    c = np.ascontiguousarray(c[synth.shuffle_rows(len(c), 500 + idx)])
    full_check(c, w.res, w.batch, w.cin, w.cout, "bf16", w.value_seed + 1, w.bias, w.weight_std)


def test_forward_shuffled_rows_permute_output():
    w, c = synth.workload(2)
    p = synth.shuffle_rows(len(c), 77)
    feats, weight, b = synth.make_values(len(c), 64, 64, 0)
    tf, tw, tb, _, _ = device_values(feats, weight, b, "f32")
    note("shuffled rows")
    out = sc.submconv_forward(tf, tw, tb, build(c, 64, 1))
    out_p = sc.submconv_forward(tf[torch.from_numpy(p).to(DEV)].contiguous(), tw, tb, build(c[p], 64, 1))
    assert_close(to_f64(out_p), to_f64(out)[p], "f32", "row permutation")


def test_forward_alias_rejected():
    c = synth.random_coords(100, 8, 1, 1)
    rb = build(c, 8, 1)
    f = torch.zeros((100, 32), device=DEV)
    note("alias")
    with pytest.raises(sc.SubmconvError) as e:
        sc.submconv_forward(f, torch.zeros((32, 3, 3, 3, 32), device=DEV), None, rb, out=f)
    assert e.value.status == -5


def test_rulebook_cache_reuse():
    w, c = synth.workload(1)
    cache = sc.RulebookCache()
    t = coords_dev(c)
    a = cache.get("subm0", t, w.res, 1)
    b = cache.get("subm0", t, w.res, 1)
    assert a is b and len(cache) == 1
    cache.clear()
    assert len(cache) == 0


def test_rulebook_cache_rebuilds_for_another_set_of_the_same_size():
    """Under one key, a different coordinate set with the same row count (another
    tensor, or the same tensor changed in place) must get its own map, never the
    cached one."""
    n = 3000
    c1 = synth.random_coords(n, 24, 1, 61)
    c2 = synth.random_coords(n, 24, 1, 62)
    assert not np.array_equal(c1, c2)
    cache = sc.RulebookCache()
    t1, t2 = coords_dev(c1), coords_dev(c2)
    note("rulebook cache: same size, other set")
    a = cache.get("k", t1, 24, 1)
    np.testing.assert_array_equal(a.neighbors().cpu().numpy(), dense.neighbor_table(c1, 24, 1))
    b = cache.get("k", t2, 24, 1)
    assert b is not a and len(cache) == 1
    np.testing.assert_array_equal(b.neighbors().cpu().numpy(), dense.neighbor_table(c2, 24, 1))
    t2.copy_(t1)                       # in place: the version counter moves, the map is rebuilt
    c = cache.get("k", t2, 24, 1)
    assert c is not b
    np.testing.assert_array_equal(c.neighbors().cpu().numpy(), dense.neighbor_table(c1, 24, 1))
    assert cache.get("k", t2, 24, 1) is c
    cache.clear()


def test_builds_on_several_host_threads():
    """Bitmap-path and single-block builds post their status to a mailbox of the
    calling host thread: builds running on four threads at once, each on its own
    stream, return exact tables and their own present counts."""
    import threading
    w2, c2 = synth.workload(2)
    w3, c3 = synth.workload(3)
    w1, c1 = synth.workload(1)
    cs = synth.random_coords(1500, 64, 2, 9)   # single block, sort (19 key bits)
    e2 = dense.neighbor_table(c2, w2.res, 1)
    e3 = dense.neighbor_table(c3, w3.res, 1)
    e1 = dense.neighbor_table(c1, w1.res, 1)
    es = dense.neighbor_table(cs, 64, 2)
    jobs = {"64^3": (c2, w2.res, 1, e2), "128^3": (c3, w3.res, 1, e3), "16^3": (c1, w1.res, 1, e1),
            "small sort": (cs, 64, 2, es)}
    got = {}

    def work(name):
        c, res, batch, e = jobs[name]
        s = torch.cuda.Stream()
        ok = True
        with torch.cuda.stream(s):
            for it in range(6):
                rb = sc.submconv_build_map(coords_dev(c), res, batch)
                table = rb.neighbors()
                s.synchronize()
                ok = ok and np.array_equal(table.cpu().numpy(), e) and rb.taps_present == int((e >= 0).sum())
                rb.free()
        s.synchronize()
        got[name] = ok

    note("builds on four host threads")
    threads = [threading.Thread(target=work, args=(name,)) for name in jobs]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert got == {name: True for name in jobs}


def test_block_cache_limit_and_cross_stream_reuse():
    """With caching off every block goes back to the driver; with it on, a block freed
    on one stream (work still queued there) is reused on another only after that work:
    the tables built on the second stream stay exact."""
    w2, c2 = synth.workload(2)
    e2 = dense.neighbor_table(c2, w2.res, 1)
    feats, weight, b = synth.make_values(len(c2), 64, 64, 3)
    tf, tw, tb, f64, w64 = device_values(feats, weight, b, "f32")
    expect = dense.forward(f64, w64, b, e2)
    note("block cache limit 0")
    sc.set_cache_limit(0)
    rb = build(c2, w2.res, 1)
    np.testing.assert_array_equal(rb.neighbors().cpu().numpy(), e2)
    rb.free()
    sc.set_cache_limit(2 << 30)
    note("block cache cross-stream reuse")
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    outs = []
    for it in range(3):
        with torch.cuda.stream(s1):
            rb = sc.submconv_build_map(coords_dev(c2), w2.res, 1)
            out = sc.submconv_forward(tf, tw, tb, rb)
            outs.append(out)
            rb.free()                  # queued forward still reads it; an event guards reuse
        with torch.cuda.stream(s2):
            rb2 = sc.submconv_build_map(coords_dev(c2), w2.res, 1)
            got = rb2.neighbors()
            rb2.free()
        s2.synchronize()
        np.testing.assert_array_equal(got.cpu().numpy(), e2)
    s1.synchronize()
    for out in outs:
        assert_close(to_f64(out), expect, "f32", "forward before a cross-stream reuse")
    with pytest.raises(sc.SubmconvError):
        sc.set_cache_limit(-1)


# ---------------------------------------------------------------- helpers

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("ch", [6, 32])
def test_subdivide(dtype, ch):
    c = synth.random_coords(777, 16, 2, 4)
    feats, _, _ = synth.make_values(777, ch, 1, 4)
    tf, _, _, f64, _ = device_values(feats, np.zeros((1, 3, 3, 3, ch), np.float32), None, dtype)
    note("subdivide %s c=%d" % (dtype, ch))
    kc, kf = sc.submconv_subdivide(coords_dev(c), tf)
    ec, ef = ref.subdivide(c, f64)
    np.testing.assert_array_equal(kc.cpu().numpy(), ec)
    np.testing.assert_array_equal(to_f64(kf), ef)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("n,res,batch,ch", [(1, 2, 1, 5), (900, 12, 2, 5), (5000, 33, 1, 5), (3000, 2048, 2, 5),
                                            (900, 12, 2, 32), (3000, 2048, 2, 32), (200000, 128, 1, 32)])
def test_space_to_depth_and_back(dtype, n, res, batch, ch):
    """Dense coarse key spaces group through a bitmap, sparse ones (2048^3) through a sort.
    5 channels take the per-element kernels, 32 the 16-byte vector ones; 200k voxels make
    the output kernels, which walk the device-side coarse count in grid-sized strides, take
    several strides."""
    c = synth.random_coords(n, res, batch, 8)
    feats, _, _ = synth.make_values(n, ch, 1, 8)
    tf, _, _, f64, _ = device_values(feats, np.zeros((1, 3, 3, 3, ch), np.float32), None, dtype)
    note("s2d %s n=%d res=%d ch=%d" % (dtype, n, res, ch))
    cc, cf, mask = sc.submconv_space_to_depth(coords_dev(c), tf, res, batch)
    ecc, ecf, emask = ref.space_to_depth(c, f64)
    np.testing.assert_array_equal(cc.cpu().numpy(), ecc)
    np.testing.assert_array_equal(to_f64(cf), ecf)
    np.testing.assert_array_equal(mask.cpu().numpy(), emask)
    # masked inverse gives back the fine set (coarse-major, slot order)
    bc, bf = sc.submconv_depth_to_space(cc, cf, mask)
    ebc, ebf = ref.depth_to_space(ecc, ecf, emask)
    np.testing.assert_array_equal(bc.cpu().numpy(), ebc)
    np.testing.assert_array_equal(to_f64(bf), ebf)
    # unmasked: every slot
    ac, af = sc.submconv_depth_to_space(cc, cf)
    eac, eaf = ref.depth_to_space(ecc, ecf)
    np.testing.assert_array_equal(ac.cpu().numpy(), eac)
    np.testing.assert_array_equal(to_f64(af), eaf)


@pytest.mark.parametrize("res", [4, 2048])
def test_space_to_depth_errors(res):
    """A duplicate row and an out-of-range row are reported on both groupings: the coarse
    bitmap (res 4) and the sort (res 2048, a sparse coarse key space)."""
    note("s2d errors res=%d" % res)
    c = np.array([[0, 1, 1, 1], [0, 3, 2, 1], [0, 1, 1, 1]], np.int32)
    f = torch.zeros((3, 4), device=DEV)
    with pytest.raises(sc.SubmconvError) as e:
        sc.submconv_space_to_depth(coords_dev(c), f, res, 1)
    assert e.value.status == -3
    with pytest.raises(sc.SubmconvError) as e:
        sc.submconv_space_to_depth(coords_dev(np.array([[0, 1, 1, 1], [0, res, 1, 1]], np.int32)), f[:2], res, 1)
    assert e.value.status == -2


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("n,c", [(1, 8), (900, 5), (900, 8), (5000, 32), (20000, 64)])
def test_upsample_masked(dtype, n, c):
    """Masked expansion (a copy): bit-exact against the oracle, including voxels that
    flag no child and voxels that flag all eight; c = 5 takes the per-element path,
    the others whole 16-byte vectors."""
    coords = synth.random_coords(n, 64, 2, 21)
    feats, _, _ = synth.make_values(n, c, 1, 21)
    rng = np.random.default_rng(21)
    mask = (rng.random((n, 8)) < 0.4).astype(np.uint8)
    mask[::7] = 0
    mask[3::11] = 1
    tf, _, _, f64, _ = device_values(feats, np.zeros((1, 3, 3, 3, c), np.float32), None, dtype)
    note("upsample_masked %s n=%d c=%d" % (dtype, n, c))
    kc, kf = sc.submconv_upsample_masked(coords_dev(coords), tf, torch.from_numpy(mask).to(DEV))
    ec, ef = ref.upsample_masked(coords, f64, mask)
    assert len(ec) == int(mask.astype(bool).sum())
    np.testing.assert_array_equal(kc.cpu().numpy(), ec)
    np.testing.assert_array_equal(to_f64(kf), ef)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("mode", ["max", "mean"])
@pytest.mark.parametrize("n,res,batch,c", [(1, 2, 1, 4), (900, 12, 2, 5), (5000, 33, 1, 32), (60000, 64, 2, 64),
                                           (3000, 2048, 2, 8), (60000, 2048, 1, 16)])
def test_downsample(dtype, mode, n, res, batch, c):
    """Pooling by 2: coarse coords exact and ascending; max exact; mean within the
    feature tolerance (fp32 sum in slot order vs the oracle's fp64 mean).  The two
    60000-voxel sets (bitmap and sort grouping) make the pooling kernels, which walk the
    device-side coarse count in grid-sized strides, take more than one stride."""
    coords = synth.random_coords(n, res, batch, 22)
    coords = coords[synth.shuffle_rows(len(coords), 22)]
    feats, _, _ = synth.make_values(len(coords), c, 1, 22)
    tf, _, _, f64, _ = device_values(feats, np.zeros((1, 3, 3, 3, c), np.float32), None, dtype)
    note("downsample %s %s n=%d res=%d c=%d" % (dtype, mode, len(coords), res, c))
    gc, gf = sc.submconv_downsample(coords_dev(coords), tf, res, batch, mode)
    ec, ef = ref.downsample(coords, f64, mode)
    np.testing.assert_array_equal(gc.cpu().numpy(), ec)
    if mode == "max":
        np.testing.assert_array_equal(to_f64(gf), ef)
    else:
        assert_close(to_f64(gf), ef, dtype, "downsample mean")


@pytest.mark.parametrize("res", [4, 2048])
def test_downsample_errors(res):
    """As for space-to-depth: errors on the bitmap (res 4) and the sort (res 2048) groupings."""
    note("downsample errors res=%d" % res)
    f = torch.zeros((3, 4), device=DEV)
    with pytest.raises(sc.SubmconvError) as e:
        sc.submconv_downsample(coords_dev(np.array([[0, 1, 1, 1], [0, 2, 3, 1], [0, 1, 1, 1]], np.int32)), f, res, 1,
                               "max")
    assert e.value.status == -3
    with pytest.raises(sc.SubmconvError) as e:
        sc.submconv_downsample(coords_dev(np.array([[0, 1, 1, 1], [0, 1, res + 5, 1]], np.int32)), f[:2], res, 1,
                               "mean")
    assert e.value.status == -2
    with pytest.raises(ValueError):
        sc.submconv_downsample(coords_dev(np.array([[0, 1, 1, 1]], np.int32)), f[:1], 4, 1, "sum")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("flip", [False, True])
def test_weight_convert(dtype, flip):
    """Conv3d [O,I,kz,ky,kx] and KRSC weights to KRSC, optionally mirrored: a copy, so
    bit-exact against the oracle's layout definitions."""
    rng = np.random.default_rng(61)
    wc = rng.standard_normal((16, 8, 3, 3, 3)).astype(np.float32)
    krsc = ref.conv3d_to_krsc(wc)
    note("weight_convert %s flip=%d" % (dtype, flip))
    for src, layout in ((wc, "oidhw"), (krsc, "krsc")):
        if dtype == "f32":
            t = torch.from_numpy(np.ascontiguousarray(src)).to(DEV)
        else:
            t = torch.from_numpy(synth.bf16_bits(np.ascontiguousarray(src)).view(np.int16)).view(torch.bfloat16).to(DEV)
        got = sc.weight_to_krsc(t, layout=layout if layout == "krsc" else None, flip=flip)
        expect = ref.mirror_krsc(krsc) if flip else krsc
        if dtype == "bf16":
            expect = synth.bf16_to_f32(synth.bf16_bits(expect))
        np.testing.assert_array_equal(got.float().cpu().numpy(), expect)


def test_flip_ab_orientations():
    """flip_ab's two outputs are the oracle's correlation and convolution forwards, and
    the convolution one equals the correlation forward with the mirrored weights."""
    w, c = synth.workload(1)
    feats, weight, bias = synth.make_values(len(c), 16, 16, 71)
    tf, tw, tb, f64, w64 = device_values(feats, weight, bias, "f32")
    note("flip_ab workload 1")
    rb = build(c, w.res, 1)
    ab = sc.flip_ab(tf, tw, tb, rb)
    nbr = dense.neighbor_table(c, w.res, 1)
    assert_close(to_f64(ab["corr"]), ref.forward(f64, w64, bias, nbr, flip=False), "f32", "corr")
    assert_close(to_f64(ab["conv"]), ref.forward(f64, w64, bias, nbr, flip=True), "f32", "conv")
    mirrored = sc.submconv_forward(tf, sc.weight_to_krsc(tw, layout="krsc", flip=True), tb, rb)
    assert_close(to_f64(mirrored), to_f64(ab["conv"]), "f32", "mirror vs flip")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_chain_small(dtype):
    """The decoder-like chain at oracle size (16^3 -> 64^3, three levels, six layers):
    per level a map, its layers on that map, then subdivide.  The oracle chain keeps
    fp64 sums and, for bf16, rounds each layer's output to bf16 as the GPU stores it."""
    levels = synth.CHAIN_SMALL
    c0 = synth.chain_start(16)
    feats, layers = synth.chain_values(levels, len(c0))
    note("chain %s n0=%d" % (dtype, len(c0)))
    zero_w = np.zeros((1, 3, 3, 3, feats.shape[1]), np.float32)
    x, _, _, x64, _ = device_values(feats, zero_w, None, dtype)
    dev_layers = []
    for li, w, b in layers:
        _, tw, tb, _, w64 = device_values(feats[:1, :w.shape[4]], w, b, dtype)
        dev_layers.append((li, tw, tb, w64, b.astype(np.float64)))
    coords, cc = coords_dev(c0), c0
    for li, (res, ch, convs) in enumerate(levels):
        rb = build(cc, res, 1)
        nbr = dense.neighbor_table(cc, res, 1)
        for lj, tw, tb, w64, b64 in dev_layers:
            if lj != li:
                continue
            x = sc.submconv_forward(x, tw, tb, rb)
            x64 = dense.forward(x64, w64, b64, nbr)
            if dtype == "bf16":
                x64 = synth.bf16_to_f32(synth.bf16_bits(x64.astype(np.float32))).astype(np.float64)
        rb.free()
        if li + 1 < len(levels):
            coords, x = sc.submconv_subdivide(coords, x)
            cc, x64 = ref.subdivide(cc, x64)
            np.testing.assert_array_equal(coords.cpu().numpy(), cc)
    assert_close(to_f64(x), x64, dtype, "chain output")


def test_block_cache_reuse_across_sizes_and_streams():
    """Builds that reuse the library's cached blocks (large and small sets in turn, a
    second stream, after an explicit release) give the same tables as fresh ones."""
    w2, c2 = synth.workload(2)
    w1, c1 = synth.workload(1)
    e2 = dense.neighbor_table(c2, w2.res, 1)
    e1 = dense.neighbor_table(c1, w1.res, 1)
    note("block cache")
    for it in range(3):
        for c, w, e in ((c2, w2, e2), (c1, w1, e1)):
            rb = build(c, w.res, 1)
            np.testing.assert_array_equal(rb.neighbors().cpu().numpy(), e)
            rb.free()
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        rb = sc.submconv_build_map(coords_dev(c2), w2.res, 1)
        got = rb.neighbors().cpu().numpy()
        rb.free()
    side.synchronize()
    np.testing.assert_array_equal(got, e2)
    sc.release_cache()
    rb = build(c1, w1.res, 1)
    np.testing.assert_array_equal(rb.neighbors().cpu().numpy(), e1)
    rb.free()


def test_rulebook_neighbors_pointer_matches_copy():
    """submconv_rulebook_neighbors builds the input-order table once and hands out
    a device pointer; its bytes equal the copy API's and the oracle's."""
    import ctypes
    w, c = synth.workload(2)
    rb = build(c[synth.shuffle_rows(len(c), 5)], w.res, 1)
    lib = sc.load_library()
    ptr, n = ctypes.c_void_p(), ctypes.c_int64()
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    note("rulebook_neighbors pointer")
    assert lib.submconv_rulebook_neighbors(rb.handle, stream, ctypes.byref(ptr), ctypes.byref(n)) == 0
    ptr2 = ctypes.c_void_p()
    assert lib.submconv_rulebook_neighbors(rb.handle, stream, ctypes.byref(ptr2), ctypes.byref(n)) == 0
    assert ptr.value == ptr2.value and n.value == rb.n
    torch.cuda.synchronize()
    hip = ctypes.CDLL("libamdhip64.so")
    host = np.empty((rb.n, 27), np.int32)
    assert hip.hipMemcpy(host.ctypes.data_as(ctypes.c_void_p), ptr, ctypes.c_size_t(host.nbytes), 2) == 0
    np.testing.assert_array_equal(host, rb.neighbors().cpu().numpy())
