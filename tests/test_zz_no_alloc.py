"""The allocation-free masked upsample (submconv_upsample_masked_noalloc) against the
allocating entry point (submconv_upsample_masked), called through the C ABI: two calls
in a row, the second on a smaller input, so stale scratch from the first call would
show; children and counts must agree exactly (pure copy and index work)."""
import ctypes

import numpy as np
import pytest
import torch

import synth
import submanifold_sparse_convolution_submconv3d_amd as sc

from gpu_common import note

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
MAX_N = 4000000           # SUBMCONV_NOALLOC_MAX_N


def _inputs(n, c, res, seed, dtype):
    coords = torch.from_numpy(synth.random_coords(n, res, 2, seed)).to(DEV)
    feats = torch.from_numpy(np.random.default_rng(seed).standard_normal((n, c)).astype(np.float32)).to(DEV)
    if dtype == torch.bfloat16:
        feats = feats.to(torch.bfloat16)
    mask = torch.from_numpy((np.random.default_rng(seed + 1).random((n, 8)) < 0.4).astype(np.uint8)).to(DEV)
    return coords, feats, mask


def _noalloc(lib, coords, feats, mask):
    n, c = feats.shape
    out_c = torch.full((max(8 * n, 1), 4), -7, dtype=torch.int32, device=DEV)
    out_f = torch.zeros((max(8 * n, 1), c), dtype=feats.dtype, device=DEV)
    cnt = ctypes.c_int64(-1)
    dt = 0 if feats.dtype == torch.float32 else 1
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    rc = lib.submconv_upsample_masked_noalloc(
        ctypes.c_void_p(coords.data_ptr()), ctypes.c_void_p(feats.data_ptr()), ctypes.c_void_p(mask.data_ptr()),
        n, c, dt, ctypes.c_void_p(out_c.data_ptr()), ctypes.c_void_p(out_f.data_ptr()), ctypes.byref(cnt), stream)
    assert rc == 0, lib.submconv_last_error().decode()
    return out_c, out_f, cnt.value


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_noalloc_matches_allocating_entry_point(dtype):
    lib = sc.load_library()
    for n, c, res, seed in ((600000, 32, 128, 3), (20001, 6, 48, 4)):   # the second call is smaller
        coords, feats, mask = _inputs(n, c, res, seed, dtype)
        note("noalloc upsample n=%d c=%d %s" % (n, c, dtype))
        ref_c, ref_f = sc.submconv_upsample_masked(coords, feats, mask)
        out_c, out_f, k = _noalloc(lib, coords, feats, mask)
        torch.cuda.synchronize()
        assert k == ref_c.shape[0] == int(mask.sum().item())
        assert torch.equal(out_c[:k], ref_c)
        assert torch.equal(out_f[:k].view(torch.int16) if dtype == torch.bfloat16 else out_f[:k],
                           ref_f.view(torch.int16) if dtype == torch.bfloat16 else ref_f)
        assert bool((out_c[k:] == -7).all())           # nothing written past the children


def test_noalloc_limits_and_empty():
    lib = sc.load_library()
    cnt = ctypes.c_int64(-1)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    note("noalloc limits")
    # above the limit: refused on the host before any device work
    assert lib.submconv_upsample_masked_noalloc(None, None, None, MAX_N + 1, 8, 0, None, None,
                                                ctypes.byref(cnt), stream) == -4
    assert lib.submconv_upsample_masked_noalloc(None, None, None, 0, 8, 0, None, None,
                                                ctypes.byref(cnt), stream) == 0
    assert cnt.value == 0
    # at the limit: runs, and agrees with the allocating entry point
    coords, feats, mask = _inputs(MAX_N, 2, 256, 9, torch.float32)
    note("noalloc at the limit n=%d" % MAX_N)
    ref_c, ref_f = sc.submconv_upsample_masked(coords, feats, mask)
    out_c, out_f, k = _noalloc(lib, coords, feats, mask)
    torch.cuda.synchronize()
    assert k == ref_c.shape[0]
    assert torch.equal(out_c[:k], ref_c) and torch.equal(out_f[:k], ref_f)
