"""The C-ABI library loads and exports every declared symbol; host-side argument
checks fail with the documented status before any HIP call.  CPU only."""
import ctypes
import os
import re

import pytest

import torch  # noqa: F401  (loads the HIP runtime the library links against)

import submanifold_sparse_convolution_submconv3d_amd as sc

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "submconv.h")

E_INVALID_ARG, E_COORD_RANGE, E_DUPLICATE, E_UNSUPPORTED, E_ALIAS, E_OOM, E_HIP = -1, -2, -3, -4, -5, -6, -7


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(sc.lib_path()):
        pytest.fail("libsubmconv.so is not built; run __graft_entry__.build()")
    return sc.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(submconv_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for required in ("submconv_build_map", "submconv_forward", "submconv_rulebook_neighbors",
                     "submconv_rulebook_free", "submconv_subdivide", "submconv_space_to_depth",
                     "submconv_depth_to_space", "submconv_upsample_masked", "submconv_downsample",
                     "submconv_status_string"):
        assert required in names


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_status_strings(lib):
    for code in (0, -1, -2, -3, -4, -5, -6, -7):
        s = lib.submconv_status_string(code).decode()
        assert s and s != "unknown status"
    assert lib.submconv_status_string(-99).decode() == "unknown status"
    assert b"gfx950" in lib.submconv_version()


def _rb_ptr():
    return ctypes.c_void_p()


def test_build_map_argument_errors(lib):
    rb = ctypes.c_void_p()
    fake = ctypes.c_void_p(0x1000)            # never dereferenced: checks fail first
    assert lib.submconv_build_map(fake, 10, 16, 1, None, None) == E_INVALID_ARG
    assert lib.submconv_build_map(fake, -1, 16, 1, None, ctypes.byref(rb)) == E_INVALID_ARG
    assert lib.submconv_build_map(fake, 1 << 31, 16, 1, None, ctypes.byref(rb)) == E_INVALID_ARG
    assert lib.submconv_build_map(None, 10, 16, 1, None, ctypes.byref(rb)) == E_INVALID_ARG
    assert lib.submconv_build_map(ctypes.c_void_p(0x1004), 10, 16, 1, None, ctypes.byref(rb)) == E_INVALID_ARG
    assert lib.submconv_build_map(fake, 10, 0, 1, None, ctypes.byref(rb)) == E_INVALID_ARG
    assert lib.submconv_build_map(fake, 10, 16, 0, None, ctypes.byref(rb)) == E_INVALID_ARG
    # 3 * 21 bits + 2 batch bits > 64
    assert lib.submconv_build_map(fake, 10, 1 << 21, 4, None, ctypes.byref(rb)) == E_UNSUPPORTED
    assert rb.value is None
    assert b"key bits" in lib.submconv_last_error()


def test_forward_argument_errors(lib):
    fake = ctypes.c_void_p(0x1000)
    assert lib.submconv_forward(fake, fake, None, None, fake, 16, 16, 0, 0, None) == E_INVALID_ARG
    assert lib.submconv_forward_variant(fake, fake, None, None, fake, 16, 16, 0, 0, 0, None) == E_INVALID_ARG


def test_helper_argument_errors(lib):
    fake = ctypes.c_void_p(0x1000)
    m = ctypes.c_int64()
    assert lib.submconv_subdivide(fake, None, -1, 0, 0, fake, None, None) == E_INVALID_ARG
    assert lib.submconv_subdivide(None, None, 3, 0, 0, fake, None, None) == E_INVALID_ARG
    assert lib.submconv_subdivide(fake, None, 4, 0, 0, fake, None, None) == E_ALIAS
    assert lib.submconv_space_to_depth(fake, fake, 4, 8, 0, 16, 1, fake, fake, None, None, None) == E_INVALID_ARG
    assert lib.submconv_space_to_depth(fake, fake, 4, 8, 7, 16, 1, fake, fake, None, ctypes.byref(m), None) == E_UNSUPPORTED
    assert lib.submconv_space_to_depth(fake, fake, 4, 0, 0, 16, 1, fake, fake, None, ctypes.byref(m), None) == E_INVALID_ARG
    assert lib.submconv_depth_to_space(fake, fake, None, 4, 8, 0, fake, fake, None, None) == E_INVALID_ARG
    assert lib.submconv_depth_to_space(fake, fake, None, -2, 8, 0, fake, fake, ctypes.byref(m), None) == E_INVALID_ARG
    assert lib.submconv_upsample_masked(fake, fake, fake, 4, 8, 0, fake, fake, None, None) == E_INVALID_ARG
    assert lib.submconv_upsample_masked(fake, fake, None, 4, 8, 0, fake, fake, ctypes.byref(m), None) == E_INVALID_ARG
    assert lib.submconv_upsample_masked(fake, fake, fake, 4, 8, 3, fake, fake, ctypes.byref(m), None) == E_UNSUPPORTED
    assert lib.submconv_upsample_masked(fake, fake, fake, 4, 8, 0, fake, fake, ctypes.byref(m), None) == E_ALIAS
    assert lib.submconv_downsample(fake, fake, 4, 8, 0, 16, 1, 0, fake, fake, None, None) == E_INVALID_ARG
    assert lib.submconv_downsample(fake, fake, 4, 8, 0, 16, 1, 2, fake, fake, ctypes.byref(m), None) == E_INVALID_ARG
    assert lib.submconv_downsample(fake, fake, 4, 8, 0, 0, 1, 0, fake, fake, ctypes.byref(m), None) == E_INVALID_ARG
    assert lib.submconv_downsample(fake, fake, 4, 8, 0, 16, 1, 1, fake, fake, ctypes.byref(m), None) == E_ALIAS
    assert lib.submconv_rulebook_neighbors(None, None, None, None) == E_INVALID_ARG
    assert lib.submconv_rulebook_info(None, None, None, None, None) == E_INVALID_ARG
    assert lib.submconv_rulebook_free(None, None) == 0


def test_empty_inputs_are_no_ops(lib):
    m = ctypes.c_int64(5)
    assert lib.submconv_subdivide(None, None, 0, 0, 0, None, None, None) == 0
    assert lib.submconv_space_to_depth(None, None, 0, 4, 0, 16, 1, None, None, None, ctypes.byref(m), None) == 0
    assert m.value == 0
    m.value = 5
    assert lib.submconv_depth_to_space(None, None, None, 0, 4, 0, None, None, ctypes.byref(m), None) == 0
    assert m.value == 0
    m.value = 5
    assert lib.submconv_upsample_masked(None, None, None, 0, 4, 0, None, None, ctypes.byref(m), None) == 0
    assert m.value == 0
    m.value = 5
    assert lib.submconv_downsample(None, None, 0, 4, 1, 16, 1, 0, None, None, ctypes.byref(m), None) == 0
    assert m.value == 0


def test_classify_5d(lib):
    """Host-only: the layout of a 5-D 3x3x3 weight shape, and the ambiguous [O,3,3,3,3]."""
    def cls(shape, hint=-1):
        arr = (ctypes.c_int64 * 5)(*shape)
        out = ctypes.c_int32(-9)
        return lib.submconv_classify_5d(arr, hint, ctypes.byref(out)), out.value
    assert cls((64, 3, 3, 3, 32)) == (0, 0)          # KRSC
    assert cls((64, 32, 3, 3, 3)) == (0, 1)          # Conv3d
    assert cls((64, 3, 3, 3, 32), 0) == (0, 0)
    assert cls((64, 3, 3, 3, 3))[0] == E_INVALID_ARG  # fits both: needs the module's hint
    assert cls((64, 3, 3, 3, 3), 1) == (0, 1)
    assert cls((64, 3, 3, 3, 3), 0) == (0, 0)
    assert cls((64, 3, 3, 3, 32), 1)[0] == E_INVALID_ARG  # hint contradicts the shape
    assert cls((64, 5, 5, 5, 32))[0] == E_UNSUPPORTED
    assert cls((64, 0, 3, 3, 3))[0] == E_INVALID_ARG
    assert cls((64, 3, 3, 3, 32), 7)[0] == E_INVALID_ARG
    assert sc.classify_5d((16, 8, 3, 3, 3)) == "oidhw"
    assert sc.classify_5d((16, 3, 3, 3, 3), hint="krsc") == "krsc"
    with pytest.raises(sc.SubmconvError):
        sc.classify_5d((16, 3, 3, 3, 3))
    fake = ctypes.c_void_p(0x1000)
    assert lib.submconv_weight_convert(fake, 2, 4, 4, 0, 0, fake, None) == E_INVALID_ARG
    assert lib.submconv_weight_convert(fake, 0, 4, 4, 5, 0, fake, None) == E_UNSUPPORTED
    assert lib.submconv_weight_convert(fake, 0, 4, 4, 0, 0, fake, None) == E_ALIAS


def test_binding_requires_device_tensors():
    with pytest.raises(TypeError):
        sc.submconv_build_map(torch.zeros((3, 4), dtype=torch.int32), 16, 1)


def test_product_path_does_not_reference_the_oracle():
    pkg = os.path.dirname(sc.__file__)
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f)).read()
                assert "import oracle" not in text and "from oracle" not in text, f
                assert "dense_oracle" not in text, f


def test_noalloc_upsample_host_checks(lib):
    """The allocation-free masked upsample refuses sizes above its scratch limit and
    bad arguments on the host, before any device work."""
    cnt = ctypes.c_int64(-1)
    assert lib.submconv_upsample_masked_noalloc(None, None, None, 4000001, 8, 0, None, None,
                                                ctypes.byref(cnt), None) == E_UNSUPPORTED
    assert lib.submconv_upsample_masked_noalloc(None, None, None, 5, 8, 0, None, None,
                                                ctypes.byref(cnt), None) == E_INVALID_ARG
    assert lib.submconv_upsample_masked_noalloc(None, None, None, 5, 8, 0, None, None, None, None) == E_INVALID_ARG
    assert lib.submconv_upsample_masked_noalloc(None, None, None, 0, 8, 0, None, None,
                                                ctypes.byref(cnt), None) == 0 and cnt.value == 0
