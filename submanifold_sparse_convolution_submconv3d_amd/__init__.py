"""MI355X (gfx950) submanifold 3x3x3 sparse convolution: Python binding.

A thin ctypes binding over the C ABI in include/submconv.h.  It only
marshals arguments (torch tensors -> device pointers, the current HIP stream,
status codes -> exceptions); every step of the computation runs in the HIP
library `_lib/libsubmconv.so`.  PyTorch provides device memory and streams.

If the library has not been built, every call raises: there is no CPU or
PyTorch fallback.

Functions carry the C names:

    submconv_build_map(coords, res, batch)        -> Rulebook
    submconv_forward(feats, weight, bias, rb, ...) -> out
    submconv_subdivide(coords, feats=None)          -> (coords8, feats8)
    submconv_space_to_depth(coords, feats, res, batch) -> (coarse, feats8c, mask)
    submconv_depth_to_space(coarse, feats8c, mask=None) -> (coords, feats)
    submconv_upsample_masked(coords, feats, mask)   -> (coords, feats)
    submconv_downsample(coords, feats, res, batch, mode) -> (coarse, feats)
    classify_5d(shape, hint=None)                   -> "krsc" | "oidhw"
    weight_to_krsc(weight, layout=None, hint=None, flip=False) -> KRSC weight
    flip_ab(feats, weight, bias, rb)                -> {"corr": out, "conv": out} for an A/B

`RulebookCache` keeps one rulebook per coordinate set, keyed like the
upstream library's indice_key, so every convolution on a set reuses its map
(lato.2_mrp_mlx working notes, commit summary).
"""
from __future__ import annotations

import ctypes
import os
import weakref
from typing import Optional

import torch

__all__ = [
    "SubmconvError", "Rulebook", "RulebookCache", "lib_path", "load_library",
    "submconv_build_map", "submconv_forward", "submconv_subdivide",
    "submconv_space_to_depth", "submconv_depth_to_space", "submconv_upsample_masked", "submconv_downsample",
    "POOL_MAX", "POOL_MEAN", "classify_5d", "weight_to_krsc", "flip_ab", "release_cache", "set_cache_limit",
    "KERNEL_AUTO", "KERNEL_GENERIC", "KERNEL_LOWC", "KERNEL_MFMA", "KERNEL_WINDOW", "KERNEL_PERSISTENT",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "_lib", "libsubmconv.so")

F32, BF16 = 0, 1
KERNEL_AUTO, KERNEL_GENERIC, KERNEL_LOWC, KERNEL_MFMA, KERNEL_WINDOW, KERNEL_PERSISTENT = 0, 1, 2, 3, 4, 5

_lib = None


class SubmconvError(RuntimeError):
    """A non-zero status returned by the library."""

    def __init__(self, status: int, where: str, detail: str):
        self.status = status
        super().__init__("%s failed: %s (%d): %s" % (where, _status_name(status), status, detail))


def lib_path() -> str:
    return _LIB_PATH


def load_library():
    """Load libsubmconv.so (torch's HIP runtime is already loaded by `import torch`)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError("libsubmconv.so is not built (%s); run "
                           "`python -m submanifold_sparse_convolution_submconv3d_amd._build`" % _LIB_PATH)
    lib = ctypes.CDLL(_LIB_PATH)
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    i64p, i32p = ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_int32)
    sig = {
        "submconv_build_map": [vp, i64, i32, i32, vp, ctypes.POINTER(vp)],
        "submconv_rulebook_neighbors": [vp, vp, ctypes.POINTER(vp), i64p],
        "submconv_rulebook_copy_neighbors": [vp, vp, vp],
        "submconv_rulebook_info": [vp, i64p, i32p, i32p, i64p],
        "submconv_rulebook_free": [vp, vp],
        "submconv_forward": [vp, vp, vp, vp, vp, i32, i32, i32, i32, vp],
        "submconv_forward_variant": [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, vp],
        "submconv_subdivide": [vp, vp, i64, i32, i32, vp, vp, vp],
        "submconv_space_to_depth": [vp, vp, i64, i32, i32, i32, i32, vp, vp, vp, i64p, vp],
        "submconv_depth_to_space": [vp, vp, vp, i64, i32, i32, vp, vp, i64p, vp],
        "submconv_upsample_masked": [vp, vp, vp, i64, i32, i32, vp, vp, i64p, vp],
        "submconv_upsample_masked_noalloc": [vp, vp, vp, i64, i32, i32, vp, vp, i64p, vp],
        "submconv_downsample": [vp, vp, i64, i32, i32, i32, i32, i32, vp, vp, i64p, vp],
        "submconv_classify_5d": [i64p, i32, i32p],
        "submconv_release_cache": [i32],
        "submconv_set_cache_limit": [i64],
        "submconv_weight_convert": [vp, i32, i32, i32, i32, i32, vp, vp],
    }
    for name, args in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = ctypes.c_int
    for name in ("submconv_status_string",):
        getattr(lib, name).argtypes = [ctypes.c_int]
        getattr(lib, name).restype = ctypes.c_char_p
    for name in ("submconv_last_error", "submconv_version"):
        getattr(lib, name).argtypes = []
        getattr(lib, name).restype = ctypes.c_char_p
    _lib = lib
    return lib


def _status_name(status: int) -> str:
    try:
        return load_library().submconv_status_string(status).decode()
    except Exception:  # pragma: no cover - library missing
        return "status"


def _check(status: int, where: str):
    if status != 0:
        raise SubmconvError(status, where, load_library().submconv_last_error().decode())


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise TypeError("feature tensors must be float32 or bfloat16, got %s" % t.dtype)


def _dev(t: torch.Tensor, name: str, dtype=None) -> torch.Tensor:
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError("%s must be a GPU tensor" % name)
    if dtype is not None and t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    return t


def _raw_stream(index: int) -> int:
    """The current HIP stream of device `index` as an integer handle."""
    get = getattr(torch._C, "_cuda_getCurrentRawStream", None)
    if get is not None:
        return get(index)
    return torch.cuda.current_stream(index).cuda_stream


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(_raw_stream(torch.device(device).index))


class Rulebook:
    """A neighbour map built on the device for one coordinate set."""

    def __init__(self, handle: ctypes.c_void_p, device: torch.device, stream: int, n: int, res: int, batch: int):
        self._h = handle
        self.device = device
        self._stream = stream          # raw handle of the stream it was built on
        self.n, self.res, self.batch = n, res, batch
        self._taps = None

    @property
    def taps_present(self) -> int:
        """P, the number of entries of the neighbour table that are not -1."""
        if self._taps is None:
            taps = ctypes.c_int64()
            _check(load_library().submconv_rulebook_info(self.handle, None, None, None, ctypes.byref(taps)),
                   "submconv_rulebook_info")
            self._taps = taps.value
        return self._taps

    @property
    def handle(self) -> ctypes.c_void_p:
        if self._h is None:
            raise RuntimeError("rulebook already freed")
        return self._h

    def neighbors(self) -> torch.Tensor:
        """A copy of the int32 [n,27] neighbour table (row i, tap k -> row or -1)."""
        out = torch.empty((self.n, 27), dtype=torch.int32, device=self.device)
        with _on_device(self.device):
            _check(load_library().submconv_rulebook_copy_neighbors(self.handle, ctypes.c_void_p(out.data_ptr()),
                                                                   _stream(self.device)),
                   "submconv_rulebook_copy_neighbors")
        return out

    def free(self, stream: Optional[torch.cuda.Stream] = None):
        """Release the map, ordered on `stream` (default: the current stream of its
        device).  Work on other streams that still reads it must be ordered before
        that stream first, as for any stream-ordered free."""
        if self._h is not None and _lib is not None:
            with _on_device(self.device):
                s = stream.cuda_stream if stream is not None else _raw_stream(self.device.index)
                _lib.submconv_rulebook_free(self._h, ctypes.c_void_p(s))
        self._h = None

    def __del__(self):
        try:
            if self._h is not None and _lib is not None:
                # garbage collection: the release is ordered on the stream the map was built on
                _lib.submconv_rulebook_free(self._h, ctypes.c_void_p(self._stream))
                self._h = None
        except Exception:
            pass


class _on_device:
    """`with torch.cuda.device(d)` without its cost when d is already current."""

    __slots__ = ("_ctx",)

    def __init__(self, device: torch.device):
        idx = device.index
        self._ctx = None if idx is None or idx == torch.cuda.current_device() else torch.cuda.device(idx)

    def __enter__(self):
        if self._ctx is not None:
            self._ctx.__enter__()

    def __exit__(self, *exc):
        if self._ctx is not None:
            self._ctx.__exit__(*exc)


def submconv_build_map(coords: torch.Tensor, res: int, batch: Optional[int] = None) -> Rulebook:
    """Build the rulebook of int32 coords [N,4] (b, z, y, x) on a res^3 grid.

    `batch` is the number of batch entries; None reads max(b)+1 from the device."""
    _dev(coords, "coords", torch.int32)
    if coords.dim() != 2 or coords.shape[1] != 4:
        raise ValueError("coords must be [N,4]")
    if batch is None:
        batch = int(coords[:, 0].max().item()) + 1 if coords.shape[0] else 1
    lib = _lib if _lib is not None else load_library()
    h = ctypes.c_void_p()
    dev = coords.device
    n, res, batch = coords.shape[0], int(res), int(batch)
    with _on_device(dev):
        stream = _raw_stream(dev.index)
        _check(lib.submconv_build_map(coords.data_ptr(), n, res, batch, stream, ctypes.byref(h)),
               "submconv_build_map")
        return Rulebook(h, dev, stream, n, res, batch)


def submconv_forward(feats: torch.Tensor, weight: torch.Tensor, bias: Optional[torch.Tensor], rb: Rulebook,
                     out: Optional[torch.Tensor] = None, flip: bool = False,
                     variant: int = KERNEL_AUTO) -> torch.Tensor:
    """out[i] = bias + sum_k W[k] . feats[nbr[i,k]]; feats [N,Cin], weight KRSC [Cout,3,3,3,Cin]."""
    _dev(feats, "feats")
    _dev(weight, "weight", feats.dtype)
    if feats.dim() != 2 or feats.shape[0] != rb.n:
        raise ValueError("feats must be [N,Cin] with N = %d" % rb.n)
    cin = feats.shape[1]
    if weight.dim() != 5 or tuple(weight.shape[1:]) != (3, 3, 3, cin):
        raise ValueError("weight must be KRSC [Cout,3,3,3,%d]" % cin)
    cout = weight.shape[0]
    if bias is not None:
        _dev(bias, "bias", torch.float32)
        if bias.shape != (cout,):
            raise ValueError("bias must be fp32 [Cout]")
    if out is None:
        out = torch.empty((rb.n, cout), dtype=feats.dtype, device=feats.device)
    else:
        _dev(out, "out", feats.dtype)
        if tuple(out.shape) != (rb.n, cout):
            raise ValueError("out must be [N,Cout]")
    with _on_device(feats.device):
        _check(load_library().submconv_forward_variant(
            ctypes.c_void_p(feats.data_ptr()), ctypes.c_void_p(weight.data_ptr()),
            ctypes.c_void_p(bias.data_ptr() if bias is not None else None), rb.handle,
            ctypes.c_void_p(out.data_ptr()), cin, cout, _dtype_code(feats), int(bool(flip)), int(variant),
            _stream(feats.device)), "submconv_forward")
    return out


def submconv_subdivide(coords: torch.Tensor, feats: Optional[torch.Tensor] = None):
    """Children of every voxel: (int32 [8N,4], feats [8N,C] or None), parent-major, C order."""
    _dev(coords, "coords", torch.int32)
    n = coords.shape[0]
    out_c = torch.empty((8 * n, 4), dtype=torch.int32, device=coords.device)
    out_f, fp, ofp, c, dt = None, None, None, 0, F32
    if feats is not None:
        _dev(feats, "feats")
        c, dt = feats.shape[1], _dtype_code(feats)
        out_f = torch.empty((8 * n, c), dtype=feats.dtype, device=feats.device)
        fp, ofp = feats.data_ptr(), out_f.data_ptr()
    with _on_device(coords.device):
        _check(load_library().submconv_subdivide(ctypes.c_void_p(coords.data_ptr()), ctypes.c_void_p(fp), n, c, dt,
                                                 ctypes.c_void_p(out_c.data_ptr()), ctypes.c_void_p(ofp),
                                                 _stream(coords.device)), "submconv_subdivide")
    return out_c, out_f


def submconv_space_to_depth(coords: torch.Tensor, feats: torch.Tensor, res: int, batch: int):
    """Factor-2 sparse space-to-depth: (coarse int32 [M,4], feats [M,8C], uint8 mask [M,8])."""
    _dev(coords, "coords", torch.int32)
    _dev(feats, "feats")
    n, c = feats.shape
    out_c = torch.empty((max(n, 1), 4), dtype=torch.int32, device=coords.device)
    out_f = torch.empty((max(n, 1), 8 * c), dtype=feats.dtype, device=feats.device)
    mask = torch.empty((max(n, 1), 8), dtype=torch.uint8, device=feats.device)
    m = ctypes.c_int64()
    with _on_device(coords.device):
        _check(load_library().submconv_space_to_depth(
            ctypes.c_void_p(coords.data_ptr()), ctypes.c_void_p(feats.data_ptr()), n, c, _dtype_code(feats),
            int(res), int(batch), ctypes.c_void_p(out_c.data_ptr()), ctypes.c_void_p(out_f.data_ptr()),
            ctypes.c_void_p(mask.data_ptr()), ctypes.byref(m), _stream(coords.device)), "submconv_space_to_depth")
    m = m.value
    return out_c[:m], out_f[:m], mask[:m]


def submconv_depth_to_space(coarse: torch.Tensor, coarse_feats: torch.Tensor, mask: Optional[torch.Tensor] = None):
    """Inverse of space-to-depth: every slot (mask None) or the masked ones -> (coords, feats)."""
    _dev(coarse, "coarse", torch.int32)
    _dev(coarse_feats, "coarse_feats")
    m, c8 = coarse_feats.shape
    if c8 % 8:
        raise ValueError("coarse_feats must be [M, 8C]")
    c = c8 // 8
    mp = None
    if mask is not None:
        _dev(mask, "mask", torch.uint8)
        if tuple(mask.shape) != (m, 8):
            raise ValueError("mask must be uint8 [M,8]")
        mp = mask.data_ptr()
    out_c = torch.empty((max(8 * m, 1), 4), dtype=torch.int32, device=coarse.device)
    out_f = torch.empty((max(8 * m, 1), c), dtype=coarse_feats.dtype, device=coarse.device)
    cnt = ctypes.c_int64()
    with _on_device(coarse.device):
        _check(load_library().submconv_depth_to_space(
            ctypes.c_void_p(coarse.data_ptr()), ctypes.c_void_p(coarse_feats.data_ptr()), ctypes.c_void_p(mp), m, c,
            _dtype_code(coarse_feats), ctypes.c_void_p(out_c.data_ptr()), ctypes.c_void_p(out_f.data_ptr()),
            ctypes.byref(cnt), _stream(coarse.device)), "submconv_depth_to_space")
    k = cnt.value
    return out_c[:k], out_f[:k]


class RulebookCache:
    """One rulebook per coordinate set, looked up by a caller-chosen key
    (the upstream library's indice_key), built on first use.

    A cached map is reused only for the very coordinate tensor it was built from
    (the same tensor object, not modified in place since: its version counter is
    unchanged) and the same grid and batch count.  Any other tensor under the key,
    even one of the same size, rebuilds the map and replaces the entry."""

    def __init__(self):
        self._maps = {}

    def get(self, key, coords: torch.Tensor, res: int, batch: Optional[int] = None) -> Rulebook:
        entry = self._maps.get(key)
        if entry is not None:
            rb, ref, version, r, b = entry
            if (ref() is coords and coords._version == version and r == int(res)
                    and (batch is None or b == int(batch))):
                return rb
            self.drop(key)
        rb = submconv_build_map(coords, res, batch)
        self._maps[key] = (rb, weakref.ref(coords), coords._version, int(res), rb.batch)
        return rb

    def drop(self, key):
        entry = self._maps.pop(key, None)
        if entry is not None:
            entry[0].free()

    def clear(self):
        for k in list(self._maps):
            self.drop(k)

    def __len__(self):
        return len(self._maps)


POOL_MAX, POOL_MEAN = 0, 1  # submconv_downsample modes (SUBMCONV_POOL_*)


def submconv_upsample_masked(coords: torch.Tensor, feats: torch.Tensor, mask: torch.Tensor):
    """Masked expansion: voxel i emits child s iff mask[i, s] (axis 0 fastest), feats copied -> (coords, feats)."""
    _dev(coords, "coords", torch.int32)
    _dev(feats, "feats")
    _dev(mask, "mask", torch.uint8)
    n, c = feats.shape
    if tuple(mask.shape) != (n, 8) or coords.shape[0] != n:
        raise ValueError("coords [N,4], feats [N,C] and mask uint8 [N,8] must agree")
    out_c = torch.empty((max(8 * n, 1), 4), dtype=torch.int32, device=coords.device)
    out_f = torch.empty((max(8 * n, 1), c), dtype=feats.dtype, device=feats.device)
    cnt = ctypes.c_int64()
    with _on_device(coords.device):
        _check(load_library().submconv_upsample_masked(
            ctypes.c_void_p(coords.data_ptr()), ctypes.c_void_p(feats.data_ptr()), ctypes.c_void_p(mask.data_ptr()),
            n, c, _dtype_code(feats), ctypes.c_void_p(out_c.data_ptr()), ctypes.c_void_p(out_f.data_ptr()),
            ctypes.byref(cnt), _stream(coords.device)), "submconv_upsample_masked")
    k = cnt.value
    return out_c[:k], out_f[:k]


def submconv_downsample(coords: torch.Tensor, feats: torch.Tensor, res: int, batch: int, mode: str):
    """Factor-2 pooling of each coarse voxel's children, mode 'max' or 'mean' -> (coarse int32 [M,4], feats [M,C])."""
    if mode not in ("max", "mean"):
        raise ValueError("mode must be 'max' or 'mean' (it differs between models, so it has no default)")
    _dev(coords, "coords", torch.int32)
    _dev(feats, "feats")
    n, c = feats.shape
    out_c = torch.empty((max(n, 1), 4), dtype=torch.int32, device=coords.device)
    out_f = torch.empty((max(n, 1), c), dtype=feats.dtype, device=feats.device)
    m = ctypes.c_int64()
    with _on_device(coords.device):
        _check(load_library().submconv_downsample(
            ctypes.c_void_p(coords.data_ptr()), ctypes.c_void_p(feats.data_ptr()), n, c, _dtype_code(feats),
            int(res), int(batch), POOL_MAX if mode == "max" else POOL_MEAN, ctypes.c_void_p(out_c.data_ptr()),
            ctypes.c_void_p(out_f.data_ptr()), ctypes.byref(m), _stream(coords.device)), "submconv_downsample")
    k = m.value
    return out_c[:k], out_f[:k]


_LAYOUTS = {"krsc": 0, "oidhw": 1}


def classify_5d(shape, hint: Optional[str] = None) -> str:
    """"krsc" ([O,kz,ky,kx,I], spconv) or "oidhw" ([O,I,kz,ky,kx], torch Conv3d) for a
    5-D 3x3x3 weight shape; `hint` is the layout the caller's module implies, needed
    when the shape fits both ([O,3,3,3,3])."""
    if len(shape) != 5:
        raise ValueError("a 5-D weight shape is expected")
    arr = (ctypes.c_int64 * 5)(*[int(d) for d in shape])
    out = ctypes.c_int32(-1)
    h = -1 if hint is None else _LAYOUTS[hint]
    _check(load_library().submconv_classify_5d(arr, h, ctypes.byref(out)), "submconv_classify_5d")
    return "krsc" if out.value == 0 else "oidhw"


def weight_to_krsc(weight: torch.Tensor, layout: Optional[str] = None, hint: Optional[str] = None,
                   flip: bool = False) -> torch.Tensor:
    """KRSC copy of a 3x3x3 weight in either layout (classified from its shape when
    `layout` is None), mirrored (tap k -> 26 - k) when `flip`."""
    _dev(weight, "weight")
    if weight.dim() != 5:
        raise ValueError("a 5-D weight is expected")
    layout = layout or classify_5d(tuple(weight.shape), hint)
    if layout == "krsc":
        cout, cin = weight.shape[0], weight.shape[4]
    else:
        cout, cin = weight.shape[0], weight.shape[1]
    out = torch.empty((cout, 3, 3, 3, cin), dtype=weight.dtype, device=weight.device)
    with _on_device(weight.device):
        _check(load_library().submconv_weight_convert(
            ctypes.c_void_p(weight.data_ptr()), _LAYOUTS[layout], cout, cin, _dtype_code(weight), int(bool(flip)),
            ctypes.c_void_p(out.data_ptr()), _stream(weight.device)), "submconv_weight_convert")
    return out


def flip_ab(feats: torch.Tensor, weight: torch.Tensor, bias: Optional[torch.Tensor], rb: "Rulebook") -> dict:
    """Both kernel orientations on the same input, for an end-to-end A/B (the caller
    compares them downstream): "corr" reads feats[c + d] (flip 0), "conv" feats[c - d]
    (flip 1, the mirrored kernel)."""
    return {"corr": submconv_forward(feats, weight, bias, rb, flip=False),
            "conv": submconv_forward(feats, weight, bias, rb, flip=True)}


def release_cache(device: int = -1) -> None:
    """Return the device blocks the library keeps for reuse (all devices when -1)."""
    _check(load_library().submconv_release_cache(int(device)), "submconv_release_cache")


def set_cache_limit(nbytes: int) -> None:
    """Per-device limit of the library's block cache in bytes (0: no caching)."""
    _check(load_library().submconv_set_cache_limit(int(nbytes)), "submconv_set_cache_limit")
