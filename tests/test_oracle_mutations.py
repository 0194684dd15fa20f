"""Plant plausible mistakes in the Python oracle (on the CPU) and check that the
pins catch each one: swapped axes in the tap order, the mirrored orientation,
a transposed weight tap, a dropped bias, an off-by-one offset, a dropped tap."""
import json
import os

import numpy as np
import pytest

import synth
from oracle import reference as ref

from test_oracle_pins import brute_force_nbr, dense_conv_at_sites

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _pins_pass(monkeypatch_ctx=None):
    """True iff the hand example, brute force and dense conv3d pins all hold."""
    g = json.load(open(os.path.join(GOLDEN, "hand_example.json")))
    coords = np.array(g["coords"], np.int32)
    w = np.zeros((1, 3, 3, 3, 1))
    for kz in range(3):
        for ky in range(3):
            for kx in range(3):
                w[0, kz, ky, kx, 0] = 9 * kz + 3 * ky + kx + 1
    try:
        nbr = ref.neighbor_table(coords, 4, 1)
        if not np.array_equal(ref.forward(np.array(g["feats"]), w, np.array(g["bias"]), nbr)[:, 0],
                              np.array(g["out_corr"])):
            return False
        c2 = synth.random_coords(300, 8, 2, 2)
        if not np.array_equal(ref.neighbor_table(c2, 8, 2), brute_force_nbr(c2)):
            return False
        c3 = synth.random_coords(400, 10, 1, 3)
        f, wt, b = synth.make_values(400, 5, 7, 3)
        got = ref.forward(f, wt, b, ref.neighbor_table(c3, 10, 1))
        return np.allclose(got, dense_conv_at_sites(c3, f, wt, b, 10, False), rtol=1e-10, atol=1e-10)
    except Exception:
        return False


def test_unmutated_oracle_passes():
    assert _pins_pass()


def _swap_axes(k):
    return (k % 3 - 1, (k // 3) % 3 - 1, k // 9 - 1)


def _off_by_one(k):
    dz, dy, dx = (k // 9 - 1, (k // 3) % 3 - 1, k % 3 - 1)
    return (dz, dy, dx + (1 if k == 5 else 0))


_orig_weight_tap = ref.weight_tap
_orig_forward = ref.forward


def _mirrored(weight, k, flip):
    return _orig_weight_tap(weight, k, not flip)


def _transposed(weight, k, flip):
    wk = _orig_weight_tap(weight, k, flip)
    return wk.T[: wk.shape[0], : wk.shape[1]] if wk.shape[0] == wk.shape[1] else wk.T.reshape(wk.shape)


def _no_bias(feats, weight, bias, nbr, flip=False):
    return _orig_forward(feats, weight, None, nbr, flip)


def _drop_tap(feats, weight, bias, nbr, flip=False):
    nb = nbr.copy()
    nb[:, 26] = -1
    return _orig_forward(feats, weight, bias, nb, flip)


@pytest.mark.parametrize("name,attr,impl", [
    ("swapped axes", "tap_offset", _swap_axes),
    ("off-by-one offset", "tap_offset", _off_by_one),
    ("mirrored orientation", "weight_tap", _mirrored),
    ("transposed weight tap", "weight_tap", _transposed),
    ("dropped bias", "forward", _no_bias),
    ("dropped tap", "forward", _drop_tap),
])
def test_planted_mistake_is_caught(monkeypatch, name, attr, impl):
    monkeypatch.setattr(ref, attr, impl)
    assert not _pins_pass(), name


@pytest.mark.parametrize("perm", [(0, 4, 3, 2, 1), (0, 3, 2, 4, 1), (0, 2, 4, 3, 1)])
def test_weight_layout_mutations_are_caught(monkeypatch, perm):
    """A Conv3d -> KRSC conversion with two kernel axes swapped keeps every shape valid;
    the dense conv3d pin must reject it."""
    import test_oracle_pins as pins
    monkeypatch.setattr(ref, "conv3d_to_krsc", lambda w: np.ascontiguousarray(np.transpose(np.asarray(w), perm)))
    with pytest.raises(AssertionError):
        pins.test_weight_layouts_against_dense_conv3d()


def test_partial_mirror_is_caught(monkeypatch):
    """A mirror over two of the three kernel axes must fail the mirror pin."""
    import test_oracle_pins as pins
    monkeypatch.setattr(ref, "mirror_krsc", lambda w: np.ascontiguousarray(np.asarray(w)[:, ::-1, ::-1, :, :]))
    with pytest.raises(AssertionError):
        pins.test_weight_layouts_against_dense_conv3d()


def _c_order_child(slot, f=2):
    return (slot // (f * f) % f, (slot // f) % f, slot % f)


def _c_order_slot(z, y, x, f=2):
    return (z % f) * f * f + (y % f) * f + (x % f)


@pytest.mark.parametrize("attr,impl", [("child_offset", _c_order_child), ("s2d_slot", _c_order_slot)])
def test_c_order_slot_mutations_are_caught(monkeypatch, attr, impl):
    """Decoding or encoding the slot in C order (subdivide's order) instead of axis 0
    fastest must fail the hand-worked space-to-depth example."""
    import test_oracle_pins as pins
    monkeypatch.setattr(ref, attr, impl)
    with pytest.raises(AssertionError):
        pins.test_s2d_hand_example_golden()
