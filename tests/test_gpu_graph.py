"""The forward inside a HIP graph.

`submconv_forward` is one kernel launch on the caller's stream: it neither
synchronises nor allocates nor clears memory, so a caller can capture it in a HIP
graph (here `torch.cuda.CUDAGraph`) and replay it, as a serving loop would.  Each
test captures one forward per kernel family, replays it three times with the
program's own eager work and synchronisations in between, writes new feature values
into the captured input buffer before the later replays, and checks every replay bit
for bit against an eager call on the same inputs; the first replay is also checked
against the C oracle."""
import numpy as np
import pytest
import torch

import synth
import submanifold_sparse_convolution_submconv3d_amd as sc
from oracle import dense

from gpu_common import assert_close, device_values, note, to_f64

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")

VARIANTS = {"generic": sc.KERNEL_GENERIC, "lowc": sc.KERNEL_LOWC, "mfma": sc.KERNEL_MFMA,
            "window": sc.KERNEL_WINDOW, "persistent": sc.KERNEL_PERSISTENT, "auto": sc.KERNEL_AUTO}


@pytest.fixture(scope="module", autouse=True)
def _gpu(oracle_built):
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    sc.load_library()


@pytest.mark.parametrize("kernel,cin,cout,dtype", [
    ("generic", 3, 5, "f32"), ("lowc", 16, 16, "f32"), ("mfma", 64, 64, "f32"), ("auto", 128, 128, "f32"),
    ("persistent", 64, 64, "bf16"), ("persistent", 128, 128, "bf16"), ("mfma", 64, 64, "bf16"),
    ("window", 32, 32, "bf16")])
def test_forward_graph_replays(kernel, cin, cout, dtype):
    res, batch = 40, 2
    c = synth.random_coords(20000, res, batch, 71)
    feats, weight, bias = synth.make_values(len(c), cin, cout, 71)
    tf, tw, tb, f64, w64 = device_values(feats, weight, bias, dtype)
    rb = sc.submconv_build_map(torch.from_numpy(c).to(DEV), res, batch)
    torch.cuda.synchronize()
    variant = VARIANTS[kernel]
    out_g = torch.empty((len(c), cout), dtype=tf.dtype, device=DEV)
    note("graph forward %s %d->%d %s n=%d" % (kernel, cin, cout, dtype, len(c)))
    # an eager call first, so the library's one-time set-up happens outside the capture
    sc.submconv_forward(tf, tw, tb, rb, out=out_g, variant=variant)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        sc.submconv_forward(tf, tw, tb, rb, out=out_g, variant=variant)
    torch.cuda.synchronize()
    for rep in range(3):
        if rep:
            nf, _, _ = synth.make_values(len(c), cin, cout, 71 + rep)
            tf.copy_(device_values(nf, weight, bias, dtype)[0])
            f64 = None
        eager = sc.submconv_forward(tf, tw, tb, rb, variant=variant)
        out_g.zero_()
        torch.cuda.synchronize()
        note("graph replay %d" % rep)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_g, eager), "replay %d differs from the eager call" % rep
        if f64 is not None:
            expect = dense.forward(f64, w64, bias, dense.neighbor_table(c, res, batch), 0)
            assert_close(to_f64(out_g), expect, dtype, "graph replay %s %d->%d %s" % (kernel, cin, cout, dtype))
    g.reset()
    rb.free()
