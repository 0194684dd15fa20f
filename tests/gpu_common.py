"""Shared helpers of the GPU parity tests: input preparation from the seeded
generators and the comparison rules.  The expected values always come from
the CPU oracle; nothing here computes the method."""
import sys

import numpy as np
import torch

import synth

TOL = {"f32": 1e-4, "bf16": 2e-2}     # max|gpu - oracle| <= TOL * max|oracle|


def note(msg):
    """Name the case before a GPU step, flushed, so a failure can be placed."""
    print("[case] " + msg, flush=True)
    sys.stdout.flush()


def device_values(feats, weight, bias, dtype):
    """Device tensors of the given dtype and the float64 values the oracle sees
    (the bf16-decoded inputs for bf16, so input rounding is not counted as error)."""
    dev = torch.device("cuda:0")
    if dtype == "f32":
        f64, w64 = feats.astype(np.float64), weight.astype(np.float64)
        tf = torch.from_numpy(np.ascontiguousarray(feats)).to(dev)
        tw = torch.from_numpy(np.ascontiguousarray(weight)).to(dev)
    else:
        fb, wb = synth.bf16_bits(feats), synth.bf16_bits(weight)
        f64, w64 = synth.bf16_to_f32(fb).astype(np.float64), synth.bf16_to_f32(wb).astype(np.float64)
        tf = torch.from_numpy(fb.view(np.int16)).view(torch.bfloat16).to(dev).reshape(feats.shape)
        tw = torch.from_numpy(wb.view(np.int16)).view(torch.bfloat16).to(dev).reshape(weight.shape)
    tb = None if bias is None else torch.from_numpy(np.ascontiguousarray(bias, dtype=np.float32)).to(dev)
    return tf, tw, tb, f64, w64


def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def assert_close(got, expect, dtype, what=""):
    scale = float(np.max(np.abs(expect))) if expect.size else 0.0
    err = float(np.max(np.abs(got - expect))) if expect.size else 0.0
    bound = TOL[dtype] * max(scale, 1e-30)
    assert err <= bound, "%s: max err %.3e > %.3e (max|out| %.3e)" % (what, err, bound, scale)
    return err / max(scale, 1e-30)
