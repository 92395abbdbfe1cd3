"""Helpers of the GPU parity tests: host <-> device transfer and the
tolerance rule for floating-point outputs.

Tolerance (fp32 accumulation, one rounding to the output type):
  |gpu - oracle| <= rtol * |oracle| + 1e-5 * S
where S is the oracle's sum of the magnitudes of the terms of that output
(the forward-error scale of a sum or dot product). rtol is 1e-5 for float32
outputs (wgrad always), 2e-2 for bfloat16 outputs and 2e-3 for float16
outputs (one float16 ulp is 2^-10 of the value).
"""
import numpy as np
import torch

import workloads as W

RTOL = {W.F32: 1e-5, W.BF16: 2e-2, W.F16: 2e-3}
ATOL_SCALE = 1e-5
TORCH_DT = {W.F32: torch.float32, W.BF16: torch.bfloat16, W.F16: torch.float16}

DEV = torch.device("cuda:0")


def to_dev(a, dtype=None):
    """numpy -> device tensor; uint16 storage becomes bf16/f16 when dtype says so."""
    a = np.ascontiguousarray(a)
    if dtype in (W.BF16, W.F16):
        return torch.from_numpy(a.view(np.int16)).view(TORCH_DT[dtype]).to(DEV)
    return torch.from_numpy(a).to(DEV)


def to_host(t):
    """device tensor -> numpy; bf16/f16 come back as uint16 bit patterns."""
    t = t.detach().contiguous().cpu()
    if t.dtype in (torch.bfloat16, torch.float16):
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def assert_close(gpu, want, scale, dtype, what):
    """The tolerance rule above; NaN never allowed on either side."""
    g = W.to_f32(gpu, dtype).astype(np.float64)
    o = W.to_f32(want, dtype).astype(np.float64)
    assert not np.isnan(g).any(), f"{what}: NaN in GPU output"
    assert not np.isnan(o).any(), f"{what}: NaN in oracle output"
    bound = RTOL[dtype] * np.abs(o) + ATOL_SCALE * scale
    err = np.abs(g - o)
    bad = err > bound
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError(f"{what}: {int(bad.sum())} elements out of tolerance; first at {tuple(i)}: "
                             f"gpu={g[tuple(i)]!r} oracle={o[tuple(i)]!r} bound={bound[tuple(i)]!r}")


def bits_equal(gpu, want, what):
    g = np.ascontiguousarray(gpu)
    w = np.ascontiguousarray(want)
    assert g.shape == w.shape, f"{what}: shape {g.shape} vs {w.shape}"
    gv = g.view(np.uint8).reshape(-1)
    wv = w.view(np.uint8).reshape(-1)
    if not np.array_equal(gv, wv):
        raise AssertionError(f"{what}: not bit-exact ({int(np.sum(gv != wv))} bytes differ)")
