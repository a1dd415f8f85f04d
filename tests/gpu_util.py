"""Helpers for the GPU tests: move seeded inputs to the device, run a path
through the C ABI, and measure the error against the oracle."""
from __future__ import annotations

import numpy as np
import torch

import token_level_head_mhla_amd as m
from mhla_inputs import DTYPE_BF16, Inputs

# Parity gates: max over (b, h) slices of max|y - y_ref| / max|y_ref|.
TOL = {0: 1e-5, 1: 1e-2}


def to_device(inp: Inputs):
    def t(x):
        if inp.wl.dtype == DTYPE_BF16:
            return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(np.ascontiguousarray(x)).cuda()
    return t(inp.q), t(inp.k), t(inp.v), torch.from_numpy(inp.w).cuda()


def run(inp: Inputs, path=m.MHLA_PATH_AUTO, dev=None, stream=None, skip_unsupported=False):
    """Run one path through the C ABI.  With skip_unsupported, a path that
    rejects the shape (MHLA_ERR_UNSUPPORTED, nothing enqueued) skips the test."""
    q, k, v, w = dev if dev is not None else to_device(inp)
    out = torch.empty_like(q)
    try:
        if inp.wl.flags:
            m.mhla_forward_ex(q, k, v, w, out, (inp.wl.grid, inp.wl.block), inp.wl.phi,
                              inp.wl.flags, path, stream=stream)
        else:
            m.mhla_forward_path(q, k, v, w, out, (inp.wl.grid, inp.wl.block), inp.wl.phi, path,
                                stream=stream)
    except m.MhlaError as e:
        if skip_unsupported and e.code == m.MHLA_ERR_UNSUPPORTED:
            import pytest
            pytest.skip("path %d does not take this shape" % path)
        raise
    torch.cuda.synchronize()
    return out


def to_f64(out: torch.Tensor) -> np.ndarray:
    return out.float().cpu().numpy().astype(np.float64)


def slice_error(y: np.ndarray, ref: np.ndarray) -> float:
    """max over slices of the infinity-norm error relative to the slice's max."""
    y = y.reshape(-1, y.shape[-2] * y.shape[-1])
    ref = ref.reshape(-1, ref.shape[-2] * ref.shape[-1])
    num = np.abs(y - ref).max(axis=1)
    den = np.abs(ref).max(axis=1)
    den = np.where(den == 0, 1.0, den)
    return float((num / den).max())
