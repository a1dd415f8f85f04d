"""GPU parity of the backward pass (mhla_backward through the C ABI) against
the fp64 oracle's gradients (chain rule through the three forward steps of
the MHLA paper §4.1; the oracle is pinned by finite differences and autograd).

Gate: 1e-2 for bf16, per gradient: max over (batch, head) slices of
max|g - g_oracle| / max|g_oracle| for dQ, dK, dV.  dW is a dot product over
all d*d + d state entries (and the batch) of bf16-rounded factors, whose
error is bounded relative to the sum of the absolute products, not to the
result (with the normaliser a row of dW sums to zero against W, and for
M = 1 it is exactly 0); its gate is max|dW - dW_oracle| per head over the
largest such absolute sum of that head.
"""
import numpy as np
import pytest
import torch

import oracle
import token_level_head_mhla_amd as m
from mhla_inputs import (DTYPE_BF16, FLAG_CAUSAL, FLAG_NO_NORM, PHI_ELU1, PHI_RELU, WORKLOADS,
                         bf16_bits_to_f32, custom_workload, make_inputs, make_upstream_grad)
from gpu_util import TOL, slice_error, to_device, to_f64

pytestmark = pytest.mark.gpu


def _bf16_dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def _run_backward(inp, gbits, flags=0):
    q, k, v, w = to_device(inp)
    dy = _bf16_dev(gbits)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    dw = torch.empty_like(w)
    m.mhla_backward(q, k, v, w, dy, dq, dk, dv, dw, (inp.wl.grid, inp.wl.block), inp.wl.phi,
                    flags)
    torch.cuda.synchronize()
    return to_f64(dq), to_f64(dk), to_f64(dv), dw.cpu().numpy().astype(np.float64)


def _head_error(a, ref, scale):
    num = np.abs(a - ref).reshape(a.shape[0], -1).max(axis=1)
    den = np.abs(scale).reshape(scale.shape[0], -1).max(axis=1)
    return float((num / np.where(den == 0, 1.0, den)).max())


def _check(wl, flags=0, label=""):
    inp = make_inputs(wl)
    gbits = make_upstream_grad(wl)
    got = _run_backward(inp, gbits, flags)
    G = bf16_bits_to_f32(gbits).astype(np.float64)
    ref = oracle.np_backward(inp.q_f64, inp.k_f64, inp.v_f64, inp.w_f64, G, wl.grid, wl.block,
                             wl.phi, norm=not (flags & FLAG_NO_NORM), dw_abs=True)
    errs = [slice_error(got[i], ref[i]) for i in range(3)] + [_head_error(got[3], ref[3], ref[4])]
    # reported beside the gate: dW's error relative to max|dW| per head (for
    # M = 1 with the normaliser dW is exactly 0 and this reads as the raw error)
    dw_rel_max = _head_error(got[3], ref[3], ref[3])
    print("PARITY backward %s %s %s d=%d phi=%d M=%d flags=%d errs dQ %.2e dK %.2e dV %.2e dW %.2e"
          " (dW / max|dW| %.2e)"
          % (label, wl.grid, wl.block, wl.d, wl.phi, wl.M, flags, *errs, dw_rel_max))
    for g in got:
        assert np.all(np.isfinite(g))
    for e in errs:
        assert e <= TOL[DTYPE_BF16]


BACKWARD_CASES = [
    # (B, H, grid, block, d, phi)
    (2, 3, (1, 14, 14), (1, 7, 7), 64, PHI_ELU1),    # DeiT-like, ragged 49-token blocks
    (2, 2, (1, 16, 16), (1, 4, 4), 72, PHI_RELU),    # DiT-like, 16-token blocks: token-pair backward
    (1, 2, (1, 32, 32), (1, 8, 8), 64, PHI_RELU),    # M = 16
    (2, 2, (1, 40, 52), (1, 4, 4), 32, PHI_ELU1),    # M = 130: partial dW tiles
    (2, 2, (1, 8, 8), (1, 8, 8), 16, PHI_ELU1),      # M = 1, d = 16 padded to 32
    (2, 3, (4, 8, 8), (2, 4, 4), 48, PHI_RELU),      # 3-D blocks, d = 48
    (1, 2, (1, 16, 16), (1, 16, 8), 96, PHI_ELU1),   # 128-token blocks, d = 96
    (1, 2, (1, 32, 32), (1, 2, 2), 32, PHI_ELU1),    # M = 256: large-M mixing, both directions
    (2, 2, (1, 48, 48), (1, 2, 4), 64, PHI_RELU),    # M = 288: partial 128-row dW tiles, d = 64
    (2, 2, (1, 20, 16), (1, 4, 4), 64, PHI_ELU1),    # M = 20: streamed mixing, both directions
    (2, 2, (1, 32, 32), (1, 4, 8), 96, PHI_ELU1),    # 32-token blocks, d = 96, M = 32: dW in 8 parts
    (1, 2, (1, 32, 64), (1, 4, 8), 72, PHI_RELU),    # d = 72 padded to 96, M = 64, B = 1, 8 parts
    (1, 32, (1, 60, 128), (1, 4, 8), 32, PHI_ELU1),  # M = 240, B = 1, 32 slices: one part, dW
                                                     # written directly, partial 64-row tiles
    (2, 2, (1, 32, 64), (1, 2, 4), 96, PHI_RELU),    # M = 256, d = 96: large-M mixing at DP = 96
]


@pytest.mark.parametrize("norm", [True, False])
@pytest.mark.parametrize("B,H,grid,block,d,phi", BACKWARD_CASES)
def test_backward_shapes(B, H, grid, block, d, phi, norm):
    wl = custom_workload(B, H, d, grid, block, phi, DTYPE_BF16, index=hash((grid, d)) % 953)
    _check(wl, 0 if norm else FLAG_NO_NORM)


def test_backward_mixing_many_slices():
    """M = 256, 64 slices, d = 32: the transposed large-M mixing runs 72 tiles
    per XCD, a second, ragged round of workgroups."""
    wl = custom_workload(1, 64, 32, (1, 1, 1024), (1, 1, 4), PHI_ELU1, DTYPE_BF16, index=461)
    _check(wl, 0)


PAIRS_BACKWARD_CASES = [
    # (B, H, grid, block, d, phi): blocks of at most 16 tokens take the
    # token-pair backward (two kernels, no d x d state)
    (2, 2, (1, 16, 16), (1, 4, 4), 72, PHI_ELU1),    # DiT-like: M = 16, d = 72 (16-wide tail)
    (2, 3, (1, 12, 16), (1, 3, 4), 64, PHI_RELU),    # 12-token blocks, M = 16
    (2, 2, (1, 6, 9), (1, 3, 3), 96, PHI_ELU1),      # 9-token blocks, M = 6, d = 96
    (3, 2, (4, 8, 8), (1, 2, 4), 32, PHI_RELU),      # M = 32: four query blocks per wave, B = 3
    (2, 2, (1, 4, 4), (1, 1, 1), 16, PHI_ELU1),      # one token per block, M = 16
    (2, 2, (1, 8, 8), (1, 4, 4), 48, PHI_RELU),      # M = 4: waves without a block
    (2, 2, (1, 10, 16), (1, 2, 8), 80, PHI_ELU1),    # d = 80, M = 10
    (2, 2, (1, 9, 15), (1, 3, 5), 48, PHI_ELU1),     # odd M = 9, 15-token blocks
    (1, 3, (1, 16, 16), (1, 4, 4), 64, PHI_RELU),    # one batch item: dW written directly
]


@pytest.mark.parametrize("norm", [True, False])
@pytest.mark.parametrize("B,H,grid,block,d,phi", PAIRS_BACKWARD_CASES)
def test_pairs_backward_shapes(B, H, grid, block, d, phi, norm):
    wl = custom_workload(B, H, d, grid, block, phi, DTYPE_BF16, index=hash((grid, d, 7)) % 951)
    _check(wl, 0 if norm else FLAG_NO_NORM, "pairs")


def test_pairs_backward_zero_denominator_rows():
    """ReLU queries with no positive feature have a 0/0 row (returned as 0):
    they must pass no gradient on the token-pair path either."""
    wl = custom_workload(2, 2, 48, (1, 8, 8), (1, 4, 4), PHI_RELU, DTYPE_BF16, index=17)
    inp = make_inputs(wl)
    bits = inp.q.copy()
    # make tokens 3 and 40 of every slice all-negative
    bits[:, :, [3, 40], :] = bits[:, :, [3, 40], :] | np.uint16(0x8000)
    inp.q = bits
    gbits = make_upstream_grad(wl)
    got = _run_backward(inp, gbits, 0)
    G = bf16_bits_to_f32(gbits).astype(np.float64)
    ref = oracle.np_backward(inp.q_f64, inp.k_f64, inp.v_f64, inp.w_f64, G, wl.grid, wl.block,
                             wl.phi, norm=True, dw_abs=True)
    errs = [slice_error(got[i], ref[i]) for i in range(3)] + [_head_error(got[3], ref[3], ref[4])]
    print("PARITY pairs backward zero-den errs", errs)
    assert np.all(got[0][:, :, [3, 40], :] == 0.0)
    for e in errs:
        assert e <= TOL[DTYPE_BF16]


@pytest.mark.parametrize("name,B,H", [("deit_t", 8, 3), ("dit_xl2", 4, 16), ("hires", 1, 4)])
def test_backward_workload_shapes(name, B, H):
    """The workloads' geometry and d with a reduced batch (the oracle's
    gradient materialises per-token states)."""
    wl = WORKLOADS[name]
    import dataclasses
    _check(dataclasses.replace(wl, B=B, H=H), 0, name)


@pytest.mark.parametrize("B,H,grid,block,d", [
    (2, 2, (1, 32, 32), (1, 2, 2), 64),   # M = 256: k_dw_big, partials summed by k_dw_reduce
    (2, 3, (1, 32, 64), (1, 4, 8), 64),   # M = 64: the split dW and its reduction
    (2, 2, (1, 16, 16), (1, 4, 4), 72),   # 16-token blocks: the token-pair backward
])
def test_backward_deterministic(B, H, grid, block, d):
    """Two calls on the same inputs give bit-identical dQ, dK, dV and dW: every
    partial sum is combined in a fixed order (no atomics)."""
    wl = custom_workload(B, H, d, grid, block, PHI_ELU1, DTYPE_BF16, index=613)
    inp = make_inputs(wl)
    gbits = make_upstream_grad(wl)
    q, k, v, w = to_device(inp)
    dy = _bf16_dev(gbits)
    outs = []
    for _ in range(2):
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        dw = torch.empty_like(w)
        m.mhla_backward(q, k, v, w, dy, dq, dk, dv, dw, (grid, block), wl.phi, 0)
        outs.append((dq, dk, dv, dw))
    torch.cuda.synchronize()
    for a, b in zip(*outs):
        assert torch.equal(a.view(torch.int32) if a.dtype == torch.float32 else a.view(torch.int16),
                           b.view(torch.int32) if b.dtype == torch.float32 else b.view(torch.int16))


def test_backward_rejects():
    wl = custom_workload(1, 1, 64, (1, 1, 128), (1, 1, 32), PHI_ELU1, DTYPE_BF16, index=2)
    inp = make_inputs(wl)
    with pytest.raises(m.MhlaError) as e:
        _run_backward(inp, make_upstream_grad(wl), FLAG_CAUSAL)
    assert e.value.code == m.MHLA_ERR_UNSUPPORTED
    q, k, v, w = to_device(inp)
    dy = _bf16_dev(make_upstream_grad(wl))
    with pytest.raises(m.MhlaError) as e:   # dQ aliases K
        m.mhla_backward(q, k, v, w, dy, k, torch.empty_like(k), torch.empty_like(v),
                        torch.empty_like(w), (wl.grid, wl.block), wl.phi)
    assert e.value.code == m.MHLA_ERR_ALIAS
