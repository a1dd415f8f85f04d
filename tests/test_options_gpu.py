"""GPU parity of the options: the normaliser switch on every path and the
chunkwise causal form, through mhla_forward_ex, against the fp64 oracle.

Same gate as the plain forward: max over (batch, head) slices of
max|y - y_oracle| / max|y_oracle| <= 1e-5 (fp32 inputs), 1e-2 (bf16 inputs).
"""
import numpy as np
import pytest
import torch

import oracle
import token_level_head_mhla_amd as m
from mhla_inputs import (DTYPE_BF16, DTYPE_F32, FLAG_CAUSAL, FLAG_NO_NORM, PHI_ELU1, PHI_RELU,
                         WORKLOADS, custom_workload, make_inputs)
from gpu_util import TOL, run, slice_error, to_device, to_f64

pytestmark = pytest.mark.gpu


def _oracle(inp, sl=None):
    wl = inp.wl
    q, k, v = inp.q_f64, inp.k_f64, inp.v_f64
    w = inp.w_f64
    if sl is not None:
        b, h = sl
        q, k, v = (x[b:b + 1, h:h + 1] for x in (q, k, v))
        w = w[h:h + 1]
    return oracle.blockwise(q, k, v, w, wl.grid, wl.block, wl.phi, norm=wl.norm,
                            causal=wl.causal)


NO_NORM_CASES = [
    # (B, H, grid, block, d, phi, dtype, path)
    (1, 2, (1, 8, 8), (1, 4, 4), 16, PHI_RELU, DTYPE_F32, m.MHLA_PATH_GENERIC),
    (2, 2, (1, 6, 10), (1, 3, 5), 24, PHI_ELU1, DTYPE_BF16, m.MHLA_PATH_GENERIC),
    (4, 3, (1, 14, 14), (1, 7, 7), 64, PHI_ELU1, DTYPE_BF16, m.MHLA_PATH_FUSED),
    (3, 2, (1, 8, 8), (1, 4, 8), 32, PHI_RELU, DTYPE_BF16, m.MHLA_PATH_FUSED),
    (2, 4, (1, 16, 16), (1, 4, 4), 72, PHI_RELU, DTYPE_BF16, m.MHLA_PATH_PAIRS),
    (2, 3, (1, 9, 9), (1, 3, 3), 48, PHI_ELU1, DTYPE_BF16, m.MHLA_PATH_PAIRS),
    (1, 4, (1, 32, 32), (1, 8, 8), 64, PHI_RELU, DTYPE_BF16, m.MHLA_PATH_BLOCKED),
    (2, 2, (2, 16, 16), (1, 4, 8), 96, PHI_ELU1, DTYPE_BF16, m.MHLA_PATH_BLOCKED),
    (1, 4, (1, 32, 32), (1, 8, 8), 64, PHI_RELU, DTYPE_BF16, m.MHLA_PATH_COLUMNS),
    (2, 2, (2, 16, 16), (1, 4, 8), 40, PHI_ELU1, DTYPE_BF16, m.MHLA_PATH_COLUMNS),
]


@pytest.mark.parametrize("B,H,grid,block,d,phi,dtype,path", NO_NORM_CASES)
def test_no_norm_paths(B, H, grid, block, d, phi, dtype, path):
    wl = custom_workload(B, H, d, grid, block, phi, dtype, index=hash((grid, d, path)) % 977,
                         flags=FLAG_NO_NORM)
    inp = make_inputs(wl)
    y = to_f64(run(inp, path))
    err = slice_error(y, _oracle(inp))
    print("PARITY no-norm %s %s d=%d path=%d err=%.3e" % (grid, block, d, path, err))
    assert np.all(np.isfinite(y))
    assert err <= TOL[dtype]


CAUSAL_CASES = [
    # (grid, block, d, phi): blocks must be runs of consecutive tokens
    ((1, 1, 256), (1, 1, 64), 64, PHI_ELU1),    # 4 chunks of 64 (the LM chunk)
    ((1, 1, 96), (1, 1, 32), 32, PHI_RELU),     # d = 32
    ((1, 1, 120), (1, 1, 40), 64, PHI_ELU1),    # ragged chunk: 40 tokens
    ((1, 8, 24), (1, 2, 24), 48, PHI_RELU),     # 2-D grid, two full rows per block
    ((4, 8, 8), (1, 8, 8), 72, PHI_ELU1),       # whole frames, d = 72 padded to 96
    ((1, 1, 256), (1, 1, 256), 64, PHI_ELU1),   # one chunk of the maximum 256 tokens
    ((1, 1, 40), (1, 1, 1), 16, PHI_ELU1),      # one token per chunk, M = 40
    ((1, 1, 1200), (1, 1, 24), 96, PHI_RELU),   # M = 50, d = 96
    ((1, 1, 8192), (1, 1, 32), 32, PHI_ELU1),   # M = 256: the large-M prefix mixing
    ((1, 1, 4608), (1, 1, 16), 16, PHI_RELU),   # M = 288: a partial query-block tile
    ((1, 1, 20480), (1, 1, 64), 64, PHI_ELU1),  # M = 320, d = 64 (the video entry width)
]


@pytest.mark.parametrize("norm", [True, False])
@pytest.mark.parametrize("grid,block,d,phi", CAUSAL_CASES)
def test_causal_shapes(grid, block, d, phi, norm):
    flags = FLAG_CAUSAL | (0 if norm else FLAG_NO_NORM)
    wl = custom_workload(2, 3, d, grid, block, phi, DTYPE_BF16,
                         index=hash((grid, block, d)) % 967, flags=flags)
    inp = make_inputs(wl)
    y = to_f64(run(inp, m.MHLA_PATH_AUTO))
    assert np.all(np.isfinite(y))
    err = slice_error(y, _oracle(inp))
    print("PARITY causal %s %s d=%d phi=%d norm=%d M=%d err=%.3e"
          % (grid, block, d, phi, norm, wl.M, err))
    assert err <= TOL[DTYPE_BF16]


@pytest.mark.parametrize("n,chunk", [(512, 64), (8192, 32)])
def test_causal_ignores_upper_triangle(n, chunk):
    """W[i,b] for b > i never enters the causal form: the output is bit-identical
    when those entries change (M = 8, and M = 256 for the large-M mixing)."""
    wl = custom_workload(2, 2, 64, (1, 1, n), (1, 1, chunk), PHI_ELU1, DTYPE_BF16, index=31,
                         flags=FLAG_CAUSAL)
    inp = make_inputs(wl)
    q, k, v, w = to_device(inp)
    y1 = run(inp, dev=(q, k, v, w))
    w2 = w.clone()
    iu = torch.triu_indices(wl.M, wl.M, 1)
    w2[:, iu[0], iu[1]] = 7.0
    y2 = run(inp, dev=(q, k, v, w2))
    assert torch.equal(y1, y2)


def test_lm_causal_workload_sampled():
    """The language-model workload at full size (chunkwise causal, no
    normaliser): whole sampled slices against the chunkwise oracle and random
    rows against the masked brute force."""
    wl = WORKLOADS["lm_causal"]
    inp = make_inputs(wl)
    y = to_f64(run(inp, m.MHLA_PATH_AUTO))
    assert np.all(np.isfinite(y))
    rng = np.random.default_rng(5)
    S = wl.B * wl.H
    err = 0.0
    for s in sorted({0, S - 1, *rng.choice(S, 3, replace=False).tolist()}):
        b, h = divmod(s, wl.H)
        err = max(err, slice_error(y[b:b + 1, h:h + 1], _oracle(inp, (b, h))))
    rows = rng.choice(S * wl.N, size=128, replace=False)
    ref_rows = oracle.rows(inp.q_f64, inp.k_f64, inp.v_f64, inp.w_f64, wl.grid, wl.block, wl.phi,
                           rows, norm=False, causal=True)
    yr = y.reshape(-1, wl.d)[rows]
    scale = np.abs(y.reshape(-1, wl.d)).max()
    err_rows = float(np.abs(yr - ref_rows).max() / scale)
    print("PARITY lm_causal slices_err=%.3e rows_err=%.3e" % (err, err_rows))
    assert err <= TOL[DTYPE_BF16]
    assert err_rows <= TOL[DTYPE_BF16]


def test_options_rejected_before_launch():
    wl = custom_workload(1, 1, 64, (1, 14, 14), (1, 7, 7), PHI_ELU1, DTYPE_BF16, index=3,
                         flags=FLAG_CAUSAL)
    inp = make_inputs(wl)
    with pytest.raises(m.MhlaError) as e:
        run(inp)
    assert e.value.code == m.MHLA_ERR_SHAPE
    wl = custom_workload(1, 1, 64, (1, 1, 256), (1, 1, 64), PHI_ELU1, DTYPE_BF16, index=3,
                         flags=FLAG_CAUSAL)
    for path in (m.MHLA_PATH_FUSED, m.MHLA_PATH_PAIRS, m.MHLA_PATH_GENERIC, m.MHLA_PATH_COLUMNS):
        with pytest.raises(m.MhlaError) as e:
            run(make_inputs(wl), path)
        assert e.value.code == m.MHLA_ERR_UNSUPPORTED
