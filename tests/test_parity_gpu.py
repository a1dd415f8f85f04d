"""GPU parity: the HIP path (called through the C ABI) against the fp64 oracle.

Gate (floating point): max over (batch, head) slices of
max|y - y_oracle| / max|y_oracle| <= 1e-5 for fp32 inputs, 1e-2 for bf16
inputs.  Each test prints the measured error.
"""
import numpy as np
import pytest
import torch

import oracle
import token_level_head_mhla_amd as m
from mhla_inputs import (DTYPE_BF16, DTYPE_F32, PHI_ELU1, PHI_RELU, WORKLOADS, custom_workload,
                         make_inputs)
from gpu_util import TOL, run, slice_error, to_device, to_f64

pytestmark = pytest.mark.gpu

ALL_PATHS = [m.MHLA_PATH_GENERIC, m.MHLA_PATH_FUSED, m.MHLA_PATH_BLOCKED, m.MHLA_PATH_PAIRS,
             m.MHLA_PATH_COLUMNS]
# paths that take only some shapes: an unsupported shape skips the case
PARTIAL_PATHS = (m.MHLA_PATH_PAIRS, m.MHLA_PATH_COLUMNS)


def _oracle_full(inp):
    wl = inp.wl
    return oracle.blockwise(inp.q_f64, inp.k_f64, inp.v_f64, inp.w_f64, wl.grid, wl.block, wl.phi)


def _check_sampled(inp, y, n_slices, n_rows, seed=0):
    """Compare whole sampled slices (blockwise oracle) and brute-force rows."""
    wl = inp.wl
    rng = np.random.default_rng(seed)
    S = wl.B * wl.H
    picks = sorted(set([0, S - 1] + rng.choice(S, size=min(S, n_slices), replace=False).tolist()))
    q, k, v = inp.q_f64, inp.k_f64, inp.v_f64
    err = 0.0
    for s in picks:
        b, h = divmod(s, wl.H)
        ref = oracle.blockwise(q[b:b + 1, h:h + 1], k[b:b + 1, h:h + 1], v[b:b + 1, h:h + 1],
                               inp.w_f64[h:h + 1], wl.grid, wl.block, wl.phi)
        err = max(err, slice_error(y[b:b + 1, h:h + 1], ref))
    rows = rng.choice(S * wl.N, size=n_rows, replace=False)
    ref_rows = oracle.rows(q, k, v, inp.w_f64, wl.grid, wl.block, wl.phi, rows)
    yr = y.reshape(-1, wl.d)[rows]
    # rows are judged against their own slice's max (from the sampled slices' scale)
    scale = np.abs(ref_rows).max()
    err_rows = float(np.abs(yr - ref_rows).max() / scale)
    return err, err_rows


@pytest.mark.parametrize("name", ["tiny", "deit_t", "dit_xl2", "hires"])
@pytest.mark.parametrize("path", [m.MHLA_PATH_AUTO, m.MHLA_PATH_GENERIC, m.MHLA_PATH_BLOCKED,
                                  m.MHLA_PATH_PAIRS, m.MHLA_PATH_COLUMNS])
def test_workload_full(name, path):
    if path != m.MHLA_PATH_AUTO and path != m.MHLA_PATH_GENERIC and \
            WORKLOADS[name].dtype != DTYPE_BF16:
        pytest.skip("the MFMA paths take bf16 inputs")
    wl = WORKLOADS[name]
    inp = make_inputs(wl)
    y = to_f64(run(inp, path, skip_unsupported=(path in PARTIAL_PATHS)))
    ref = _oracle_full(inp)
    err = slice_error(y, ref)
    print("PARITY %s path=%d err=%.3e elementwise_floor1e-3=%.3e" % (name, path, err,
                                                                     _elementwise_info(y, ref)))
    assert np.all(np.isfinite(y))
    assert err <= TOL[wl.dtype]


def _elementwise_info(y, ref):
    """Elementwise relative error with a floor of 1e-3 of the slice's max|y|
    (reported only; the gate is the per-slice infinity-norm error)."""
    yr = y.reshape(-1, y.shape[-2] * y.shape[-1])
    rr = ref.reshape(-1, ref.shape[-2] * ref.shape[-1])
    floor = 1e-3 * np.abs(rr).max(axis=1, keepdims=True)
    return float((np.abs(yr - rr) / np.maximum(np.abs(rr), floor)).max())


def test_video_full():
    """The video-latent workload at full size (B1 H24 N32768, M = 512) in the
    launch configuration the benchmark times (the automatic path): all 24
    heads against the blockwise oracle (MHLA paper §4.1), and 256 brute-force
    rows of the explicit token-pair matrix (§4.2 Eq. 5) on each of four heads
    (the first, the last and two drawn at random)."""
    wl = WORKLOADS["video"]
    inp = make_inputs(wl)
    y = to_f64(run(inp, m.MHLA_PATH_AUTO))
    assert np.all(np.isfinite(y))
    q, k, v, w = inp.q_f64, inp.k_f64, inp.v_f64, inp.w_f64
    ref = oracle.blockwise(q, k, v, w, wl.grid, wl.block, wl.phi)
    err = slice_error(y, ref)
    info = _elementwise_info(y, ref)
    del ref
    rng = np.random.default_rng(7)
    S = wl.B * wl.H
    heads = [0, S - 1] + sorted(rng.choice(np.arange(1, S - 1), size=2, replace=False).tolist())
    err_rows = 0.0
    for s in heads:
        rows = s * wl.N + rng.choice(wl.N, size=256, replace=False)
        ref_rows = oracle.rows(q, k, v, w, wl.grid, wl.block, wl.phi, rows)
        b, h = divmod(s, wl.H)
        scale = np.abs(y[b, h]).max()
        err_rows = max(err_rows, float(np.abs(y.reshape(-1, wl.d)[rows] - ref_rows).max() / scale))
    print("PARITY video path=auto heads=%d full_err=%.3e rows_err=%.3e (4 heads x 256 rows) "
          "elementwise_floor1e-3=%.3e" % (S, err, err_rows, info))
    assert err <= TOL[wl.dtype]
    assert err_rows <= TOL[wl.dtype]


def test_video_generic_sampled():
    """The VALU path on the video workload, as a second GPU implementation:
    whole sampled heads plus brute-force rows."""
    wl = WORKLOADS["video"]
    inp = make_inputs(wl)
    y = to_f64(run(inp, m.MHLA_PATH_GENERIC))
    assert np.all(np.isfinite(y))
    err, err_rows = _check_sampled(inp, y, n_slices=1, n_rows=96)
    print("PARITY video path=generic slices_err=%.3e rows_err=%.3e" % (err, err_rows))
    assert err <= TOL[wl.dtype]
    assert err_rows <= TOL[wl.dtype]


FUSED_CASES = [
    # (grid, block, d, phi)
    ((1, 14, 14), (1, 7, 7), 64, PHI_ELU1),   # DeiT-like, ragged 49-token blocks
    ((1, 10, 10), (1, 5, 5), 64, PHI_RELU),   # 25-token blocks
    ((1, 8, 8), (1, 8, 8), 32, PHI_ELU1),     # M = 1: global linear attention
    ((1, 6, 9), (1, 3, 3), 16, PHI_RELU),     # M = 6, 9 tokens per block
    ((2, 8, 8), (1, 4, 8), 56, PHI_ELU1),     # 3-D grid, M = 4
    ((1, 4, 16), (1, 2, 4), 8, PHI_RELU),     # M = 8, d = 8
    ((1, 12, 12), (1, 6, 4), 40, PHI_ELU1),   # M = 6, 24 tokens, d = 40
    ((1, 1, 64), (1, 1, 32), 24, PHI_RELU),   # 1-D sequence chunks
]


@pytest.mark.parametrize("grid,block,d,phi", FUSED_CASES)
@pytest.mark.parametrize("path", ALL_PATHS)
def test_small_shapes(grid, block, d, phi, path):
    wl = custom_workload(3, 2, d, grid, block, phi, DTYPE_BF16, index=hash((grid, block, d)) % 997)
    inp = make_inputs(wl)
    y = to_f64(run(inp, path, skip_unsupported=(path in PARTIAL_PATHS)))
    err = slice_error(y, _oracle_full(inp))
    print("PARITY small %s %s d=%d phi=%d path=%d err=%.3e" % (grid, block, d, phi, path, err))
    assert err <= TOL[DTYPE_BF16]


BLOCKED_CASES = [
    # (grid, block, d, phi): shapes the three-kernel MFMA path must handle
    ((1, 16, 16), (1, 16, 8), 64, PHI_ELU1),   # 128-token blocks: two staging chunks
    ((1, 16, 16), (1, 4, 4), 72, PHI_RELU),    # d = 72 padded to 96 (DiT-like)
    ((1, 12, 12), (1, 3, 4), 96, PHI_ELU1),    # d = 96, 12-token blocks
    ((1, 40, 52), (1, 4, 4), 32, PHI_RELU),    # M = 130: partial mixing tiles
    ((4, 16, 16), (2, 4, 4), 64, PHI_ELU1),    # 3-D blocks, M = 32
    ((1, 1, 300), (1, 1, 5), 16, PHI_RELU),    # 1-D, M = 60, d = 16 padded to 32
    ((3, 8, 8), (1, 8, 8), 48, PHI_ELU1),      # whole-frame blocks, M = 3
    # M >= 256: bf16 coefficients and the large-tile mixing GEMM
    ((1, 32, 32), (1, 2, 2), 32, PHI_ELU1),    # M = 256, one query-block tile
    ((1, 48, 48), (1, 2, 4), 16, PHI_RELU),    # M = 288: a partial query-block tile
    ((4, 32, 32), (1, 4, 4), 64, PHI_ELU1),    # M = 256, d = 64 (the video entry width)
    ((1, 32, 64), (1, 2, 4), 96, PHI_RELU),    # M = 256, d = 96
    ((1, 1, 6656), (1, 1, 16), 64, PHI_ELU1),  # M = 416: a partial 128-block z chunk
]


@pytest.mark.parametrize("grid,block,d,phi", BLOCKED_CASES)
def test_blocked_shapes(grid, block, d, phi):
    wl = custom_workload(2, 2, d, grid, block, phi, DTYPE_BF16, index=hash((grid, block, d)) % 991)
    inp = make_inputs(wl)
    y = to_f64(run(inp, m.MHLA_PATH_BLOCKED))
    assert np.all(np.isfinite(y))
    err = slice_error(y, _oracle_full(inp))
    print("PARITY blocked %s %s d=%d phi=%d M=%d err=%.3e" % (grid, block, d, phi, wl.M, err))
    assert err <= TOL[DTYPE_BF16]


# M >= 256 with many slices: the large-M mixing runs several rounds of
# workgroups on each XCD (one 256-query-block x 128-entry tile each; an XCD
# takes ceil(B * H / 8) * (d * d / 128) * ceil(M / 256) of them, 64 at a time
# on 256 CUs), including a ragged last round and partial query tiles.
# (B, H, grid, block, d, phi)
MANY_SLICE_CASES = [
    (5, 8, (1, 1, 1152), (1, 1, 4), 32, PHI_RELU),   # M = 288: 80 tiles per XCD
    (12, 8, (1, 1, 1280), (1, 1, 4), 32, PHI_ELU1),  # M = 320: 192 tiles per XCD
    (25, 8, (1, 1, 1024), (1, 1, 4), 32, PHI_ELU1),  # M = 256: 200 tiles per XCD
    (9, 8, (1, 1, 1664), (1, 1, 4), 32, PHI_RELU),   # M = 416: 144 tiles per XCD
]


@pytest.mark.parametrize("B,H,grid,block,d,phi", MANY_SLICE_CASES)
def test_blocked_many_slices(B, H, grid, block, d, phi):
    wl = custom_workload(B, H, d, grid, block, phi, DTYPE_BF16, index=hash((B, grid, d)) % 997)
    inp = make_inputs(wl)
    y = to_f64(run(inp, m.MHLA_PATH_BLOCKED))
    assert np.all(np.isfinite(y))
    err = slice_error(y, _oracle_full(inp))
    print("PARITY blocked B=%d H=%d %s d=%d M=%d err=%.3e" % (B, H, grid, d, wl.M, err))
    assert err <= TOL[DTYPE_BF16]


PAIRS_CASES = [
    # (grid, block, d, phi): blocks of at most 16 tokens, the token-pair order
    ((1, 16, 16), (1, 4, 4), 72, PHI_ELU1),    # DiT-like, d = 72 (16-wide tail step)
    ((1, 12, 20), (1, 3, 4), 64, PHI_RELU),    # 12-token blocks, M = 20 (odd pairs)
    ((1, 9, 9), (1, 3, 3), 96, PHI_ELU1),      # 9-token blocks, M = 9 (odd M)
    ((4, 8, 8), (1, 2, 4), 32, PHI_RELU),      # 3-D grid, M = 32 (4 query blocks per wave)
    ((1, 4, 4), (1, 1, 1), 16, PHI_ELU1),      # one token per block, M = 16
    ((1, 8, 8), (1, 4, 4), 48, PHI_RELU),      # M = 4 (waves without a query block)
    ((1, 10, 16), (1, 2, 8), 80, PHI_ELU1),    # d = 80: a second O^T row tile
]


@pytest.mark.parametrize("grid,block,d,phi", PAIRS_CASES)
def test_pairs_shapes(grid, block, d, phi):
    wl = custom_workload(2, 3, d, grid, block, phi, DTYPE_BF16, index=hash((grid, block, d)) % 983)
    inp = make_inputs(wl)
    y = to_f64(run(inp, m.MHLA_PATH_PAIRS))
    assert np.all(np.isfinite(y))
    err = slice_error(y, _oracle_full(inp))
    print("PARITY pairs %s %s d=%d phi=%d M=%d err=%.3e" % (grid, block, d, phi, wl.M, err))
    assert err <= TOL[DTYPE_BF16]


COLS_CASES = [
    # (grid, block, d, phi): the column-split path, up to 64 blocks and d <= 64
    ((1, 64, 64), (1, 8, 8), 64, PHI_RELU),     # the 4096-token image geometry, M = 64
    ((1, 32, 48), (1, 4, 8), 64, PHI_ELU1),     # M = 48: a partial second block group
    ((1, 33, 8), (1, 1, 8), 40, PHI_RELU),      # M = 33: one block in the second group
    ((1, 20, 20), (1, 10, 10), 56, PHI_ELU1),   # 100-token blocks: four 32-token steps
    ((1, 28, 28), (1, 7, 7), 64, PHI_RELU),     # M = 16, 49-token ragged blocks
    ((4, 16, 16), (2, 4, 4), 32, PHI_ELU1),     # 3-D blocks, M = 32, d = 32
    ((1, 1, 600), (1, 1, 24), 16, PHI_RELU),    # 1-D chunks, M = 25, d = 16
    ((3, 8, 12), (1, 4, 4), 24, PHI_ELU1),      # 3-D grid, M = 18, d = 24 (partial chunk)
    ((1, 12, 12), (1, 12, 12), 8, PHI_RELU),    # M = 1, d = 8
    ((2, 24, 24), (1, 6, 6), 48, PHI_RELU),     # M = 32 exactly, 36-token blocks
    ((1, 64, 64), (1, 16, 16), 64, PHI_ELU1),   # 256-token blocks: the largest the path takes
]


def test_cols_largest_shape():
    """M = 64 blocks of 256 tokens, d = 64: the largest LDS footprint and the
    longest summary and readout loops of the column-split path."""
    wl = custom_workload(1, 2, 64, (1, 128, 128), (1, 16, 16), PHI_RELU, DTYPE_BF16, index=13)
    inp = make_inputs(wl)
    y = to_f64(run(inp, m.MHLA_PATH_COLUMNS))
    assert np.all(np.isfinite(y))
    err = slice_error(y, _oracle_full(inp))
    print("PARITY cols largest M=%d nb=%d err=%.3e" % (wl.M, wl.nb, err))
    assert err <= TOL[DTYPE_BF16]


@pytest.mark.parametrize("grid,block,d,phi", COLS_CASES)
def test_cols_shapes(grid, block, d, phi):
    wl = custom_workload(3, 2, d, grid, block, phi, DTYPE_BF16, index=hash((grid, block, d)) % 971)
    inp = make_inputs(wl)
    y = to_f64(run(inp, m.MHLA_PATH_COLUMNS))
    assert np.all(np.isfinite(y))
    err = slice_error(y, _oracle_full(inp))
    print("PARITY cols %s %s d=%d phi=%d M=%d err=%.3e" % (grid, block, d, phi, wl.M, err))
    assert err <= TOL[DTYPE_BF16]


def test_cols_odd_slice_count():
    """B*H = 7 slices: the XCD-grouped grid has workgroups with no slice."""
    wl = custom_workload(7, 1, 64, (1, 32, 32), (1, 8, 8), PHI_ELU1, DTYPE_BF16, index=12)
    inp = make_inputs(wl)
    y = to_f64(run(inp, m.MHLA_PATH_COLUMNS))
    err = slice_error(y, _oracle_full(inp))
    print("PARITY cols 7 slices err=%.3e" % err)
    assert err <= TOL[DTYPE_BF16]


@pytest.mark.parametrize("kind", ["identity", "sparse_rows", "unnormalised"])
def test_pairs_special_mixing_matrices(kind):
    wl = custom_workload(2, 2, 72, (1, 16, 16), (1, 4, 4), PHI_RELU, DTYPE_BF16, index=8)
    inp = make_inputs(wl)
    M = wl.M
    if kind == "identity":
        inp.w = np.broadcast_to(np.eye(M, dtype=np.float32), (wl.H, M, M)).copy()
    elif kind == "sparse_rows":
        inp.w[:, :, 3] = 0.0
        inp.w[:, 5, :] = 0.0
        inp.w[:, 5, 11] = 1.0
    else:
        inp.w = (inp.w * np.float32(11.0)).astype(np.float32)
    y = to_f64(run(inp, m.MHLA_PATH_PAIRS))
    err = slice_error(y, _oracle_full(inp))
    print("PARITY pairs W=%s err=%.3e" % (kind, err))
    assert err <= TOL[DTYPE_BF16]


@pytest.mark.parametrize("d", [1, 5, 16, 17, 64, 128])
def test_fp32_generic_any_d(d):
    wl = custom_workload(2, 2, d, (1, 6, 10), (1, 3, 5), PHI_ELU1, DTYPE_F32, index=d)
    inp = make_inputs(wl)
    y = to_f64(run(inp, m.MHLA_PATH_GENERIC))
    err = slice_error(y, _oracle_full(inp))
    print("PARITY fp32 d=%d err=%.3e" % (d, err))
    assert err <= TOL[DTYPE_F32]


@pytest.mark.parametrize("path", [p for p in ALL_PATHS if p != m.MHLA_PATH_PAIRS])
@pytest.mark.parametrize("kind", ["identity", "sparse_rows", "unnormalised"])
def test_special_mixing_matrices(path, kind):
    """W = I (block-local), rows with zeros, and rows that do not sum to 1."""
    wl = custom_workload(2, 3, 64, (1, 14, 14), (1, 7, 7), PHI_ELU1, DTYPE_BF16, index=5)
    inp = make_inputs(wl)
    M = wl.M
    if kind == "identity":
        inp.w = np.broadcast_to(np.eye(M, dtype=np.float32), (wl.H, M, M)).copy()
    elif kind == "sparse_rows":
        inp.w[:, :, 1] = 0.0
        inp.w[:, 2, :] = 0.0
        inp.w[:, 2, 3] = 1.0
    else:
        inp.w = (inp.w * np.float32(37.0)).astype(np.float32)
    y = to_f64(run(inp, path))
    err = slice_error(y, _oracle_full(inp))
    print("PARITY W=%s path=%d err=%.3e" % (kind, path, err))
    assert err <= TOL[DTYPE_BF16]


@pytest.mark.parametrize("path", ALL_PATHS)
def test_zero_denominator_rows(path):
    if path == m.MHLA_PATH_PAIRS:
        pytest.skip("covered with 16-token blocks in test_pairs_zero_denominator_rows")
    """ReLU query with every coordinate <= 0: phi(q) = 0, the row is written as 0."""
    wl = custom_workload(1, 2, 32, (1, 8, 8), (1, 4, 4), PHI_RELU, DTYPE_BF16, index=6)
    inp = make_inputs(wl)
    from mhla_inputs import bf16_round_bits
    qf = -np.abs(np.random.default_rng(0).standard_normal((wl.d,))).astype(np.float32)
    inp.q[0, 1, 7] = bf16_round_bits(qf)
    inp.q[0, 0, 63] = bf16_round_bits(np.zeros(wl.d, np.float32))
    y = to_f64(run(inp, path))
    assert np.all(y[0, 1, 7] == 0.0) and np.all(y[0, 0, 63] == 0.0)
    err = slice_error(y, _oracle_full(inp))
    assert err <= TOL[DTYPE_BF16]


def test_pairs_zero_denominator_rows():
    wl = custom_workload(1, 2, 32, (1, 8, 8), (1, 4, 4), PHI_RELU, DTYPE_BF16, index=9)
    inp = make_inputs(wl)
    from mhla_inputs import bf16_round_bits
    inp.q[0, 1, 7] = bf16_round_bits(-np.abs(np.random.default_rng(1).standard_normal(wl.d)).astype(np.float32))
    y = to_f64(run(inp, m.MHLA_PATH_PAIRS))
    assert np.all(y[0, 1, 7] == 0.0)
    assert slice_error(y, _oracle_full(inp)) <= TOL[DTYPE_BF16]


def test_fp32_zero_denominator_rows():
    wl = custom_workload(1, 1, 16, (1, 8, 8), (1, 4, 4), PHI_RELU, DTYPE_F32, index=7)
    inp = make_inputs(wl)
    inp.q[0, 0, 9] = -np.abs(inp.q[0, 0, 9])
    y = to_f64(run(inp, m.MHLA_PATH_GENERIC))
    assert np.all(y[0, 0, 9] == 0.0)
    assert slice_error(y, _oracle_full(inp)) <= TOL[DTYPE_F32]


@pytest.mark.parametrize("name", ["deit_t", "hires"])
def test_deterministic(name):
    inp = make_inputs(WORKLOADS[name], B=2)
    dev = to_device(inp)
    a = run(inp, dev=dev)
    b = run(inp, dev=dev)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_side_stream():
    inp = make_inputs(WORKLOADS["deit_t"], B=4)
    dev = to_device(inp)
    ref = run(inp, dev=dev)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        out = torch.empty_like(dev[0])
        m.mhla_forward(*dev, out, (inp.wl.grid, inp.wl.block), inp.wl.phi)
    s.synchronize()
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))


def test_errors_enqueue_nothing():
    inp = make_inputs(WORKLOADS["deit_t"], B=1)
    q, k, v, w = to_device(inp)
    before = q.clone()
    with pytest.raises(m.MhlaError) as ei:
        m.mhla_forward(q, k, v, w, q, (inp.wl.grid, inp.wl.block), inp.wl.phi)
    assert ei.value.code == m.MHLA_ERR_ALIAS
    out = torch.empty_like(q)
    with pytest.raises(m.MhlaError) as ei:
        m.mhla_forward(q, k, v, w, out, ((1, 14, 14), (1, 4, 7)), inp.wl.phi)
    assert ei.value.code == m.MHLA_ERR_SHAPE
    # 2x2 blocks of the 14x14 grid: M = 49 is more blocks than the fused path
    # keeps on chip (with a W of the matching H*M*M size)
    w49 = torch.full((inp.wl.H, 49, 49), 1.0 / 49, dtype=torch.float32, device=q.device)
    with pytest.raises(m.MhlaError) as ei:
        m.mhla_forward_path(q, k, v, w49, out, ((1, 14, 14), (1, 2, 2)), inp.wl.phi,
                            m.MHLA_PATH_FUSED)
    assert ei.value.code == m.MHLA_ERR_UNSUPPORTED
    torch.cuda.synchronize()
    assert torch.equal(q.view(torch.int16), before.view(torch.int16))


def test_binding_rejects_wrong_mixing_matrix_size():
    """The library reads H*M*M floats of Wmix (and the backward writes as many
    of dWmix) and cannot see the buffer's size: the binding checks it."""
    inp = make_inputs(WORKLOADS["deit_t"], B=1)
    q, k, v, w = to_device(inp)
    out = torch.empty_like(q)
    for bad in (w[:, :3, :3].contiguous(), w.reshape(-1)[:-1].contiguous(),
                torch.zeros((inp.wl.H + 1, 4, 4), dtype=torch.float32, device=q.device)):
        with pytest.raises(ValueError):
            m.mhla_forward(q, k, v, bad, out, (inp.wl.grid, inp.wl.block), inp.wl.phi)
        with pytest.raises(ValueError):
            m.mhla_backward(q, k, v, bad, q, torch.empty_like(q), torch.empty_like(q),
                            torch.empty_like(q), torch.empty_like(w), (inp.wl.grid, inp.wl.block),
                            inp.wl.phi)
    with pytest.raises(ValueError):
        m.mhla_backward(q, k, v, w, q, torch.empty_like(q), torch.empty_like(q),
                        torch.empty_like(q), w[:2].contiguous(), (inp.wl.grid, inp.wl.block),
                        inp.wl.phi)
    # the 49-block shape needs a 3x49x49 W
    with pytest.raises(ValueError):
        m.mhla_forward(q, k, v, w, out, ((1, 14, 14), (1, 2, 2)), inp.wl.phi)
    torch.cuda.synchronize()


def test_profiled_call_matches_forward():
    """mhla_forward_profiled gives the same output as mhla_forward_ex and
    names its launches; the recorded events are ordered."""
    import ctypes
    hip = ctypes.CDLL("libamdhip64.so")
    evs = []
    for _ in range(m.MHLA_MAX_LAUNCHES + 1):
        e = ctypes.c_void_p()
        assert hip.hipEventCreate(ctypes.byref(e)) == 0
        evs.append(e.value)
    try:
        for name in ("tiny", "deit_t", "hires"):
            inp = make_inputs(WORKLOADS[name], B=1)
            dev = to_device(inp)
            ref = run(inp, dev=dev)
            out = torch.empty_like(dev[0])
            names = m.mhla_forward_profiled(*dev, out, (inp.wl.grid, inp.wl.block), inp.wl.phi,
                                            0, m.MHLA_PATH_AUTO, evs)
            torch.cuda.synchronize()
            assert torch.equal(out.view(torch.int16) if out.dtype == torch.bfloat16 else out,
                               ref.view(torch.int16) if ref.dtype == torch.bfloat16 else ref)
            assert 1 <= len(names) <= m.MHLA_MAX_LAUNCHES
            for a in range(len(names)):
                ms = ctypes.c_float()
                assert hip.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(evs[a]),
                                               ctypes.c_void_p(evs[a + 1])) == 0
                assert ms.value >= 0.0
            print("PROFILED %s: %s" % (name, names))
    finally:
        for e in evs:
            hip.hipEventDestroy(ctypes.c_void_p(e))
