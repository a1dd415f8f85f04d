"""Pins of the fp64 oracle to facts fixed by the pages and by the mathematics.

Each test names the passage it follows.  "MHLA paper" is "MHLA: Restoring
Expressivity of Linear Attention via Token-Level Multi-Head" (arXiv 2601.07832).
None of these tests uses the GPU or the HIP library.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from mhla_inputs import PHI_ELU1, PHI_RELU

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _rand_case(rng, B, H, grid, block, d, phi, w_kind="softmax"):
    N = int(np.prod(grid))
    M = oracle.num_blocks(grid, block)
    Q = rng.standard_normal((B, H, N, d))
    K = rng.standard_normal((B, H, N, d))
    V = rng.standard_normal((B, H, N, d))
    if w_kind == "softmax":
        L = rng.standard_normal((H, M, M))
        W = np.exp(L) / np.exp(L).sum(-1, keepdims=True)
    elif w_kind == "raw":  # any sign, not normalised: the forward is defined for any W
        W = rng.standard_normal((H, M, M)) + 1.5
    else:
        raise ValueError(w_kind)
    return Q, K, V, W


# ---------------------------------------------------------------- worked examples

@pytest.mark.parametrize("name", ["worked_relu_2x2.json", "worked_elu1_1x2.json"])
def test_worked_example(name):
    """Hand-derived examples of MHLA paper §4.1 (fixtures cite the passage)."""
    g = _load(name)
    Q = np.array(g["Q"], dtype=np.float64)[None, None]
    K = np.array(g["K"], dtype=np.float64)[None, None]
    V = np.array(g["V"], dtype=np.float64)[None, None]
    W = np.array(g["W"], dtype=np.float64)[None]
    exp = np.array([[float(Fraction(n, dd)) for n, dd in zip(rn, rd)]
                    for rn, rd in zip(g["Y_num"], g["Y_den"])])
    Yb = oracle.blockwise(Q, K, V, W, g["grid"], g["block"], g["phi"])[0, 0]
    np.testing.assert_allclose(Yb, exp, rtol=0, atol=1e-14)
    N = Q.shape[2]
    Yr = oracle.rows(Q, K, V, W, g["grid"], g["block"], g["phi"], np.arange(N))
    np.testing.assert_allclose(Yr, exp, rtol=0, atol=1e-14)
    Yn = oracle.numpy_bruteforce(Q, K, V, W, g["grid"], g["block"], g["phi"])[0, 0]
    np.testing.assert_allclose(Yn, exp, rtol=0, atol=1e-14)


def test_geometry_fixture():
    """Block membership: spatial tiles in raster order (MHLA paper §1, §4.1, Fig. 4b)."""
    for case in _load("geometry_blocks.json")["cases"]:
        grid, block = case["grid"], case["block"]
        N = int(np.prod(grid))
        M = oracle.num_blocks(grid, block)
        assert M == len(case["members"])
        got = [[] for _ in range(M)]
        for t in range(N):
            got[oracle.block_of_token(grid, block, t)].append(t)
        assert got == case["members"]
        bm = oracle.np_block_map(grid, block)
        assert [sorted(np.nonzero(bm == b)[0].tolist()) for b in range(M)] == case["members"]


def test_phi_definitions():
    """ReLU and elu+1 (alpha = 1) from the attention-variants tutorial."""
    for x in [-3.0, -0.5, 0.0, 0.25, 2.0]:
        assert oracle.phi(PHI_RELU, x) == max(x, 0.0)
        assert oracle.phi(PHI_ELU1, x) == (x + 1.0 if x > 0 else float(np.exp(x)))
    # elu+1 is continuous at 0 and strictly positive
    assert oracle.phi(PHI_ELU1, 0.0) == 1.0
    assert oracle.phi(PHI_ELU1, -50.0) > 0.0


# ---------------------------------------------------------------- blockwise == brute force

GEOMS = [
    ((1, 8, 8), (1, 4, 4)),     # the tiny fp32 workload's geometry
    ((1, 6, 10), (1, 3, 5)),    # non-square grid and blocks
    ((2, 4, 6), (1, 2, 3)),     # 3-D grid, per-frame blocks
    ((3, 4, 4), (3, 2, 2)),     # 3-D blocks spanning frames
    ((1, 1, 12), (1, 1, 4)),    # 1-D sequence chunks
    ((1, 5, 7), (1, 5, 7)),     # M = 1
    ((1, 4, 4), (1, 1, 1)),     # M = N, one token per block
]


@pytest.mark.parametrize("grid,block", GEOMS)
@pytest.mark.parametrize("phi", [PHI_RELU, PHI_ELU1])
def test_blockwise_equals_bruteforce(grid, block, phi):
    """The blockwise order equals the token-expanded form (MHLA paper §4.2 Eq. 5)."""
    rng = np.random.default_rng(hash((grid, block, phi)) % 2**32)
    Q, K, V, W = _rand_case(rng, 2, 2, grid, block, 5, phi, "raw")
    Yb = oracle.blockwise(Q, K, V, W, grid, block, phi)
    Yn = oracle.numpy_bruteforce(Q, K, V, W, grid, block, phi)
    np.testing.assert_allclose(Yb, Yn, rtol=1e-11, atol=1e-11)
    N = Q.shape[2]
    rows = np.arange(2 * 2 * N)
    Yr = oracle.rows(Q, K, V, W, grid, block, phi, rows).reshape(Yb.shape)
    np.testing.assert_allclose(Yr, Yn, rtol=1e-11, atol=1e-11)


# ---------------------------------------------------------------- special cases

def _linear_attention(Q, K, V, phi):
    """Global kernelised linear attention, MHLA paper §3.1 (second display)."""
    pq, pk = oracle.np_phi(phi, Q), oracle.np_phi(phi, K)
    G = np.einsum("bhnk,bhnc->bhkc", pk, V)
    z = pk.sum(axis=2)
    num = np.einsum("bhnk,bhkc->bhnc", pq, G)
    den = np.einsum("bhnk,bhk->bhn", pq, z)
    return num / den[..., None]


@pytest.mark.parametrize("phi", [PHI_RELU, PHI_ELU1])
def test_m1_is_global_linear_attention(phi):
    """With one block MHLA is plain linear attention (blog review, §4.2 checklist;
    MHLA paper §3.1)."""
    rng = np.random.default_rng(7)
    grid = (1, 6, 6)
    Q, K, V, W = _rand_case(rng, 2, 3, grid, grid, 8, phi)
    Q = np.abs(Q) + 0.1  # keep ReLU denominators away from 0
    Y = oracle.blockwise(Q, K, V, W, grid, grid, phi)
    np.testing.assert_allclose(Y, _linear_attention(Q, K, V, phi), rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("phi", [PHI_RELU, PHI_ELU1])
def test_constant_w_is_global_linear_attention(phi):
    """Equal mixing weights give every query block the global summary
    (derived: S~_i = c * sum_b S_b)."""
    rng = np.random.default_rng(8)
    grid, block = (1, 8, 8), (1, 2, 4)
    Q, K, V, W = _rand_case(rng, 1, 2, grid, block, 6, phi)
    Q = np.abs(Q) + 0.1
    W[:] = 0.37
    Y = oracle.blockwise(Q, K, V, W, grid, block, phi)
    np.testing.assert_allclose(Y, _linear_attention(Q, K, V, phi), rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("phi", [PHI_RELU, PHI_ELU1])
def test_identity_w_is_block_local_attention(phi):
    """With W = I only the local summaries remain: block-local linear attention
    (blog review §2.2, first sentence)."""
    rng = np.random.default_rng(9)
    case = _load("geometry_blocks.json")["cases"][1]  # 4x6 grid, 2x3 blocks
    grid, block, members = case["grid"], case["block"], case["members"]
    M = len(members)
    Q, K, V, _ = _rand_case(rng, 2, 2, grid, block, 4, phi)
    Q, K = np.abs(Q) + 0.1, K + 1.0   # no 0/0 rows within the small blocks
    W = np.broadcast_to(np.eye(M), (2, M, M)).copy()
    Y = oracle.blockwise(Q, K, V, W, grid, block, phi)
    ref = np.empty_like(Y)
    for toks in members:
        t = np.array(toks)
        ref[:, :, t] = _linear_attention(Q[:, :, t], K[:, :, t], V[:, :, t], phi)
    np.testing.assert_allclose(Y, ref, rtol=1e-11, atol=1e-12)


def test_token_blocks_reproduce_softmax_attention():
    """With one token per block (M = N), W is a free N x N matrix; choosing
    W[i,j] = exp(q_i.k_j/sqrt(d)) / (phi(q_i).phi(k_j)) turns the unified form of
    MHLA paper §3.1 (first display) into softmax attention.  This pins W's
    orientation (row = query block) and the normaliser against a library routine."""
    rng = np.random.default_rng(10)
    grid = (1, 3, 5)
    N, d = 15, 6
    q = rng.standard_normal((N, d))
    k = rng.standard_normal((N, d))
    v = rng.standard_normal((N, d))
    pq, pk = oracle.np_phi(PHI_ELU1, q), oracle.np_phi(PHI_ELU1, k)
    W = np.exp(q @ k.T / np.sqrt(d)) / (pq @ pk.T)
    Y = oracle.blockwise(q[None, None], k[None, None], v[None, None], W[None],
                         grid, (1, 1, 1), PHI_ELU1)[0, 0]
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None, None], torch.from_numpy(k)[None, None],
        torch.from_numpy(v)[None, None])[0, 0].numpy()
    np.testing.assert_allclose(Y, ref, rtol=1e-12, atol=1e-12)


def test_zero_denominator_row_is_zero():
    """Reading taken (pages give no epsilon): a query whose phi is all zero
    (ReLU, all coordinates <= 0) has a 0/0 row; it is returned as 0."""
    rng = np.random.default_rng(11)
    grid, block = (1, 4, 4), (1, 2, 2)
    Q, K, V, W = _rand_case(rng, 1, 1, grid, block, 4, PHI_RELU)
    Q[0, 0, 5] = -np.abs(Q[0, 0, 5]) - 0.1
    Y = oracle.blockwise(Q, K, V, W, grid, block, PHI_RELU)
    assert np.all(Y[0, 0, 5] == 0.0)
    Yr = oracle.rows(Q, K, V, W, grid, block, PHI_RELU, [5])
    assert np.all(Yr == 0.0)
    assert np.all(np.isfinite(Y))


# ---------------------------------------------------------------- rank bounds

def _stochastic_matrix(grid, block, d_eff, phi, M1=False, seed=12):
    """Read the row-normalised attention matrix out of the blockwise oracle by
    feeding V = identity (Y is linear in V).  Q and K carry only d_eff non-zero
    features, so the kernel rank is at most d_eff."""
    rng = np.random.default_rng(seed)
    N = int(np.prod(grid))
    d = N
    Q = np.zeros((1, 1, N, d))
    K = np.zeros((1, 1, N, d))
    Q[..., :d_eff] = rng.standard_normal((N, d_eff)) + 1.0
    K[..., :d_eff] = rng.standard_normal((N, d_eff)) + 1.0
    if phi == PHI_ELU1:
        raise ValueError("elu+1 maps 0 to 1; use ReLU for the padded features")
    V = np.eye(N)[None, None]
    blk = grid if M1 else block
    M = oracle.num_blocks(grid, blk)
    L = rng.standard_normal((1, M, M))
    W = np.exp(L) / np.exp(L).sum(-1, keepdims=True)
    return oracle.blockwise(Q, K, V, W, grid, blk, phi)[0, 0]


def test_rank_linear_attention_bounded_by_d():
    """rank(A_lin) <= d (MHLA paper §3.2, rank limitation)."""
    P = _stochastic_matrix((1, 4, 8), None, 3, PHI_RELU, M1=True)
    assert np.linalg.matrix_rank(P) <= 3
    assert np.linalg.matrix_rank(P) == 3   # generic inputs reach the bound


def test_rank_mhla_bound_and_attained():
    """rank(A_MHLA) <= min(N, sum_b min(n_b, d)), attainable for generic inputs
    (MHLA paper §4.3 and Table 1)."""
    grid, block, d_eff = (1, 4, 8), (1, 2, 4), 3   # M = 4 blocks of 8 tokens
    P = _stochastic_matrix(grid, block, d_eff, PHI_RELU)
    bound = min(32, 4 * min(8, d_eff))
    r = np.linalg.matrix_rank(P)
    assert r <= bound
    assert r == bound
    assert r > d_eff  # strictly above linear attention's cap


# ---------------------------------------------------------------- invariants

@pytest.mark.parametrize("phi", [PHI_RELU, PHI_ELU1])
def test_invariants(phi):
    """Derived from the definition: rows of the normalised matrix sum to one
    (shift equivariance in V), Y is linear in V, a positive per-row scale of W
    cancels, and (batch, head) slices are independent."""
    rng = np.random.default_rng(13)
    grid, block = (1, 6, 6), (1, 3, 2)
    Q, K, V, W = _rand_case(rng, 2, 3, grid, block, 5, phi)
    Q = np.abs(Q) + 0.1
    Y = oracle.blockwise(Q, K, V, W, grid, block, phi)
    c = rng.standard_normal(5)
    np.testing.assert_allclose(oracle.blockwise(Q, K, V + c, W, grid, block, phi), Y + c,
                               rtol=1e-11, atol=1e-11)
    V2 = rng.standard_normal(V.shape)
    Y2 = oracle.blockwise(Q, K, V2, W, grid, block, phi)
    np.testing.assert_allclose(oracle.blockwise(Q, K, 2.0 * V - 3.0 * V2, W, grid, block, phi),
                               2.0 * Y - 3.0 * Y2, rtol=1e-10, atol=1e-10)
    scale = rng.uniform(0.1, 10.0, size=W.shape[:2] + (1,))
    np.testing.assert_allclose(oracle.blockwise(Q, K, V, W * scale, grid, block, phi), Y,
                               rtol=1e-11, atol=1e-12)
    Ys = oracle.blockwise(Q[1:2, 2:3], K[1:2, 2:3], V[1:2, 2:3], W[2:3], grid, block, phi)
    np.testing.assert_allclose(Ys[0, 0], Y[1, 2], rtol=0, atol=0)


def test_rejects_bad_geometry():
    Q = np.zeros((1, 1, 12, 2))
    with pytest.raises(ValueError):
        oracle.blockwise(Q, Q, Q, np.ones((1, 4, 4)), (1, 3, 4), (1, 2, 2), PHI_RELU)
    with pytest.raises(ValueError):
        oracle.blockwise(Q, Q, Q, np.ones((1, 4, 4)), (1, 4, 4), (1, 2, 2), PHI_RELU)
