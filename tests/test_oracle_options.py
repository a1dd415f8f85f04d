"""Pins of the oracle's options: the normaliser switch, the chunkwise causal
form, and the locality-biased initial mixing matrix.

"MHLA paper" is "MHLA: Restoring Expressivity of Linear Attention via
Token-Level Multi-Head" (arXiv 2601.07832); "blog review" is the Chinese
review page of the same paper.  CPU only.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
from mhla_inputs import PHI_ELU1, PHI_RELU

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _arr(g, key):
    return np.array(g[key], dtype=np.float64)[None, None]


def _rand(rng, B, H, N, d, M, w_kind="softmax"):
    Q, K, V = (rng.standard_normal((B, H, N, d)) for _ in range(3))
    if w_kind == "softmax":
        L = rng.standard_normal((H, M, M))
        W = np.exp(L) / np.exp(L).sum(-1, keepdims=True)
    else:
        W = rng.uniform(0.2, 1.5, (H, M, M))
    return Q, K, V, W


# ---------------------------------------------------------------- normaliser switch

def test_no_norm_worked_example():
    """Hand-derived numerators of the §4.1 worked example: with the normaliser
    switched off (MHLA paper, language modelling and long video; blog review
    §2.2) the output is q~^T S~_i itself."""
    g = _load("worked_relu_2x2.json")
    args = (_arr(g, "Q"), _arr(g, "K"), _arr(g, "V"), np.array(g["W"])[None], g["grid"],
            g["block"], g["phi"])
    exp = np.array(g["numerator"], dtype=np.float64)
    np.testing.assert_allclose(oracle.blockwise(*args, norm=False)[0, 0], exp, rtol=0, atol=1e-14)
    np.testing.assert_allclose(oracle.rows(*args, np.arange(4), norm=False), exp, rtol=0,
                               atol=1e-14)
    np.testing.assert_allclose(oracle.numpy_bruteforce(*args, norm=False)[0, 0], exp, rtol=0,
                               atol=1e-14)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("phi", [PHI_RELU, PHI_ELU1])
def test_no_norm_ones_column_gives_denominator(phi, causal):
    """Derived: the numerator is linear in V, so with a column of ones in V that
    column of the un-normalised output is the denominator; dividing the other
    columns by it must give the normalised output."""
    rng = np.random.default_rng(21 + phi + 2 * causal)
    grid, block = (1, 4, 6), (1, 2, 6)
    M = oracle.num_blocks(grid, block)
    Q, K, V, W = _rand(rng, 2, 2, 24, 6, M)
    Q, K = np.abs(Q) + 0.1, np.abs(K)   # no zero denominators
    V[..., 5] = 1.0
    num = oracle.blockwise(Q, K, V, W, grid, block, phi, norm=False, causal=causal)
    Y = oracle.blockwise(Q, K, V, W, grid, block, phi, causal=causal)
    np.testing.assert_allclose(num[..., :5] / num[..., 5:], Y[..., :5], rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(Y[..., 5], 1.0, rtol=0, atol=1e-13)


@pytest.mark.parametrize("phi", [PHI_RELU, PHI_ELU1])
def test_no_norm_scales_with_w(phi):
    """Derived: without the normaliser the output is linear in W (a scale of W
    scales Y), while with it a positive row scale cancels."""
    rng = np.random.default_rng(22)
    grid, block = (1, 6, 6), (1, 3, 2)
    M = oracle.num_blocks(grid, block)
    Q, K, V, W = _rand(rng, 1, 2, 36, 4, M)
    Y = oracle.blockwise(Q, K, V, W, grid, block, phi, norm=False)
    np.testing.assert_allclose(oracle.blockwise(Q, K, V, 2.5 * W, grid, block, phi, norm=False),
                               2.5 * Y, rtol=1e-12, atol=1e-12)
    W2 = rng.uniform(0.1, 1.0, W.shape)
    np.testing.assert_allclose(
        oracle.blockwise(Q, K, V, W + W2, grid, block, phi, norm=False),
        Y + oracle.blockwise(Q, K, V, W2, grid, block, phi, norm=False), rtol=1e-10, atol=1e-10)


# ---------------------------------------------------------------- causal (chunkwise) form

@pytest.mark.parametrize("norm", [True, False])
def test_causal_worked_example(norm):
    """Hand-derived chunkwise example (MHLA paper §4.2 chunkwise form, App. C)."""
    g = _load("worked_causal_relu_1x4.json")
    args = (_arr(g, "Q"), _arr(g, "K"), _arr(g, "V"), np.array(g["W"])[None], g["grid"],
            g["block"], g["phi"])
    num = np.array(g["numerator"], dtype=np.float64)
    den = np.array(g["denominator"], dtype=np.float64)
    exp = num / den[:, None] if norm else num
    np.testing.assert_allclose(oracle.blockwise(*args, norm=norm, causal=True)[0, 0], exp,
                               rtol=0, atol=1e-14)
    np.testing.assert_allclose(oracle.rows(*args, np.arange(4), norm=norm, causal=True), exp,
                               rtol=0, atol=1e-14)
    np.testing.assert_allclose(oracle.numpy_bruteforce(*args, norm=norm, causal=True)[0, 0], exp,
                               rtol=0, atol=1e-14)


CAUSAL_GEOMS = [
    ((1, 1, 24), (1, 1, 6)),    # 1-D sequence, 4 chunks
    ((1, 1, 20), (1, 1, 20)),   # one chunk
    ((1, 1, 9), (1, 1, 1)),     # one token per chunk
    ((1, 4, 6), (1, 2, 6)),     # 2-D grid, blocks of whole rows
    ((3, 2, 4), (1, 2, 4)),     # 3-D grid, one frame per block
]


@pytest.mark.parametrize("grid,block", CAUSAL_GEOMS)
@pytest.mark.parametrize("phi", [PHI_RELU, PHI_ELU1])
@pytest.mark.parametrize("norm", [True, False])
def test_causal_chunkwise_equals_masked_bruteforce(grid, block, phi, norm):
    """The chunkwise order (prefix mixing + causal own chunk) equals the token
    form with the mask j <= q (MHLA paper §4.2 Eq. 5, chunkwise form)."""
    rng = np.random.default_rng(hash((grid, block, phi, norm)) % 2**32)
    N = int(np.prod(grid))
    M = oracle.num_blocks(grid, block)
    Q, K, V, W = _rand(rng, 2, 2, N, 5, M, "raw")
    Yb = oracle.blockwise(Q, K, V, W, grid, block, phi, norm=norm, causal=True)
    Yn = oracle.numpy_bruteforce(Q, K, V, W, grid, block, phi, norm=norm, causal=True)
    np.testing.assert_allclose(Yb, Yn, rtol=1e-11, atol=1e-11)
    Yr = oracle.rows(Q, K, V, W, grid, block, phi, np.arange(4 * N), norm=norm,
                     causal=True).reshape(Yb.shape)
    np.testing.assert_allclose(Yr, Yn, rtol=1e-11, atol=1e-11)


def _causal_linear_attention(Q, K, V, phi, norm):
    """Textbook causal linear attention as a recurrence over tokens: running
    state S_t = S_{t-1} + phi(k_t) v_t^T and z_t = z_{t-1} + phi(k_t)
    (attention-variants tutorial, linear attention section)."""
    B, H, N, d = Q.shape
    Y = np.zeros_like(Q)
    for b in range(B):
        for h in range(H):
            S = np.zeros((d, d))
            z = np.zeros(d)
            for t in range(N):
                pk = oracle.np_phi(phi, K[b, h, t])
                S += np.outer(pk, V[b, h, t])
                z += pk
                pq = oracle.np_phi(phi, Q[b, h, t])
                Y[b, h, t] = pq @ S / (pq @ z) if norm else pq @ S
    return Y


@pytest.mark.parametrize("phi", [PHI_RELU, PHI_ELU1])
@pytest.mark.parametrize("norm", [True, False])
def test_causal_constant_w_is_causal_linear_attention(phi, norm):
    """Equal mixing weights (all entries c) reduce chunkwise MHLA to c times
    causal linear attention without the normaliser and to it exactly with it."""
    rng = np.random.default_rng(23)
    grid, block = (1, 1, 32), (1, 1, 8)
    Q, K, V, W = _rand(rng, 1, 2, 32, 6, 4)
    Q = np.abs(Q) + 0.1
    W[:] = 0.6
    Y = oracle.blockwise(Q, K, V, W, grid, block, phi, norm=norm, causal=True)
    ref = _causal_linear_attention(Q, K, V, phi, norm)
    np.testing.assert_allclose(Y, ref if norm else 0.6 * ref, rtol=1e-11, atol=1e-11)


@pytest.mark.parametrize("phi", [PHI_RELU, PHI_ELU1])
def test_causal_ignores_upper_triangle_and_future(phi):
    """Derived from the mask: W[i,b] with b > i is never used, and no output at
    position q depends on keys or values after q."""
    rng = np.random.default_rng(24)
    grid, block = (1, 1, 30), (1, 1, 5)
    Q, K, V, W = _rand(rng, 1, 2, 30, 4, 6)
    Y = oracle.blockwise(Q, K, V, W, grid, block, phi, causal=True)
    W2 = W.copy()
    iu = np.triu_indices(6, 1)
    W2[:, iu[0], iu[1]] = rng.uniform(5, 9, (2, len(iu[0])))
    np.testing.assert_array_equal(oracle.blockwise(Q, K, V, W2, grid, block, phi, causal=True), Y)
    t = 17
    K2, V2 = K.copy(), V.copy()
    K2[:, :, t:] = rng.standard_normal(K2[:, :, t:].shape)
    V2[:, :, t:] = rng.standard_normal(V2[:, :, t:].shape)
    Y2 = oracle.blockwise(Q, K2, V2, W, grid, block, phi, causal=True)
    np.testing.assert_array_equal(Y2[:, :, :t], Y[:, :, :t])
    assert not np.allclose(Y2[:, :, t:], Y[:, :, t:])


@pytest.mark.parametrize("norm", [True, False])
def test_causal_last_token_sees_everything(norm):
    """The last query of the last chunk sees every key with the full last row
    of W, so it equals the non-causal output there."""
    rng = np.random.default_rng(25)
    grid, block = (2, 3, 4), (1, 3, 4)
    Q, K, V, W = _rand(rng, 2, 2, 24, 5, 2)
    Yc = oracle.blockwise(Q, K, V, W, grid, block, PHI_ELU1, norm=norm, causal=True)
    Y = oracle.blockwise(Q, K, V, W, grid, block, PHI_ELU1, norm=norm)
    np.testing.assert_allclose(Yc[:, :, -1], Y[:, :, -1], rtol=1e-12, atol=1e-12)


def test_causal_rejects_non_contiguous_blocks():
    """2-D tiles narrower than the grid are not runs of consecutive tokens, so
    the chunkwise form does not apply to them."""
    Q = np.zeros((1, 1, 16, 2))
    with pytest.raises(ValueError):
        oracle.blockwise(Q, Q, Q, np.ones((1, 4, 4)), (1, 4, 4), (1, 2, 2), PHI_RELU, causal=True)


# ---------------------------------------------------------------- LB-init

def test_lb_init_line_of_three():
    """m0 for three blocks on a line (MHLA paper §4.2): distances 0, 1, 2 from
    an end block give 1, 1/2, 0 before normalisation; the middle block is
    equally far (1) from both ends, so only its own weight survives."""
    m = oracle.np_lb_init((1, 1, 3), (1, 1, 1))
    exp = np.array([[2 / 3, 1 / 3, 0], [0, 1, 0], [0, 1 / 3, 2 / 3]])
    np.testing.assert_allclose(m, exp, rtol=0, atol=1e-15)


def test_lb_init_two_by_two():
    """2 x 2 block grid: distances 0, 1, 1, sqrt(2) from a corner."""
    m = oracle.np_lb_init((1, 4, 4), (1, 2, 2))
    r = 1 - 1 / math.sqrt(2)
    row0 = np.array([1, r, r, 0]) / (1 + 2 * r)
    np.testing.assert_allclose(m[0], row0, rtol=0, atol=1e-15)
    np.testing.assert_allclose(m[3], row0[::-1], rtol=0, atol=1e-15)


def test_lb_init_degenerate_sizes():
    """One block gives [[1]]; two blocks are each other's farthest block, so m0
    is the identity."""
    np.testing.assert_array_equal(oracle.np_lb_init((1, 4, 4), (1, 4, 4)), [[1.0]])
    np.testing.assert_array_equal(oracle.np_lb_init((1, 1, 8), (1, 1, 4)), np.eye(2))


@pytest.mark.parametrize("grid,block", [((1, 14, 14), (1, 7, 7)), ((1, 16, 16), (1, 4, 4)),
                                        ((8, 64, 64), (1, 8, 8)), ((1, 6, 10), (1, 3, 5))])
def test_lb_init_properties(grid, block):
    """Rows sum to 1, entries are in [0, 1), every row's largest entry is its
    own block and its farthest block gets 0 (MHLA paper §4.2 and Fig. 4b)."""
    m = oracle.np_lb_init(grid, block)
    M = oracle.num_blocks(grid, block)
    assert m.shape == (M, M)
    np.testing.assert_allclose(m.sum(axis=1), 1.0, rtol=0, atol=1e-12)
    assert np.all(m >= 0) and np.all(m < 1)
    assert np.all(np.argmax(m, axis=1) == np.arange(M))
    assert np.all(m.min(axis=1) == 0.0)
    np.testing.assert_allclose(m, m[::-1, ::-1], rtol=0, atol=1e-15)   # point symmetry


# ---------------------------------------------------------------- incremental inference

@pytest.mark.parametrize("norm", [True, False])
def test_decode_worked_example(norm):
    """The hand-derived chunkwise example, produced token by token (MHLA paper
    App. C, causal inference)."""
    g = _load("worked_causal_relu_1x4.json")
    num = np.array(g["numerator"], dtype=np.float64)
    den = np.array(g["denominator"], dtype=np.float64)
    exp = num / den[:, None] if norm else num
    Y = oracle.np_decode(_arr(g, "Q"), _arr(g, "K"), _arr(g, "V"), np.array(g["W"])[None], 2,
                         g["phi"], norm=norm)[0, 0]
    np.testing.assert_allclose(Y, exp, rtol=0, atol=1e-14)


@pytest.mark.parametrize("nb", [1, 6, 8, 24])
@pytest.mark.parametrize("phi", [PHI_RELU, PHI_ELU1])
@pytest.mark.parametrize("norm", [True, False])
def test_decode_equals_causal_forward(nb, phi, norm):
    """Streaming inference reproduces the chunkwise causal forward (C blockwise
    oracle) and the masked token form (NumPy brute force) at every position."""
    rng = np.random.default_rng(26 + nb + 3 * phi)
    N = 24
    M = N // nb
    Q, K, V, W = _rand(rng, 2, 2, N, 5, M, "raw")
    Yd = oracle.np_decode(Q, K, V, W, nb, phi, norm=norm)
    Yc = oracle.blockwise(Q, K, V, W, (1, 1, N), (1, 1, nb), phi, norm=norm, causal=True)
    np.testing.assert_allclose(Yd, Yc, rtol=1e-11, atol=1e-11)
    Yn = oracle.numpy_bruteforce(Q, K, V, W, (1, 1, N), (1, 1, nb), phi, norm=norm, causal=True)
    np.testing.assert_allclose(Yd, Yn, rtol=1e-11, atol=1e-11)


DECODE_MUTANTS = {
    "prefix_uses_w_column": ('P = np.einsum("b,bfc->fc", W[h, i, :i], S[:i])',
                             'P = np.einsum("b,bfc->fc", W[h, :i, i], S[:i])'),
    "own_unweighted": ("num = pq @ (P + W[h, i, i] * S[i])", "num = pq @ (P + S[i])"),
    "den_prefix_dropped": ("den = pq @ (p + W[h, i, i] * z[i])", "den = pq @ (W[h, i, i] * z[i])"),
    "chunk_never_reset": ("if t % nb == 0:", "if t == 0:"),
}


@pytest.mark.parametrize("name", sorted(DECODE_MUTANTS))
def test_pins_catch_decode_mutant(name):
    """Planted mistakes in a copy of np_decode fail the comparison with the
    causal blockwise oracle."""
    import inspect
    import textwrap
    old, new = DECODE_MUTANTS[name]
    src = textwrap.dedent(inspect.getsource(oracle.np_decode))
    assert src.count(old) == 1, old
    ns = dict(vars(oracle))
    exec(src.replace(old, new), ns)
    rng = np.random.default_rng(27)
    Q, K, V, W = _rand(rng, 1, 2, 24, 4, 4, "raw")
    ref = oracle.blockwise(Q, K, V, W, (1, 1, 24), (1, 1, 6), PHI_ELU1, causal=True)
    assert not np.allclose(ns["np_decode"](Q, K, V, W, 6, PHI_ELU1), ref, rtol=1e-8, atol=1e-8)
