"""Pins of the oracle's backward pass (CPU only).

The pages print no backward; np_backward applies the chain rule to the three
forward steps of "MHLA: Restoring Expressivity of Linear Attention via
Token-Level Multi-Head" §4.1.  It is pinned to things it does not share code
with:
  * central finite differences of the C forward oracle (blockwise order);
  * torch autograd through the explicit token-pair form of §4.2 Eq. 5
    (an N x N matrix, a different formulation of the same function);
  * the closed form dV = A^T G of the un-normalised form, which is linear in V.
Planted mistakes in a copy of np_backward must fail these pins.
"""
import inspect
import textwrap

import numpy as np
import pytest
import torch

import oracle
from mhla_inputs import PHI_ELU1, PHI_RELU

GEOMS = [((1, 4, 6), (1, 2, 3)), ((2, 2, 4), (1, 2, 2)), ((1, 1, 10), (1, 1, 5))]


def _case(seed, grid, block, d, phi, B=2, H=2):
    rng = np.random.default_rng(seed)
    N = int(np.prod(grid))
    M = oracle.num_blocks(grid, block)
    Q, K, V, G = (rng.standard_normal((B, H, N, d)) for _ in range(4))
    if phi == PHI_RELU:
        Q = np.abs(Q) + 0.1   # no 0/0 rows, so that autograd is defined everywhere
        K = np.where(np.abs(K) < 1e-2, 0.5, K)
    W = rng.uniform(0.2, 1.0, (H, M, M))
    return Q, K, V, W, G


def _autograd(Q, K, V, W, G, grid, block, phi, norm):
    """torch autograd of sum(G * Y) with Y from the explicit attention matrix."""
    t = lambda x: torch.tensor(x, dtype=torch.float64, requires_grad=True)
    q, k, v, w = t(Q), t(K), t(V), t(W)
    bm = torch.from_numpy(oracle.np_block_map(grid, block))
    if phi == PHI_RELU:
        f = torch.relu
    else:
        f = lambda x: torch.where(x > 0, x + 1.0, torch.exp(torch.clamp(x, max=0.0)))
    A = w[:, bm][:, :, bm][None] * (f(q) @ f(k).transpose(-1, -2))
    num = A @ v
    Y = num / A.sum(-1, keepdim=True) if norm else num
    (Y * torch.from_numpy(G)).sum().backward()
    return q.grad.numpy(), k.grad.numpy(), v.grad.numpy(), w.grad.numpy()


@pytest.mark.parametrize("grid,block", GEOMS)
@pytest.mark.parametrize("phi", [PHI_RELU, PHI_ELU1])
@pytest.mark.parametrize("norm", [True, False])
def test_backward_matches_autograd_of_token_form(grid, block, phi, norm):
    Q, K, V, W, G = _case(hash((grid, phi, norm)) % 2**32, grid, block, 5, phi)
    got = oracle.np_backward(Q, K, V, W, G, grid, block, phi, norm)
    ref = _autograd(Q, K, V, W, G, grid, block, phi, norm)
    for name, a, b in zip("QKVW", got, ref):
        np.testing.assert_allclose(a, b, rtol=1e-10, atol=1e-10, err_msg="d" + name)


def _loss(Q, K, V, W, G, grid, block, phi, norm):
    return float((oracle.blockwise(Q, K, V, W, grid, block, phi, norm=norm) * G).sum())


@pytest.mark.parametrize("phi", [PHI_RELU, PHI_ELU1])
@pytest.mark.parametrize("norm", [True, False])
def test_backward_matches_finite_differences(phi, norm):
    """Central differences of the C forward oracle, every coordinate of a tiny
    case; the step h = 1e-6 keeps the truncation error near h^2."""
    grid, block = (1, 3, 4), (1, 3, 2)
    Q, K, V, W, G = _case(41 + phi + 2 * norm, grid, block, 3, phi, B=2, H=1)
    grads = oracle.np_backward(Q, K, V, W, G, grid, block, phi, norm)
    h = 1e-6
    for which, g in zip(range(4), grads):
        args = [Q, K, V, W]
        x = args[which]
        fd = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            ap, am = list(args), list(args)
            ap[which], am[which] = xp, xm
            fd[idx] = (_loss(*ap, G, grid, block, phi, norm)
                       - _loss(*am, G, grid, block, phi, norm)) / (2 * h)
        np.testing.assert_allclose(g, fd, rtol=1e-6, atol=1e-7, err_msg="d" + "QKVW"[which])


@pytest.mark.parametrize("phi", [PHI_RELU, PHI_ELU1])
def test_no_norm_dv_is_attention_transpose_times_g(phi):
    """Without the normaliser Y = A V with the explicit matrix A of Eq. 5, so
    dV = A^T G exactly."""
    grid, block = (1, 4, 4), (1, 2, 2)
    Q, K, V, W, G = _case(43, grid, block, 4, phi)
    dV = oracle.np_backward(Q, K, V, W, G, grid, block, phi, norm=False)[2]
    for b in range(2):
        for h in range(2):
            A = oracle.np_attention_matrix(Q[b, h], K[b, h], W[h], grid, block, phi)
            np.testing.assert_allclose(dV[b, h], A.T @ G[b, h], rtol=1e-12, atol=1e-12)


def test_zero_denominator_row_passes_no_gradient():
    """A ReLU query with no positive feature has a 0/0 row, returned as 0 (a
    constant), so its upstream gradient must not reach any input."""
    grid, block = (1, 4, 4), (1, 2, 2)
    Q, K, V, W, G = _case(44, grid, block, 4, PHI_RELU, B=1, H=1)
    Q[0, 0, 5] = -np.abs(Q[0, 0, 5]) - 0.1
    g1 = oracle.np_backward(Q, K, V, W, G, grid, block, PHI_RELU)
    G2 = G.copy()
    G2[0, 0, 5] = 17.0
    g2 = oracle.np_backward(Q, K, V, W, G2, grid, block, PHI_RELU)
    for a, b in zip(g1, g2):
        np.testing.assert_array_equal(a, b)
    assert np.all(g1[0][0, 0, 5] == 0.0)


# ---------------------------------------------------------------- planted mistakes

BACKWARD_MUTANTS = {
    "dden_sign": ("dden = -(g * y).sum(axis=1) * rd", "dden = (g * y).sum(axis=1) * rd"),
    "dn_unscaled": ("dn = g * rd[:, None]", "dn = g"),
    "dpq_without_z": ("dpq = np.einsum(\"qfc,qc->qf\", St[bm], dn) + zt[bm] * dden[:, None]",
                      "dpq = np.einsum(\"qfc,qc->qf\", St[bm], dn)"),
    "mix_not_transposed": ("dS = np.einsum(\"ib,ifc->bfc\", w, dSt)",
                           "dS = np.einsum(\"bi,ifc->bfc\", w, dSt)"),
    "dz_not_transposed": ("dz = w.T @ dzt", "dz = w @ dzt"),
    "dw_transposed": ("dW[h] += np.einsum(\"ifc,bfc->ib\", dSt, S) + dzt @ z.T",
                      "dW[h] += np.einsum(\"ifc,bfc->bi\", dSt, S) + (dzt @ z.T).T"),
    "dw_without_z": ("dW[h] += np.einsum(\"ifc,bfc->ib\", dSt, S) + dzt @ z.T",
                     "dW[h] += np.einsum(\"ifc,bfc->ib\", dSt, S)"),
    "dpk_without_dz": ("dpk = np.einsum(\"jfc,jc->jf\", dS[bm], v) + dz[bm]",
                       "dpk = np.einsum(\"jfc,jc->jf\", dS[bm], v)"),
    "dv_state_transposed": ("dV[b, h] = np.einsum(\"jfc,jf->jc\", dS[bm], pk)",
                            "dV[b, h] = np.einsum(\"jcf,jf->jc\", dS[bm], pk)"),
    "no_phi_derivative": ("dQ[b, h] = dpq * np_dphi(phi_kind, Q[b, h])", "dQ[b, h] = dpq"),
}


def _mutant(old, new):
    src = textwrap.dedent(inspect.getsource(oracle.np_backward))
    assert src.count(old) == 1, old
    ns = dict(vars(oracle))
    exec(src.replace(old, new), ns)
    return ns["np_backward"]


@pytest.mark.parametrize("name", sorted(BACKWARD_MUTANTS))
def test_pins_catch_backward_mutant(name):
    fn = _mutant(*BACKWARD_MUTANTS[name])
    caught = False
    for phi in (PHI_RELU, PHI_ELU1):
        for grid, block in GEOMS[:2]:
            Q, K, V, W, G = _case(45, grid, block, 4, phi)
            ref = _autograd(Q, K, V, W, G, grid, block, phi, True)
            got = fn(Q, K, V, W, G, grid, block, phi, True)
            caught |= not all(np.allclose(a, b, rtol=1e-8, atol=1e-8) for a, b in zip(got, ref))
    assert caught, "mutant %s survived" % name
