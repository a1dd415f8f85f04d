"""fp64 CPU oracle for the MHLA forward -- TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The HIP library and its Python binding
never touch it, and it never touches them.

Two independent implementations live here:

* ``mhla_oracle.c`` (plain C, fp64, OpenMP over (batch, head) slices):
  ``blockwise`` follows the three steps of "MHLA: Restoring Expressivity of
  Linear Attention via Token-Level Multi-Head" §4.1 (block summaries S_b, z_b;
  multi-head mixing S~_i, z~_i; readout), and ``rows`` is brute force on rows
  of the explicit token-pair matrix of §4.2 Eq. 5.
* ``numpy_bruteforce`` (NumPy fp64): the same explicit matrix, built whole,
  for tiny inputs -- a second witness written without the C code.

Both take the two options of the method: ``norm=False`` drops the denominator
(the MHLA paper omits it for language modelling and very long video), and
``causal=True`` is the chunkwise causal form of §4.2 ("Chunkwise parallel form
of MHLA", App. C): blocks are consecutive chunks, query chunk i mixes the
summaries of chunks b < i with W[i,b] and its own chunk's keys j <= q with
W[i,i]; in the explicit matrix that is the mask A[q,j] = 0 for j > q.

``np_lb_init`` is the locality-biased initial mixing matrix of §4.2
(m0[i,j] proportional to 1 - dist(i,j) / max_k dist(i,k), rows summing to 1).

``np_decode`` is incremental (streaming) inference of the causal form, one
token at a time, in the order the MHLA paper's App. C ("Causal inference")
describes: past chunk summaries are kept, the current chunk's summary is
updated with each new token, and the current chunk's mixed state is the mix of
the past summaries plus m_ii times that running summary.

``np_backward`` gives the gradients of the (non-causal) forward for an upstream
gradient G = dL/dY.  The pages print no backward pass; it is the chain rule
applied to the three forward steps of §4.1, written out step by step in
reverse order (readout, mixing, summaries).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mhla_oracle.c")
_LIB = os.path.join(_HERE, "liboracle_mhla.so")
_lib = None

NO_NORM = 1   # option bits of blockwise / rows
CAUSAL = 2


def build(force: bool = True) -> str:
    """Compile the C oracle with gcc (fp64, -O2, OpenMP)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99",
                               "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _configure(lib):
    dp = ctypes.POINTER(ctypes.c_double)
    ip = ctypes.POINTER(ctypes.c_int)
    lp = ctypes.POINTER(ctypes.c_long)
    lib.oracle_mhla_blockwise.argtypes = [dp, dp, dp, dp, dp, ctypes.c_int, ctypes.c_int,
                                          ctypes.c_int, ctypes.c_int, ip, ip,
                                          ctypes.c_int, ctypes.c_int, ctypes.c_int]
    lib.oracle_mhla_rows.argtypes = [dp, dp, dp, dp, dp, ctypes.c_int, ctypes.c_int,
                                     ctypes.c_int, ctypes.c_int, ip, ip, ctypes.c_int,
                                     ctypes.c_int, lp, ctypes.c_int]
    lib.oracle_block_of_token.argtypes = [ip, ip, ctypes.c_long]
    lib.oracle_num_blocks.argtypes = [ip, ip]
    lib.oracle_phi.argtypes = [ctypes.c_int, ctypes.c_double]
    lib.oracle_phi.restype = ctypes.c_double
    lib.oracle_threads.argtypes = []
    return lib


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        _lib = _configure(ctypes.CDLL(_LIB))
    return _lib


def use_library(path):
    """Point the wrappers at another build of mhla_oracle.c (used by the
    mutation tests, which plant mistakes in a copy); returns the previous one."""
    global _lib
    prev = _lib
    _lib = None if path is None else _configure(ctypes.CDLL(path))
    return prev


def _dptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _g3(x: Sequence[int]):
    x = tuple(int(v) for v in x)
    x = (1,) * (3 - len(x)) + x
    return (ctypes.c_int * 3)(*x)


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float64)


def threads() -> int:
    return int(_load().oracle_threads())


def phi(kind: int, x: float) -> float:
    return float(_load().oracle_phi(kind, float(x)))


def num_blocks(grid, block) -> int:
    return int(_load().oracle_num_blocks(_g3(grid), _g3(block)))


def block_of_token(grid, block, t: int) -> int:
    return int(_load().oracle_block_of_token(_g3(grid), _g3(block), int(t)))


def _flags(norm: bool, causal: bool) -> int:
    return (0 if norm else NO_NORM) | (CAUSAL if causal else 0)


def blockwise(Q, K, V, W, grid, block, phi_kind: int, nthreads: int = 0, norm: bool = True,
              causal: bool = False) -> np.ndarray:
    """Q,K,V: [B,H,N,d]; W: [H,M,M].  Returns Y [B,H,N,d] fp64."""
    Q, K, V, W = _f64(Q), _f64(K), _f64(V), _f64(W)
    B, H, N, d = Q.shape
    Y = np.empty_like(Q)
    rc = _load().oracle_mhla_blockwise(_dptr(Q), _dptr(K), _dptr(V), _dptr(W), _dptr(Y),
                                       B, H, N, d, _g3(grid), _g3(block), int(phi_kind),
                                       _flags(norm, causal), int(nthreads))
    if rc != 0:
        raise ValueError("oracle_mhla_blockwise rejected the arguments")
    return Y


def rows(Q, K, V, W, grid, block, phi_kind: int, flat_rows, norm: bool = True,
         causal: bool = False) -> np.ndarray:
    """Brute-force rows.  flat_rows[r] = (b*H + h)*N + q.  Returns [nrows, d]."""
    Q, K, V, W = _f64(Q), _f64(K), _f64(V), _f64(W)
    B, H, N, d = Q.shape
    r = np.ascontiguousarray(flat_rows, dtype=np.int64)
    out = np.empty((len(r), d), dtype=np.float64)
    rc = _load().oracle_mhla_rows(_dptr(Q), _dptr(K), _dptr(V), _dptr(W), _dptr(out),
                                  B, H, N, d, _g3(grid), _g3(block), int(phi_kind),
                                  _flags(norm, causal),
                                  r.ctypes.data_as(ctypes.POINTER(ctypes.c_long)), len(r))
    if rc != 0:
        raise ValueError("oracle_mhla_rows rejected the arguments")
    return out


# ---------------------------------------------------------------------------
# NumPy witness (independent of the C file).
# ---------------------------------------------------------------------------

def np_phi(kind: int, x: np.ndarray) -> np.ndarray:
    if kind == 0:
        return np.maximum(x, 0.0)
    return np.where(x > 0.0, x + 1.0, np.exp(np.minimum(x, 0.0)))


def np_block_map(grid, block) -> np.ndarray:
    """Token -> block index via np.unravel_index / np.ravel_multi_index."""
    g = (1,) * (3 - len(grid)) + tuple(grid)
    b = (1,) * (3 - len(block)) + tuple(block)
    coords = np.unravel_index(np.arange(g[0] * g[1] * g[2]), g)
    bc = tuple(c // s for c, s in zip(coords, b))
    return np.ravel_multi_index(bc, tuple(gi // bi for gi, bi in zip(g, b)))


def np_attention_matrix(q, k, w, grid, block, phi_kind, causal=False) -> np.ndarray:
    """Explicit A[q,j] = W[blk(q), blk(j)] * phi(q).phi(k_j) for one slice
    (zero above the diagonal in the causal form)."""
    bm = np_block_map(grid, block)
    kern = np_phi(phi_kind, q) @ np_phi(phi_kind, k).T
    A = w[np.ix_(bm, bm)] * kern
    return np.tril(A) if causal else A


def numpy_bruteforce(Q, K, V, W, grid, block, phi_kind, norm=True, causal=False) -> np.ndarray:
    Q, K, V, W = _f64(Q), _f64(K), _f64(V), _f64(W)
    B, H, N, d = Q.shape
    Y = np.zeros_like(Q)
    for b in range(B):
        for h in range(H):
            A = np_attention_matrix(Q[b, h], K[b, h], W[h], grid, block, phi_kind, causal)
            num = A @ V[b, h]
            if not norm:
                Y[b, h] = num
                continue
            den = A.sum(axis=1)
            safe = np.where(den == 0.0, 1.0, den)
            Y[b, h] = np.where((den == 0.0)[:, None], 0.0, num / safe[:, None])
    return Y


def np_lb_init(grid, block) -> np.ndarray:
    """Locality-biased initial mixing matrix [M, M] (MHLA paper §4.2): blocks sit
    at their integer coordinates on the block grid (raster order, x fastest);
    m0[i,j] is proportional to 1 - dist(i,j) / max_k dist(i,k) with dist the
    Euclidean distance, and each row is scaled to sum to 1.  With one block the
    matrix is [[1]]."""
    g = (1,) * (3 - len(grid)) + tuple(grid)
    b = (1,) * (3 - len(block)) + tuple(block)
    shape = tuple(gi // bi for gi, bi in zip(g, b))
    M = shape[0] * shape[1] * shape[2]
    pos = np.stack(np.unravel_index(np.arange(M), shape), axis=1).astype(np.float64)
    dist = np.sqrt(((pos[:, None, :] - pos[None, :, :]) ** 2).sum(-1))
    far = dist.max(axis=1, keepdims=True)
    if M == 1:
        return np.ones((1, 1))
    m = 1.0 - dist / far
    return m / m.sum(axis=1, keepdims=True)


def np_dphi(kind: int, x: np.ndarray) -> np.ndarray:
    """Derivative of the feature map: ReLU' = 1 for x > 0 else 0; (elu+1)' =
    1 for x > 0 else exp(x)."""
    if kind == 0:
        return (x > 0.0).astype(np.float64)
    return np.where(x > 0.0, 1.0, np.exp(np.minimum(x, 0.0)))


def np_backward(Q, K, V, W, G, grid, block, phi_kind, norm=True, dw_abs=False):
    """Gradients (dQ, dK, dV, dW) of L = sum(G * Y) for the non-causal forward.
    With dw_abs=True a fifth array is returned: the sum of the absolute values
    of the products that make up each dW entry (the scale of the error bound
    of that dot product when it is evaluated in finite precision).

    Forward, per (batch, head) slice, with phi applied to Q and K:
      S_b = phi(K_b)^T V_b, z_b = phi(K_b)^T 1         (summaries)
      S~_i = sum_b W[i,b] S_b, z~_i = sum_b W[i,b] z_b (mixing)
      n_q = phi(q) S~_i, den_q = phi(q).z~_i, Y_q = n_q / den_q  (readout)
    Reverse, step by step:
      readout:   dn_q = G_q / den_q, dden_q = -(G_q . Y_q) / den_q
                 (without the normaliser: dn_q = G_q, dden_q = 0; a zero
                 denominator gives a zero row and zero gradients)
                 dphi(q) = S~_i dn_q + z~_i dden_q
                 dS~_i = sum_{q in i} phi(q) dn_q^T, dz~_i = sum_{q in i} phi(q) dden_q
      mixing:    dS_b = sum_i W[i,b] dS~_i, dz_b = sum_i W[i,b] dz~_i
                 dW[i,b] += <dS~_i, S_b> + dz~_i . z_b   (W is shared over the batch)
      summaries: dphi(k_j) = dS_b v_j + dz_b, dV_j = dS_b^T phi(k_j)
      feature map: dQ = dphi(Q) * phi'(Q), dK = dphi(K) * phi'(K).
    """
    Q, K, V, W, G = _f64(Q), _f64(K), _f64(V), _f64(W), _f64(G)
    B, H, N, d = Q.shape
    bm = np_block_map(grid, block)
    M = int(bm.max()) + 1
    dQ, dK, dV = np.zeros_like(Q), np.zeros_like(K), np.zeros_like(V)
    dW = np.zeros_like(W)
    dWabs = np.zeros_like(W)
    for b in range(B):
        for h in range(H):
            pq, pk = np_phi(phi_kind, Q[b, h]), np_phi(phi_kind, K[b, h])
            v, g, w = V[b, h], G[b, h], W[h]
            S = np.zeros((M, d, d))
            z = np.zeros((M, d))
            for blk in range(M):
                sel = bm == blk
                S[blk] = pk[sel].T @ v[sel]
                z[blk] = pk[sel].sum(axis=0)
            St = np.einsum("ib,bfc->ifc", w, S)
            zt = w @ z
            n = np.einsum("qf,qfc->qc", pq, St[bm])
            den = np.einsum("qf,qf->q", pq, zt[bm])
            if norm:
                rd = np.where(den == 0.0, 0.0, 1.0 / np.where(den == 0.0, 1.0, den))
                y = n * rd[:, None]
                dn = g * rd[:, None]
                dden = -(g * y).sum(axis=1) * rd
            else:
                dn = g
                dden = np.zeros(N)
            dpq = np.einsum("qfc,qc->qf", St[bm], dn) + zt[bm] * dden[:, None]
            dSt = np.zeros((M, d, d))
            dzt = np.zeros((M, d))
            for i in range(M):
                sel = bm == i
                dSt[i] = pq[sel].T @ dn[sel]
                dzt[i] = pq[sel].T @ dden[sel]
            dS = np.einsum("ib,ifc->bfc", w, dSt)
            dz = w.T @ dzt
            dW[h] += np.einsum("ifc,bfc->ib", dSt, S) + dzt @ z.T
            dWabs[h] += np.einsum("ifc,bfc->ib", np.abs(dSt), np.abs(S)) + np.abs(dzt) @ np.abs(z).T
            dpk = np.einsum("jfc,jc->jf", dS[bm], v) + dz[bm]
            dV[b, h] = np.einsum("jfc,jf->jc", dS[bm], pk)
            dQ[b, h] = dpq * np_dphi(phi_kind, Q[b, h])
            dK[b, h] = dpk * np_dphi(phi_kind, K[b, h])
    if dw_abs:
        return dQ, dK, dV, dW, dWabs
    return dQ, dK, dV, dW


def np_decode(Q, K, V, W, nb, phi_kind, norm=True):
    """Token-by-token causal inference over a 1-D sequence cut into chunks of nb
    tokens (chunk i = tokens [i*nb, (i+1)*nb)).  Q, K, V: [B, H, N, d]; W:
    [H, M, M].  For each token t in chunk i:
      1. when t starts chunk i, the finished chunks' summaries are mixed once:
         P_i = sum_{b<i} W[i,b] S_b, p_i = sum_{b<i} W[i,b] z_b, and the
         running summary of chunk i starts at zero;
      2. S_i += phi(k_t) v_t^T, z_i += phi(k_t);
      3. y_t = phi(q_t)(P_i + W[i,i] S_i) / phi(q_t).(p_i + W[i,i] z_i)
         (the numerator alone without the normaliser; 0 for a zero denominator).
    Returns Y [B, H, N, d]."""
    Q, K, V, W = _f64(Q), _f64(K), _f64(V), _f64(W)
    B, H, N, d = Q.shape
    M = (N + nb - 1) // nb
    Y = np.zeros_like(Q)
    for b in range(B):
        for h in range(H):
            S = np.zeros((M, d, d))
            z = np.zeros((M, d))
            P = np.zeros((d, d))
            p = np.zeros(d)
            for t in range(N):
                i = t // nb
                if t % nb == 0:
                    P = np.einsum("b,bfc->fc", W[h, i, :i], S[:i])
                    p = W[h, i, :i] @ z[:i]
                pk = np_phi(phi_kind, K[b, h, t])
                S[i] += np.outer(pk, V[b, h, t])
                z[i] += pk
                pq = np_phi(phi_kind, Q[b, h, t])
                num = pq @ (P + W[h, i, i] * S[i])
                if not norm:
                    Y[b, h, t] = num
                    continue
                den = pq @ (p + W[h, i, i] * z[i])
                Y[b, h, t] = 0.0 if den == 0.0 else num / den
    return Y
