"""Planted-mistake check for the oracle's pins (CPU only).

Each mutant is a copy of oracle/mhla_oracle.c with one plausible mistake
(a transposed operand, a dropped term, a wrong index or axis).  It is built
with gcc into a temporary directory, and the pins of test_oracle_pins must
then fail on it.  The committed oracle itself is never modified.
"""
import json
import os
import subprocess

import numpy as np
import pytest
import torch

import oracle
from mhla_inputs import PHI_ELU1, PHI_RELU

SRC = os.path.join(os.path.dirname(oracle.__file__), "mhla_oracle.c")
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")

MUTANTS = {
    "w_transposed": ("double m = w[(size_t)i * M + b];", "double m = w[(size_t)b * M + i];"),
    "no_normaliser": ("den == 0.0 ? 0.0 : num[c] / den;", "den == 0.0 ? 0.0 : num[c];"),
    "phi_on_v": ("Sb[(size_t)a * d + c] += pk[a] * v[(size_t)t * d + c];",
                 "Sb[(size_t)a * d + c] += pk[a] * oracle_phi(phi, v[(size_t)t * d + c]);"),
    "summary_transposed": ("Sb[(size_t)a * d + c] += pk[a]", "Sb[(size_t)c * d + a] += pk[a]"),
    "elu_without_one": ("return x > 0.0 ? x + 1.0 : exp(x);", "return x > 0.0 ? x : exp(x);"),
    "block_axes_swapped": ("long bx = x / block[2], by = y / block[1]",
                           "long bx = x / block[1], by = y / block[2]"),
    "block_raster_swapped": ("return (int)((bz * nby + by) * nbx + bx);",
                             "return (int)((bz * nbx + bx) * nby + by);"),
    "flattened_split": ("long x = t % grid[2];",
                        "return (int)(t / ((long)block[0] * block[1] * block[2]));\n  long x = t % grid[2];"),
    "z_without_phi": ("z[(size_t)b * d + a] += pk[a];",
                      "z[(size_t)b * d + a] += k[(size_t)t * d + a];"),
    "query_phi_dropped": ("double pq = oracle_phi(phi, q[(size_t)t * d + a]);",
                          "double pq = q[(size_t)t * d + a];"),
    "mix_skips_last_block": ("for (int b = 0; b < (causal ? i : M); ++b) {",
                             "for (int b = 0; b < (causal ? i : M - 1); ++b) {"),
    # options: normaliser switch and the chunkwise causal form
    "nonorm_ignored": ("  if (flags & ORACLE_NO_NORM) {\n    for (int c = 0; c < d; ++c) y[c] = num[c];",
                       "  if (0) {\n    for (int c = 0; c < d; ++c) y[c] = num[c];"),
    "causal_prefix_includes_own": ("b < (causal ? i : M)", "b < (causal ? i + 1 : M)"),
    "causal_own_chunk_strict": ("for (int t2 = 0; t2 <= t; ++t2)", "for (int t2 = 0; t2 < t; ++t2)"),
    "causal_own_chunk_unweighted": ("double mii = w[(size_t)i * M + i];", "double mii = 1.0;"),
    "causal_own_chunk_wrong_weight": ("double mii = w[(size_t)i * M + i];",
                                      "double mii = w[(size_t)(i > 0 ? i - 1 : 0) * M + i];"),
    "rows_causal_strict": ("(jmax_causal ? qi + 1 : N)", "(jmax_causal ? qi : N)"),
    "rows_nonorm_ignored": ("    if (!(flags & ORACLE_NO_NORM))\n      for", "    if (1)\n      for"),
}


def _pins_hold() -> bool:
    """A compact run of the pins; True when all of them hold (an argument error
    raised by a mutant counts as a failed pin)."""
    try:
        return _pins_hold_inner()
    except ValueError:
        return False


def _pins_hold_inner() -> bool:
    ok = True
    for name in ["worked_relu_2x2.json", "worked_elu1_1x2.json"]:
        g = json.load(open(os.path.join(GOLDEN, name)))
        arr = lambda k: np.array(g[k], dtype=np.float64)[None, None]
        exp = np.array(g["Y_num"], dtype=np.float64) / np.array(g["Y_den"], dtype=np.float64)
        Y = oracle.blockwise(arr("Q"), arr("K"), arr("V"), np.array(g["W"])[None],
                             g["grid"], g["block"], g["phi"])[0, 0]
        ok &= bool(np.allclose(Y, exp, rtol=0, atol=1e-12))
    for case in json.load(open(os.path.join(GOLDEN, "geometry_blocks.json")))["cases"]:
        N = int(np.prod(case["grid"]))
        got = [oracle.block_of_token(case["grid"], case["block"], t) for t in range(N)]
        want = np.empty(N, dtype=int)
        for b, toks in enumerate(case["members"]):
            want[toks] = b
        ok &= got == want.tolist()
    rng = np.random.default_rng(0)
    for grid, block in [((1, 6, 10), (1, 3, 5)), ((2, 4, 6), (1, 2, 3)), ((1, 5, 7), (1, 5, 7))]:
        for phi in (PHI_RELU, PHI_ELU1):
            N = int(np.prod(grid))
            M = oracle.num_blocks(grid, block)
            Q, K, V = (rng.standard_normal((1, 2, N, 5)) for _ in range(3))
            W = rng.uniform(0.2, 1.0, (2, M, M))
            Yb = oracle.blockwise(Q, K, V, W, grid, block, phi)
            ok &= bool(np.allclose(Yb, oracle.numpy_bruteforce(Q, K, V, W, grid, block, phi),
                                   rtol=1e-10, atol=1e-10))
    # the options: hand-derived numerators and the chunkwise causal example
    g = json.load(open(os.path.join(GOLDEN, "worked_relu_2x2.json")))
    arr = lambda k: np.array(g[k], dtype=np.float64)[None, None]
    args = (arr("Q"), arr("K"), arr("V"), np.array(g["W"])[None], g["grid"], g["block"], g["phi"])
    num = np.array(g["numerator"])
    ok &= bool(np.allclose(oracle.blockwise(*args, norm=False)[0, 0], num, rtol=0, atol=1e-12))
    ok &= bool(np.allclose(oracle.rows(*args, np.arange(4), norm=False), num, rtol=0, atol=1e-12))
    g = json.load(open(os.path.join(GOLDEN, "worked_causal_relu_1x4.json")))
    args = (arr("Q"), arr("K"), arr("V"), np.array(g["W"])[None], g["grid"], g["block"], g["phi"])
    num, den = np.array(g["numerator"]), np.array(g["denominator"])[:, None]
    for norm, exp in ((True, num / den), (False, num)):
        ok &= bool(np.allclose(oracle.blockwise(*args, norm=norm, causal=True)[0, 0], exp,
                               rtol=0, atol=1e-12))
        ok &= bool(np.allclose(oracle.rows(*args, np.arange(4), norm=norm, causal=True), exp,
                               rtol=0, atol=1e-12))
    for grid, block in [((1, 1, 24), (1, 1, 6)), ((2, 3, 4), (1, 3, 4))]:
        N, M = int(np.prod(grid)), oracle.num_blocks(grid, block)
        Q, K, V = (rng.standard_normal((1, 2, N, 4)) for _ in range(3))
        W = rng.uniform(0.2, 1.0, (2, M, M))
        for norm in (True, False):
            ref = oracle.numpy_bruteforce(Q, K, V, W, grid, block, PHI_ELU1, norm=norm, causal=True)
            Yb = oracle.blockwise(Q, K, V, W, grid, block, PHI_ELU1, norm=norm, causal=True)
            Yr = oracle.rows(Q, K, V, W, grid, block, PHI_ELU1, np.arange(2 * N), norm=norm,
                             causal=True).reshape(ref.shape)
            ok &= bool(np.allclose(Yb, ref, rtol=1e-10, atol=1e-10))
            ok &= bool(np.allclose(Yr, ref, rtol=1e-10, atol=1e-10))
    # softmax reduction with one token per block
    q, k, v = (rng.standard_normal((12, 4)) for _ in range(3))
    pq, pk = oracle.np_phi(PHI_ELU1, q), oracle.np_phi(PHI_ELU1, k)
    W = np.exp(q @ k.T / 2.0) / (pq @ pk.T)
    Y = oracle.blockwise(q[None, None], k[None, None], v[None, None], W[None], (1, 3, 4),
                         (1, 1, 1), PHI_ELU1)[0, 0]
    ref = torch.nn.functional.scaled_dot_product_attention(
        *(torch.from_numpy(x)[None, None] for x in (q, k, v)))[0, 0].numpy()
    ok &= bool(np.allclose(Y, ref, rtol=1e-10, atol=1e-10))
    return ok


def test_pins_hold_on_committed_oracle():
    assert _pins_hold()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, "mutation site not found: " + name
    mut = tmp_path / "mutant.c"
    mut.write_text(src.replace(old, new))
    so = tmp_path / "libmutant.so"
    subprocess.check_call(["gcc", "-O1", "-fopenmp", "-fPIC", "-shared", "-std=c99", "-o",
                           str(so), str(mut), "-lm"])
    prev = oracle.use_library(str(so))
    try:
        assert not _pins_hold(), "mutant %s survived the pins" % name
    finally:
        oracle._lib = prev
