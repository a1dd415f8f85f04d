"""A lane-level NumPy model of the gfx950 operand layouts the kernels rely on
(CPU only), and of the fragment helpers in csrc/mhla_mfma.hpp, k_pairs.hpp
and k_pairs_bwd.hpp that build operands for them.

v_mfma_f32_16x16x32_bf16, lane l = s + 16 g (s = l % 16, g = l / 16):
  A: lane holds A[s][8g + e], e = 0..7     (16 x 32)
  B: lane holds B[8g + e][s]                (32 x 16)
  D: lane holds D[4g + r][s], r = 0..3      (16 x 16)
v_mfma_f32_16x16x16_bf16: A[s][4g + e], B[4g + e][s], e = 0..3; D as above.
ds_read_b64_tr_b16, within each 16-lane group: lane s supplies the address of
four consecutive 16-bit values and receives, as element e, value s % 4 of
the four that lane 4e + s // 4 supplied.

The MFMA layouts were checked on an MI355X with exact small-integer data
(every case below that issues MFMAs of one shape, or separates two shapes,
gave the exact product).  The same check showed that a dependent MFMA of the
other 16x16 shape -- 16x16x16 reading the accumulator of a 16x16x32 right
after it, or the reverse -- gets a wrong accumulator when it issues back to
back, and hipcc puts no wait states between them; so the library uses the
16x16x32 shape only (test_device_code.py checks the built code object).
Each test below runs a live helper combination through the model and
compares with the plain matrix product it must equal; two more show why a
16-feature tail may only pair operands that hold the same feature indices.
"""
import numpy as np
import pytest

RNG = np.random.default_rng(1234)


def lanes():
    l = np.arange(64)
    return l % 16, l // 16


# ----------------------------------------------------------------- instructions

def mfma_16x16x32(a, b, c):
    """a, b: [64, 8] lane registers; c: [64, 4]. Returns D lanes [64, 4]."""
    s, g = lanes()
    A = np.zeros((16, 32))
    B = np.zeros((32, 16))
    C = np.zeros((16, 16))
    for l in range(64):
        A[s[l], 8 * g[l]:8 * g[l] + 8] = a[l]
        B[8 * g[l]:8 * g[l] + 8, s[l]] = b[l]
        C[4 * g[l]:4 * g[l] + 4, s[l]] = c[l]
    D = A @ B + C
    return np.stack([D[4 * g[l]:4 * g[l] + 4, s[l]] for l in range(64)])


def mfma_16x16x16(a, b, c):
    """a, b: [64, 4] lane registers; c: [64, 4]."""
    s, g = lanes()
    A = np.zeros((16, 16))
    B = np.zeros((16, 16))
    C = np.zeros((16, 16))
    for l in range(64):
        A[s[l], 4 * g[l]:4 * g[l] + 4] = a[l]
        B[4 * g[l]:4 * g[l] + 4, s[l]] = b[l]
        C[4 * g[l]:4 * g[l] + 4, s[l]] = c[l]
    D = A @ B + C
    return np.stack([D[4 * g[l]:4 * g[l] + 4, s[l]] for l in range(64)])


def ds_read_tr4(mem, addr):
    """ds_read_b64_tr_b16: addr[l] = element address supplied by lane l."""
    out = np.zeros((64, 4))
    for l in range(64):
        grp, s = l // 16, l % 16
        for e in range(4):
            src = 16 * grp + 4 * e + s // 4
            out[l, e] = mem[addr[src] + s % 4]
    return out


# ----------------------------------------------------------------- helpers

def lds_tr8(mem, base, rs, r0, c0):
    """mhla_mfma.hpp lds_tr8: lane (s, g) receives column c0 + s of rows
    r0 + 8g .. r0 + 8g + 7 (two transposing reads, rows 4 apart)."""
    s, g = lanes()
    p = base + (r0 + 8 * g + (s >> 2)) * rs + c0 + 4 * (s & 3)
    return np.concatenate([ds_read_tr4(mem, p), ds_read_tr4(mem, p + 4 * rs)], axis=1)


def lds_tr8_rows(mem, base_lane, rs, r0, r1):
    """lds_tr8_rows: base_lane[l] already points at column c0 + 4 (s % 4); lane
    l passes rows r0[l] and r1[l] for the two reads."""
    return np.concatenate([ds_read_tr4(mem, base_lane + r0 * rs),
                           ds_read_tr4(mem, base_lane + r1 * rs)], axis=1)


def pack_acc8(a, b):
    """Two accumulator tiles (rows 4g..4g+3 each) as one 8-element operand."""
    return np.concatenate([a, b], axis=1)


def acc8_row(mem, row_base, m, ct):
    """k_pairs_bwd.hpp acc8_row: elements 0..3 = row[32m + 4g ..], 4..7 =
    row[32m + 16 + 4g ..] (zero when tile 2m + 1 does not exist)."""
    s, g = lanes()
    lo = np.stack([mem[row_base[l] + 32 * m + 4 * g[l] + np.arange(4)] for l in range(64)])
    if 2 * m + 1 < ct:
        hi = np.stack([mem[row_base[l] + 32 * m + 16 + 4 * g[l] + np.arange(4)] for l in range(64)])
    else:
        hi = np.zeros((64, 4))
    return np.concatenate([lo, hi], axis=1)


def feat_row(mem, row_base, ks, ks_full):
    """k_pairs.hpp feat_row: features 32 ks + 8g .. +7 of a row; the half-empty
    tail step (ks == ks_full) leaves groups 2 and 3 zero."""
    s, g = lanes()
    out = np.zeros((64, 8))
    for l in range(64):
        if ks == ks_full and g[l] >= 2:
            continue
        out[l] = mem[row_base[l] + 32 * ks + 8 * g[l] + np.arange(8)]
    return out


def store_row_tiles(tiles, limit):
    """mhla_mfma.hpp store_row_tiles: tiles[j] lane (s, g) element r holds row
    s, entry 16j + 4g + r.  Lane groups g and g^1 swap halves so that each lane
    stores 8 consecutive entries.  Returns the 16 stored rows."""
    nt = len(tiles)
    rows = np.full((16, 16 * nt), np.nan)
    s, g = lanes()
    for j in range(0, nt - 1, 2):
        a, b = tiles[j], tiles[j + 1]
        for l in range(64):
            odd = g[l] & 1
            partner = l ^ 16
            if odd:
                v = np.concatenate([b[partner], b[l]])
                c = 16 * (j + 1) + 4 * (g[l] - 1)
            else:
                v = np.concatenate([a[l], a[partner]])
                c = 16 * j + 4 * g[l]
            if c < limit:
                rows[s[l], c:c + 8] = v
    if nt % 2:
        for l in range(64):
            c = 16 * (nt - 1) + 4 * g[l]
            if c < limit:
                rows[s[l], c:c + 4] = tiles[nt - 1][l]
    return rows


def tile_of(D):
    """The D lanes of a 16 x 16 matrix."""
    s, g = lanes()
    return np.stack([D[4 * g[l]:4 * g[l] + 4, s[l]] for l in range(64)])


def matrix_of(d):
    s, g = lanes()
    D = np.zeros((16, 16))
    for l in range(64):
        D[4 * g[l]:4 * g[l] + 4, s[l]] = d[l]
    return D


# ----------------------------------------------------------------- checks

def test_mfma_model_is_the_matrix_product():
    A, B = RNG.standard_normal((16, 32)), RNG.standard_normal((32, 16))
    s, g = lanes()
    a = np.stack([A[s[l], 8 * g[l]:8 * g[l] + 8] for l in range(64)])
    b = np.stack([B[8 * g[l]:8 * g[l] + 8, s[l]] for l in range(64)])
    np.testing.assert_allclose(matrix_of(mfma_16x16x32(a, b, np.zeros((64, 4)))), A @ B)


def test_lds_tr8_reads_a_column_slice():
    rs = 40
    mem = RNG.standard_normal(64 * rs)
    out = lds_tr8(mem, 0, rs, 32, 16)
    M = mem.reshape(64, rs)
    s, g = lanes()
    for l in range(64):
        np.testing.assert_array_equal(out[l], M[32 + 8 * g[l]:32 + 8 * g[l] + 8, 16 + s[l]])


def test_summary_product():
    """k_summary_mfma: A = tr8 of phi(K) (features x tokens), B = tr8 of V
    (tokens x columns) over two 32-token steps; D = S[feature][column]."""
    RS = 64 + 16
    K = RNG.standard_normal((64, RS))
    V = RNG.standard_normal((64, RS))
    mk, mv = K.ravel(), V.ravel()
    for kt in range(4):
        for ct in range(4):
            acc = np.zeros((64, 4))
            for st in range(2):
                acc = mfma_16x16x32(lds_tr8(mk, 0, RS, 32 * st, 16 * kt),
                                    lds_tr8(mv, 0, RS, 32 * st, 16 * ct), acc)
            S = K[:, 16 * kt:16 * kt + 16].T @ V[:, 16 * ct:16 * ct + 16]
            np.testing.assert_allclose(matrix_of(acc), S, atol=1e-12)


def test_mixing_product():
    """k_mix_big / k_mix_mfma: A = tr8 of the S tile (rows = key blocks,
    columns = entries), B = W rows (8 consecutive key blocks per lane group);
    D[entry][query block]."""
    SRS, WRS = 128 + 8, 32 + 16
    S = RNG.standard_normal((32, SRS))
    W = RNG.standard_normal((128, WRS))
    s, g = lanes()
    for a_t in range(3):
        for c in range(3):
            af = lds_tr8(S.ravel(), 0, SRS, 0, 16 * a_t)
            bw = np.stack([W[16 * c + s[l], 8 * g[l]:8 * g[l] + 8] for l in range(64)])
            D = matrix_of(mfma_16x16x32(af, bw, np.zeros((64, 4))))
            ref = S[:, 16 * a_t:16 * a_t + 16].T @ W[16 * c:16 * c + 16, :32].T
            np.testing.assert_allclose(D, ref, atol=1e-12)


def test_readout_product_and_store():
    """k_readout_mfma: A = rows of S~^T read straight from the transposed
    workspace row (value column 16ct + s, features 32ks + 8g ..), B = phi(Q)
    rows (token s, the same features); D = Y^T; store_row_tiles writes each
    token's row in order."""
    DP, d = 64, 64
    St = RNG.standard_normal((d, DP))          # St[c][f] = S~[f][c]
    Qf = RNG.standard_normal((16, d))          # 16 tokens
    s, g = lanes()
    tiles = []
    for ct in range(4):
        o = np.zeros((64, 4))
        for ks in range(2):
            af = np.stack([St[16 * ct + s[l], 32 * ks + 8 * g[l]:32 * ks + 8 * g[l] + 8]
                           for l in range(64)])
            bq = np.stack([Qf[s[l], 32 * ks + 8 * g[l]:32 * ks + 8 * g[l] + 8] for l in range(64)])
            o = mfma_16x16x32(af, bq, o)
        tiles.append(o)
    Y = Qf @ St.T                               # Y[token][c]
    rows = store_row_tiles(tiles, d)
    np.testing.assert_allclose(rows, Y, atol=1e-12)


@pytest.mark.parametrize("nt", [1, 3, 4, 5])
def test_store_row_tiles_covers_every_entry(nt):
    tiles = [RNG.standard_normal((64, 4)) for _ in range(nt)]
    rows = store_row_tiles(tiles, 16 * nt)
    s, g = lanes()
    for j in range(nt):
        for l in range(64):
            np.testing.assert_array_equal(rows[s[l], 16 * j + 4 * g[l]:16 * j + 4 * g[l] + 4],
                                          tiles[j][l])


def prow(r, rs):
    return r * rs + (r >> 3) * 8


@pytest.mark.parametrize("dk", [16, 48, 64, 80, 96])
def test_token_pair_products(dk):
    """k_pairs: P'^T = phi(K) phi(Q)^T over features in 32-steps with a
    half-empty last step (feat_row / feat operands), then O^T = V^T P' with
    V^T from lds_tr8_rows and P' packed by pack_acc8 (keys 4g..4g+3 of two
    key blocks).  nb = 16 tokens per block, two key blocks."""
    nb = 16
    KS, TAIL = dk // 32, dk % 32 != 0
    KSF = KS + (1 if TAIL else 0)
    RSK = (dk + 15) // 32 * 32 + 16
    DO = 32
    RSV = (DO + 15) // 32 * 32 + 16
    N = 2 * nb
    Kf = np.zeros((N, RSK))
    Kf[:, :dk] = RNG.standard_normal((N, dk))
    Qf = np.zeros((16, RSK))
    Qf[:, :dk] = RNG.standard_normal((16, dk))
    V = RNG.standard_normal((N, DO))
    memK = np.zeros(prow(N + 1, RSK) + 8)
    memV = np.zeros(prow(N + 1, RSV) + 8)
    for r in range(N):
        memK[prow(r, RSK):prow(r, RSK) + RSK] = Kf[r]
        memV[prow(r, RSV):prow(r, RSV) + DO] = V[r]
    s, g = lanes()
    p = []
    for hb in range(2):
        kr = hb * nb + s
        acc = np.zeros((64, 4))
        for ks in range(KSF):
            ka = feat_row(memK, prow(kr, RSK), ks, KS)
            qf = feat_row(Qf.ravel(), s * RSK, ks, KS)
            acc = mfma_16x16x32(ka, qf, acc)
        ref = Kf[hb * nb:hb * nb + 16, :dk] @ Qf[:, :dk].T     # [key][query]
        np.testing.assert_allclose(matrix_of(acc), ref, atol=1e-12)
        p.append(acc)
    pb = pack_acc8(p[0], p[1])
    vj = 4 * g + (s >> 2)
    for c in range(DO // 16):
        va = lds_tr8_rows(memV, 16 * c + 4 * (s & 3), 1, prow(vj, RSV), prow(nb + vj, RSV))
        o = matrix_of(mfma_16x16x32(va, pb, np.zeros((64, 4))))
        P = np.concatenate([matrix_of(p[0]), matrix_of(p[1])], axis=0)   # [32 keys][query]
        ref = V[:, 16 * c:16 * c + 16].T @ P
        np.testing.assert_allclose(o, ref, atol=1e-12)


def test_acc8_row_pairs_with_pack_acc8():
    """k_pairs_bwd: contraction over value columns in the acc8 order -- an
    operand from two accumulator tiles (columns 4g.. and 16 + 4g..) against
    acc8_row of a bf16 row (the same columns), including an odd last tile."""
    for ct in (2, 3):
        G = RNG.standard_normal((16, 16 * ct))      # [query][column]
        Vr = RNG.standard_normal((16, 32 * ((ct + 1) // 2)))   # [key][column]
        Vr[:, 16 * ct:] = 0.0
        s, g = lanes()
        acc = np.zeros((64, 4))
        for m in range((ct + 1) // 2):
            t0 = tile_of(G[:, 32 * m:32 * m + 16].T)
            t1 = tile_of(G[:, 32 * m + 16:32 * m + 32].T) if 2 * m + 1 < ct else np.zeros((64, 4))
            # A operand: row = query s; the accumulator tiles hold columns as rows
            a = pack_acc8(t0, t1)
            b = acc8_row(Vr.ravel(), s * Vr.shape[1], m, ct)
            acc = mfma_16x16x32(a, b, acc)
        np.testing.assert_allclose(matrix_of(acc), G @ Vr[:, :16 * ct].T, atol=1e-12)


def test_16_feature_tail_pairing():
    """A 16-feature tail on the 16x16x16 shape is right only when both
    operands hold features 4g .. 4g+3 (the old forward's 8-byte loads); the
    first half of an 8g-style operand holds 8g .. 8g+3 and pairs wrongly with
    a 4g-style one, and two such halves drop features 4..7 and 12..15.  (The
    library avoids the shape altogether: its tail is a 16x16x32 step with
    groups 2 and 3 zero, see test_token_pair_products.)"""
    A = RNG.standard_normal((16, 16))
    B = RNG.standard_normal((16, 16))
    s, g = lanes()
    four = lambda M, rowmajor: np.stack([(M[s[l], 4 * g[l]:4 * g[l] + 4] if rowmajor
                                          else M[4 * g[l]:4 * g[l] + 4, s[l]]) for l in range(64)])

    def eight_half(M, rowmajor):
        out = np.zeros((64, 4))
        for l in range(64):
            if g[l] < 2:
                out[l] = M[s[l], 8 * g[l]:8 * g[l] + 4] if rowmajor else M[8 * g[l]:8 * g[l] + 4, s[l]]
        return out

    zero = np.zeros((64, 4))
    good = matrix_of(mfma_16x16x16(four(A, True), four(B, False), zero))
    np.testing.assert_allclose(good, A @ B, atol=1e-12)
    mixed = matrix_of(mfma_16x16x16(eight_half(A, True), four(B, False), zero))
    assert not np.allclose(mixed, A @ B)
    halves = matrix_of(mfma_16x16x16(eight_half(A, True), eight_half(B, False), zero))
    keep = np.r_[0:4, 8:12]
    np.testing.assert_allclose(halves, A[:, keep] @ B[keep, :], atol=1e-12)
