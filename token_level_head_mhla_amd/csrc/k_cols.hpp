// k_cols.hpp -- single-kernel MHLA forward split by value columns (bf16 in/out,
// gfx950), for block counts up to 64 and head dims up to 64.
//
// One workgroup of 8 waves per (batch-head slice, chunk of 16 value columns).
// The output columns of "MHLA: Restoring Expressivity of Linear Attention via
// Token-Level Multi-Head" §4.1 are independent given the normaliser: column c
// of Y_q needs only column c of every S_b and the whole z_b.  So each
// workgroup forms S_b[:, chunk] and z_b for every block of its slice, mixes
// them with the head's coefficients and reads out its 16 columns of every
// query, all on chip: there is no workspace.  K and Q are read by every chunk
// of a slice; the grid places the chunks of a slice on one XCD so that the
// re-reads can hit in its L2.  (Measured on the 4096-token image shape this is
// slower than the three-kernel blocked path, so it is an explicit path only.)
//
//   0. Block bases and member offsets go to a small LDS table once, so the
//      loops below do no integer division.
//   1. Wave w summarises blocks b = w, w + 8, ... in 32-token steps: K rows
//      (phi applied) and the chunk's V columns go to the wave's own LDS
//      staging area with 16-byte writes; transpose reads give the MFMA
//      operands, D[c][k] = sum_t V[t][c] phi(K)[t][k] and, with one-hot
//      rows of ones as the other operand, z_b[k].  The finished S_b[:, chunk]
//      and z_b are written as bf16 into column b % 32 of an entry-major table
//      (entry e = c*DP + k, then DP entries of z).
//   2. Every 32 blocks the table is mixed on MFMA:
//      S~[i][e] += sum_b W[i][b] S[b][e] (W rounded to bf16), with the
//      accumulators for all query blocks i of the wave's entries in
//      registers (wave w owns value columns 2w, 2w+1 and z features
//      16w..16w+15).
//   3. S~ (and z~) go to LDS as bf16, laid out [i][c][k] (c = 16 is z~).
//   4. Readout: work item = 16 queries of one block.  Y^T[c][q] =
//      S~_i^T phi(Q)^T on MFMA with phi(Q) loaded straight from global memory
//      (8 consecutive features per lane); a second accumulator whose A
//      operand holds z~_i in row 0 gives the denominators phi(q).z~_i; the
//      divide and the bf16 rounding are fused into 8-byte stores.
//
// A denominator of exactly 0 (ReLU with phi(q) = 0) writes a zero row.
#pragma once

#include "mhla_mfma.hpp"

namespace mhla {

constexpr int kColsWaves = 8;
constexpr int kColsMaxM = 64;
constexpr int kColsMaxNb = 256;  // tokens per block (the member-offset table)

template <int DP>
struct ColsLayout {
  static constexpr int NKT = DP / 16;        // 16-feature tiles
  static constexpr int RK = DP + 16;         // phi(K) staging row stride (elements)
  static constexpr int RV = 16;              // V staging row stride
  static constexpr int STAGE = 32 * RK + 32 * RV;  // per-wave staging (elements)
  static constexpr int E = 17 * DP;          // 16 value columns x DP features, then z
  static constexpr int RB = 40;              // entry table row: 32 blocks + 8 pad
  static constexpr int RS = DP + 8;          // S~ row stride
  static constexpr int CR = 17;              // S~ rows per query block (16 columns + z~)
  __host__ __device__ static constexpr size_t table_off() {
    return (size_t)kColsWaves * STAGE * 2;
  }
  __host__ __device__ static size_t phase1() { return table_off() + (size_t)E * RB * 2; }
  __host__ __device__ static size_t phase3(int M) { return (size_t)M * CR * RS * 2; }
  // block bases [kColsMaxM] and member offsets [kColsMaxNb] (int) after both
  __host__ __device__ static size_t index_off(int M) {
    const size_t a = phase1(), b = phase3(M);
    return a > b ? a : b;
  }
  __host__ __device__ static size_t total(int M) {
    return index_off(M) + (size_t)(kColsMaxM + kColsMaxNb) * 4;
  }
};

template <int DP, int MT, int PHI>
__global__ __launch_bounds__(64 * kColsWaves) void k_cols(
    const bf16_t* __restrict__ Q, const bf16_t* __restrict__ K, const bf16_t* __restrict__ V,
    const float* __restrict__ W, bf16_t* __restrict__ Y, Geo g, int H, int N, int d,
    long slices, int NC) {
  using L = ColsLayout<DP>;
  constexpr int NKT = L::NKT, RK = L::RK, RV = L::RV, RB = L::RB, RS = L::RS, CR = L::CR;
  constexpr int NE = 2 * NKT + 1;  // entry tiles per wave: two value columns, one z tile
  constexpr int DS = DP / 32;      // 32-feature steps of the readout
  constexpr int PF = (DP == 64 && MT == 4) ? 1 : 2;  // summary units in flight
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int M = g.M, nb = g.nb;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int s = lane & 15, grp = lane >> 4;

  // Workgroup x runs on XCD x % 8; the NC chunks of one slice get the same
  // x % 8, so their K and Q reads meet in one L2.
  const int x = blockIdx.x;
  const int xcd = x & 7, loc = x >> 3;
  const int sgrp = loc / NC;
  const long slice = (long)sgrp * 8 + xcd;
  const int chunk = loc - sgrp * NC;
  if (slice >= slices) return;  // whole workgroup, before any barrier
  const int c0 = 16 * chunk;
  const int h = (int)(slice % H);
  const bf16_t* Qs = Q + (size_t)slice * N * d;
  const bf16_t* Ks = K + (size_t)slice * N * d;
  const bf16_t* Vs = V + (size_t)slice * N * d;
  bf16_t* Ys = Y + (size_t)slice * N * d;
  const float* Wh = W + (size_t)h * M * M;

  bf16_t* stK = reinterpret_cast<bf16_t*>(smem) + wave * L::STAGE;
  bf16_t* stV = stK + 32 * RK;
  bf16_t* tab = reinterpret_cast<bf16_t*>(smem + L::table_off());
  bf16_t* sT = reinterpret_cast<bf16_t*>(smem);  // step 3 onwards: S~ [M][CR][RS]
  int* ibase = reinterpret_cast<int*>(smem + L::index_off(M));  // first token of block b
  int* ioff = ibase + kColsMaxM;  // offset of member j (clamped to the last member)

  const int F8 = d >> 3;
  const int KS = (nb + 31) >> 5;  // 32-token steps per block
  const int QT = (nb + 15) >> 4;  // 16-query tiles per block

  // geometry tables, once per workgroup (no divisions in the loops below)
  for (int t = tid; t < M; t += 64 * kColsWaves) ibase[t] = g.blockbase(t);
  for (int t = tid; t < 32 * KS; t += 64 * kColsWaves) ioff[t] = g.tokoff(min(t, nb - 1));

  f32x4_t acc[MT][NE];
#pragma unroll
  for (int it = 0; it < MT; ++it)
#pragma unroll
    for (int et = 0; et < NE; ++et) acc[it][et] = zero4();

  // staging lanes: K rows t = lane/8 + 8q (q = 0..3), feature octet lane % 8;
  // V row t = lane / 2, columns c0 + 8 (lane % 2) .. + 7
  const int kt0 = lane >> 3, koct = lane & 7;
  const int vt = lane >> 1, vcol = c0 + 8 * (lane & 1);
  const bool koct_ok = koct < F8, vcol_ok = vcol < d;
  const int kcol = 8 * min(koct, F8 - 1), vcolc = min(vcol, d - 8);
  // A operands with row ft of ones (z_b accumulates in one tile: row ft of dz
  // holds z_b[16 ft .. 16 ft + 15])
  const uint32_t onehot_bits = 0x3f803f80u;
  lds_barrier();

  const int ngroups = (M + 31) >> 5;
  for (int G = 0; G < ngroups; ++G) {
    if (32 * G + 32 > M) {
      // a partial group: the table's unused block columns must read as 0
      constexpr int chunks = L::E * RB * 2 / 16;
      for (int e = tid; e < chunks; e += 64 * kColsWaves)
        reinterpret_cast<u32x4_t*>(tab)[e] = u32x4_t{0u, 0u, 0u, 0u};
      lds_barrier();
    }
    // ---- 1. summaries of this wave's blocks in the group ----------------------
    // Units (block jb, 32-token step st) of this wave's blocks
    // b = 32 G + wave + 8 jb, in order.  PF units are in flight: the loads of
    // the unit PF ahead are issued as soon as a unit is staged (PF = 1 where
    // the mixing accumulators leave no registers for a second set).  Loads are
    // never skipped (the position is clamped to the last unit) so that the
    // waits count exactly the loads of one unit.
    int nblk = 0;
    while (nblk < 4 && 32 * G + wave + 8 * nblk < M) ++nblk;
    if (nblk > 0) {
      f32x4_t dsv[NKT], dz = zero4();
#pragma unroll
      for (int ft = 0; ft < NKT; ++ft) dsv[ft] = zero4();
      auto issue = [&](u32x4_t(&kr)[4], u32x4_t& vr, int jb, int st) {
        if (jb >= nblk) { jb = nblk - 1; st = KS - 1; }
        const int base = ibase[32 * G + wave + 8 * jb];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int tok = base + ioff[32 * st + kt0 + 8 * q];
          kr[q] = *reinterpret_cast<const u32x4_t*>(Ks + (size_t)tok * d + kcol);
        }
        const int tok = base + ioff[32 * st + vt];
        vr = *reinterpret_cast<const u32x4_t*>(Vs + (size_t)tok * d + vcolc);
      };
      auto stage = [&](const u32x4_t(&kr)[4], const u32x4_t& vr, int st) {
        const u32x4_t z4 = {0u, 0u, 0u, 0u};
        if (koct < DP / 8) {
#pragma unroll
          for (int q = 0; q < 4; ++q)
            *reinterpret_cast<u32x4_t*>(stK + (kt0 + 8 * q) * RK + 8 * koct) =
                (koct_ok && 32 * st + kt0 + 8 * q < nb) ? phi8<PHI>(kr[q]) : z4;
        }
        *reinterpret_cast<u32x4_t*>(stV + vt * RV + 8 * (lane & 1)) =
            (vcol_ok && 32 * st + vt < nb) ? vr : z4;
      };
      auto compute = [&](int jb, int st) {
        // the staging area is private to this wave: LDS keeps one wave's
        // accesses in order, so only the compiler must not move them
        __asm__ volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        const u16x8_t av = lds_tr8(stV, RV, 0, 0, lane);
#pragma unroll
        for (int ft = 0; ft < NKT; ++ft) {
          const u16x8_t bk = lds_tr8(stK, RK, 0, 16 * ft, lane);
          dsv[ft] = mfma_bf16(av, bk, dsv[ft]);
          const uint32_t o = s == ft ? onehot_bits : 0u;
          dz = mfma_bf16(__builtin_bit_cast(u16x8_t, u32x4_t{o, o, o, o}), bk, dz);
        }
        __asm__ volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        if (st == KS - 1) {
          // D[c = 4 grp + r][k = 16 ft + s] -> entry c*DP + k, column b % 32
          bf16_t* col = tab + wave + 8 * jb;
#pragma unroll
          for (int ft = 0; ft < NKT; ++ft) {
            const uint32_t p01 = pack2(dsv[ft][0], dsv[ft][1]);
            const uint32_t p23 = pack2(dsv[ft][2], dsv[ft][3]);
            bf16_t* e = col + ((4 * grp) * DP + 16 * ft + s) * RB;
            e[0] = (bf16_t)p01;
            e[DP * RB] = (bf16_t)(p01 >> 16);
            e[2 * DP * RB] = (bf16_t)p23;
            e[3 * DP * RB] = (bf16_t)(p23 >> 16);
            dsv[ft] = zero4();
          }
          // row ft of dz sits in lane group 0, element ft
          if (grp == 0) {
            const uint32_t z01 = pack2(dz[0], dz[1]), z23 = pack2(dz[2], dz[3]);
            bf16_t* e = col + (16 * DP + s) * RB;
            e[0] = (bf16_t)z01;
            if (NKT > 1) e[16 * RB] = (bf16_t)(z01 >> 16);
            if (NKT > 2) e[32 * RB] = (bf16_t)z23;
            if (NKT > 3) e[48 * RB] = (bf16_t)(z23 >> 16);
          }
          dz = zero4();
        }
      };
      if constexpr (PF == 2) {
        u32x4_t ka[4], va, kb[4], vb;
        // (jb, st) of the units in the two register sets and of the next issue
        int ja = 0, sa = 0, jn = 0, sn = 0;
        auto advance = [&](int& j, int& st) { if (++st == KS) { st = 0; ++j; } };
        issue(ka, va, jn, sn); advance(jn, sn);
        int jbb = jn, sbb = sn;
        issue(kb, vb, jn, sn); advance(jn, sn);
        while (ja < nblk) {
          stage(ka, va, sa);
          const int jc = ja, sc = sa;
          ja = jn; sa = sn;
          issue(ka, va, jn, sn); advance(jn, sn);
          compute(jc, sc);
          const bool has_b = jbb < nblk;
          if (has_b) stage(kb, vb, sbb);
          const int jd = jbb, sd = sbb;
          jbb = jn; sbb = sn;
          issue(kb, vb, jn, sn); advance(jn, sn);
          if (has_b) compute(jd, sd);
        }
      } else {
        u32x4_t ka[4], va;
        int jb = 0, st = 0;
        issue(ka, va, 0, 0);
        while (jb < nblk) {
          stage(ka, va, st);
          int jn = jb, sn = st + 1;
          if (sn == KS) { sn = 0; ++jn; }
          issue(ka, va, jn, sn);
          compute(jb, st);
          jb = jn; st = sn;
        }
      }
    }
    lds_barrier();

    // ---- 2. mixing of this group's 32 blocks ------------------------------------
    // W is read unconditionally (clamped) and masked on its bits, so the loads
    // stay in straight-line code.
    u16x8_t aw[MT];
#pragma unroll
    for (int it = 0; it < MT; ++it) {
      const int i = 16 * it + s;
      uint32_t w8[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int bb = 32 * G + 8 * grp + e;
        const float w = Wh[(size_t)min(i, M - 1) * M + min(bb, M - 1)];
        w8[e] = __float_as_uint(w) & ((i < M && bb < M) ? 0xffffffffu : 0u);
      }
      aw[it] = __builtin_bit_cast(
          u16x8_t, u32x4_t{pack2(__uint_as_float(w8[0]), __uint_as_float(w8[1])),
                           pack2(__uint_as_float(w8[2]), __uint_as_float(w8[3])),
                           pack2(__uint_as_float(w8[4]), __uint_as_float(w8[5])),
                           pack2(__uint_as_float(w8[6]), __uint_as_float(w8[7]))});
    }
#pragma unroll
    for (int et = 0; et < NE; ++et) {
      if (et == NE - 1 && wave >= NKT) break;  // z tiles belong to waves 0..NKT-1
      const int e0 = et < 2 * NKT ? (2 * wave + et / NKT) * DP + 16 * (et % NKT)
                                  : 16 * DP + 16 * wave;
      const u16x8_t bs = *reinterpret_cast<const u16x8_t*>(tab + (e0 + s) * RB + 8 * grp);
#pragma unroll
      for (int it = 0; it < MT; ++it) acc[it][et] = mfma_bf16(aw[it], bs, acc[it][et]);
    }
    lds_barrier();  // the table is rewritten by the next group (or by step 3)
  }

  // ---- 3. S~ and z~ to LDS as bf16, [i][c][k] ---------------------------------
#pragma unroll
  for (int it = 0; it < MT; ++it)
#pragma unroll
    for (int et = 0; et < NE; ++et) {
      if (et == NE - 1 && wave >= NKT) break;
      const int c = et < 2 * NKT ? 2 * wave + et / NKT : 16;
      const int k = et < 2 * NKT ? 16 * (et % NKT) + s : 16 * wave + s;
      const uint32_t p01 = pack2(acc[it][et][0], acc[it][et][1]);
      const uint32_t p23 = pack2(acc[it][et][2], acc[it][et][3]);
      const uint32_t pv[2] = {p01, p23};
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 16 * it + 4 * grp + r;
        if (i < M) sT[(i * CR + c) * RS + k] = (bf16_t)(pv[r >> 1] >> (16 * (r & 1)));
      }
    }
  lds_barrier();

  // ---- 4. readout ----------------------------------------------------------------
  // Work items (query block i, 16-query tile qt) in order; wave w takes a
  // contiguous range.  Items go in batches of RU with two batches of Q rows in
  // flight (positions clamped to the wave's last item, loads never skipped).
  // The denominator comes out of the same MFMA chain: an A operand whose row 0
  // is z~_i gives phi(q).z~_i in row 0 of a second accumulator.
  const int items = M * QT;
  const int ipw = (items + kColsWaves - 1) / kColsWaves;
  const int i0 = wave * ipw, i1 = min(items, i0 + ipw);
  constexpr int RU = 4;
  if (i1 > i0) {
    int cur = -1;
    u16x8_t as[DS], az[DS];
    // the batch positions as (block, tile) pairs, advanced without divisions
    int bi = i0 / QT, bq = i0 - bi * QT;  // next item to issue
    const int li = (i1 - 1) / QT, lq = (i1 - 1) - li * QT;  // the wave's last item
    auto issue_q = [&](u32x4_t(&qr)[RU][DS], int(&tk)[RU], int(&ib)[RU]) {
#pragma unroll
      for (int r = 0; r < RU; ++r) {
        const bool past = bi > li || (bi == li && bq > lq);
        const int i = past ? li : bi, qt = past ? lq : bq;
        ib[r] = past ? -1 : i;
        const int jq = 16 * qt + s;
        tk[r] = jq < nb ? ibase[i] + ioff[jq] : -1;
        const int tok = ibase[i] + ioff[min(jq, nb - 1)];
#pragma unroll
        for (int ks = 0; ks < DS; ++ks)
          qr[r][ks] = *reinterpret_cast<const u32x4_t*>(Qs + (size_t)tok * d +
                                                         min(32 * ks + 8 * grp, d - 8));
        if (++bq == QT) { bq = 0; ++bi; }
      }
    };
    auto consume_q = [&](const u32x4_t(&qr)[RU][DS], const int(&tk)[RU], const int(&ib)[RU]) {
#pragma unroll
      for (int r = 0; r < RU; ++r) {
        const int i = ib[r];
        if (i < 0) break;
        u16x8_t bqv[DS];
#pragma unroll
        for (int ks = 0; ks < DS; ++ks)
          bqv[ks] = (32 * ks + 8 * grp < d) ? __builtin_bit_cast(u16x8_t, phi8<PHI>(qr[r][ks]))
                                            : u16x8_t{0, 0, 0, 0, 0, 0, 0, 0};
        if (i != cur) {
          cur = i;
#pragma unroll
          for (int ks = 0; ks < DS; ++ks) {
            as[ks] =
                *reinterpret_cast<const u16x8_t*>(sT + (i * CR + s) * RS + 32 * ks + 8 * grp);
            const u16x8_t zr =
                *reinterpret_cast<const u16x8_t*>(sT + (i * CR + 16) * RS + 32 * ks + 8 * grp);
            az[ks] = s == 0 ? zr : u16x8_t{0, 0, 0, 0, 0, 0, 0, 0};
          }
        }
        f32x4_t o = zero4(), oz = zero4();
#pragma unroll
        for (int ks = 0; ks < DS; ++ks) {
          o = mfma_bf16(as[ks], bqv[ks], o);
          oz = mfma_bf16(az[ks], bqv[ks], oz);
        }
        // row 0 of oz (lane group 0, element 0) holds the denominators
        const float rd = out_scale(g, __shfl(oz[0], s));
        // D[c = 4 grp + r][q = s]: four consecutive columns of query s
        const int col = c0 + 4 * grp;
        if (tk[r] >= 0 && col < d)
          *reinterpret_cast<uint2*>(Ys + (size_t)tk[r] * d + col) =
              make_uint2(pack2(o[0] * rd, o[1] * rd), pack2(o[2] * rd, o[3] * rd));
      }
    };
    u32x4_t qa[RU][DS], qb[RU][DS];
    int ta[RU], tb[RU], ia[RU], ibb[RU];
    issue_q(qa, ta, ia);
    issue_q(qb, tb, ibb);
    for (int first = i0; first < i1; first += 2 * RU) {
      consume_q(qa, ta, ia);
      issue_q(qa, ta, ia);
      consume_q(qb, tb, ibb);
      issue_q(qb, tb, ibb);
    }
  }
}

inline int cols_dp(int d) { return d <= 32 ? 32 : 64; }
inline int cols_mt(int M) { return M <= 16 ? 1 : (M <= 32 ? 2 : 4); }

inline size_t cols_lds(int d, int M) {
  return cols_dp(d) == 32 ? ColsLayout<32>::total(M) : ColsLayout<64>::total(M);
}

inline bool cols_supports(int dtype, int d, int M, int nb, long slices) {
  if (dtype != 1 || d % 8 != 0 || d > 64 || M < 1 || M > kColsMaxM) return false;
  if (nb < 1 || nb > kColsMaxNb) return false;
  const long nc = (d + 15) / 16;
  if (((slices + 7) / 8) * 8 * nc > 0x7fffffffL) return false;
  return cols_lds(d, M) <= kLdsLimit;
}

template <int DP, int MT, int PHI>
int launch_cols_t(long slices, int H, int N, int d, const Geo& g, const bf16_t* Q,
                  const bf16_t* K, const bf16_t* V, const float* W, bf16_t* Y, hipStream_t st) {
  const size_t lds = ColsLayout<DP>::total(g.M);
  static std::atomic<bool> attr_set[64];
  if (lds_limit_once(reinterpret_cast<const void*>(&k_cols<DP, MT, PHI>), attr_set,
                     (int)kLdsLimit) != 0)
    return -1;
  const int NC = (d + 15) / 16;
  const long grid = ((slices + 7) / 8) * 8 * NC;
  k_cols<DP, MT, PHI><<<dim3((unsigned)grid), dim3(64 * kColsWaves), lds, st>>>(
      Q, K, V, W, Y, g, H, N, d, slices, NC);
  launch_mark(st, "k_cols");
  return 0;
}

template <int DP, int PHI>
int launch_cols_m(long slices, int H, int N, int d, const Geo& g, const bf16_t* Q,
                  const bf16_t* K, const bf16_t* V, const float* W, bf16_t* Y, hipStream_t st) {
  switch (cols_mt(g.M)) {
    case 1: return launch_cols_t<DP, 1, PHI>(slices, H, N, d, g, Q, K, V, W, Y, st);
    case 2: return launch_cols_t<DP, 2, PHI>(slices, H, N, d, g, Q, K, V, W, Y, st);
    default: return launch_cols_t<DP, 4, PHI>(slices, H, N, d, g, Q, K, V, W, Y, st);
  }
}

inline int launch_cols(long slices, int H, int N, int d, const Geo& g, int phi, const bf16_t* Q,
                       const bf16_t* K, const bf16_t* V, const float* W, bf16_t* Y,
                       hipStream_t st) {
  const bool d32 = cols_dp(d) == 32;
  if (phi == PHI_RELU)
    return d32 ? launch_cols_m<32, PHI_RELU>(slices, H, N, d, g, Q, K, V, W, Y, st)
               : launch_cols_m<64, PHI_RELU>(slices, H, N, d, g, Q, K, V, W, Y, st);
  return d32 ? launch_cols_m<32, PHI_ELU1>(slices, H, N, d, g, Q, K, V, W, Y, st)
             : launch_cols_m<64, PHI_ELU1>(slices, H, N, d, g, Q, K, V, W, Y, st);
}

}  // namespace mhla
