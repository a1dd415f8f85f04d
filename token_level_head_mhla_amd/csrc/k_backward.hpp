// k_backward.hpp -- backward pass of the (non-causal) MHLA forward, bf16 in
// and out, fp32 dW, gfx950 MFMA.  The pages print no backward; this is the
// chain rule through the three forward steps of "MHLA: Restoring
// Expressivity of Linear Attention via Token-Level Multi-Head" §4.1, taken in
// reverse order.  With phi applied to Q and K and G = dL/dY:
//
//   readout   dn_q = G_q / den_q, dden_q = -(G_q . Y_q) / den_q
//             (normaliser off: dn_q = G_q, dden_q = 0; den_q = 0: both 0)
//             dphi(q) = S~_i dn_q + z~_i dden_q
//             dS~_i = sum_{q in i} phi(q) dn_q^T,  dz~_i = sum_{q in i} dden_q phi(q)
//   mixing    dS_b = sum_i W[i,b] dS~_i (and dz_b);
//             dW[i,b] = sum over the batch of <dS~_i, S_b> + dz~_i . z_b
//   summaries dphi(k_j) = dS_b v_j + dz_b,  dV_j = dS_b^T phi(k_j)
//   phi       dQ = dphi(Q) * phi'(Q),  dK = dphi(K) * phi'(K)
//
// Treating z as one more value column ([S | z], [V | 1], [dn | dden]) makes
// every step one of the forward's building blocks:
//   1. S, S~          summary kernel, then the mixing GEMM in its precise
//                     form (W as two bf16 parts, S~ in fp32)
//   2. dn, dden, dQ   k_bwd_q, one pass over the query blocks: the readout
//                     recomputed, the two formulas, then dphi(Q) from S~
//                     staged in LDS (hi + lo bf16, read transposed) times G
//                     (exact bf16) on MFMA, scaled by 1/den per token in
//                     fp32, plus z~ dden in fp32, times phi'(Q)
//   3. dS~, dz~       summary kernel with (phi(Q), dN) and dden as z weights
//   4. dS, dz         mixing GEMM with W transposed
//   5. dW             k_dw_partial16 (M <= 16), k_dw_partial (16 < M < 256)
//                     or k_dw_big (M >= 256): per slice, the rows of dS~
//                     against the rows of S over all d*d + d entries (for
//                     16 < M < 256 in up to 8 parts), and k_dw_reduce (sum
//                     over the parts and the batch, fixed order:
//                     deterministic)
//   6. dK, dV         k_bwd_kv, one pass over the key blocks: dS staged in
//                     LDS; dV^T = dS^T phi(K)^T (the readout with K for Q, dS
//                     for S~ and no normaliser), and dphi(K) from dS read
//                     transposed times V on MFMA, plus dz, times phi'(K).
#pragma once

#include "k_blocked.hpp"

namespace mhla {

template <int PHI>
__device__ __forceinline__ float dphi_apply(float x) {
  if constexpr (PHI == PHI_RELU) return x > 0.0f ? 1.0f : 0.0f;
  return x > 0.0f ? 1.0f : __expf(x);
}

// ---------------------------------------------------------------------------
// Steps 6 and 7 in one pass over the key blocks (they read the same dS rows
// and K): per 16-token tile of key block b,
//   dV^T = dS_b^T phi(K)^T (the readout of phi(K) against dS, without the
//       normaliser), and
//   dphi(k)[f] = sum_c dS_b[f][c] v[c] + dz_b[f], times phi'(k) -> dK.
// grid = (M, slices), block = 256: one workgroup per key block.  The block's
// dS row (rows c = value column, entries f; row DP = dz) is staged in LDS: its
// rows are the A operand of dV, and read transposed (A[f][c]) that of dK;
// wave w takes the block's 16-token tiles w, w + 4, ...  phi(K), V and K at
// the output features come straight from global memory (the wave's first
// tile requested before the state is staged); the dz term is added in fp32.
// d = 64: held to 80 VGPRs for six workgroups per CU, as for k_bwd_q.
template <int DP, int PHI>
__global__ __launch_bounds__(kBlkThreads, DP == 64 ? 6 : 1) void k_bwd_kv(const bf16_t* __restrict__ K,
                                                        const bf16_t* __restrict__ V,
                                                        const bf16_t* __restrict__ dS,
                                                        bf16_t* __restrict__ dK,
                                                        bf16_t* __restrict__ dV, Geo g, int N,
                                                        int d) {
  using D = BlockedDims<DP>;
  constexpr int NT = D::NT, DS = D::DS, EP = D::EP, RS = D::RS;
  __shared__ __attribute__((aligned(16))) bf16_t sT[DP * RS];  // rows c, entries f
  __shared__ __attribute__((aligned(16))) float sz[DP];         // dz
  // rows of 128 or 64 bytes (d == DP = 64 or 32) are stored whole, through a
  // per-wave LDS staging area (consecutive lanes on consecutive bytes)
  constexpr bool STAGED = DP == 64 || DP == 32;
  __shared__ __attribute__((aligned(16))) bf16_t stage_all[STAGED ? kBlkWaves * 16 * (DP + 8) : 1];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int s = lane & 15, grp = lane >> 4;
  bf16_t* stage = stage_all + (STAGED ? wave * 16 * (DP + 8) : 0);
  const bool whole_rows = STAGED && d == DP;
  const long slice = blockIdx.y;
  const int blk = blockIdx.x;
  const size_t off = (size_t)slice * N * d;
  const bf16_t* row = dS + ((size_t)slice * g.M + blk) * EP;
  constexpr int F8P = DP / 8;
  const int bb = g.blockbase(blk);
  // Loads of one 16-token tile: K and V as B operands (features
  // 32k + 8grp .. +7 of token s) and K at this lane's output features
  // (16ft + 4grp .. +3).  Rows and features are clamped in bounds, so every
  // load is issued; pad tokens and features are masked when used.
  int tq;
  u32x4_t kb[DS];
  u16x8_t vb[DS];
  uint2 xv[NT];
  auto load_tile = [&](int t0) {
    const int j = t0 + s;
    tq = j < g.nb ? bb + g.tokoff(j) : -1;
    const int tc = bb + g.tokoff(min(j, g.nb - 1));
    const bf16_t* kr = K + off + (size_t)tc * d;
    const bf16_t* vr = V + off + (size_t)tc * d;
#pragma unroll
    for (int ks = 0; ks < DS; ++ks) {
      kb[ks] = *reinterpret_cast<const u32x4_t*>(kr + min(32 * ks + 8 * grp, d - 8));
      vb[ks] = *reinterpret_cast<const u16x8_t*>(vr + min(32 * ks + 8 * grp, d - 8));
    }
#pragma unroll
    for (int ft = 0; ft < NT; ++ft)
      xv[ft] = *reinterpret_cast<const uint2*>(kr + min(16 * ft + 4 * grp, d - 4));
  };
  const int first = 16 * wave;
  if (first < g.nb) load_tile(first);
  for (int it = tid; it < DP * F8P; it += kBlkThreads) {
    const int c = it / F8P, f = it - (it / F8P) * F8P;
    *reinterpret_cast<u32x4_t*>(sT + c * RS + 8 * f) =
        *reinterpret_cast<const u32x4_t*>(row + c * DP + 8 * f);
  }
  for (int f = tid; f < DP; f += kBlkThreads) sz[f] = bf16_to_f32(row[DP * DP + f]);
  lds_barrier();
  const u16x8_t zero8 = {0, 0, 0, 0, 0, 0, 0, 0};
  for (int t0 = first; t0 < g.nb; t0 += 16 * kBlkWaves) {
    if (t0 != first) load_tile(t0);
    u16x8_t bk[DS], bm[DS];
#pragma unroll
    for (int ks = 0; ks < DS; ++ks) {
      const bool ok = tq >= 0 && 32 * ks + 8 * grp < d;
      bk[ks] = __builtin_bit_cast(u16x8_t, phi8<PHI>(ok ? kb[ks] : u32x4_t{0u, 0u, 0u, 0u}));
      bm[ks] = ok ? vb[ks] : zero8;
    }
    // dV^T: rows c = value column, column = token s
    f32x4_t o[NT];
#pragma unroll
    for (int ct = 0; ct < NT; ++ct) {
      o[ct] = zero4();
#pragma unroll
      for (int ks = 0; ks < DS; ++ks)
        o[ct] = mfma_bf16(*reinterpret_cast<const u16x8_t*>(sT + (16 * ct + s) * RS + 32 * ks +
                                                           8 * grp),
                          bk[ks], o[ct]);
    }
    bf16_t* vrow = tq >= 0 ? dV + off + (size_t)tq * d : nullptr;
    if constexpr (STAGED) {
      if (whole_rows) store_rows_staged<NT, false>(vrow, stage, o, 1.0f, lane);
      else store_row_tiles<NT>(vrow, d, o, 1.0f, grp);
    } else {
      store_row_tiles<NT>(vrow, d, o, 1.0f, grp);
    }
    // dK
    const float uem = tq >= 0 ? 1.0f : 0.0f;
    f32x4_t dk[NT];
#pragma unroll
    for (int ft = 0; ft < NT; ++ft) {
      f32x4_t acc = zero4();
#pragma unroll
      for (int kc = 0; kc < DS; ++kc)
        acc = mfma_bf16(lds_tr8(sT, RS, 32 * kc, 16 * ft, lane), bm[kc], acc);
      // acc lane (s, grp) element r = sum_c dS[f][c] v[token t0 + s][c], f = 16ft + 4grp + r
      const int f = 16 * ft + 4 * grp;
      const float x[4] = {lo_f32(xv[ft].x), hi_f32(xv[ft].x), lo_f32(xv[ft].y), hi_f32(xv[ft].y)};
#pragma unroll
      for (int r = 0; r < 4; ++r) dk[ft][r] = (acc[r] + sz[f + r] * uem) * dphi_apply<PHI>(x[r]);
    }
    bf16_t* krow = tq >= 0 ? dK + off + (size_t)tq * d : nullptr;
    if constexpr (STAGED) {
      if (whole_rows) store_rows_staged<NT, false>(krow, stage, dk, 1.0f, lane);
      else store_row_tiles<NT>(krow, d, dk, 1.0f, grp);
    } else {
      store_row_tiles<NT>(krow, d, dk, 1.0f, grp);
    }
  }
}

// ---------------------------------------------------------------------------
// Steps 2 and 6 in one pass over the query blocks (they read the same S~ rows,
// Q and G): per 16-token tile of block i,
//   o^T = S~_i^T phi(Q)^T and den = phi(q).z~_i with S~, z~ rounded to bf16
//       (the recomputed readout),
//   dden = -(G . o) / den^2 (0 without the normaliser), dN = G / den (G
//       without it), stored through LDS as whole rows,
//   dphi(q)[f] = (1/den) sum_c S~[f][c] G[c] + z~[f] dden, with S~ as two
//       bf16 parts (hi + lo) and the per-token factors in fp32, times phi'(q),
//       stored as dQ.
// So the fp32 S~ rows, Q and G are read once instead of twice, and the
// per-token factor 1/den never goes through memory.  grid = (M, slices),
// block = 256: one workgroup per query block, the block's S~ row staged in
// LDS as hi and lo parts (rows c = value column, entries f); wave w takes the
// 16-token tiles w, w + 4, ...  Loads are unconditional (token and feature
// clamped in range) and masked where used.
// d = 64: the compiler is held to 96 VGPRs (91 used, no spills), so that five
// workgroups share a CU (LDS allows five): the kernel is bound by its memory
// streams, and a fifth workgroup keeps more of them in flight.
template <int DP, int PHI>
__global__ __launch_bounds__(kBlkThreads, DP == 64 ? 5 : 1) void k_bwd_q(
    const bf16_t* __restrict__ Q, const float* __restrict__ St, const bf16_t* __restrict__ G,
    bf16_t* __restrict__ dN, float* __restrict__ dden, bf16_t* __restrict__ dQ, Geo g, int N,
    int d) {
  using D = BlockedDims<DP>;
  constexpr int NT = D::NT, DS = D::DS, EP = D::EP, RS = D::RS;
  __shared__ __attribute__((aligned(16))) bf16_t sT[2][DP * RS];  // hi, lo: rows c, entries f
  __shared__ __attribute__((aligned(16))) float sz[DP];            // z~ (fp32)
  __shared__ __attribute__((aligned(16))) bf16_t szb[DP];          // z~ rounded to bf16
  // rows of 128 or 64 bytes (d == DP = 64 or 32) are stored whole, through a
  // per-wave LDS staging area (consecutive lanes on consecutive bytes)
  constexpr bool STAGED = DP == 64 || DP == 32;
  __shared__ __attribute__((aligned(16))) bf16_t stage_all[STAGED ? kBlkWaves * 16 * (DP + 8) : 1];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int s = lane & 15, grp = lane >> 4;
  bf16_t* stage = stage_all + (STAGED ? wave * 16 * (DP + 8) : 0);
  const bool whole_rows = STAGED && d == DP;
  const long slice = blockIdx.y;
  const int blk = blockIdx.x;
  const size_t off = (size_t)slice * N * d;
  const float* row = St + ((size_t)slice * g.M + blk) * EP;
  constexpr int F8P = DP / 8;
  const int bb = g.blockbase(blk);
  // Loads of one 16-token tile, all issued before any is used: phi(Q) and G
  // as B operands (features 32k + 8grp .. +7 of token s), G in the
  // accumulator layout (features 16ct + 4grp .. +3) and Q at the same
  // features.  The wave's first tile is requested before the state is
  // staged, so that both transfers are in flight together.
  int tq;
  u32x4_t qv[DS];
  u16x8_t gb[DS];
  uint2 gu[NT], xv[NT];
  auto load_tile = [&](int t0) {
    const int j = t0 + s;
    tq = j < g.nb ? bb + g.tokoff(j) : -1;
    const int tc = bb + g.tokoff(min(j, g.nb - 1));
    const bf16_t* qr = Q + off + (size_t)tc * d;
    const bf16_t* gr = G + off + (size_t)tc * d;
#pragma unroll
    for (int ks = 0; ks < DS; ++ks) {
      qv[ks] = *reinterpret_cast<const u32x4_t*>(qr + min(32 * ks + 8 * grp, d - 8));
      gb[ks] = *reinterpret_cast<const u16x8_t*>(gr + min(32 * ks + 8 * grp, d - 8));
    }
#pragma unroll
    for (int ct = 0; ct < NT; ++ct) {
      gu[ct] = *reinterpret_cast<const uint2*>(gr + min(16 * ct + 4 * grp, d - 4));
      xv[ct] = *reinterpret_cast<const uint2*>(qr + min(16 * ct + 4 * grp, d - 4));
    }
  };
  const int first = 16 * wave;
  if (first < g.nb) load_tile(first);
  for (int it = tid; it < DP * F8P; it += kBlkThreads) {
    const int c = it / F8P, f = it - (it / F8P) * F8P;
    const f32x4_t x0 = *reinterpret_cast<const f32x4_t*>(row + c * DP + 8 * f);
    const f32x4_t x1 = *reinterpret_cast<const f32x4_t*>(row + c * DP + 8 * f + 4);
    const u32x4_t hi = u32x4_t{pack2(x0[0], x0[1]), pack2(x0[2], x0[3]), pack2(x1[0], x1[1]),
                               pack2(x1[2], x1[3])};
    const u32x4_t lo = u32x4_t{pack2(x0[0] - lo_f32(hi[0]), x0[1] - hi_f32(hi[0])),
                               pack2(x0[2] - lo_f32(hi[1]), x0[3] - hi_f32(hi[1])),
                               pack2(x1[0] - lo_f32(hi[2]), x1[1] - hi_f32(hi[2])),
                               pack2(x1[2] - lo_f32(hi[3]), x1[3] - hi_f32(hi[3]))};
    *reinterpret_cast<u32x4_t*>(sT[0] + c * RS + 8 * f) = hi;
    *reinterpret_cast<u32x4_t*>(sT[1] + c * RS + 8 * f) = lo;
  }
  for (int f = 2 * tid; f < DP; f += 2 * kBlkThreads) {
    const float z0 = row[DP * DP + f], z1 = row[DP * DP + f + 1];
    sz[f] = z0;
    sz[f + 1] = z1;
    *reinterpret_cast<uint32_t*>(szb + f) = pack2(z0, z1);
  }
  lds_barrier();
  const u16x8_t zero8 = {0, 0, 0, 0, 0, 0, 0, 0};
  for (int t0 = first; t0 < g.nb; t0 += 16 * kBlkWaves) {
    if (t0 != first) load_tile(t0);
    u16x8_t bq[DS];
#pragma unroll
    for (int ks = 0; ks < DS; ++ks) {
      const bool ok = tq >= 0 && 32 * ks + 8 * grp < d;
      bq[ks] = __builtin_bit_cast(u16x8_t, phi8<PHI>(ok ? qv[ks] : u32x4_t{0u, 0u, 0u, 0u}));
      gb[ks] = ok ? gb[ks] : zero8;
    }
    // the recomputed readout: o^T (rows c = value column, column = token s)
    f32x4_t o[NT], oz = zero4();
#pragma unroll
    for (int ct = 0; ct < NT; ++ct) {
      o[ct] = zero4();
#pragma unroll
      for (int ks = 0; ks < DS; ++ks)
        o[ct] = mfma_bf16(*reinterpret_cast<const u16x8_t*>(sT[0] + (16 * ct + s) * RS + 32 * ks +
                                                           8 * grp),
                          bq[ks], o[ct]);
    }
#pragma unroll
    for (int ks = 0; ks < DS; ++ks) {
      const u16x8_t az = s == 0 ? *reinterpret_cast<const u16x8_t*>(szb + 32 * ks + 8 * grp)
                                : zero8;
      oz = mfma_bf16(az, bq[ks], oz);
    }
    const float rd = out_scale(g, __shfl(oz[0], s));
    // G^T in the accumulator layout: lane (s, grp) holds G[t0+s][16ct+4grp .. +3]
    float gv[NT][4];
    float dot = 0.0f;
#pragma unroll
    for (int ct = 0; ct < NT; ++ct) {
      const bool ok = tq >= 0 && 16 * ct + 4 * grp < d;
      const uint2 u = ok ? gu[ct] : make_uint2(0u, 0u);
      gv[ct][0] = lo_f32(u.x); gv[ct][1] = hi_f32(u.x);
      gv[ct][2] = lo_f32(u.y); gv[ct][3] = hi_f32(u.y);
#pragma unroll
      for (int r = 0; r < 4; ++r) dot += gv[ct][r] * (o[ct][r] * rd);
    }
    // sum over the four lanes of token s (groups 0..3)
    dot += __shfl_xor(dot, 16);
    dot += __shfl_xor(dot, 32);
    const float scale = g.norm ? rd : 1.0f;
    const float dd = g.norm ? -dot * rd : 0.0f;
    {
      f32x4_t gt[NT];
#pragma unroll
      for (int ct = 0; ct < NT; ++ct) gt[ct] = f32x4_t{gv[ct][0], gv[ct][1], gv[ct][2], gv[ct][3]};
      bf16_t* nrow = tq >= 0 ? dN + off + (size_t)tq * d : nullptr;
      if constexpr (STAGED) {
        if (whole_rows) store_rows_staged<NT, false>(nrow, stage, gt, scale, lane);
        else store_row_tiles<NT>(nrow, d, gt, scale, grp);
      } else {
        store_row_tiles<NT>(nrow, d, gt, scale, grp);
      }
    }
    if (tq >= 0 && grp == 0) dden[(size_t)slice * N + tq] = dd;
    // dQ against the precise S~ (hi + lo), the per-token factors in fp32
    const float usm = tq >= 0 ? scale : 1.0f, uem = tq >= 0 ? dd : 0.0f;
    f32x4_t oq[NT];
#pragma unroll
    for (int ft = 0; ft < NT; ++ft) {
      f32x4_t acc = zero4();
#pragma unroll
      for (int p = 0; p < 2; ++p)
#pragma unroll
        for (int kc = 0; kc < DS; ++kc)
          acc = mfma_bf16(lds_tr8(sT[p], RS, 32 * kc, 16 * ft, lane), gb[kc], acc);
      // acc lane (s, grp) element r = sum_c S~[f][c] G[token t0 + s][c], f = 16ft + 4grp + r
      const int f = 16 * ft + 4 * grp;
      const float x[4] = {lo_f32(xv[ft].x), hi_f32(xv[ft].x), lo_f32(xv[ft].y), hi_f32(xv[ft].y)};
#pragma unroll
      for (int r = 0; r < 4; ++r)
        oq[ft][r] = (acc[r] * usm + sz[f + r] * uem) * dphi_apply<PHI>(x[r]);
    }
    bf16_t* xrow = tq >= 0 ? dQ + off + (size_t)tq * d : nullptr;
    if constexpr (STAGED) {
      if (whole_rows) {
        store_rows_staged<NT, false>(xrow, stage, oq, 1.0f, lane);
        continue;
      }
    }
    store_row_tiles<NT>(xrow, d, oq, 1.0f, grp);
  }
}

// ---------------------------------------------------------------------------
// Step 5, M <= 16.  P[slice][i][b] = sum_{e < DP*DP + DP} A[slice][i][e]
// B[slice][b][e] over the workspace rows (A = dS~, B = S).  grid =
// (ceil(M/16)^2, slices),
// block = 256: a 16 x 16 output tile per workgroup, the contraction split over
// the four waves (steps of 32 entries, wave w takes steps w, w + 4, ...) and
// summed in LDS.  Rows past M are clamped on load and never stored.
template <int DP>
__global__ __launch_bounds__(kBlkThreads) void k_dw_partial16(const bf16_t* __restrict__ A,
                                                            const bf16_t* __restrict__ Bm,
                                                            float* __restrict__ P, int M) {
  using D = BlockedDims<DP>;
  constexpr int EP = D::EP, E = DP * DP + DP, NSTEP = E / 32;
  static_assert(E % 32 == 0, "contraction steps");
  __shared__ float red[kBlkWaves][256];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int s = lane & 15, grp = lane >> 4;
  const long slice = blockIdx.y;
  const int nt = (M + 15) / 16;
  const int i0 = 16 * (blockIdx.x / nt), b0 = 16 * (blockIdx.x % nt);
  const bf16_t* arow = A + ((size_t)slice * M + min(i0 + s, M - 1)) * EP + 8 * grp;
  const bf16_t* brow = Bm + ((size_t)slice * M + min(b0 + s, M - 1)) * EP + 8 * grp;
  // four independent accumulators, four steps' loads issued together
  f32x4_t acc4[4] = {zero4(), zero4(), zero4(), zero4()};
  int k = wave;
  for (; k + 3 * kBlkWaves < NSTEP; k += 4 * kBlkWaves) {
    u16x8_t av[4], bv[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      av[u] = *reinterpret_cast<const u16x8_t*>(arow + 32 * (k + u * kBlkWaves));
      bv[u] = *reinterpret_cast<const u16x8_t*>(brow + 32 * (k + u * kBlkWaves));
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) acc4[u] = mfma_bf16(av[u], bv[u], acc4[u]);
  }
  for (; k < NSTEP; k += kBlkWaves)
    acc4[0] = mfma_bf16(*reinterpret_cast<const u16x8_t*>(arow + 32 * k),
                        *reinterpret_cast<const u16x8_t*>(brow + 32 * k), acc4[0]);
  const f32x4_t acc = (acc4[0] + acc4[1]) + (acc4[2] + acc4[3]);
  // acc lane (s, grp) element r = P[i0 + 4grp + r][b0 + s]
#pragma unroll
  for (int r = 0; r < 4; ++r) red[wave][(4 * grp + r) * 16 + s] = acc[r];
  __syncthreads();
  if (tid < 256) {
    const int ii = tid / 16, bl = tid % 16;
    const float v = red[0][tid] + red[1][tid] + red[2][tid] + red[3][tid];
    if (i0 + ii < M && b0 + bl < M) P[((size_t)slice * M + i0 + ii) * M + b0 + bl] = v;
  }
}

// ---------------------------------------------------------------------------
// Step 5, 16 < M < 256.  P[slice][i][b] = sum_{e < DP*DP + DP} A[slice][i][e] B[slice][b][e]
// over the workspace rows (A = dS~, B = S).  grid = (ceil(M/T)^2 * nsplit,
// slices), block = 256: a T x T output tile per workgroup (T = 64; the
// kernel also takes T = 128), a (T/2) x (T/2) quarter per wave.  Both operands are
// contiguous in e, so the MFMA fragments are 16-byte row reads of an LDS tile
// (no transpose); 32-entry steps pass through a double-buffered tile, loaded
// one step ahead.  Each operand row is read once per T output columns (the
// 16 x 16-tile kernel above reads it once per 16: 6.5 GB through L2 and
// 712 us on the video shape, against 122 us here with T = 128, which
// k_dw_big has since replaced for M >= 256).  For 16 < M < 256 the
// contraction is split into nsplit parts (dw_split) that write separate
// partial sums, so that the few 64 x 64 tiles still give enough workgroups
// (4096-token image backward: 0.242 against 0.249 ms with the 16 x 16
// kernel).  Rows past M are clamped on load and never stored.
template <int DP, int T>
__global__ __launch_bounds__(kBlkThreads) void k_dw_partial(const bf16_t* __restrict__ A,
                                                            const bf16_t* __restrict__ Bm,
                                                            float* __restrict__ P, int M,
                                                            int nsplit, size_t pstride) {
  using D = BlockedDims<DP>;
  constexpr int EP = D::EP, E = DP * DP + DP, NSTEP = E / 32;
  static_assert(E % 32 == 0, "contraction steps");
  constexpr int WT = T / 2, FT = WT / 16;        // wave tile and its 16-row fragments
  constexpr int RS = 32 + 16;                    // LDS row stride (elements)
  constexpr int CH = 2 * T * 32 / 8 / kBlkThreads;  // 16-byte chunks per thread per step
  static_assert(CH * 8 * kBlkThreads == 2 * T * 32, "tile");
  __shared__ __attribute__((aligned(16))) bf16_t sm[2][2 * T * RS];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int s = lane & 15, grp = lane >> 4;
  const int wi = wave >> 1, wb = wave & 1;
  const long slice = blockIdx.y;
  const int nt = (M + T - 1) / T;
  // blockIdx.x = tile * nsplit + part: part takes steps [k0, k1) of the
  // contraction and writes its partial sums at P + part * pstride
  const int tile = blockIdx.x / nsplit, part = blockIdx.x - tile * nsplit;
  const int i0 = T * (tile / nt), b0 = T * (tile % nt);
  const int k0 = part * NSTEP / nsplit, k1 = (part + 1) * NSTEP / nsplit;
  P += (size_t)part * pstride;
  // chunk u of a step: LDS row r = c / 4 (rows 0..T-1 hold A rows i0.., rows
  // T..2T-1 hold B rows b0..), 16-byte piece c % 4 of the step's 32 entries.
  // Rows past M are clamped in bounds; they feed outputs that are not stored.
  const bf16_t* src[CH];
  int dst[CH];
#pragma unroll
  for (int u = 0; u < CH; ++u) {
    const int c = tid + kBlkThreads * u, r = c >> 2, f = c & 3;
    const bool isa = r < T;
    const int row = min((isa ? i0 + r : b0 + r - T), M - 1);
    src[u] = (isa ? A : Bm) + ((size_t)slice * M + row) * EP + 8 * f;
    dst[u] = r * RS + 8 * f;
  }
  u32x4_t ld[CH];
  auto gload = [&](int k) {
#pragma unroll
    for (int u = 0; u < CH; ++u) ld[u] = *reinterpret_cast<const u32x4_t*>(src[u] + 32 * k);
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int u = 0; u < CH; ++u) *reinterpret_cast<u32x4_t*>(sm[buf] + dst[u]) = ld[u];
  };
  f32x4_t acc[FT][FT];
#pragma unroll
  for (int a = 0; a < FT; ++a)
#pragma unroll
    for (int b = 0; b < FT; ++b) acc[a][b] = zero4();
  gload(k0);
  lstore(0);
  lds_barrier();
  // Step k reads LDS buffer (k - k0) & 1; the loads of step k + 1 (clamped,
  // never skipped) land in the other buffer after this step's fragment reads.
  for (int k = k0; k < k1; ++k) {
    const int buf = (k - k0) & 1;
    gload(k + 1 < k1 ? k + 1 : k);
    // A fragment: row i (lane s), entries 8grp .. 8grp+7; B likewise for row b
    u16x8_t af[FT], bf[FT];
#pragma unroll
    for (int t = 0; t < FT; ++t) {
      af[t] = *reinterpret_cast<const u16x8_t*>(sm[buf] + (WT * wi + 16 * t + s) * RS + 8 * grp);
      bf[t] = *reinterpret_cast<const u16x8_t*>(sm[buf] + (T + WT * wb + 16 * t + s) * RS +
                                                8 * grp);
    }
#pragma unroll
    for (int a = 0; a < FT; ++a)
#pragma unroll
      for (int b = 0; b < FT; ++b) acc[a][b] = mfma_bf16(af[a], bf[b], acc[a][b]);
    lstore(buf ^ 1);
    lds_barrier();
  }
  // acc[a][b] lane (s, grp) element r = P[i0 + WT wi + 16a + 4grp + r][b0 + WT wb + 16b + s]
#pragma unroll
  for (int a = 0; a < FT; ++a)
#pragma unroll
    for (int b = 0; b < FT; ++b) {
      const int bc = b0 + WT * wb + 16 * b + s;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = i0 + WT * wi + 16 * a + 4 * grp + r;
        if (i < M && bc < M) P[((size_t)slice * M + i) * M + bc] = acc[a][b][r];
      }
    }
}

// Step 5, M >= 256: the same P[slice][i][b] = sum_e A[slice][i][e] B[slice][b][e]
// as k_dw_partial, on large-M mixing's pattern.  A workgroup (4 waves) computes
// a 256 (i) x 128 (b) tile, a wave 128 x 64 (32 accumulator tiles, 32 MFMAs per
// 32 entries).  Entries advance KB per step through a ring of three LDS
// stages filled by global-to-LDS loads (global_load_lds_dwordx4) two steps
// ahead, one barrier per step: no register staging and no LDS store
// instructions.  KB = 64 where the contraction length allows (d = 64): each
// step then reads whole 128-byte pieces of the operand rows, which lie 8 KB
// and more apart, so that every visit to a row is one DRAM access; pieces of
// 64 bytes cost a second access per line when the rows come from HBM.  The
// stages (48 KB each) then hold one workgroup per CU; with KB = 32 (24 KB
// stages) two.  Rows are kept unpadded with 16-byte chunk f of row r at slot
// f ^ ((r / (8 / CPR)) % CPR), CPR = KB / 8 chunks per row, so that the
// fragment reads (16 rows, one chunk each) spread over all banks; the lane
// that loads a slot fetches the chunk that belongs there.  Rows past M are
// clamped in bounds and never stored.  grid = 8 ceil(slices / 8) *
// ceil(M / 256) * ceil(M / 128) (the workgroups of one slice share an XCD and
// its L2), block = 256.
template <int EP, int KB>
__device__ __forceinline__ void dw_big_loop(bf16_t* __restrict__ ring,
                                            const bf16_t* __restrict__ Ab,
                                            const bf16_t* __restrict__ Bb, int M, int i0, int b0,
                                            int nk, int wave, int lane, f32x4_t (&acc)[8][4]) {
  constexpr int TI = 256, TB = 128, STAGE = (TI + TB) * KB;
  constexpr int CPR = KB / 8, RPL = 64 / CPR;  // chunks per row, rows per load
  constexpr int LA = TI / 4 / RPL, LB = TB / 4 / RPL, NL = LA + LB;
  // wait for this thread's loads of step k; those of step k + 1 may stay in flight
  constexpr int WAIT = (NL & 15) | 0x70 | ((NL >> 4) << 14);  // vmcnt(NL) lgkmcnt(0)
  const int s = lane & 15, grp = lane >> 4;
  const int wi = wave >> 1, wb = wave & 1;
  // Wave w loads A rows 64w .. 64w+63 and B rows 32w .. 32w+31, RPL rows per
  // load: lane L's 16 bytes land at slot L of the 1 KB, row L / CPR, slot
  // L % CPR, holding the chunk that belongs there.
  const bf16_t* ap[LA];
  const bf16_t* bp[LB];
#pragma unroll
  for (int u = 0; u < LA; ++u) {
    const int r = TI / 4 * wave + RPL * u + lane / CPR;
    ap[u] = Ab + (size_t)(i0 + r < M ? i0 + r : M - 1) * EP +
            8 * ((lane % CPR) ^ ((r / (8 / CPR)) % CPR));
  }
#pragma unroll
  for (int u = 0; u < LB; ++u) {
    const int r = TB / 4 * wave + RPL * u + lane / CPR;
    bp[u] = Bb + (size_t)(b0 + r < M ? b0 + r : M - 1) * EP +
            8 * ((lane % CPR) ^ ((r / (8 / CPR)) % CPR));
  }
  auto issue = [&](bf16_t* st, int k) {
#pragma unroll
    for (int u = 0; u < LA; ++u)
      __builtin_amdgcn_global_load_lds(
          (const void*)(ap[u] + KB * k),
          (__attribute__((address_space(3))) void*)(st + (TI / 4 * wave + RPL * u) * KB), 16, 0,
          0);
#pragma unroll
    for (int u = 0; u < LB; ++u)
      __builtin_amdgcn_global_load_lds(
          (const void*)(bp[u] + KB * k),
          (__attribute__((address_space(3))) void*)(st + (TI + TB / 4 * wave + RPL * u) * KB), 16,
          0, 0);
  };
  // per 32 entries h: A fragment t: row 128wi + 16t + s, entries 32h + 8grp
  // .. +7; B fragment u: row TI + 64wb + 16u + s, the same entries
  auto compute = [&](const bf16_t* st) {
#pragma unroll
    for (int h = 0; h < KB / 32; ++h) {
      const int sw = 8 * ((4 * h + grp) ^ ((s / (8 / CPR)) % CPR));
      u16x8_t bf[4];
#pragma unroll
      for (int u = 0; u < 4; ++u)
        bf[u] = *reinterpret_cast<const u16x8_t*>(st + (TI + 64 * wb + 16 * u + s) * KB + sw);
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const u16x8_t af =
            *reinterpret_cast<const u16x8_t*>(st + (128 * wi + 16 * t + s) * KB + sw);
#pragma unroll
        for (int u = 0; u < 4; ++u) acc[t][u] = mfma_bf16(af, bf[u], acc[t][u]);
      }
    }
  };
  // as in mix_big_loop: wait for step k's loads, barrier, refill the stage
  // read in step k - 1 with step k + 2 (past the end: the last step again,
  // into a stage no one reads), multiply
  auto step = [&](bf16_t* cur, bf16_t* next2, int k) {
    __builtin_amdgcn_s_waitcnt(WAIT);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    issue(next2, k + 2 < nk ? k + 2 : nk - 1);
    compute(cur);
  };
  bf16_t* const ring0 = ring;
  bf16_t* const ring1 = ring + STAGE;
  bf16_t* const ring2 = ring + 2 * STAGE;
  issue(ring0, 0);
  issue(ring1, nk > 1 ? 1 : 0);
  int k = 0;
  for (; k + 3 <= nk; k += 3) {
    step(ring0, ring2, k);
    step(ring1, ring0, k + 1);
    step(ring2, ring1, k + 2);
  }
  if (k < nk) step(ring0, ring2, k);
  if (k + 1 < nk) step(ring1, ring0, k + 1);
  __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0): no load is left in flight
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// entries per step of k_dw_big: 64 where d^2 + d allows it
template <int DP>
constexpr int dw_big_kb() {
  return (DP * DP + DP) % 64 == 0 ? 64 : 32;
}

template <int DP>
__global__ __launch_bounds__(256, dw_big_kb<DP>() == 64 ? 1 : 2) void k_dw_big(
    const bf16_t* __restrict__ A, const bf16_t* __restrict__ Bm, float* __restrict__ P, int M,
    long nslices) {
  using D = BlockedDims<DP>;
  constexpr int EP = D::EP, E = DP * DP + DP, KB = dw_big_kb<DP>(), NSTEP = E / KB;
  constexpr int TI = 256, TB = 128;
  static_assert(E % KB == 0, "contraction steps");
  __shared__ __attribute__((aligned(16))) bf16_t ring[3 * (TI + TB) * KB];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int s = lane & 15, grp = lane >> 4;
  const int wi = wave >> 1, wb = wave & 1;
  const int nti = (M + TI - 1) / TI, ntb = (M + TB - 1) / TB, per = nti * ntb;
  const int xcd = blockIdx.x & 7, j = blockIdx.x >> 3;
  const long slice = (long)(j / per) * 8 + xcd;
  if (slice >= nslices) return;  // before any barrier
  const int rem = j - (j / per) * per;
  const int i0 = TI * (rem / ntb), b0 = TB * (rem % ntb);
  f32x4_t acc[8][4];
#pragma unroll
  for (int t = 0; t < 8; ++t)
#pragma unroll
    for (int u = 0; u < 4; ++u) acc[t][u] = zero4();
  dw_big_loop<EP, KB>(ring, A + (size_t)slice * M * EP, Bm + (size_t)slice * M * EP, M, i0, b0,
                      NSTEP, wave, lane, acc);
  // acc[t][u] lane (s, grp) element r = P[i0 + 128wi + 16t + 4grp + r][b0 + 64wb + 16u + s]
  float* Ps = P + (size_t)slice * M * M;
#pragma unroll
  for (int t = 0; t < 8; ++t)
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int bc = b0 + 64 * wb + 16 * u + s;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = i0 + 128 * wi + 16 * t + 4 * grp + r;
        if (i < M && bc < M) Ps[(size_t)i * M + bc] = acc[t][u][r];
      }
    }
}

// dW[h][i][b] = sum over the parts of the contraction and over the batch of
// P[part][batch * H + h][i][b], in a fixed order: term q (part q / B, batch
// item q % B) goes to partial sum q % 8, and the eight partial sums meet in a
// fixed tree.  The terms are fetched eight at a time, with no branch among
// the eight loads (indices past the last term are clamped and masked), so
// that eight loads are in flight per thread.
__global__ __launch_bounds__(256) void k_dw_reduce(const float* __restrict__ P,
                                                   float* __restrict__ dW, int B, int H, int M,
                                                   int nsplit, size_t pstride) {
  const long e = (long)blockIdx.x * 256 + threadIdx.x;
  const long MM = (long)M * M;
  if (e >= (long)H * MM) return;
  const long h = e / MM, ib = e - h * MM;
  const int n = nsplit * B;
  // term q0's address, advanced by one batch item (db) or, after the last
  // batch item, to the first of the next part (dsp)
  const float* first = P + h * MM + ib;
  const float* ptr = first;
  const long db = (long)H * MM, dsp = (long)pstride - (long)(B - 1) * db;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  int b = 0;  // batch item of term q0
  for (int q0 = 0; q0 < n; q0 += 8) {
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const bool ok = q0 + u < n;
      v[u] = *(ok ? ptr : first);
      v[u] = ok ? v[u] : 0.0f;
      const bool wrap = b + 1 == B;
      ptr += wrap ? dsp : db;
      b = wrap ? 0 : b + 1;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) acc[u] += v[u];
  }
  dW[e] = ((acc[0] + acc[1]) + (acc[2] + acc[3])) + ((acc[4] + acc[5]) + (acc[6] + acc[7]));
}

// Parts of the dW contraction for 16 < M < 256, where the 64 x 64 tiles
// alone give few workgroups (one per slice at M = 64): about 512 workgroups,
// at most 8 parts.
inline int dw_split(long slices, int M) {
  if (M <= 16 || M >= 256) return 1;
  const long tiles = slices * (long)((M + 63) / 64) * ((M + 63) / 64);
  const long sp = (512 + tiles - 1) / tiles;
  return (int)(sp < 1 ? 1 : (sp > 8 ? 8 : sp));
}

// ---------------------------------------------------------------------------
inline bool backward_supports(int dtype, int d, int M, long slices) {
  if (!blocked_supports(dtype, d, M, slices)) return false;
  // the precise mixing GEMM runs 64 query blocks per workgroup on a 1-D grid,
  // and the dW tile grid along x is ceil(M/16)^2 (M <= 16) or ceil(M/64)^2
  // times the contraction parts (16 < M < 256), both at most ceil(M/16)^2; for
  // M >= 256 the dW grid is 1-D (k_dw_big)
  const long n = (slices + 7) / 8 * 8 * (long)(blocked_ws_elems(d) / kMixEB) * ((M + 63) / 64);
  const long ndw = (slices + 7) / 8 * 8 * (long)((M + 255) / 256) * ((M + 127) / 128);
  return n * kBlkThreads < (1L << 31) && ndw < (1L << 31) &&
         (long)((M + 15) / 16) * ((M + 15) / 16) < (1L << 31);
}

// Workspace: S, dS~, dS ([slices][M][EP] bf16 each), the precise S~
// ([slices][M][EP] fp32), dN ([slices][N][d] bf16), dden ([slices][N] fp32),
// P ([slices][M][M] fp32), the mixing's coefficient scratch (two sets for the
// precise large-M mixing).
inline size_t backward_workspace(long slices, int H, int M, int N, int d) {
  const size_t rows = (size_t)slices * M * blocked_ws_elems(d) * sizeof(bf16_t);
  const size_t al = 256;
  auto up = [&](size_t x) { return (x + al - 1) / al * al; };
  return 3 * up(rows) + up(2 * rows) + up((size_t)slices * N * d * sizeof(bf16_t)) +
         up((size_t)slices * N * sizeof(float)) +
         up((size_t)dw_split(slices, M) * slices * M * M * sizeof(float)) +
         mix_coef2_bytes(H, M);
}

template <int DP, int PHI>
int launch_backward_t(long slices, int B, int H, int N, int d, const Geo& g, const bf16_t* Q,
                      const bf16_t* K, const bf16_t* V, const float* W, const bf16_t* dY,
                      bf16_t* dQ, bf16_t* dK, bf16_t* dV, float* dW, void* ws, hipStream_t st) {
  using D = BlockedDims<DP>;
  const int M = g.M;
  const size_t al = 256;
  auto up = [&](size_t x) { return (x + al - 1) / al * al; };
  const size_t rows = (size_t)slices * M * D::EP;
  char* p = static_cast<char*>(ws);
  bf16_t* S = reinterpret_cast<bf16_t*>(p);
  p += up(rows * sizeof(bf16_t));
  bf16_t* dSt = reinterpret_cast<bf16_t*>(p);
  p += up(rows * sizeof(bf16_t));
  bf16_t* dS = reinterpret_cast<bf16_t*>(p);
  p += up(rows * sizeof(bf16_t));
  float* St32 = reinterpret_cast<float*>(p);
  p += up(rows * sizeof(float));
  bf16_t* dN = reinterpret_cast<bf16_t*>(p);
  p += up((size_t)slices * N * d * sizeof(bf16_t));
  float* dden = reinterpret_cast<float*>(p);
  p += up((size_t)slices * N * sizeof(float));
  float* P = reinterpret_cast<float*>(p);
  const int nsp = dw_split(slices, M);
  const size_t pstride = (size_t)slices * M * M;
  p += up((size_t)nsp * pstride * sizeof(float));
  bf16_t* wc = reinterpret_cast<bf16_t*>(p);
  const unsigned nsl = (unsigned)slices;
  // 1. forward state: S, and the precise S~ (fp32, W in two bf16 parts),
  //    which serves both the recomputed readout and dQ in step 2
  k_summary_mfma<DP, PHI><<<dim3((unsigned)M, nsl), 64 * D::NT, 0, st>>>(K, V, S, g, N, d,
                                                                           nullptr);
  launch_mix_f32<DP>(slices, H, M, S, W, St32, wc, st);
  // 2. dn, dden and dQ in one pass over the query blocks
  const unsigned nbw = (unsigned)((M + kBlkWaves - 1) / kBlkWaves);
  k_bwd_q<DP, PHI><<<dim3((unsigned)M, nsl), kBlkThreads, 0, st>>>(Q, St32, dY, dN, dden, dQ, g,
                                                                   N, d);
  // 3. dS~ = phi(Q)^T dN per query block, dz~ weighted by dden
  k_summary_mfma<DP, PHI><<<dim3((unsigned)M, nsl), 64 * D::NT, 0, st>>>(Q, dN, dSt, g, N, d,
                                                                           dden);
  // 4. dS = W^T-mixing of dS~
  launch_mix<DP>(slices, H, M, dSt, W, dS, kMixTransposed, wc, st);
  // 5. dW (with one batch item and one part the partials are dW itself)
  const bool direct = B == 1 && nsp == 1;
  float* Pd = direct ? dW : P;
  if (M >= 256) {
    const unsigned nb = (unsigned)((slices + 7) / 8 * 8 * ((M + 255) / 256) * ((M + 127) / 128));
    k_dw_big<DP><<<dim3(nb), 256, 0, st>>>(dSt, S, Pd, M, slices);
  } else if (M > 16) {
    const unsigned nt = (unsigned)((M + 63) / 64);
    k_dw_partial<DP, 64><<<dim3(nt * nt * nsp, nsl), kBlkThreads, 0, st>>>(dSt, S, Pd, M, nsp,
                                                                          pstride);
  } else {
    const unsigned nt = (unsigned)((M + 15) / 16);
    k_dw_partial16<DP><<<dim3(nt * nt, nsl), kBlkThreads, 0, st>>>(dSt, S, Pd, M);
  }
  if (!direct) {
    const long nw = (long)H * M * M;
    k_dw_reduce<<<dim3((unsigned)((nw + 255) / 256)), 256, 0, st>>>(P, dW, B, H, M, nsp,
                                                                    pstride);
  }
  // 6. dK and dV in one pass over the key blocks
  k_bwd_kv<DP, PHI><<<dim3((unsigned)M, nsl), kBlkThreads, 0, st>>>(K, V, dS, dK, dV, g, N, d);
  return 0;
}

template <int PHI>
int launch_backward_p(long slices, int B, int H, int N, int d, const Geo& g, const bf16_t* Q,
                      const bf16_t* K, const bf16_t* V, const float* W, const bf16_t* dY,
                      bf16_t* dQ, bf16_t* dK, bf16_t* dV, float* dW, void* ws, hipStream_t st) {
  switch (blocked_dp(d)) {
    case 32: return launch_backward_t<32, PHI>(slices, B, H, N, d, g, Q, K, V, W, dY, dQ, dK, dV, dW, ws, st);
    case 64: return launch_backward_t<64, PHI>(slices, B, H, N, d, g, Q, K, V, W, dY, dQ, dK, dV, dW, ws, st);
    default: return launch_backward_t<96, PHI>(slices, B, H, N, d, g, Q, K, V, W, dY, dQ, dK, dV, dW, ws, st);
  }
}

inline int launch_backward(long slices, int B, int H, int N, int d, const Geo& g, int phi,
                           const bf16_t* Q, const bf16_t* K, const bf16_t* V, const float* W,
                           const bf16_t* dY, bf16_t* dQ, bf16_t* dK, bf16_t* dV, float* dW,
                           void* ws, hipStream_t st) {
  if (phi == PHI_RELU)
    return launch_backward_p<PHI_RELU>(slices, B, H, N, d, g, Q, K, V, W, dY, dQ, dK, dV, dW, ws, st);
  return launch_backward_p<PHI_ELU1>(slices, B, H, N, d, g, Q, K, V, W, dY, dQ, dK, dV, dW, ws, st);
}

}  // namespace mhla
