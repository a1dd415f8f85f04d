// k_blocked.hpp -- three-kernel MHLA forward for any number of blocks M
// (bf16 in/out, gfx950 MFMA), the three steps of "MHLA: Restoring
// Expressivity of Linear Attention via Token-Level Multi-Head" §4.1:
//
//   k_summary_mfma : S_b = phi(K_b)^T V_b and z_b = sum_j phi(K_b)[j]
//                    (one wave per key block, operands through LDS with
//                    transpose reads, fp32 accumulation, bf16 result)
//   k_mix_mfma     : S~_i = sum_b W[i,b] S_b, z~_i = sum_b W[i,b] z_b, one
//                    GEMM per (batch, head) slice over all d*d + d entries
//                    (k_mix_small for M <= 16; for M >= 256, k_mix_prep
//                    (bf16 coefficients and z~) + k_mix_big, a larger-tile
//                    GEMM over the d*d entries of S)
//   k_readout_mfma : Y_q = phi(Q_q) S~_i / (phi(Q_q) . z~_i), one wave per
//                    query block, operands straight from global memory
//
// Workspace rows: one row of EP bf16 per (slice, block).  Entry c*DP + k holds
// S[k][c] (value column c, key feature k: the transpose of the summary, so
// that the readout's A operand reads 8 consecutive features of one column),
// entries DP*DP + k hold z[k], the rest up to EP is padding that is computed
// but never read.  The same layout serves S (summary -> mixing) and S~
// (mixing -> readout); the mixing GEMM treats the rows as plain vectors.
#pragma once

#include "mhla_mfma.hpp"

namespace mhla {

constexpr int kBlkThreads = 256;
constexpr int kBlkWaves = kBlkThreads / 64;
constexpr int kMixEB = 128;  // entries per mixing workgroup
constexpr int kMixKB = 32;   // key blocks per mixing step

template <int DP>
struct BlockedDims {
  static constexpr int NT = DP / 16;   // 16-wide tiles along d
  static constexpr int DS = DP / 32;   // 32-feature contraction steps
  static constexpr int RS = DP + 16;   // LDS row stride (elements) of staged K, V
  static constexpr int E = DP * DP + DP;
  static constexpr int EP = (E + kMixEB - 1) / kMixEB * kMixEB;
};

inline int blocked_dp(int d) { return (d + 31) / 32 * 32; }

// ---------------------------------------------------------------------------
// Summaries.  grid = (M, slices), block = 64 * NT: one workgroup per key block
// and one wave per 16-column tile ct of the value dimension.  The block's
// tokens are staged in LDS (phi applied to K) 64 at a time; wave ct forms
// S[:, 16ct .. 16ct+15] from transpose-read operands, and wave 0 also forms
// z_b (a ones B operand).  For d = 64 the compiler is held to 80 VGPRs (76
// used, no spills) so that six workgroups (24 waves) share a CU, next to 20 KB
// of LDS each: the more blocks are in flight, the better this bandwidth-bound
// kernel hides its load latency (at 104 VGPRs only four fitted).
//
// zw == nullptr gives z_b = sum_j phi(K_j); otherwise z_b = sum_j zw[j] phi(K_j)
// with zw a per-token fp32 weight ([slices, N]); the backward pass uses this
// for dz~_i = sum_q dden_q phi(Q_q).  STREAM = true reads K and V with the
// nontemporal hint (see blocked_stream).
template <int DP, int PHI, bool STREAM = false>
__global__ __launch_bounds__(64 * (DP / 16), DP == 64 ? 6 : 1) void k_summary_mfma(
    const bf16_t* __restrict__ K, const bf16_t* __restrict__ V, bf16_t* __restrict__ S, Geo g,
    int N, int d, const float* __restrict__ zw) {
  using D = BlockedDims<DP>;
  constexpr int NT = D::NT, RS = D::RS, EP = D::EP;
  constexpr int NTHR = 64 * NT;
  constexpr int F8P = DP / 8;
  constexpr int UCH = 64 * F8P / NTHR;  // 16-byte chunks per thread and tensor (= 2)
  __shared__ __attribute__((aligned(16))) bf16_t sk[64 * RS];
  __shared__ __attribute__((aligned(16))) bf16_t sv[64 * RS];
  __shared__ __attribute__((aligned(16))) bf16_t szw[64];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int ct = __builtin_amdgcn_readfirstlane(tid >> 6);
  const long slice = blockIdx.y;
  const int b = blockIdx.x;
  const size_t off = (size_t)slice * N * d;
  const int F8 = d >> 3;
  const float inv8 = 1.0f / (float)F8;
  const int bb = g.blockbase(b);

  if (d < DP) {  // feature columns d .. DP-1 stay zero for every chunk
    for (int e = tid; e < 64 * RS / 8; e += NTHR) {
      reinterpret_cast<u32x4_t*>(sk)[e] = u32x4_t{0u, 0u, 0u, 0u};
      reinterpret_cast<u32x4_t*>(sv)[e] = u32x4_t{0u, 0u, 0u, 0u};
    }
  }
  f32x4_t acc[NT], zacc[NT];
#pragma unroll
  for (int kt = 0; kt < NT; ++kt) acc[kt] = zacc[kt] = zero4();
  const u16x8_t ones = {0x3f80, 0x3f80, 0x3f80, 0x3f80, 0x3f80, 0x3f80, 0x3f80, 0x3f80};

  for (int c0 = 0; c0 < g.nb; c0 += 64) {
    // chunk it = tid + NTHR u of the 64-token chunk: token jl = it / F8, chunk f
    u32x4_t kr[UCH], vr[UCH];
    int dst[UCH];
#pragma unroll
    for (int u = 0; u < UCH; ++u) {
      const int it = tid + NTHR * u;
      const int jl = (int)(((float)it + 0.5f) * inv8);
      const int f = it - jl * F8;
      const int j = c0 + jl;
      dst[u] = (it < 64 * F8) ? jl * RS + 8 * f : -1;
      kr[u] = vr[u] = u32x4_t{0u, 0u, 0u, 0u};
      if (it < 64 * F8 && j < g.nb) {
        const size_t src = off + (size_t)(bb + g.tokoff(j)) * d + 8 * f;
        if constexpr (STREAM) {
          kr[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(K + src));
          vr[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(V + src));
        } else {
          kr[u] = *reinterpret_cast<const u32x4_t*>(K + src);
          vr[u] = *reinterpret_cast<const u32x4_t*>(V + src);
        }
      }
    }
    float wz = 0.0f;
    if (zw != nullptr && tid < 64 && c0 + tid < g.nb)
      wz = zw[(size_t)slice * N + bb + g.tokoff(c0 + tid)];
    // the previous chunk's reads (or, for d < DP, the zero fill) are done
    if (c0 > 0 || d < DP) lds_barrier();
    if (zw != nullptr && tid < 64) szw[tid] = f32_to_bf16(wz);
#pragma unroll
    for (int u = 0; u < UCH; ++u) {
      if (dst[u] >= 0) {
        const bool real = c0 + (int)(((float)(tid + NTHR * u) + 0.5f) * inv8) < g.nb;
        *reinterpret_cast<u32x4_t*>(sk + dst[u]) = real ? phi8<PHI>(kr[u]) : u32x4_t{0u, 0u, 0u, 0u};
        *reinterpret_cast<u32x4_t*>(sv + dst[u]) = vr[u];
      }
    }
    lds_barrier();
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      const u16x8_t bv = lds_tr8(sv, RS, 32 * st, 16 * ct, lane);
      // B operand of the z column: ones, or the chunk's token weights
      const u16x8_t bz = zw == nullptr
          ? ones
          : *reinterpret_cast<const u16x8_t*>(szw + 32 * st + 8 * (lane >> 4));
#pragma unroll
      for (int kt = 0; kt < NT; ++kt) {
        const u16x8_t a = lds_tr8(sk, RS, 32 * st, 16 * kt, lane);
        acc[kt] = mfma_bf16(a, bv, acc[kt]);
        if (ct == 0) zacc[kt] = mfma_bf16(a, bz, zacc[kt]);
      }
    }
  }
  // acc[kt] lane (s, grp) element r = S[16kt + 4grp + r][16ct + s]: four
  // consecutive features of value column 16ct + s.
  const int s = lane & 15, grp = lane >> 4;
  bf16_t* row = S + ((size_t)slice * g.M + b) * EP;
  store_row_tiles<NT>(row + (16 * ct + s) * DP, DP, acc, 1.0f, grp);
  if (ct == 0 && s == 0) {
#pragma unroll
    for (int kt = 0; kt < NT; ++kt)
      *reinterpret_cast<uint2*>(row + DP * DP + 16 * kt + 4 * grp) =
          make_uint2(pack2(zacc[kt][0], zacc[kt][1]), pack2(zacc[kt][2], zacc[kt][3]));
  }
}

// ---------------------------------------------------------------------------
// Mixing: per slice, S~[i][e] = sum_b W[h][i][b] S[b][e], computed as the
// transposed product S~^T = S^T W^T so that each lane stores four consecutive
// entries.  1-D grid of 8 * ceil(slices / 8) * nE * nI workgroups (nE = EP /
// 128 entry tiles, nI = ceil(M / IB) query-block tiles), block = 256.
// Workgroups are dealt to the 8 XCDs round-robin (id % 8), so workgroup id
// maps to XCD x = id % 8 and that XCD walks slices x, x + 8, ... in turn;
// within a slice the nI query-block tiles of one entry tile are adjacent.
// A slice's W (and each S entry column) is therefore fetched into one XCD's
// L2 and reused there.  The workgroup tile is 128 entries x IB query blocks;
// wave (we, wi) owns EW entries x IW query blocks: (EW, IW) = (64, 64) for
// IB = 128 and (32, 64) for IB = 64.  The key
// blocks are walked in steps of 32: the next step's S and W tiles are loaded
// into registers while the current step's tiles (double-buffered in LDS) feed
// the MFMAs, so there is one barrier per step.
//
// MODE selects the coefficient of S[b] in output row i: kMixPlain W[i,b];
// kMixCausal W[i,b] for b < i and 0 otherwise (the prefix mixture of the
// chunkwise causal form); kMixTransposed W[b,i] (the backward pass's
// dS_b = sum_i W[i,b] dS~_i).
//
// OutT = float is the precise variant used by the backward pass: the
// coefficients enter as two bf16 parts (w = hi + lo, two MFMAs per step) and
// S~ is stored in fp32, so that the only rounding left is that of S.
enum { kMixPlain = 0, kMixCausal = 1, kMixTransposed = 2 };

// With 64 query blocks per workgroup and bf16 output (plain and transposed
// modes) the compiler is held to 96 VGPRs (no spills): five workgroups per CU
// instead of four, which LDS allows (4096-token image mixing 16.6 -> 15.9 us).
template <int EP, int IB, int MODE, typename OutT = bf16_t, bool WVEC = true>
__global__ __launch_bounds__(kBlkThreads,
                             IB == 64 && sizeof(OutT) == 2 && MODE != kMixCausal ? 5 : 1) void
k_mix_mfma(const bf16_t* __restrict__ S,
                                                          const float* __restrict__ W,
                                                          OutT* __restrict__ St, int M, int H,
                                                          long nslices) {
  constexpr bool PREC = sizeof(OutT) == 4;
  constexpr int WSPLIT = PREC ? 2 : 1;
  constexpr int EB = kMixEB, KB = kMixKB;
  constexpr int EW = IB == 64 ? 32 : 64, IW = 64;
  constexpr int AT = EW / 16, BT = IW / 16;        // MFMA tiles per wave along e and i
  constexpr int NWE = EB / EW;                      // waves along e
  constexpr int SRS = EB + 16;  // LDS row stride of the S tile (rows = key blocks)
  constexpr int WRS = KB + 16;  // LDS row stride of the W tile: 16-byte reads of 16
                                // consecutive rows are free of bank conflicts
  constexpr int SCH = KB * EB / 8 / kBlkThreads;   // 16-byte S chunks per thread per step
  constexpr int WCH = IB * KB / 4 / kBlkThreads;   // 4-float W chunks per thread per step
  static_assert(SCH * 8 * kBlkThreads == KB * EB && WCH * 4 * kBlkThreads == IB * KB, "tiles");
  __shared__ __attribute__((aligned(16))) bf16_t sS[2][KB * SRS];
  __shared__ __attribute__((aligned(16))) bf16_t sW[2][WSPLIT][IB * WRS];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int s = lane & 15, grp = lane >> 4;
  const int we = wave % NWE, wi = wave / NWE;
  const int nE = EP / EB, nI = (M + IB - 1) / IB;
  const int xcd = blockIdx.x & 7, j = blockIdx.x >> 3;
  const int per = nE * nI;
  const long slice = (long)(j / per) * 8 + xcd;
  if (slice >= nslices) return;  // no barrier has been reached yet
  const int rem = j - (j / per) * per;
  const int e0 = (rem / nI) * EB, i0 = (rem - (rem / nI) * nI) * IB;
  const int h = (int)(slice % H);
  const bf16_t* Ss = S + (size_t)slice * M * EP;
  const float* Wh = W + (size_t)h * M * M;
  // WVEC (M % 4 == 0, not transposed): W rows are read as 16-byte vectors
  static_assert(!WVEC || MODE != kMixTransposed, "vector W loads read rows");

  f32x4_t acc[AT][BT];
#pragma unroll
  for (int a = 0; a < AT; ++a)
#pragma unroll
    for (int c = 0; c < BT; ++c) acc[a][c] = zero4();

  u32x4_t sr[SCH], sr1[SCH];
  f32x4_t wr[WCH], wr1[WCH];
  // Loads are unconditional, at clamped rows and columns, so that every load
  // of a step is in flight before the first wait; the zeros (key blocks past
  // M, query blocks past M, the prefix mask) are applied when the tiles are
  // written to LDS.
#define MHLA_MIX_GLOAD(b0, sr, wr)                                                        \
  _Pragma("unroll") for (int u = 0; u < SCH; ++u) {                                       \
    const int c = tid + kBlkThreads * u;                                                  \
    const int r = c / (EB / 8), f = c % (EB / 8);                                         \
    sr[u] = *reinterpret_cast<const u32x4_t*>(Ss + (size_t)min((b0) + r, M - 1) * EP + e0 + \
                                              8 * f);                                     \
  }                                                                                       \
  _Pragma("unroll") for (int u = 0; u < WCH; ++u) {                                       \
    const int c = tid + kBlkThreads * u;                                                  \
    const int r = c / (KB / 4), f = c % (KB / 4);                                         \
    const int ic = min(i0 + r, M - 1), bc = (b0) + 4 * f;                                 \
    f32x4_t v;                                                                            \
    if constexpr (WVEC) {                                                                 \
      v = *reinterpret_cast<const f32x4_t*>(Wh + (size_t)ic * M + min(bc, M - 4));        \
    } else if constexpr (MODE == kMixTransposed) {                                        \
      _Pragma("unroll") for (int q = 0; q < 4; ++q)                                       \
        v[q] = Wh[(size_t)min(bc + q, M - 1) * M + ic];                                   \
    } else {                                                                              \
      _Pragma("unroll") for (int q = 0; q < 4; ++q)                                       \
        v[q] = Wh[(size_t)ic * M + min(bc + q, M - 1)];                                   \
    }                                                                                     \
    wr[u] = v;                                                                            \
  }
#define MHLA_MIX_LSTORE(buf, sr, wr, b0)                                                  \
  _Pragma("unroll") for (int u = 0; u < SCH; ++u) {                                       \
    const int c = tid + kBlkThreads * u;                                                  \
    const int r = c / (EB / 8), f = c % (EB / 8);                                         \
    *reinterpret_cast<u32x4_t*>(sS[buf] + r * SRS + 8 * f) =                              \
        (b0) + r < M ? sr[u] : u32x4_t{0u, 0u, 0u, 0u};                                    \
  }                                                                                       \
  _Pragma("unroll") for (int u = 0; u < WCH; ++u) {                                       \
    const int c = tid + kBlkThreads * u;                                                  \
    const int r = c / (KB / 4), f = c % (KB / 4);                                         \
    const int i = i0 + r, bc = (b0) + 4 * f;                                              \
    f32x4_t w = wr[u];                                                                    \
    _Pragma("unroll") for (int q = 0; q < 4; ++q) {                                       \
      const bool keep = i < M && bc + q < M && (MODE != kMixCausal || bc + q < i);        \
      w[q] = keep ? w[q] : 0.0f;                                                          \
    }                                                                                     \
    const uint2 hi_ = make_uint2(pack2(w[0], w[1]), pack2(w[2], w[3]));                   \
    *reinterpret_cast<uint2*>(sW[buf][0] + r * WRS + 4 * f) = hi_;                        \
    if constexpr (PREC) {                                                                 \
      *reinterpret_cast<uint2*>(sW[buf][WSPLIT - 1] + r * WRS + 4 * f) =                  \
          make_uint2(pack2(w[0] - lo_f32(hi_.x), w[1] - hi_f32(hi_.x)),                   \
                     pack2(w[2] - lo_f32(hi_.y), w[3] - hi_f32(hi_.y)));                  \
    }                                                                                     \
  }

  const int nk = (M + KB - 1) / KB;
  // A = S^T (rows e, contraction b via transpose reads: b = 8grp .. 8grp+7),
  // B = W^T (column i, the same b: W[i][8grp .. 8grp+7] is contiguous).
  auto compute = [&](int buf) {
    u16x8_t af[AT], bw[BT];
#pragma unroll
    for (int a = 0; a < AT; ++a) af[a] = lds_tr8(sS[buf], SRS, 0, EW * we + 16 * a, lane);
#pragma unroll
    for (int c = 0; c < BT; ++c)
      bw[c] = *reinterpret_cast<const u16x8_t*>(sW[buf][0] + (IW * wi + 16 * c + s) * WRS + 8 * grp);
#pragma unroll
    for (int a = 0; a < AT; ++a)
#pragma unroll
      for (int c = 0; c < BT; ++c) acc[a][c] = mfma_bf16(af[a], bw[c], acc[a][c]);
    if constexpr (PREC) {
#pragma unroll
      for (int c = 0; c < BT; ++c)
        bw[c] = *reinterpret_cast<const u16x8_t*>(sW[buf][WSPLIT - 1] +
                                                  (IW * wi + 16 * c + s) * WRS + 8 * grp);
#pragma unroll
      for (int a = 0; a < AT; ++a)
#pragma unroll
        for (int c = 0; c < BT; ++c) acc[a][c] = mfma_bf16(af[a], bw[c], acc[a][c]);
    }
  };
  if (nk <= 2) {
    // M <= 64: both steps' loads go out together (the second one repeats the
    // first when nk = 1; loads stay unconditional so the waits are exact)
    MHLA_MIX_GLOAD(0, sr, wr)
    MHLA_MIX_GLOAD((nk - 1) * KB, sr1, wr1)
    MHLA_MIX_LSTORE(0, sr, wr, 0)
    MHLA_MIX_LSTORE(1, sr1, wr1, (nk - 1) * KB)
    lds_barrier();
    compute(0);
    if (nk == 2) compute(1);
  } else {
    MHLA_MIX_GLOAD(0, sr, wr)
    MHLA_MIX_LSTORE(0, sr, wr, 0)
    lds_barrier();
    for (int k = 0; k < nk; ++k) {
      const int buf = k & 1;
      if (k + 1 < nk) { MHLA_MIX_GLOAD((k + 1) * KB, sr, wr) }
      compute(buf);
      if (k + 1 < nk) { MHLA_MIX_LSTORE(buf ^ 1, sr, wr, (k + 1) * KB) }
      lds_barrier();
    }
  }
#undef MHLA_MIX_GLOAD
#undef MHLA_MIX_LSTORE
  // acc[a][c] lane (s, grp) element r = S~[i = 16c + s][e = 16a + 4grp + r]:
  // consecutive lanes hold different rows.  The stores go through the S
  // tiles' LDS (idle after the barrier below), 16 rows at a time in a
  // wave-private area, so that each store instruction writes whole rows of
  // the wave's EW entries with consecutive lanes on consecutive bytes.
  lds_barrier();  // every wave is done reading the tiles
  if constexpr (PREC) {
    constexpr int RSF = EW + 4;    // staging row stride (floats)
    constexpr int LPR = EW / 4;    // lanes per row, 16 bytes each
    constexpr int RPI = 64 / LPR;  // rows per store instruction
    static_assert(kBlkWaves * 16 * RSF * 4 <= 2 * KB * SRS * 2, "staging fits the S tiles");
    float* sw = reinterpret_cast<float*>(&sS[0][0]) + wave * 16 * RSF;
    const int rr = lane / LPR, cq = 4 * (lane % LPR);
    OutT* ob = St + ((size_t)slice * M + i0 + IW * wi + rr) * EP + e0 + EW * we + cq;
#pragma unroll
    for (int c = 0; c < BT; ++c) {
#pragma unroll
      for (int a = 0; a < AT; ++a)
        *reinterpret_cast<f32x4_t*>(sw + s * RSF + 16 * a + 4 * grp) = acc[a][c];
      __builtin_amdgcn_wave_barrier();  // LDS operations of one wave run in order
      f32x4_t v[16 / RPI];
#pragma unroll
      for (int hq = 0; hq < 16 / RPI; ++hq)
        v[hq] = *reinterpret_cast<const f32x4_t*>(sw + (RPI * hq + rr) * RSF + cq);
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int hq = 0; hq < 16 / RPI; ++hq)
        if (i0 + IW * wi + 16 * c + RPI * hq + rr < M)
          *reinterpret_cast<f32x4_t*>(ob + (size_t)(16 * c + RPI * hq) * EP) = v[hq];
    }
  } else {
    static_assert(kBlkWaves * 16 * (16 * AT + 8) <= 2 * KB * SRS, "staging fits the S tiles");
    bf16_t* stage = &sS[0][0] + wave * 16 * (16 * AT + 8);
#pragma unroll
    for (int c = 0; c < BT; ++c) {
      const int i = i0 + IW * wi + 16 * c + s;
      f32x4_t t[AT];
#pragma unroll
      for (int a = 0; a < AT; ++a) t[a] = acc[a][c];
      store_rows_staged<AT, false>(i < M ? St + ((size_t)slice * M + i) * EP + e0 + EW * we : nullptr,
                                   stage, t, 1.0f, lane);
    }
  }
}

// ---------------------------------------------------------------------------
// Mixing for many blocks (M >= kMixBigM, M % 32 == 0; plain, prefix and
// transposed modes).  k_mix_prep (plain, prefix) or k_mix_coef_t (transposed)
// first writes the coefficient matrix of the mode in bf16 (Wc[h][i][b] =
// coef(i, b)), so that the GEMM streams two bf16 operands with unconditional
// 16-byte loads.  k_mix_big: one workgroup (4
// waves) computes 256 query blocks x 128 entries of one slice; wave (we, wi)
// owns 64 entries x 128 query blocks (32 accumulator tiles), which keeps it
// within 256 registers, so two workgroups share a CU and one's barrier waits
// overlap the other's MFMAs.  Key blocks advance 32 per step through a ring
// of three LDS stages (72 KB) filled by global-to-LDS loads
// (global_load_lds_dwordx4, no register round trip): the loads of step k + 2
// are issued while step k is multiplied, one barrier per step.  In the
// prefix mode a tile stops at the last key block its rows can use.
constexpr int kMixBigM = 256;

// Coefficient layout of the large-M mixing: for every head, query-block tile
// (256 rows, padded with zero rows past M) and 32-block step, one contiguous
// 256 x 32 bf16 tile (16 KB), so that each mixing step loads whole cache lines.
__host__ __device__ inline size_t coef_tiled(int M, int h, int i, int b) {
  const int nit = (M + 255) / 256, nk = M / 32;
  return (((size_t)h * nit + i / 256) * nk + b / 32) * 8192 + (size_t)(i % 256) * 32 + b % 32;
}

// Coefficients and mixed normalisers of the large-M mixing, plain and
// prefix modes.  A workgroup owns the 16 query blocks i0 .. i0+15 of head h
// (rows past M are the zero padding of the coefficient tiles):
//   - it converts their rows of W to the bf16 coefficients of the mode
//     (coef(i, b) = W[h][i][b], zero for b >= i in the prefix mode) and
//     writes them in the tiled layout of coef_tiled;
//   - for every slice of head h it forms z~_i = sum_b coef(i, b) z_b on MFMA
//     (the same bf16 coefficients as the GEMM, fp32 accumulation) and stores
//     it as the z part of row i of S~ (entries DP*DP .. DP*DP + DP - 1).
// k_mix_big then mixes only the DP*DP entries of S, which are a whole number
// of its 128-entry tiles.  The key blocks go in steps of 32; wave w takes
// steps w, w + 4, ...; the z_b rows of 128 key blocks (one step per wave) are
// staged in LDS and read as transposed B operands; the four waves' partial
// sums meet in LDS.  Each chunk's z rows and W pieces are requested while the
// previous chunk is multiplied (a workgroup used to wait for two round trips
// per chunk: the z rows, then, after staging them, the W pieces).  grid =
// H8 * MI / 16 (H8 = H rounded up to 8, MI = M rounded up to 256; the
// workgroups of one head share an XCD), block = 256, M % 32 == 0.
template <int DP, int MODE>
__global__ __launch_bounds__(256) void k_mix_prep(const float* __restrict__ W,
                                                  const bf16_t* __restrict__ S,
                                                  bf16_t* __restrict__ St,
                                                  bf16_t* __restrict__ Wc, int M, int H,
                                                  long nslices) {
  static_assert(MODE == kMixPlain || MODE == kMixCausal, "plain and prefix modes only");
  constexpr int EP = BlockedDims<DP>::EP;
  constexpr int NT = DP / 16;        // 16-feature output tiles
  constexpr int ZR = DP + 8;         // LDS row stride of the staged z rows
  constexpr int CH = 128;            // key blocks staged per chunk
  constexpr int ZCH = CH * DP / 8 / 256;  // 16-byte z pieces per thread per chunk
  __shared__ __attribute__((aligned(16))) bf16_t sz[CH * ZR];
  __shared__ __attribute__((aligned(16))) float sacc[4][16][DP + 4];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int s = lane & 15, grp = lane >> 4;
  const int nti = (M + 255) / 256 * 16;  // 16-row tiles per head
  // XCD-aware: the nti workgroups of a head share blockIdx.x % 8, so that
  // one L2 holds the head's z rows, which every one of them reads
  const int xcd = blockIdx.x & 7, j = blockIdx.x >> 3;
  const int h = xcd + 8 * (j / nti);
  if (h >= H) return;  // padding of the grid to whole groups of 8 heads (no barrier yet)
  const int i0 = (j - (j / nti) * nti) * 16;
  const int i = i0 + s;                  // this lane's row of the A operand
  const int nk = M / 32, nch = (M + CH - 1) / CH;
  const float* Wr = W + ((size_t)h * M + (i < M ? i : 0)) * M;
  // The work is a sequence of (slice, chunk) pairs: slices h, h + H, ...,
  // chunks of CH key blocks.  The z rows and W pieces of the next pair are
  // requested as soon as the current pair is staged, so that they arrive
  // while it is multiplied.
  u32x4_t zr[ZCH];
  f32x4_t w0, w1;
  auto fetch = [&](long sl, int c0) {
    const bf16_t* Zs = S + (size_t)sl * M * EP + DP * DP;
#pragma unroll
    for (int u = 0; u < ZCH; ++u) {
      const int pc = tid + 256 * u;
      const int r = pc / (DP / 8), f = pc - (pc / (DP / 8)) * (DP / 8);
      zr[u] = c0 + r < M ? *reinterpret_cast<const u32x4_t*>(Zs + (size_t)(c0 + r) * EP + 8 * f)
                         : u32x4_t{0u, 0u, 0u, 0u};
    }
    const int b = c0 + 32 * wave + 8 * grp;  // A: row i, key blocks b .. b+7
    w0 = w1 = zero4();
    if (c0 / 32 + wave < nk && i < M) {
      w0 = *reinterpret_cast<const f32x4_t*>(Wr + b);
      w1 = *reinterpret_cast<const f32x4_t*>(Wr + b + 4);
    }
  };
  f32x4_t acc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) acc[t] = zero4();
  long slice = h;
  int c = 0;
  fetch(slice, 0);
  for (;;) {
    const int c0 = c * CH;
    const int k = c0 / 32 + wave;        // this wave's step of the chunk
    const int b = 32 * k + 8 * grp;
    lds_barrier();  // the previous chunk's reads of sz are done
#pragma unroll
    for (int u = 0; u < ZCH; ++u) {
      const int pc = tid + 256 * u;
      const int r = pc / (DP / 8), f = pc - (pc / (DP / 8)) * (DP / 8);
      *reinterpret_cast<u32x4_t*>(sz + r * ZR + 8 * f) = zr[u];
    }
    f32x4_t v0 = w0, v1 = w1;
    if constexpr (MODE == kMixCausal) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (b + q >= i) v0[q] = 0.0f;
        if (b + 4 + q >= i) v1[q] = 0.0f;
      }
    }
    const u32x4_t a32 = {pack2(v0[0], v0[1]), pack2(v0[2], v0[3]), pack2(v1[0], v1[1]),
                         pack2(v1[2], v1[3])};
    // the coefficient tiles are written once, with the head's first slice
    if (slice == h && k < nk) *reinterpret_cast<u32x4_t*>(Wc + coef_tiled(M, h, i, b)) = a32;
    lds_barrier();
    long slice2 = slice;
    int c2 = c + 1;
    if (c2 == nch) {
      c2 = 0;
      slice2 += H;
    }
    if (slice2 < nslices) fetch(slice2, c2 * CH);
    if (k < nk) {
      const u16x8_t a = __builtin_bit_cast(u16x8_t, a32);
#pragma unroll
      for (int t = 0; t < NT; ++t)
        acc[t] = mfma_bf16(a, lds_tr8(sz, ZR, 32 * wave, 16 * t, lane), acc[t]);
    }
    if (c + 1 == nch) {
      // acc[t] lane (s, grp) element r = z~[i0 + 4grp + r][16t + s] (partial)
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) sacc[wave][4 * grp + r][16 * t + s] = acc[t][r];
      lds_barrier();
      for (int e = tid; e < 16 * DP / 2; e += 256) {
        const int row = e / (DP / 2), cc = 2 * (e - row * (DP / 2));
        if (i0 + row < M) {
          float x0 = 0.0f, x1 = 0.0f;
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            x0 += sacc[w][row][cc];
            x1 += sacc[w][row][cc + 1];
          }
          *reinterpret_cast<uint32_t*>(St + ((size_t)slice * M + i0 + row) * EP + DP * DP + cc) =
              pack2(x0, x1);
        }
      }
      lds_barrier();  // sacc is rewritten by the next slice
#pragma unroll
      for (int t = 0; t < NT; ++t) acc[t] = zero4();
    }
    if (slice2 >= nslices) break;
    slice = slice2;
    c = c2;
  }
}

// Mixing for 16 < M <= 32 (MP = 32, M padded): the contraction is a single
// 32-block step, so a workgroup that takes a single 128-entry tile spends its
// life waiting for one load.  Here a workgroup (4 waves) loads the
// head's coefficients into LDS once (bf16, the mode applied, zero past M) and
// then streams kStreamTiles consecutive 128-entry tiles of one slice: the S
// tile of tile t + 1 is loaded into registers while tile t is multiplied.
// Wave w owns entries 32w .. 32w+31 of a tile for all MP query blocks.
// grid = xslices * ceil(nE / kStreamTiles), XCD-aware like k_mix_mfma.
// Same-box A/B against k_mix_mfma: the LM shape (M = 32) 127.5 against
// 129.8 us per step; with MP = 64 the 4096-token image shape (M = 64) was
// 2.6% slower, so k_mix_mfma keeps M > 32.
constexpr int kStreamTiles = 3;

template <int EP, int MODE, int MP>
__global__ __launch_bounds__(kBlkThreads) void k_mix_stream(const bf16_t* __restrict__ S,
                                                            const float* __restrict__ W,
                                                            bf16_t* __restrict__ St, int M,
                                                            int H, long nslices) {
  constexpr int TE = 128, KS = MP / 32, BT = MP / 16, AT = 2;
  constexpr int SRS = TE + 8;          // S tile row stride (rows = key blocks)
  constexpr int WRS = MP + 16;         // coefficient row stride (rows = query blocks)
  constexpr int SCH = MP * TE / 8 / kBlkThreads;  // 16-byte S chunks per thread per tile
  constexpr int nE = EP / TE;
  constexpr int NG = (nE + kStreamTiles - 1) / kStreamTiles;  // tile groups per slice
  __shared__ __attribute__((aligned(16))) bf16_t sS[2][MP * SRS];
  __shared__ __attribute__((aligned(16))) bf16_t sW[MP * WRS];
  __shared__ __attribute__((aligned(16))) bf16_t stage_all[kBlkWaves * 16 * (16 * AT + 8)];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  bf16_t* stage = stage_all + wave * 16 * (16 * AT + 8);
  const int s = lane & 15, grp = lane >> 4;
  const int xcd = blockIdx.x & 7, j = blockIdx.x >> 3;
  const long slice = (long)(j / NG) * 8 + xcd;
  if (slice >= nslices) return;  // before any barrier
  const int t0 = (j - (j / NG) * NG) * kStreamTiles;
  const int nt = min(kStreamTiles, nE - t0);
  const int h = (int)(slice % H);
  const bf16_t* Ss = S + (size_t)slice * M * EP;
  const float* Wh = W + (size_t)h * M * M;

  // coefficients coef(i, b) as bf16, [i][b]; zero for i, b >= M.  All of a
  // thread's W loads are issued first, then the first S tile's (sload(0)
  // below), so that the coefficient wait does not cover the tile.
  constexpr int WPT = MP * MP / kBlkThreads;  // coefficients per thread
  static_assert(WPT * kBlkThreads == MP * MP, "coefficients per thread");
  // (loads unconditional at clamped indices; the mode's zeros are applied
  // when the coefficients are written)
  float wv[WPT];
#pragma unroll
  for (int q = 0; q < WPT; ++q) {
    const int e = tid + q * kBlkThreads;
    const int i = min(e / MP, M - 1), b = min(e - (e / MP) * MP, M - 1);
    if constexpr (MODE == kMixTransposed) wv[q] = Wh[(size_t)b * M + i];
    else wv[q] = Wh[(size_t)i * M + b];
  }
  // S chunk u of a tile: key-block row r (clamped in bounds; its coefficients
  // are zero past M), 16-byte piece f
  u32x4_t sr[SCH];
  auto sload = [&](int t) {
    const int e0 = (t0 + min(t, nt - 1)) * TE;
#pragma unroll
    for (int u = 0; u < SCH; ++u) {
      const int c = tid + kBlkThreads * u;
      const int r = c / (TE / 8), f = c % (TE / 8);
      sr[u] = *reinterpret_cast<const u32x4_t*>(Ss + (size_t)min(r, M - 1) * EP + e0 + 8 * f);
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int u = 0; u < SCH; ++u) {
      const int c = tid + kBlkThreads * u;
      const int r = c / (TE / 8), f = c % (TE / 8);
      *reinterpret_cast<u32x4_t*>(sS[buf] + r * SRS + 8 * f) = sr[u];
    }
  };
  sload(0);
#pragma unroll
  for (int q = 0; q < WPT; ++q) {
    const int e = tid + q * kBlkThreads;
    const int i = e / MP, b = e - (e / MP) * MP;
    const bool keep = i < M && b < M && (MODE != kMixCausal || b < i);
    sW[i * WRS + b] = f32_to_bf16(keep ? wv[q] : 0.0f);
  }
  lstore(0);
  lds_barrier();
  for (int t = 0; t < nt; ++t) {
    const int buf = t & 1;
    sload(t + 1);  // clamped: the last tile repeats, harmlessly
    // A = S^T (rows e, contraction b via transpose reads), B = coef^T (column
    // i, b contiguous in the [i][b] tile)
    f32x4_t acc[AT][BT];
#pragma unroll
    for (int a = 0; a < AT; ++a)
#pragma unroll
      for (int c = 0; c < BT; ++c) acc[a][c] = zero4();
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u16x8_t af[AT], bw[BT];
#pragma unroll
      for (int a = 0; a < AT; ++a) af[a] = lds_tr8(sS[buf], SRS, 32 * ks, 32 * wave + 16 * a, lane);
#pragma unroll
      for (int c = 0; c < BT; ++c)
        bw[c] = *reinterpret_cast<const u16x8_t*>(sW + (16 * c + s) * WRS + 32 * ks + 8 * grp);
#pragma unroll
      for (int a = 0; a < AT; ++a)
#pragma unroll
        for (int c = 0; c < BT; ++c) acc[a][c] = mfma_bf16(af[a], bw[c], acc[a][c]);
    }
    // acc[a][c] lane (s, grp) element r = S~[i = 16c + s][e = 32 wave + 16a + 4grp + r];
    // stored through the wave's LDS staging area, so that each store
    // instruction writes whole 64-byte row pieces with consecutive lanes on
    // consecutive bytes
    const int e0 = (t0 + t) * TE + 32 * wave;
#pragma unroll
    for (int c = 0; c < BT; ++c) {
      const int i = 16 * c + s;
      f32x4_t tt[AT];
#pragma unroll
      for (int a = 0; a < AT; ++a) tt[a] = acc[a][c];
      store_rows_staged<AT, false>(i < M ? St + ((size_t)slice * M + i) * EP + e0 : nullptr,
                                   stage, tt, 1.0f, lane);
    }
    lstore(buf ^ 1);
    lds_barrier();
  }
}

// The transposed coefficients coef(i, b) = W[h][b][i] (the backward's dS
// mixing), through a 32 x 32 LDS tile so that both the fp32 reads and the bf16
// writes are coalesced rows (reading W down its columns took 36 us on the
// video shape, against 8.5 us for the plain conversion).  grid =
// H * (MI/32) * (M/32) (head-major; MI = M rounded up to 256, the tiles past
// M write the zero padding rows), block = 256; M % 32 == 0.
__global__ __launch_bounds__(256) void k_mix_coef_t(const float* __restrict__ W,
                                                    bf16_t* __restrict__ Wc, int M) {
  __shared__ float tile[32][33];
  const int nti = (M + 255) / 256 * 8, ntb = M / 32;
  const int h = blockIdx.x / (nti * ntb), rem = blockIdx.x - h * nti * ntb;
  const int b0 = 32 * (rem / nti), i0 = 32 * (rem % nti);
  const int t = threadIdx.x, r = t >> 3, c4 = 4 * (t & 7);
  if (i0 < M) {  // uniform: read row b0 + r of W, columns i0 + c4 .. + 3
    const f32x4_t v =
        *reinterpret_cast<const f32x4_t*>(W + ((size_t)h * M + b0 + r) * M + i0 + c4);
#pragma unroll
    for (int q = 0; q < 4; ++q) tile[r][c4 + q] = v[q];
  } else {
#pragma unroll
    for (int q = 0; q < 4; ++q) tile[r][c4 + q] = 0.0f;
  }
  __syncthreads();
  // coefficient row i0 + r, columns b0 + c4 .. + 3: tile[c4 + q][r]
  *reinterpret_cast<uint2*>(Wc + coef_tiled(M, h, i0 + r, b0 + c4)) =
      make_uint2(pack2(tile[c4][r], tile[c4 + 1][r]), pack2(tile[c4 + 2][r], tile[c4 + 3][r]));
}

// The pipelined main loop of k_mix_big.  The three stages are separate
// restrict-qualified arrays so that the compiler's wait insertion can tell
// a stage being read from the stages whose loads are still in flight.
template <int EP>
__device__ __forceinline__ void mix_big_loop(bf16_t* __restrict__ ring0, bf16_t* __restrict__ ring1,
                                             bf16_t* __restrict__ ring2,
                                             const bf16_t* __restrict__ Ss,
                                             const bf16_t* __restrict__ Wt, int nk, int e0,
                                             int wave, int lane, f32x4_t (&acc)[4][8]) {
  constexpr int TI = 256, TE = 128, KB = 32, EW = TE / 2, AT = EW / 16;
  constexpr int SST = KB * TE;
  const int s = lane & 15, grp = lane >> 4;
  const int we = wave & 1, wi = wave >> 1;
  static_assert(TI * KB == 8192, "coefficient tile");
  // Step k's tiles into stage `st`: wave w moves S rows 8w .. 8w+7 (two
  // 1 KB loads of four rows) and W rows 64w .. 64w+63 (four loads of 16
  // rows); lane L's 16 bytes land at slot L of the load's 1 KB.  Six loads
  // per thread per step.
  auto issue = [&](bf16_t* st, int k) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int r = 8 * wave + 4 * u + (lane >> 4);
      const int f = ((lane & 15) - r) & 15;
      __builtin_amdgcn_global_load_lds(
          (const void*)(Ss + (size_t)(k * KB + r) * EP + e0 + 8 * f),
          (__attribute__((address_space(3))) void*)(st + (8 * wave + 4 * u) * TE), 16, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = 64 * wave + 16 * u + (lane >> 2);
      const int f = (lane & 3) ^ ((i >> 1) & 3);
      __builtin_amdgcn_global_load_lds(
          (const void*)(Wt + (size_t)k * 8192 + i * KB + 8 * f),
          (__attribute__((address_space(3))) void*)(st + SST + (64 * wave + 16 * u) * KB), 16, 0,
          0);
    }
  };
  // A = S^T (rows e, contraction b via transpose reads), B = W^T (column i,
  // the same b: W[i][8grp .. 8grp+7] is one chunk)
  auto compute = [&](const bf16_t* st) {
    const bf16_t* sS = st;
    const bf16_t* sW = st + SST;
    u16x8_t bw[8];
#pragma unroll
    for (int c = 0; c < 8; ++c)
      bw[c] = *reinterpret_cast<const u16x8_t*>(sW + (128 * wi + 16 * c + s) * KB +
                                                8 * (grp ^ ((s >> 1) & 3)));
    // lane (s, grp) of a transpose read supplies row 8grp + s/4 (+4 for the
    // second read), entries c0 + 4 (s % 4) .. + 3: chunk c0 / 8 + (s % 4) / 2
    const int r_lo = 8 * grp + (s >> 2), half = 4 * (s & 1);
#pragma unroll
    for (int a = 0; a < AT; ++a) {
      const int f = (EW * we + 16 * a) / 8 + ((s & 3) >> 1);
      const i16x4_t lo = lds_tr4(sS + r_lo * TE + 8 * ((f + r_lo) & 15) + half);
      const i16x4_t hi = lds_tr4(sS + (r_lo + 4) * TE + 8 * ((f + r_lo + 4) & 15) + half);
      const u16x8_t af =
          __builtin_bit_cast(u16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
      for (int c = 0; c < 8; ++c) acc[a][c] = mfma_bf16(af, bw[c], acc[a][c]);
    }
  };
  // Step k: wait for this thread's loads of step k (the six of step k + 1
  // may still be in flight), barrier (every wave's step-k tiles are in LDS
  // and every wave is done reading step k - 1's stage), refill that stage
  // with step k + 2 (past the end: the last step again, into a stage no one
  // reads), multiply.  Every step issues six loads, so the wait is always
  // vmcnt(6).  The barrier is a plain s_barrier after explicit counter
  // waits: a workgroup fence would also wait for step k + 1's loads.
  auto step = [&](bf16_t* cur, bf16_t* next2, int k) {
    __builtin_amdgcn_s_waitcnt(0x0076);  // vmcnt(6) lgkmcnt(0)
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    issue(next2, k + 2 < nk ? k + 2 : nk - 1);
    compute(cur);
  };
  // stage of step k: k % 3; the main loop is unrolled by three so that
  // every stage is a fixed array and the body has no branches
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

template <int EP, int MODE, int NE = EP / 128>
__global__ __launch_bounds__(256, 2) void k_mix_big(const bf16_t* __restrict__ S,
                                                    const bf16_t* __restrict__ Wc,
                                                    bf16_t* __restrict__ St, int M, int H,
                                                    long nslices) {
  constexpr int TI = 256, TE = 128, KB = 32;
  constexpr int EW = TE / 2, AT = EW / 16;  // entries and A tiles per wave
  constexpr int nE = NE;                    // entry tiles computed (the first NE of the row)
  static_assert(EP % TE == 0 && NE * TE <= EP, "tiles");
  // One stage of the ring: the S tile (KB key blocks x TE entries, rows of
  // 256 bytes) and the W tile (TI query blocks x KB coefficients, rows of 64
  // bytes), both unpadded.  The global-to-LDS loads write 64 lanes x 16
  // bytes contiguously, so the bank spreading is a permutation of the
  // 16-byte chunks within a row, chosen by the lane that loads them:
  //   S row r: chunk f at slot (f + r) % 16  (the transpose reads of 4
  //            consecutive rows then fall on distinct banks, as with a
  //            16-byte row pad);
  //   W row i: chunk f at slot f ^ ((i >> 1) & 3)  (the fragment reads of 16
  //            consecutive rows, one chunk each, spread over all banks).
  constexpr int SST = KB * TE, WST = TI * KB, STAGE = SST + WST;  // elements
  __shared__ __attribute__((aligned(16))) bf16_t ring0[STAGE];
  __shared__ __attribute__((aligned(16))) bf16_t ring1[STAGE];
  __shared__ __attribute__((aligned(16))) bf16_t ring2[STAGE];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int s = lane & 15, grp = lane >> 4;
  const int we = wave & 1, wi = wave >> 1;
  const int nI = (M + TI - 1) / TI;
  const int per = nE * nI;
  const int xcd = blockIdx.x & 7, j = blockIdx.x >> 3;
  const long slice = (long)(j / per) * 8 + xcd;
  if (slice >= nslices) return;  // before any barrier
  const int rem = j - (j / per) * per;
  const int e0 = (rem / nI) * TE, i0 = (rem - (rem / nI) * nI) * TI;
  const int h = (int)(slice % H);
  const bf16_t* Ss = S + (size_t)slice * M * EP;
  // this tile's coefficients: contiguous 256 x 32 tiles, one per step
  const bf16_t* Wt = Wc + coef_tiled(M, h, i0, 0);
  int nk = M / KB;
  if constexpr (MODE == kMixCausal) {
    // coefficients vanish for b >= i: stop below the tile's last row
    const int last = i0 + TI - 1 < M - 1 ? i0 + TI - 1 : M - 1;
    const int need = (last + KB - 1) / KB;
    nk = need < nk ? need : nk;
    nk = nk > 0 ? nk : 1;
  }

  f32x4_t acc[AT][8];
#pragma unroll
  for (int a = 0; a < AT; ++a)
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[a][c] = zero4();

  mix_big_loop<EP>(ring0, ring1, ring2, Ss, Wt, nk, e0, wave, lane, acc);
  // acc[a][c] lane (s, grp) element r = S~[i = 16c + s][e = 16a + 4grp + r]:
  // consecutive lanes hold different rows.  The stores go through LDS, 16
  // rows at a time in a wave-private 16 x 72 area of the (now idle) ring:
  // v_permlane16_swap pairs lane groups g, g ^ 1 so that each lane holds 8
  // consecutive entries of its row (at column b(g) = 0, 16, 8, 24 for
  // g = 0..3, and + 32 from the second tile pair), the lane writes them, and
  // reads back 8 entries of row L / 8 (and L / 8 + 8) at column 8 (L % 8).
  // Each store instruction then writes eight whole 128-byte rows (this
  // wave's 64 entries of a row: one aligned line, as EP is a multiple of 64)
  // with consecutive lanes on consecutive bytes; storing straight from the
  // accumulators (each lane 16 bytes of a different row) took 5 us longer
  // on the video shape.
  __syncthreads();  // every wave is done reading the ring
  constexpr int RS = 72;  // staging row stride (elements)
  static_assert(4 * 16 * RS <= STAGE, "staging fits a stage");
  bf16_t* sw = ring0 + wave * 16 * RS;
  const int bcol = (grp & 1) ? 12 + 4 * grp : 4 * grp;
  const int rr = lane >> 3, ch = lane & 7;
  bf16_t* ob = St + ((size_t)slice * M + i0 + 128 * wi + rr) * EP + e0 + EW * we + 8 * ch;
#pragma unroll
  for (int c = 0; c < 8; ++c) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const f32x4_t& x = acc[2 * j][c];
      const f32x4_t& y = acc[2 * j + 1][c];
      const auto p0 =
          __builtin_amdgcn_permlane16_swap(pack2(x[0], x[1]), pack2(y[0], y[1]), false, false);
      const auto p1 =
          __builtin_amdgcn_permlane16_swap(pack2(x[2], x[3]), pack2(y[2], y[3]), false, false);
      *reinterpret_cast<u32x4_t*>(sw + s * RS + bcol + 32 * j) = u32x4_t{p0[0], p1[0], p0[1], p1[1]};
    }
    __builtin_amdgcn_wave_barrier();  // LDS operations of one wave run in order
    const u32x4_t v0 = *reinterpret_cast<const u32x4_t*>(sw + rr * RS + 8 * ch);
    const u32x4_t v1 = *reinterpret_cast<const u32x4_t*>(sw + (rr + 8) * RS + 8 * ch);
    __builtin_amdgcn_wave_barrier();
    const int ib = i0 + 128 * wi + 16 * c + rr;
    if (ib < M) *reinterpret_cast<u32x4_t*>(ob + (size_t)(16 * c) * EP) = v0;
    if (ib + 8 < M) *reinterpret_cast<u32x4_t*>(ob + (size_t)(16 * c + 8) * EP) = v1;
  }
}

// ---------------------------------------------------------------------------
// The precise large-M mixing (the backward's fp32 S~ for dQ): St = W S with
// W = hi + lo split into two bf16 coefficient sets, both in the tiled layout
// of coef_tiled (lo at Wc + lo_off), fp32 accumulation and fp32 output, over
// all EP entries of a row (the z column included).  k_mix_coef2 writes the two
// sets; k_mix_big_f32 is k_mix_big's ring with a 128 x 128 workgroup tile
// (wave (we, wi): 64 entries x 64 query blocks, each fragment pair feeding
// one MFMA per coefficient part), so that a stage (S tile, hi tile, lo tile:
// 24 KB) matches the plain kernel's and two workgroups share a CU.

// W -> hi = bf16(w), lo = bf16(w - hi), tiled; rows past M are zero.  grid =
// H * MI * M / 1024 (MI = M rounded up to 256), block = 256: one thread per
// four consecutive key blocks of one row.
__global__ __launch_bounds__(256) void k_mix_coef2(const float* __restrict__ W,
                                                   bf16_t* __restrict__ Wc, long lo_off, int M) {
  const int MI = (M + 255) / 256 * 256;
  const long t = (long)blockIdx.x * 256 + threadIdx.x;
  const int mq = M / 4;
  const long row = t / mq;  // h * MI + i
  const int b = 4 * (int)(t - row * mq);
  const int h = (int)(row / MI), i = (int)(row - (long)h * MI);
  f32x4_t w = zero4();
  if (i < M) w = *reinterpret_cast<const f32x4_t*>(W + ((size_t)h * M + i) * M + b);
  const uint2 hi = make_uint2(pack2(w[0], w[1]), pack2(w[2], w[3]));
  const uint2 lo = make_uint2(pack2(w[0] - lo_f32(hi.x), w[1] - hi_f32(hi.x)),
                              pack2(w[2] - lo_f32(hi.y), w[3] - hi_f32(hi.y)));
  const size_t o = coef_tiled(M, h, i, b);
  *reinterpret_cast<uint2*>(Wc + o) = hi;
  *reinterpret_cast<uint2*>(Wc + lo_off + o) = lo;
}

template <int EP>
__device__ __forceinline__ void mix_big_f32_loop(bf16_t* __restrict__ ring0,
                                                 bf16_t* __restrict__ ring1,
                                                 bf16_t* __restrict__ ring2,
                                                 const bf16_t* __restrict__ Ss,
                                                 const bf16_t* __restrict__ Wh,
                                                 const bf16_t* __restrict__ Wl, int nk, int e0,
                                                 int wave, int lane, f32x4_t (&acc)[4][4]) {
  constexpr int TI = 128, TE = 128, KB = 32, EW = 64, IW = 64, AT = 4, CT = 4;
  constexpr int SST = KB * TE, WST = TI * KB;  // elements of the S tile and of one W tile
  const int s = lane & 15, grp = lane >> 4;
  const int we = wave & 1, wi = wave >> 1;
  // Step k's tiles into stage `st` (S rows 8w .. 8w+7, hi and lo rows
  // 32w .. 32w+31; lane L's 16 bytes land at slot L of each 1 KB load, with
  // the chunk permutations of k_mix_big).  Six loads per thread per step.
  auto issue = [&](bf16_t* st, int k) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int r = 8 * wave + 4 * u + (lane >> 4);
      const int f = ((lane & 15) - r) & 15;
      __builtin_amdgcn_global_load_lds(
          (const void*)(Ss + (size_t)(k * KB + r) * EP + e0 + 8 * f),
          (__attribute__((address_space(3))) void*)(st + (8 * wave + 4 * u) * TE), 16, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int i = 32 * wave + 16 * u + (lane >> 2);
      const int f = (lane & 3) ^ ((i >> 1) & 3);
      const size_t src = (size_t)k * 8192 + i * KB + 8 * f;
      bf16_t* dst = st + SST + (32 * wave + 16 * u) * KB;
      __builtin_amdgcn_global_load_lds((const void*)(Wh + src),
                                       (__attribute__((address_space(3))) void*)dst, 16, 0, 0);
      __builtin_amdgcn_global_load_lds((const void*)(Wl + src),
                                       (__attribute__((address_space(3))) void*)(dst + WST), 16,
                                       0, 0);
    }
  };
  auto compute = [&](const bf16_t* st) {
    const bf16_t* sS = st;
    const bf16_t* sH = st + SST;
    const bf16_t* sL = st + SST + WST;
    u16x8_t bh[CT], bl[CT];
#pragma unroll
    for (int c = 0; c < CT; ++c) {
      const int o = (IW * wi + 16 * c + s) * KB + 8 * (grp ^ ((s >> 1) & 3));
      bh[c] = *reinterpret_cast<const u16x8_t*>(sH + o);
      bl[c] = *reinterpret_cast<const u16x8_t*>(sL + o);
    }
    const int r_lo = 8 * grp + (s >> 2), half = 4 * (s & 1);
#pragma unroll
    for (int a = 0; a < AT; ++a) {
      const int f = (EW * we + 16 * a) / 8 + ((s & 3) >> 1);
      const i16x4_t lo = lds_tr4(sS + r_lo * TE + 8 * ((f + r_lo) & 15) + half);
      const i16x4_t hi = lds_tr4(sS + (r_lo + 4) * TE + 8 * ((f + r_lo + 4) & 15) + half);
      const u16x8_t af =
          __builtin_bit_cast(u16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
      for (int c = 0; c < CT; ++c) acc[a][c] = mfma_bf16(af, bh[c], acc[a][c]);
#pragma unroll
      for (int c = 0; c < CT; ++c) acc[a][c] = mfma_bf16(af, bl[c], acc[a][c]);
    }
  };
  // the step and ring of mix_big_loop
  auto step = [&](bf16_t* cur, bf16_t* next2, int k) {
    __builtin_amdgcn_s_waitcnt(0x0076);  // vmcnt(6) lgkmcnt(0)
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    issue(next2, k + 2 < nk ? k + 2 : nk - 1);
    compute(cur);
  };
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

// grid = 8 * ceil(slices / 8) * (EP / 128) * ceil(M / 128), XCD-aware like
// k_mix_big; block = 256; M >= kMixBigM, M % 32 == 0.
template <int EP>
__global__ __launch_bounds__(256, 2) void k_mix_big_f32(const bf16_t* __restrict__ S,
                                                        const bf16_t* __restrict__ Wc, long lo_off,
                                                        float* __restrict__ St, int M, int H,
                                                        long nslices) {
  constexpr int TI = 128, TE = 128, KB = 32;
  constexpr int STAGE = KB * TE + 2 * TI * KB;  // elements: S, hi, lo tiles (24 KB)
  __shared__ __attribute__((aligned(16))) bf16_t ring0[STAGE];
  __shared__ __attribute__((aligned(16))) bf16_t ring1[STAGE];
  __shared__ __attribute__((aligned(16))) bf16_t ring2[STAGE];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int s = lane & 15, grp = lane >> 4;
  const int we = wave & 1, wi = wave >> 1;
  const int nE = EP / TE, nI = (M + TI - 1) / TI;
  const int per = nE * nI;
  const int xcd = blockIdx.x & 7, j = blockIdx.x >> 3;
  const long slice = (long)(j / per) * 8 + xcd;
  if (slice >= nslices) return;  // before any barrier
  const int rem = j - (j / per) * per;
  const int e0 = (rem / nI) * TE, i0 = (rem - (rem / nI) * nI) * TI;
  const int h = (int)(slice % H);
  const bf16_t* Ss = S + (size_t)slice * M * EP;
  // rows i0 .. i0+127 are one contiguous half of a 256-row coefficient tile
  const bf16_t* Wh = Wc + coef_tiled(M, h, i0, 0);
  f32x4_t acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[a][c] = zero4();
  mix_big_f32_loop<EP>(ring0, ring1, ring2, Ss, Wh, Wh + lo_off, M / KB, e0, wave, lane, acc);
  // acc[a][c] lane (s, grp) element r = S~[i0 + 64wi + 16c + s][e0 + 64we + 16a + 4grp + r]:
  // consecutive lanes hold different rows.  As in k_mix_big, the stores go
  // through LDS, 16 rows at a time in a wave-private 16 x 68 fp32 area of the
  // (now idle) ring, and are read back as 16 bytes of row 4h + L / 16 at
  // column 4 (L % 16): each store instruction writes four whole 256-byte rows
  // (this wave's 64 entries) with consecutive lanes on consecutive bytes.
  __syncthreads();  // every wave is done reading the ring
  constexpr int RS = 68;  // staging row stride (floats)
  static_assert(4 * 16 * RS * 4 <= STAGE * 2, "staging fits a stage");
  float* sw = reinterpret_cast<float*>(ring0) + wave * 16 * RS;
  const int rq = lane >> 4, cq = 4 * (lane & 15);
  float* ob = St + ((size_t)slice * M + i0 + 64 * wi + rq) * EP + e0 + 64 * we + cq;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
#pragma unroll
    for (int a = 0; a < 4; ++a)
      *reinterpret_cast<f32x4_t*>(sw + s * RS + 16 * a + 4 * grp) = acc[a][c];
    __builtin_amdgcn_wave_barrier();  // LDS operations of one wave run in order
    f32x4_t v[4];
#pragma unroll
    for (int hq = 0; hq < 4; ++hq)
      v[hq] = *reinterpret_cast<const f32x4_t*>(sw + (4 * hq + rq) * RS + cq);
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int hq = 0; hq < 4; ++hq)
      if (i0 + 64 * wi + 16 * c + 4 * hq + rq < M)
        *reinterpret_cast<f32x4_t*>(ob + (size_t)(16 * c + 4 * hq) * EP) = v[hq];
  }
}

// ---------------------------------------------------------------------------
// Readout.  grid = (ceil(M / 4), slices), block = 256; wave w reads out query
// block 4*blockIdx.x + w, 16 queries per step.  Y^T = S~_i^T phi(Q)^T with the
// contraction split as features 32ks + 8grp .. +7 on both operands; the z~
// row (row 0 of one more A tile) gives phi(q).z~_i.  STREAM = true reads Q
// and writes Y with the nontemporal hint (see blocked_stream).
template <int DP, int PHI, bool STREAM = false>
__global__ __launch_bounds__(kBlkThreads) void k_readout_mfma(
    const bf16_t* __restrict__ Q, const bf16_t* __restrict__ St, bf16_t* __restrict__ Y, Geo g,
    int N, int d) {
  using D = BlockedDims<DP>;
  constexpr int NT = D::NT, DS = D::DS, EP = D::EP;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int s = lane & 15, grp = lane >> 4;
  const long slice = blockIdx.y;
  const int i = blockIdx.x * kBlkWaves + wave;
  if (i >= g.M) return;  // this kernel has no barrier
  const size_t off = (size_t)slice * N * d;
  const bf16_t* row = St + ((size_t)slice * g.M + i) * EP;
  u16x8_t af[NT][DS], az[DS];
#pragma unroll
  for (int ct = 0; ct < NT; ++ct)
#pragma unroll
    for (int ks = 0; ks < DS; ++ks)
      af[ct][ks] = *reinterpret_cast<const u16x8_t*>(row + (16 * ct + s) * DP + 32 * ks + 8 * grp);
#pragma unroll
  for (int ks = 0; ks < DS; ++ks)
    az[ks] = s == 0 ? *reinterpret_cast<const u16x8_t*>(row + DP * DP + 32 * ks + 8 * grp)
                    : u16x8_t{0, 0, 0, 0, 0, 0, 0, 0};
  const int bb = g.blockbase(i);
  // rows of 128 or 64 bytes (d == DP = 64 or 32) are stored whole, through a
  // per-wave LDS staging area
  constexpr bool STAGED = DP == 64 || DP == 32;
  __shared__ __attribute__((aligned(16))) bf16_t stage_all[STAGED ? kBlkWaves * 16 * (DP + 8) : 1];
  bf16_t* stage = stage_all + wave * 16 * (DP + 8);
  const bool whole_rows = STAGED && d == DP;
  // Query tiles of 16, loaded QP tiles at a time before any of them is used,
  // so that their transfers overlap.
  constexpr int QP = 4;
  for (int q0 = 0; q0 < g.nb; q0 += 16 * QP) {
    int tq[QP];
    u16x8_t bq[QP][DS];
#pragma unroll
    for (int u = 0; u < QP; ++u) {
      const int j = q0 + 16 * u + s;
      tq[u] = j < g.nb ? bb + g.tokoff(j) : -1;
#pragma unroll
      for (int ks = 0; ks < DS; ++ks) {
        const int k0 = 32 * ks + 8 * grp;
        u32x4_t v = u32x4_t{0u, 0u, 0u, 0u};
        if (tq[u] >= 0 && k0 < d)
          v = STREAM ? __builtin_nontemporal_load(
                           reinterpret_cast<const u32x4_t*>(Q + off + (size_t)tq[u] * d + k0))
                     : *reinterpret_cast<const u32x4_t*>(Q + off + (size_t)tq[u] * d + k0);
        bq[u][ks] = __builtin_bit_cast(u16x8_t, v);
      }
    }
#pragma unroll
    for (int u = 0; u < QP; ++u) {
      if (q0 + 16 * u >= g.nb) break;
#pragma unroll
      for (int ks = 0; ks < DS; ++ks)
        bq[u][ks] = __builtin_bit_cast(u16x8_t, phi8<PHI>(__builtin_bit_cast(u32x4_t, bq[u][ks])));
      f32x4_t o[NT], oz = zero4();
#pragma unroll
      for (int ct = 0; ct < NT; ++ct) {
        o[ct] = zero4();
#pragma unroll
        for (int ks = 0; ks < DS; ++ks) o[ct] = mfma_bf16(af[ct][ks], bq[u][ks], o[ct]);
      }
#pragma unroll
      for (int ks = 0; ks < DS; ++ks) oz = mfma_bf16(az[ks], bq[u][ks], oz);
      const float den = __shfl(oz[0], s);
      const float rd = out_scale(g, den);
      bf16_t* yrow = tq[u] >= 0 ? Y + off + (size_t)tq[u] * d : nullptr;
      if constexpr (STAGED) {
        if (whole_rows) {
          store_rows_staged<NT, STREAM>(yrow, stage, o, rd, threadIdx.x & 63);
          continue;
        }
      }
      store_row_tiles<NT, STREAM>(yrow, d, o, rd, grp);
    }
  }
}

// ---------------------------------------------------------------------------
inline size_t blocked_ws_elems(int d);

// Query blocks per mixing workgroup.
inline int mix_ib(int M) { return M <= 64 ? 64 : 128; }

inline bool blocked_supports(int dtype, int d, int M, long slices) {
  if (dtype != 1 || d % 8 != 0 || d > 96 || slices > 65535) return false;
  // the mixing grid is 1-D: keep its thread count below 2^31
  const int ib = mix_ib(M);
  const long n = (slices + 7) / 8 * 8 * (long)(blocked_ws_elems(d) / kMixEB) * ((M + ib - 1) / ib);
  return n * kBlkThreads < (1L << 31);
}

inline size_t blocked_ws_elems(int d) {
  switch (blocked_dp(d)) {
    case 32: return BlockedDims<32>::EP;
    case 64: return BlockedDims<64>::EP;
    default: return BlockedDims<96>::EP;
  }
}

// Bytes of the bf16 coefficient matrix of the large-M mixing (0 where that
// kernel is not used), 256-byte aligned.
inline size_t mix_coef_bytes(int H, int M) {
  if (M < kMixBigM || M % 32 != 0) return 0;
  const size_t mi = (size_t)(M + 255) / 256 * 256;  // query-block rows, zero-padded
  return ((size_t)H * mi * M * sizeof(bf16_t) + 255) / 256 * 256;
}

// Two coefficient sets (hi and lo parts) of the precise large-M mixing.
inline size_t mix_coef2_bytes(int H, int M) { return 2 * mix_coef_bytes(H, M); }

// Workspace: S and S~, [slices][M][EP] bf16 each, then the mixing's bf16
// coefficients (large M only; tiled, see coef_tiled).
inline size_t blocked_workspace(long slices, int H, int M, int d) {
  return 2 * (size_t)slices * M * blocked_ws_elems(d) * sizeof(bf16_t) + mix_coef_bytes(H, M);
}

// One mixing GEMM over all slices: St[slice][i] = sum_b coef(i, b) S[slice][b]
// with the coefficient chosen by mode (kMixPlain, kMixCausal, kMixTransposed).
// ---------------------------------------------------------------------------
// Mixing for small M on the vector ALUs.  With M <= 16 the MFMA tiles of
// k_mix_mfma (64 query blocks, 32 key blocks per step) are at most a quarter
// used, and the mixing is bound by reading S and writing S~ once, not by its
// 2*M^2 flops per entry (measured: 4.4 TB/s at M = 16; at M = 32 the flops
// already make it slower than the MFMA GEMM).  grid = (EP / 512, slices), block = 256: each thread
// owns two adjacent entries of every row, reads them for all M key blocks and
// writes them for all M query blocks; the M x M coefficients (mode applied,
// fp32) sit in LDS and are read as broadcasts.
constexpr int kMixSmallM = 16;

template <int EP, int MODE, int MMAX, typename OutT>
__global__ __launch_bounds__(256) void k_mix_small(const bf16_t* __restrict__ S,
                                                   const float* __restrict__ W,
                                                   OutT* __restrict__ St, int M, int H) {
  __shared__ __attribute__((aligned(16))) float sw[MMAX * MMAX];
  const int tid = threadIdx.x;
  const long slice = blockIdx.y;
  const int h = (int)(slice % H);
  const float* Wh = W + (size_t)h * M * M;
  for (int e = tid; e < M * M; e += 256) {
    const int i = e / M, b = e - (e / M) * M;
    float c = MODE == kMixTransposed ? Wh[(size_t)b * M + i] : Wh[e];
    if (MODE == kMixCausal && b >= i) c = 0.0f;
    sw[i * MMAX + b] = c;
  }
  __syncthreads();
  const int e0 = (blockIdx.x * 256 + tid) * 2;
  if (e0 >= EP) return;  // after the only barrier
  const bf16_t* src = S + (size_t)slice * M * EP + e0;
  float x0[MMAX], x1[MMAX];
#pragma unroll
  for (int b = 0; b < MMAX; ++b) {
    uint32_t u = 0u;
    if (b < M) u = *reinterpret_cast<const uint32_t*>(src + (size_t)b * EP);
    x0[b] = __uint_as_float(u << 16);
    x1[b] = __uint_as_float(u & 0xffff0000u);
  }
  OutT* dst = St + (size_t)slice * M * EP + e0;
#pragma unroll
  for (int i = 0; i < MMAX; ++i) {
    if (i >= M) break;
    float a0 = 0.0f, a1 = 0.0f;
#pragma unroll
    for (int b = 0; b < MMAX; b += 4) {
      // four coefficients per LDS read (a broadcast); entries with b >= M are
      // never set and never used
      const f32x4_t c = *reinterpret_cast<const f32x4_t*>(sw + i * MMAX + b);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if (b + u < M) {
          a0 = fmaf(c[u], x0[b + u], a0);
          a1 = fmaf(c[u], x1[b + u], a1);
        }
      }
    }
    if constexpr (sizeof(OutT) == 4) {
      *reinterpret_cast<float2*>(dst + (size_t)i * EP) = make_float2(a0, a1);
    } else {
      *reinterpret_cast<uint32_t*>(dst + (size_t)i * EP) = pack2(a0, a1);
    }
  }
}

template <int EP, int MODE, typename OutT>
void launch_mix_small(long slices, int H, int M, const bf16_t* S, const float* W, OutT* St,
                      hipStream_t st) {
  const dim3 grid((unsigned)((EP + 511) / 512), (unsigned)slices);
  if (M <= 8)
    k_mix_small<EP, MODE, 8, OutT><<<grid, 256, 0, st>>>(S, W, St, M, H);
  else
    k_mix_small<EP, MODE, kMixSmallM, OutT><<<grid, 256, 0, st>>>(S, W, St, M, H);
  launch_mark(st, "k_mix_small");
}

// wc: mix_coef_bytes(H, M) bytes of scratch for the large-M kernel (which is
// used whenever those bytes are nonzero).
template <int DP, int MODE>
void launch_mix_m(long slices, int H, int M, const bf16_t* S, const float* W, bf16_t* St,
                  bf16_t* wc, hipStream_t st) {
  using D = BlockedDims<DP>;
  if (M <= kMixSmallM) {
    launch_mix_small<D::EP, MODE, bf16_t>(slices, H, M, S, W, St, st);
    return;
  }
  const long xslices = (slices + 7) / 8 * 8;
  if (mix_coef_bytes(H, M) != 0) {
    const int nit = (M + 255) / 256;
    if constexpr (MODE == kMixTransposed) {
      // the backward's transposed mixing: dz_b rides along as the last entry tile
      const long tot = (long)H * nit * 256 * M;
      k_mix_coef_t<<<dim3((unsigned)(tot / 1024)), 256, 0, st>>>(W, wc, M);
      launch_mark(st, "k_mix_coef_t");
      const unsigned nb = (unsigned)(xslices * (D::EP / 128) * nit);
      k_mix_big<D::EP, MODE><<<dim3(nb), 256, 0, st>>>(S, wc, St, M, H, slices);
    } else {
      // coefficients and z~ first; the GEMM then covers the DP*DP entries only
      const unsigned np = (unsigned)((H + 7) / 8 * 8 * nit * 16);
      k_mix_prep<DP, MODE><<<dim3(np), 256, 0, st>>>(W, S, St, wc, M, H, slices);
      launch_mark(st, "k_mix_prep");
      constexpr int NE = DP * DP / 128;
      const unsigned nb = (unsigned)(xslices * NE * nit);
      k_mix_big<D::EP, MODE, NE><<<dim3(nb), 256, 0, st>>>(S, wc, St, M, H, slices);
    }
    launch_mark(st, "k_mix_big");
    return;
  }
  if (M <= 32) {
    constexpr int NG = (D::EP / 128 + kStreamTiles - 1) / kStreamTiles;
    const unsigned n = (unsigned)(xslices * NG);
    k_mix_stream<D::EP, MODE, 32><<<dim3(n), kBlkThreads, 0, st>>>(S, W, St, M, H, slices);
    launch_mark(st, "k_mix_stream");
    return;
  }
  const int ib = mix_ib(M);
  const unsigned n = (unsigned)(xslices * (D::EP / kMixEB) * ((M + ib - 1) / ib));
  constexpr bool kVec = MODE != kMixTransposed;  // with M % 4 == 0
  if (ib == 64 && (M & 3) == 0)
    k_mix_mfma<D::EP, 64, MODE, bf16_t, kVec><<<dim3(n), kBlkThreads, 0, st>>>(S, W, St, M, H,
                                                                               slices);
  else if (ib == 64)
    k_mix_mfma<D::EP, 64, MODE, bf16_t, false><<<dim3(n), kBlkThreads, 0, st>>>(S, W, St, M, H,
                                                                                slices);
  else if ((M & 3) == 0)
    k_mix_mfma<D::EP, 128, MODE, bf16_t, kVec><<<dim3(n), kBlkThreads, 0, st>>>(S, W, St, M, H,
                                                                                slices);
  else
    k_mix_mfma<D::EP, 128, MODE, bf16_t, false><<<dim3(n), kBlkThreads, 0, st>>>(S, W, St, M,
                                                                                 H, slices);
  launch_mark(st, "k_mix_mfma");
}

template <int DP>
void launch_mix(long slices, int H, int M, const bf16_t* S, const float* W, bf16_t* St, int mode,
                bf16_t* wc, hipStream_t st) {
  if (mode == kMixCausal) launch_mix_m<DP, kMixCausal>(slices, H, M, S, W, St, wc, st);
  else if (mode == kMixTransposed) launch_mix_m<DP, kMixTransposed>(slices, H, M, S, W, St, wc, st);
  else launch_mix_m<DP, kMixPlain>(slices, H, M, S, W, St, wc, st);
}

// The precise variant (fp32 S~, coefficients split in two bf16 parts): for
// large M the ring kernel k_mix_big_f32, whose two coefficient sets take
// mix_coef2_bytes(H, M) of scratch at wc; otherwise k_mix_mfma with 64 query
// blocks per workgroup, so that both coefficient tiles fit in LDS.
template <int DP>
void launch_mix_f32(long slices, int H, int M, const bf16_t* S, const float* W, float* St,
                    bf16_t* wc, hipStream_t st) {
  using D = BlockedDims<DP>;
  if (M <= kMixSmallM) {
    launch_mix_small<D::EP, kMixPlain, float>(slices, H, M, S, W, St, st);
    return;
  }
  const long xslices = (slices + 7) / 8 * 8;
  if (mix_coef_bytes(H, M) != 0) {
    // large M: two tiled bf16 coefficient sets in wc (mix_coef2_bytes)
    const long lo_off = (long)(mix_coef_bytes(H, M) / sizeof(bf16_t));
    const int mi = (M + 255) / 256 * 256;
    k_mix_coef2<<<dim3((unsigned)((long)H * mi * M / 1024)), 256, 0, st>>>(W, wc, lo_off, M);
    launch_mark(st, "k_mix_coef2");
    const unsigned nb = (unsigned)(xslices * (D::EP / 128) * ((M + 127) / 128));
    k_mix_big_f32<D::EP><<<dim3(nb), 256, 0, st>>>(S, wc, lo_off, St, M, H, slices);
    launch_mark(st, "k_mix_big_f32");
    return;
  }
  const unsigned n = (unsigned)(xslices * (D::EP / kMixEB) * ((M + 63) / 64));
  if ((M & 3) == 0)
    k_mix_mfma<D::EP, 64, kMixPlain, float, true><<<dim3(n), kBlkThreads, 0, st>>>(S, W, St, M,
                                                                                 H, slices);
  else
    k_mix_mfma<D::EP, 64, kMixPlain, float, false><<<dim3(n), kBlkThreads, 0, st>>>(S, W, St, M,
                                                                                  H, slices);
  launch_mark(st, "k_mix_mfma");
}

// MI355X's last-level cache (the 256 MB Infinity Cache).  When a blocked call
// moves more than this (Q, K, V, Y and the S and S~ workspace), its inputs are
// read with the nontemporal hint so that they do not push the workspace out
// between the kernels that write and read it.  Below it, ordinary loads are
// faster (same-box A/B: the 4096-token image shape, about 200 MB, took 58.9
// instead of 52.8 us with the hint; the video shape, about 600 MB, 197.5
// instead of 212.7 us).
constexpr size_t kLastLevelCacheBytes = (size_t)256 << 20;

template <int DP>
bool blocked_stream(long slices, int N, int d, int M) {
  const size_t io = (size_t)4 * slices * N * d * 2;
  const size_t wsb = (size_t)2 * slices * M * BlockedDims<DP>::EP * 2;
  return io + wsb > kLastLevelCacheBytes;
}

// Summary and mixing launches shared by the plain and the causal readout; with
// causal != 0 the mixing keeps only earlier chunks.  S and S~ sit at the start
// of ws; wc is the mixing's coefficient scratch.  stream selects nontemporal
// K and V loads.  Returns S~.
template <int DP, int PHI>
bf16_t* launch_summary_mix(long slices, int H, int N, int d, const Geo& g, const bf16_t* K,
                           const bf16_t* V, const float* W, bf16_t* ws, bf16_t* wc, int causal,
                           hipStream_t st, bool stream = false) {
  using D = BlockedDims<DP>;
  bf16_t* S = ws;
  bf16_t* St = ws + (size_t)slices * g.M * D::EP;
  const dim3 grid((unsigned)g.M, (unsigned)slices);
  if (stream)
    k_summary_mfma<DP, PHI, true><<<grid, 64 * D::NT, 0, st>>>(K, V, S, g, N, d, nullptr);
  else
    k_summary_mfma<DP, PHI><<<grid, 64 * D::NT, 0, st>>>(K, V, S, g, N, d, nullptr);
  launch_mark(st, "k_summary_mfma");
  launch_mix<DP>(slices, H, g.M, S, W, St, causal ? kMixCausal : kMixPlain, wc, st);
  return St;
}

// The coefficient scratch of the blocked and causal paths: right after S~.
template <int DP>
bf16_t* blocked_coef_scratch(bf16_t* ws, long slices, int M) {
  return ws + 2 * (size_t)slices * M * BlockedDims<DP>::EP;
}

template <int DP, int PHI>
int launch_blocked_t(long slices, int H, int N, int d, const Geo& g, const bf16_t* Q,
                     const bf16_t* K, const bf16_t* V, const float* W, bf16_t* Y, bf16_t* ws,
                     hipStream_t st) {
  const bool stream = blocked_stream<DP>(slices, N, d, g.M);
  const bf16_t* St = launch_summary_mix<DP, PHI>(
      slices, H, N, d, g, K, V, W, ws, blocked_coef_scratch<DP>(ws, slices, g.M), 0, st, stream);
  const dim3 grid((unsigned)((g.M + kBlkWaves - 1) / kBlkWaves), (unsigned)slices);
  if (stream)
    k_readout_mfma<DP, PHI, true><<<grid, kBlkThreads, 0, st>>>(Q, St, Y, g, N, d);
  else
    k_readout_mfma<DP, PHI><<<grid, kBlkThreads, 0, st>>>(Q, St, Y, g, N, d);
  launch_mark(st, "k_readout_mfma");
  return 0;
}

template <int PHI>
int launch_blocked_p(long slices, int H, int N, int d, const Geo& g, const bf16_t* Q,
                     const bf16_t* K, const bf16_t* V, const float* W, bf16_t* Y, bf16_t* ws,
                     hipStream_t st) {
  switch (blocked_dp(d)) {
    case 32: return launch_blocked_t<32, PHI>(slices, H, N, d, g, Q, K, V, W, Y, ws, st);
    case 64: return launch_blocked_t<64, PHI>(slices, H, N, d, g, Q, K, V, W, Y, ws, st);
    default: return launch_blocked_t<96, PHI>(slices, H, N, d, g, Q, K, V, W, Y, ws, st);
  }
}

inline int launch_blocked(long slices, int H, int N, int d, const Geo& g, int phi,
                          const bf16_t* Q, const bf16_t* K, const bf16_t* V, const float* W,
                          bf16_t* Y, bf16_t* ws, hipStream_t st) {
  if (phi == PHI_RELU)
    return launch_blocked_p<PHI_RELU>(slices, H, N, d, g, Q, K, V, W, Y, ws, st);
  return launch_blocked_p<PHI_ELU1>(slices, H, N, d, g, Q, K, V, W, Y, ws, st);
}

}  // namespace mhla
