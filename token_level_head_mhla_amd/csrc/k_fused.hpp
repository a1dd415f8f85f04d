// k_fused.hpp -- single-kernel MHLA forward for small M (bf16 in/out, gfx950).
//
// One workgroup of 8 waves per (batch, head) slice.  The whole forward of
// "MHLA: Restoring Expressivity of Linear Attention via Token-Level
// Multi-Head" §4.1 runs on chip, and HBM sees only Q, K, V, W and Y:
//
//   A. K and V of the slice (contiguous) are read with 16-byte coalesced
//      loads, phi is applied to K in registers (bf16 result) and both are
//      written to LDS in token (raster) order; one extra all-zero row stands
//      in for the padding of short blocks.  Q is loaded in the same burst but
//      only staged after step B, so its transfer overlaps the summaries.
//   B. Work item (ct, ks) = value columns 16ct..16ct+15 and key features
//      32ks..32ks+31.  For every key block b the wave forms the two 16x16
//      tiles of S_b = phi(K_b)^T V_b with v_mfma_f32_16x16x32_bf16.  Both
//      operands are gathered from LDS with transpose reads whose row addresses
//      follow the block's tokens (blocks are tiles of the grid, numbered in
//      raster order of the block grid, Fig. 4b), and the tiles are mixed at
//      once into every query block's S~_i += W[i,b] S_b (fp32 registers, W
//      read through the scalar cache).  Waves with ct = 0 also form
//      z_b = sum phi(K_b) with a ones operand.
//   C. The mixed tiles are packed to bf16 in the A-operand layout of the
//      readout and exchanged through LDS; z~_i = sum_b W[i,b] z_b.
//   D. Work item = 16 queries of one block.  Y^T = S~_i^T phi(Q)^T on MFMA;
//      an extra operand tile whose row 0 is z~_i yields the denominator
//      phi(q).z~_i from the same product; the divide and the bf16 rounding are
//      fused into the 8-byte stores.
//
// A denominator of exactly 0 (ReLU with phi(q) = 0) writes a zero row.
#pragma once

#include "mhla_mfma.hpp"

namespace mhla {

// Waves per workgroup: 16 when M <= 4 (waves 8..15 stage phi(Q) while waves
// 0..7 form the summaries), 8 otherwise (the mixing registers of M = 5..8 need
// the larger per-wave register budget).
__host__ __device__ constexpr int fused_waves(int MM) { return MM <= 4 ? 16 : 8; }
constexpr int kFusedMaxM = 8;
constexpr size_t kLdsLimit = 160 * 1024;

// LDS layout (bytes), N tokens, M blocks:
//   [phi(Q)]   (N+1) rows x RSQ bf16, row N = 0
//   [phi(K) V] 2 x (N+1) rows x RS bf16, row N = 0; RS keeps the transpose
//              reads free of bank conflicts (rows 8 banks apart); after step B
//              the mixed A-operand fragments [M][NT][DS][64 lanes] reuse it
//   [zraw zmix] z_b and z~_i, [M][DP] fp32 each
template <int DP>
struct FusedLayout {
  static constexpr int RSQ = DP + 8;
  static constexpr int RS = DP + 16;
  static constexpr int NT = DP / 16;       // value-column tiles
  static constexpr int DS = DP / 32;       // 32-feature contraction steps
  __host__ __device__ static size_t q_bytes(int N) { return (size_t)(N + 1) * RSQ * 2; }
  __host__ __device__ static size_t kv_bytes(int N, int M) {
    const size_t kv = (size_t)2 * (N + 1) * RS * 2, fr = (size_t)M * NT * DS * 64 * 16;
    return kv > fr ? kv : fr;
  }
  __host__ __device__ static size_t z_off(int N, int M) { return q_bytes(N) + kv_bytes(N, M); }
  // zraw [M][DP], zmix [M][DP], W [M][M] (fp32)
  __host__ __device__ static size_t total(int N, int M) {
    return z_off(N, M) + (size_t)2 * M * DP * 4 + (size_t)M * M * 4;
  }
};

// First token of every block, computed on the host (uniform kernel argument).
struct FusedBases {
  int b[kFusedMaxM];
};

// floor(a / b) for 0 <= a < 2^22 with inv = fl(1/b) (see Geo::tokoff).
__device__ __forceinline__ int small_div(int a, float inv) {
  return (int)(((float)a + 0.5f) * inv);
}

template <int DP, int NBP, int MM, int PHI>
__global__ __launch_bounds__(64 * fused_waves(MM)) void k_fused(
    const bf16_t* __restrict__ Q, const bf16_t* __restrict__ K, const bf16_t* __restrict__ V,
    const float* __restrict__ W, bf16_t* __restrict__ Y, Geo g, FusedBases fb, int H, int N,
    int d) {
  using L = FusedLayout<DP>;
  constexpr int RSQ = L::RSQ, RS = L::RS, NT = L::NT, DS = L::DS;
  constexpr int KS = NBP / 32;  // 32-token contraction steps per block
  constexpr int QT = NBP / 16;  // 16-query tiles per block
  constexpr int NWAVE = fused_waves(MM), NTHR = 64 * NWAVE;
  constexpr int TPW = (MM * QT + NWAVE - 1) / NWAVE;  // max query tiles per wave
  constexpr int QW0 = NWAVE == 16 ? 8 : 0;  // first wave that stages phi(Q)
  constexpr int QTHR = NTHR - 64 * QW0;     // threads that stage phi(Q)
  constexpr int UKV = 2048 / NTHR;          // 16-byte K, V chunks per thread per batch
  constexpr int UQ = 2048 / QTHR;           // 16-byte Q chunks per thread per batch
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int M = g.M, nb = g.nb;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int s = lane & 15, grp = lane >> 4;
  const long slice = blockIdx.x;
  const int h = (int)(slice % H);
  const size_t off = (size_t)slice * N * d;
  const float* Wh = W + (size_t)h * M * M;

  bf16_t* sQ = reinterpret_cast<bf16_t*>(smem);
  bf16_t* sK = reinterpret_cast<bf16_t*>(smem + L::q_bytes(N));
  bf16_t* sV = sK + (size_t)(N + 1) * RS;
  u16x8_t* frag = reinterpret_cast<u16x8_t*>(sK);  // after step B
  float* zraw = reinterpret_cast<float*>(smem + L::z_off(N, M));
  float* zmix = zraw + M * DP;
  float* sW = zmix + M * DP;

  // ---- A. loads: K and V first, then Q; W; stage phi(K) and V -----------------
  const int F8 = d >> 3;
  const int items = N * F8;
  const float inv8 = 1.0f / (float)F8;
  const bool qwave = wave >= QW0;
  const int qtid = tid - QW0 * 64;
  u32x4_t qr[UQ], kr[UKV], vr[UKV];
#define MHLA_LOAD(dst, src_ptr, base, U, stride, id)                                     \
  _Pragma("unroll") for (int u = 0; u < U; ++u) {                                         \
    /* clamped so that every lane loads: straight-line code, all loads in flight */      \
    const size_t o = off + (size_t)min((base) + u * (stride) + (id), items - 1) * 8;     \
    dst[u] = *reinterpret_cast<const u32x4_t*>(src_ptr + o);                              \
  }
  MHLA_LOAD(kr, K, 0, UKV, NTHR, tid)
  MHLA_LOAD(vr, V, 0, UKV, NTHR, tid)
  if (qwave) { MHLA_LOAD(qr, Q, 0, UQ, QTHR, qtid) }
  // W through the scalar cache (uniform), clamped in range and masked to 0
  // for the padding rows / columns i, b >= M.
  float wr[MM][MM];
#pragma unroll
  for (int i = 0; i < MM; ++i)
#pragma unroll
    for (int b = 0; b < MM; ++b) {
      const float w = Wh[min(i, M - 1) * M + min(b, M - 1)];
      wr[i][b] = (i < M && b < M) ? w : 0.0f;
    }
  const float wv = tid < M * M ? Wh[tid] : 0.0f;

  // zero row N (and every pad column when d < DP)
  if (d < DP) {
    const int chunks = (int)((L::q_bytes(N) + (size_t)2 * (N + 1) * RS * 2) / 16);
    for (int e = tid; e < chunks; e += NTHR)
      reinterpret_cast<u32x4_t*>(smem)[e] = u32x4_t{0u, 0u, 0u, 0u};
    lds_barrier();
  } else if (tid < 3 * (DP / 8)) {
    const int m = tid / (DP / 8), f = tid - m * (DP / 8);
    bf16_t* row = m == 0 ? sQ + (size_t)N * RSQ : (m == 1 ? sK : sV) + (size_t)N * RS;
    *reinterpret_cast<u32x4_t*>(row + 8 * f) = u32x4_t{0u, 0u, 0u, 0u};
  }

  // N * d / 8 <= 8 * 64 * 64 / 8 = 4096 chunks for every shape this kernel
  // accepts, so two batches of 2048 chunks cover the slice.
#pragma unroll
  for (int bt = 0; bt < 2; ++bt) {
    const int base = bt * UKV * NTHR;
    if (base < items) {
      if (bt > 0) {
        MHLA_LOAD(kr, K, base, UKV, NTHR, tid)
        MHLA_LOAD(vr, V, base, UKV, NTHR, tid)
      }
#pragma unroll
      for (int u = 0; u < UKV; ++u) {
        const int it = base + u * NTHR + tid;
        if (it < items) {
          const int t = small_div(it, inv8);
          const int f = it - t * F8;
          *reinterpret_cast<u32x4_t*>(sK + t * RS + 8 * f) = phi8<PHI>(kr[u]);
          *reinterpret_cast<u32x4_t*>(sV + t * RS + 8 * f) = vr[u];
        }
      }
    }
  }
  lds_barrier();

  // ---- B. summaries and mixing ------------------------------------------------
  // Wave w owns item (ct, ks) = (w % NT, w / NT): value columns 16ct..16ct+15
  // and key features 32ks..32ks+31 of every S_b, mixed into every S~_i in
  // registers.  Blocks b = M .. MM-1 (when M is not a power of two) gather the
  // zero row and have W = 0.  The fragments of block b+1 are read while block
  // b is multiplied.  The wave with ct = b % NT also forms z_b for its
  // features (a ones B operand puts z_b in every column).
  const bool has_item = wave < NT * DS;
  const int ct = wave % NT, ksB = wave / NT;
  f32x4_t mix[MM][2];
#pragma unroll
  for (int i = 0; i < MM; ++i) mix[i][0] = mix[i][1] = zero4();
  if (has_item) {
    int toff[KS][2];  // this lane's tokens: member 32 st + 8 grp + 4 th + s / 4
#pragma unroll
    for (int st = 0; st < KS; ++st)
#pragma unroll
      for (int th = 0; th < 2; ++th) {
        const int j = 32 * st + 8 * grp + 4 * th + (s >> 2);
        toff[st][th] = j < nb ? g.tokoff(j) : -1;
      }
    const bf16_t* kb = sK + 4 * (s & 3) + 32 * ksB;
    const bf16_t* vb = sV + 4 * (s & 3) + 16 * ct;
    const u16x8_t ones = {0x3f80, 0x3f80, 0x3f80, 0x3f80, 0x3f80, 0x3f80, 0x3f80, 0x3f80};
    u16x8_t fa[2][KS][2], fv[2][KS];
#define MHLA_FRAGS(bk, buf)                                                                  \
  _Pragma("unroll") for (int st = 0; st < KS; ++st) {                                        \
    const int bb_ = (bk) < M ? fb.b[bk] : -1;                                                \
    const int r0 = (bb_ >= 0 && toff[st][0] >= 0) ? bb_ + toff[st][0] : N;                   \
    const int r1 = (bb_ >= 0 && toff[st][1] >= 0) ? bb_ + toff[st][1] : N;                   \
    fv[buf][st] = lds_tr8_rows(vb, RS, r0, r1);                                              \
    fa[buf][st][0] = lds_tr8_rows(kb, RS, r0, r1);                                           \
    fa[buf][st][1] = lds_tr8_rows(kb + 16, RS, r0, r1);                                      \
  }
    MHLA_FRAGS(0, 0)
#pragma unroll
    for (int b = 0; b < MM; ++b) {
      const int cb = b & 1;
      if (b + 1 < MM) { MHLA_FRAGS(b + 1, cb ^ 1) }
      f32x4_t sb[2] = {zero4(), zero4()};
#pragma unroll
      for (int st = 0; st < KS; ++st)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) sb[hh] = mfma_bf16(fa[cb][st][hh], fv[cb][st], sb[hh]);
      if (b < M && b % NT == ct) {
        f32x4_t zb[2] = {zero4(), zero4()};
#pragma unroll
        for (int st = 0; st < KS; ++st)
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) zb[hh] = mfma_bf16(fa[cb][st][hh], ones, zb[hh]);
        if (s == 0) {
#pragma unroll
          for (int hh = 0; hh < 2; ++hh)
            *reinterpret_cast<f32x4_t*>(zraw + b * DP + 32 * ksB + 16 * hh + 4 * grp) = zb[hh];
        }
      }
#pragma unroll
      for (int i = 0; i < MM; ++i) {
        mix[i][0] += wr[i][b] * sb[0];
        mix[i][1] += wr[i][b] * sb[1];
      }
    }
#undef MHLA_FRAGS
  }

  // ---- waves 8..15 stage phi(Q) meanwhile (loads issued at the start) -------
  if (qwave) {
#pragma unroll
    for (int bt = 0; bt < 2; ++bt) {
      const int base = bt * UQ * QTHR;
      if (base < items) {
        if (bt > 0) { MHLA_LOAD(qr, Q, base, UQ, QTHR, qtid) }
#pragma unroll
        for (int u = 0; u < UQ; ++u) {
          const int it = base + u * QTHR + qtid;
          if (it < items) {
            const int t = small_div(it, inv8);
            const int f = it - t * F8;
            *reinterpret_cast<u32x4_t*>(sQ + t * RSQ + 8 * f) = phi8<PHI>(qr[u]);
          }
        }
      }
    }
  }
  if (tid < M * M) sW[tid] = wv;
#undef MHLA_LOAD
  lds_barrier();  // phi(K) / V are no longer read; z_b and phi(Q) are complete

  // ---- C. exchange the mixed tiles; z~ ----------------------------------------
  if (has_item) {
#pragma unroll
    for (int i = 0; i < MM; ++i)
      if (i < M) frag[((i * NT + ct) * DS + ksB) * 64 + lane] = pack_acc8(mix[i][0], mix[i][1]);
  }
  for (int e = tid; e < M * DP; e += NTHR) {
    const int i = e / DP, k = e - i * DP;
    float acc = 0.0f;
    for (int b = 0; b < M; ++b) acc += sW[i * M + b] * zraw[b * DP + k];
    zmix[e] = acc;
  }
  lds_barrier();

  // ---- D. readout ------------------------------------------------------------
  // Wave w takes tiles w*tpw .. w*tpw+tpw-1 (16 queries each; consecutive tiles
  // share a block).  All of the wave's phi(Q) operands are read first.
  const int ntile = M * QT;
  const int tpw = (ntile + NWAVE - 1) / NWAVE;
  u16x8_t bq[TPW][DS];
  int tok[TPW];
#pragma unroll
  for (int u = 0; u < TPW; ++u) {
    const int tile = wave * tpw + u;
    const int i = tile / QT, j = (tile - i * QT) * 16 + s;
    const bool real = u < tpw && tile < ntile && j < nb;
    tok[u] = real ? fb.b[i] + g.tokoff(j) : -1;
    const int row = real ? tok[u] : N;
#pragma unroll
    for (int ks = 0; ks < DS; ++ks) {
      const bf16_t* p = sQ + row * RSQ + 32 * ks + 4 * grp;
      bq[u][ks] = from_u2x2(*reinterpret_cast<const uint2*>(p),
                            *reinterpret_cast<const uint2*>(p + 16));
    }
  }
  int cur = -1;
  u16x8_t af[NT][DS], az[DS];
#pragma unroll
  for (int u = 0; u < TPW; ++u) {
    const int tile = wave * tpw + u;
    if (u >= tpw || tile >= ntile) break;
    const int i = tile / QT, qt = tile - i * QT;
    if (qt * 16 >= nb) continue;
    if (i != cur) {
      cur = i;
#pragma unroll
      for (int c = 0; c < NT; ++c)
#pragma unroll
        for (int ks = 0; ks < DS; ++ks) af[c][ks] = frag[((i * NT + c) * DS + ks) * 64 + lane];
#pragma unroll
      for (int ks = 0; ks < DS; ++ks) {
        // the z~ operand: row 0 of an extra column tile holds z~_i, rows 1..15 are 0
        const float* zp = zmix + i * DP + 32 * ks + 4 * grp;
        az[ks] = s == 0 ? pack_acc8(*reinterpret_cast<const f32x4_t*>(zp),
                                    *reinterpret_cast<const f32x4_t*>(zp + 16))
                        : u16x8_t{0, 0, 0, 0, 0, 0, 0, 0};
      }
    }
    f32x4_t o[NT], oz = zero4();
#pragma unroll
    for (int c = 0; c < NT; ++c) {
      o[c] = zero4();
#pragma unroll
      for (int ks = 0; ks < DS; ++ks) o[c] = mfma_bf16(af[c][ks], bq[u][ks], o[c]);
    }
#pragma unroll
    for (int ks = 0; ks < DS; ++ks) oz = mfma_bf16(az[ks], bq[u][ks], oz);
    // row 0 of the z~ tile (lane s of group 0, element 0) is phi(q).z~_i
    const float den = __shfl(oz[0], s);
    const float rd = out_scale(g, den);
    store_row_tiles<NT, true>(tok[u] >= 0 ? Y + off + (size_t)tok[u] * d : nullptr, d, o, rd, grp);
  }
}

inline int fused_dp(int d) { return d <= 32 ? 32 : 64; }
inline int fused_nbp(int nb) { return nb <= 32 ? 32 : 64; }
inline int fused_mm(int M) { return M <= 2 ? 2 : (M <= 4 ? 4 : 8); }

inline size_t fused_lds(int d, int M, int nb) {
  const int N = M * nb;
  return fused_dp(d) == 32 ? FusedLayout<32>::total(N, M) : FusedLayout<64>::total(N, M);
}

inline bool fused_supports(int dtype, int d, int M, int nb) {
  if (dtype != 1 || d % 8 != 0 || d > 64 || M < 1 || M > kFusedMaxM || nb > 64) return false;
  return fused_lds(d, M, nb) <= kLdsLimit;
}

template <int DP, int NBP, int MM, int PHI>
int launch_fused_t(long slices, int H, int N, int d, const Geo& g, const bf16_t* Q,
                   const bf16_t* K, const bf16_t* V, const float* W, bf16_t* Y, hipStream_t st) {
  const size_t lds = FusedLayout<DP>::total(N, g.M);
  static std::atomic<bool> attr_set[64];
  if (lds_limit_once(reinterpret_cast<const void*>(&k_fused<DP, NBP, MM, PHI>), attr_set,
                     (int)kLdsLimit) != 0)
    return -1;
  FusedBases fb;
  for (int b = 0; b < kFusedMaxM; ++b) fb.b[b] = b < g.M ? g.blockbase(b) : 0;
  k_fused<DP, NBP, MM, PHI><<<dim3((unsigned)slices), dim3(64 * fused_waves(MM)), lds, st>>>(
      Q, K, V, W, Y, g, fb, H, N, d);
  launch_mark(st, "k_fused");
  return 0;
}

template <int DP, int NBP, int PHI>
int launch_fused_m(long slices, int H, int N, int d, const Geo& g, const bf16_t* Q,
                   const bf16_t* K, const bf16_t* V, const float* W, bf16_t* Y, hipStream_t st) {
  switch (fused_mm(g.M)) {
    case 2: return launch_fused_t<DP, NBP, 2, PHI>(slices, H, N, d, g, Q, K, V, W, Y, st);
    case 4: return launch_fused_t<DP, NBP, 4, PHI>(slices, H, N, d, g, Q, K, V, W, Y, st);
    default: return launch_fused_t<DP, NBP, 8, PHI>(slices, H, N, d, g, Q, K, V, W, Y, st);
  }
}

template <int PHI>
int launch_fused_p(long slices, int H, int N, int d, const Geo& g, const bf16_t* Q,
                   const bf16_t* K, const bf16_t* V, const float* W, bf16_t* Y, hipStream_t st) {
  const int DP = fused_dp(d), NBP = fused_nbp(g.nb);
  if (DP == 32 && NBP == 32)
    return launch_fused_m<32, 32, PHI>(slices, H, N, d, g, Q, K, V, W, Y, st);
  if (DP == 32) return launch_fused_m<32, 64, PHI>(slices, H, N, d, g, Q, K, V, W, Y, st);
  if (NBP == 32) return launch_fused_m<64, 32, PHI>(slices, H, N, d, g, Q, K, V, W, Y, st);
  return launch_fused_m<64, 64, PHI>(slices, H, N, d, g, Q, K, V, W, Y, st);
}

inline int launch_fused(long slices, int H, int N, int d, const Geo& g, int phi, const bf16_t* Q,
                        const bf16_t* K, const bf16_t* V, const float* W, bf16_t* Y,
                        hipStream_t st) {
  if (phi == PHI_RELU)
    return launch_fused_p<PHI_RELU>(slices, H, N, d, g, Q, K, V, W, Y, st);
  return launch_fused_p<PHI_ELU1>(slices, H, N, d, g, Q, K, V, W, Y, st);
}

}  // namespace mhla
