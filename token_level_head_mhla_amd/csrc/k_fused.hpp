// k_fused.hpp -- single-kernel MHLA forward for small M (bf16 in/out, gfx950).
//
// One workgroup of 8 waves per (batch, head) slice.  The whole forward of
// "MHLA: Restoring Expressivity of Linear Attention via Token-Level
// Multi-Head" §4.1 runs on chip, and HBM sees only Q, K, V, W and Y:
//
//   0. token <-> LDS-row tables: the rows of block b are b*NBP .. b*NBP+nb-1
//      (raster order inside the tile, Fig. 4b numbering of the blocks); rows
//      nb .. NBP-1 of every block are zero padding.
//   A. K and V of the slice are read with 16-byte coalesced loads (the slice
//      is contiguous), phi is applied to K in registers (bf16 result), and
//      both are written to LDS row-major in block order.
//   B. Work item (ct, ks) = value columns 16ct..16ct+15 and key features
//      32ks..32ks+31.  For every key block b the wave forms the two 16x16
//      tiles of S_b = phi(K_b)^T V_b with v_mfma_f32_16x16x32_bf16, both
//      operands taken from LDS with transpose reads, and immediately mixes
//      them into every query block's S~_i += W[i,b] S_b (fp32 registers).
//      The normaliser z_b = sum phi(K_b) rides along as one more column
//      tile (B operand = a column of ones), so z~_i = sum_b W[i,b] z_b comes
//      out of the same mixing.  The mixed tiles are packed to bf16 in the
//      A-operand layout of the readout and exchanged through LDS.
//   D. Work item (i, qt) = 16 queries of block i.  Y^T = S~_i^T phi(Q)^T on
//      MFMA; the extra z~ tile gives the denominator phi(q).z~_i as row d of
//      the same product; the divide and the bf16 rounding are fused into the
//      8-byte stores.  Q is prefetched at kernel start.
//
// A denominator of exactly 0 (ReLU with phi(q) = 0) writes a zero row.
#pragma once

#include "mhla_mfma.hpp"

namespace mhla {

constexpr int kFusedThreads = 512;
constexpr int kFusedWaves = kFusedThreads / 64;
constexpr int kFusedMaxM = 8;
constexpr size_t kLdsLimit = 160 * 1024;

template <int DP, int NBP>
struct FusedLayout {
  static constexpr int RS = DP + 8;        // LDS row stride of phi(K) and V (elements)
  static constexpr int NT = DP / 16;       // value-column tiles
  static constexpr int DS = DP / 32;       // 32-feature contraction steps
  static constexpr int KS = NBP / 32;      // 32-token contraction steps per block
  static constexpr int QT = NBP / 16;      // query tiles per block
  // byte offsets for M blocks
  __host__ __device__ static size_t kv_bytes(int M) { return (size_t)2 * M * NBP * RS * 2; }
  __host__ __device__ static size_t frag_bytes(int M) { return (size_t)M * (NT + 1) * DS * 64 * 16; }
  __host__ __device__ static size_t tab_off(int M) {
    const size_t a = kv_bytes(M), b = frag_bytes(M);
    return (a > b ? a : b);
  }
  __host__ __device__ static size_t w_off(int M) { return tab_off(M) + (size_t)2 * 2 * M * NBP; }
  __host__ __device__ static size_t total(int M) { return w_off(M) + (size_t)4 * M * M; }
};

template <int DP, int NBP, int MM, int PHI>
__global__ __launch_bounds__(kFusedThreads) void k_fused(
    const bf16_t* __restrict__ Q, const bf16_t* __restrict__ K, const bf16_t* __restrict__ V,
    const float* __restrict__ W, bf16_t* __restrict__ Y, Geo g, int H, int N, int d) {
  using L = FusedLayout<DP, NBP>;
  constexpr int RS = L::RS, NT = L::NT, DS = L::DS, KS = L::KS, QT = L::QT;
  constexpr int TPW = (MM * QT + kFusedWaves - 1) / kFusedWaves;  // query tiles per wave
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int M = g.M, nb = g.nb;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int s = lane & 15, grp = lane >> 4;
  const long slice = blockIdx.x;
  const int h = (int)(slice % H);
  const size_t off = (size_t)slice * N * d;

  bf16_t* sK = reinterpret_cast<bf16_t*>(smem);
  bf16_t* sV = sK + (size_t)M * NBP * RS;
  u16x8_t* frag = reinterpret_cast<u16x8_t*>(smem);  // aliases sK/sV after phase B
  uint16_t* rowtab = reinterpret_cast<uint16_t*>(smem + L::tab_off(M));  // token -> row
  uint16_t* toktab = rowtab + M * NBP;                                     // row -> token
  float* sW = reinterpret_cast<float*>(smem + L::w_off(M));

  // ---- 0. tables, W, zero padding -----------------------------------------
  for (int r = tid; r < M * NBP; r += kFusedThreads) toktab[r] = 0xffff;
  for (int e = tid; e < M * M; e += kFusedThreads) sW[e] = W[(size_t)h * M * M + e];
  if (d < DP) {
    const int chunks = 2 * M * NBP * RS / 8;
    for (int e = tid; e < chunks; e += kFusedThreads)
      reinterpret_cast<uint4*>(sK)[e] = make_uint4(0u, 0u, 0u, 0u);
  } else if (nb < NBP) {
    constexpr int F8 = DP / 8;
    const int pad = NBP - nb;
    for (int e = tid; e < 2 * M * pad * F8; e += kFusedThreads) {
      const int f = e % F8, r = (e / F8) % pad, b = e / (F8 * pad);
      bf16_t* base = b < M ? sK : sV;
      const int bb = b < M ? b : b - M;
      *reinterpret_cast<uint4*>(base + (bb * NBP + nb + r) * RS + 8 * f) =
          make_uint4(0u, 0u, 0u, 0u);
    }
  }
  __syncthreads();
  for (int t = tid; t < N; t += kFusedThreads) {
    const int x = t % g.Wg, y = (t / g.Wg) % g.Hg, z = t / (g.Wg * g.Hg);
    const int b = ((z / g.bt) * g.nby + y / g.bh) * g.nbx + x / g.bw;
    const int j = ((z % g.bt) * g.bh + y % g.bh) * g.bw + x % g.bw;
    const int r = b * NBP + j;
    rowtab[t] = (uint16_t)r;
    toktab[r] = (uint16_t)t;
  }
  __syncthreads();

  // ---- prefetch this wave's queries (acc8 B-operand layout) ----------------
  uint2 qraw[TPW][DS][2];
#pragma unroll
  for (int u = 0; u < TPW; ++u) {
    const int tile = wave + u * kFusedWaves;
    int t = 0xffff;
    if (tile < M * QT) t = toktab[(tile / QT) * NBP + (tile % QT) * 16 + s];
#pragma unroll
    for (int ks = 0; ks < DS; ++ks)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int k0 = 32 * ks + 16 * hh + 4 * grp;
        qraw[u][ks][hh] = (t != 0xffff && k0 < d)
                              ? *reinterpret_cast<const uint2*>(Q + off + (size_t)t * d + k0)
                              : make_uint2(0u, 0u);
      }
  }

  // ---- A. stage phi(K) and V ---------------------------------------------
  {
    const int F8 = d >> 3;
    const int items = N * F8;
    const float inv = 1.0f / (float)F8;
    constexpr int U = 4;
    for (int base = 0; base < items; base += U * kFusedThreads) {
      uint4 kr[U], vr[U];
      int it[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        // clamped so that every lane loads (straight-line, all loads in flight)
        it[u] = base + u * kFusedThreads + tid;
        const size_t src = off + (size_t)min(it[u], items - 1) * 8;
        kr[u] = *reinterpret_cast<const uint4*>(K + src);
        vr[u] = *reinterpret_cast<const uint4*>(V + src);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (it[u] < items) {
          const int t = (int)(((float)it[u] + 0.5f) * inv);
          const int f = it[u] - t * F8;
          const int r = rowtab[t];
          *reinterpret_cast<uint4*>(sK + r * RS + 8 * f) = phi8<PHI>(kr[u]);
          *reinterpret_cast<uint4*>(sV + r * RS + 8 * f) = vr[u];
        }
      }
    }
  }
  __syncthreads();

  // ---- B. summaries, mixing ----------------------------------------------
  // Each wave owns at most one (ct, ks) item when NT*DS <= 8 (all shapes this
  // kernel accepts); waves without an item idle until the exchange.
  const int item = wave;
  const bool has_item = item < NT * DS;
  const int ct = item % NT, ksB = item / NT;
  const bool ztile = has_item && ct == 0;
  f32x4_t mix[MM][2], zmix[MM][2];
#pragma unroll
  for (int i = 0; i < MM; ++i) {
    mix[i][0] = mix[i][1] = zero4();
    zmix[i][0] = zmix[i][1] = zero4();
  }
  if (has_item) {
    const uint16_t one = 0x3f80;  // bf16 1.0
    const uint16_t ov = s == 0 ? one : (uint16_t)0;
    const u16x8_t ones = {ov, ov, ov, ov, ov, ov, ov, ov};
    for (int b = 0; b < M; ++b) {
      f32x4_t sb[2] = {zero4(), zero4()}, zb[2] = {zero4(), zero4()};
#pragma unroll
      for (int st = 0; st < KS; ++st) {
        const int r0 = b * NBP + 32 * st;
        const u16x8_t bv = lds_tr8(sV, RS, r0, 16 * ct, lane);
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const u16x8_t a = lds_tr8(sK, RS, r0, 32 * ksB + 16 * hh, lane);
          sb[hh] = mfma_bf16(a, bv, sb[hh]);
          if (ztile) zb[hh] = mfma_bf16(a, ones, zb[hh]);
        }
      }
#pragma unroll
      for (int i = 0; i < MM; ++i) {
        if (i < M) {
          const float w = sW[i * M + b];
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) {
            mix[i][hh] += w * sb[hh];
            if (ztile) zmix[i][hh] += w * zb[hh];
          }
        }
      }
    }
  }
  __syncthreads();  // every wave is done reading sK / sV
  if (has_item) {
#pragma unroll
    for (int i = 0; i < MM; ++i) {
      if (i < M) {
        frag[((i * (NT + 1) + ct) * DS + ksB) * 64 + lane] = pack_acc8(mix[i][0], mix[i][1]);
        if (ztile)
          frag[((i * (NT + 1) + NT) * DS + ksB) * 64 + lane] = pack_acc8(zmix[i][0], zmix[i][1]);
      }
    }
  }
  __syncthreads();

  // ---- D. readout ----------------------------------------------------------
#pragma unroll
  for (int u = 0; u < TPW; ++u) {
    const int tile = wave + u * kFusedWaves;
    if (tile >= M * QT) break;
    const int i = tile / QT, qt = tile % QT;
    if (qt * 16 >= nb) continue;
    u16x8_t bq[DS];
#pragma unroll
    for (int ks = 0; ks < DS; ++ks)
      bq[ks] = from_u2x2(phi4<PHI>(qraw[u][ks][0]), phi4<PHI>(qraw[u][ks][1]));
    f32x4_t o[NT + 1];
#pragma unroll
    for (int c = 0; c <= NT; ++c) {
      o[c] = zero4();
#pragma unroll
      for (int ks = 0; ks < DS; ++ks)
        o[c] = mfma_bf16(frag[((i * (NT + 1) + c) * DS + ks) * 64 + lane], bq[ks], o[c]);
    }
    // row d of the product (lane s of group 0, element 0) is phi(q).z~_i
    const float den = __shfl(o[NT][0], s);
    const float rd = den == 0.0f ? 0.0f : 1.0f / den;
    const int j = qt * 16 + s;
    if (j < nb) {
      const int t = toktab[i * NBP + j];
      bf16_t* yrow = Y + off + (size_t)t * d;
#pragma unroll
      for (int c = 0; c < NT; ++c) {
        const int col = 16 * c + 4 * grp;
        if (col < d)
          *reinterpret_cast<uint2*>(yrow + col) =
              make_uint2(pack2(o[c][0] * rd, o[c][1] * rd), pack2(o[c][2] * rd, o[c][3] * rd));
      }
    }
  }
}

inline int fused_dp(int d) { return d <= 32 ? 32 : 64; }
inline int fused_nbp(int nb) { return nb <= 32 ? 32 : 64; }
inline int fused_mm(int M) { return M <= 2 ? 2 : (M <= 4 ? 4 : 8); }

inline size_t fused_lds(int d, int M, int nb) {
  const int DP = fused_dp(d), NBP = fused_nbp(nb);
  if (DP == 32)
    return NBP == 32 ? FusedLayout<32, 32>::total(M) : FusedLayout<32, 64>::total(M);
  return NBP == 32 ? FusedLayout<64, 32>::total(M) : FusedLayout<64, 64>::total(M);
}

inline bool fused_supports(int dtype, int d, int M, int nb) {
  if (dtype != 1 || d % 8 != 0 || d > 64 || M < 1 || M > kFusedMaxM || nb > 64) return false;
  return fused_lds(d, M, nb) <= kLdsLimit;
}

template <int DP, int NBP, int MM, int PHI>
int launch_fused_t(long slices, int H, int N, int d, const Geo& g, const bf16_t* Q,
                   const bf16_t* K, const bf16_t* V, const float* W, bf16_t* Y, hipStream_t st) {
  const size_t lds = FusedLayout<DP, NBP>::total(g.M);
  static bool attr_set[64] = {false};
  int dev = 0;
  (void)hipGetDevice(&dev);
  const void* fn = reinterpret_cast<const void*>(&k_fused<DP, NBP, MM, PHI>);
  if (dev < 0 || dev >= 64 || !attr_set[dev]) {
    if (hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLdsLimit) !=
        hipSuccess)
      return -1;
    if (dev >= 0 && dev < 64) attr_set[dev] = true;
  }
  k_fused<DP, NBP, MM, PHI><<<dim3((unsigned)slices), dim3(kFusedThreads), lds, st>>>(
      Q, K, V, W, Y, g, H, N, d);
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
