// k_fused.hpp -- single-kernel MHLA forward for small M (bf16, gfx950 MFMA).
//
// One workgroup per (batch, head) slice and one wave per block.  The whole
// forward of "MHLA: Restoring Expressivity of Linear Attention via
// Token-Level Multi-Head" §4.1 runs on chip:
//   1. phi(K) and V of every block are staged in LDS, transposed to
//      [feature][token] so that MFMA operands read 8 consecutive tokens;
//   2. wave b forms S_b = phi(K_b)^T V_b with v_mfma_f32_16x16x32_bf16
//      (fp32 accumulate) and z_b by summing its phi(K) rows;
//   3. the summaries are exchanged through LDS and wave i mixes
//      S~_i = sum_b W[i,b] S_b, z~_i = sum_b W[i,b] z_b in fp32 registers;
//   4. wave i reads its query block out as Y^T = S~_i^T phi(Q_i)^T on MFMA,
//      with the denominator phi(q).z~_i reduced across the wave, and the
//      divide fused before the bf16 store.
// S, S~ and z never reach HBM: the kernel reads Q, K, V, W and writes Y.
//
// MFMA operand conventions used here (16x16x32 bf16): lane l holds row
// (l % 16) of A, column (l % 16) of B, and 8 contraction elements chosen by
// lane group l / 16; A and B share that choice, so any fixed assignment of
// contraction indices to (group, element) gives the same sum.  The result
// lane l holds D[4*(l/16) + i][l % 16], i = 0..3.  A result tile can thus be
// reused as an A operand of a later product whose contraction runs over the
// tile's rows: two row-adjacent 16x16 tiles give the 8 elements
// {4g..4g+3} and {16+4g..16+4g+3}; the other operand uses the same indices.
#pragma once

#include "mhla_common.hpp"

namespace mhla {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef uint16_t u16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4_t mfma16x16x32(const u16x8_t& a, const u16x8_t& b,
                                                const f32x4_t& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

constexpr int kFusedMaxM = 8;

template <int DP, int NBP>
constexpr size_t fused_lds_bytes(int M) {
  // max(staged phi(K)^T and V^T, exchanged summaries + normalisers)
  return (size_t)M * ((size_t)2 * DP * (NBP + 8) * 2 > (size_t)DP * DP * 4 + DP * 4
                          ? (size_t)2 * DP * (NBP + 8) * 2
                          : (size_t)DP * DP * 4 + DP * 4);
}

// grid = B*H; block = 64*M threads; dynamic LDS = fused_lds_bytes<DP,NBP>(M).
template <int DP, int NBP>
__global__ __launch_bounds__(64 * kFusedMaxM) void k_fused(
    const bf16_t* __restrict__ Q, const bf16_t* __restrict__ K, const bf16_t* __restrict__ V,
    const float* __restrict__ W, bf16_t* __restrict__ Y, Geo g, int H, int N, int d, int phi) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  constexpr int RS = NBP + 8;   // LDS row length (bf16) of the transposed tiles
  constexpr int NT = DP / 16;   // 16-wide tiles along d
  constexpr int KS = NBP / 32;  // contraction steps of the summary
  constexpr int DS = DP / 32;   // contraction steps of the readout
  constexpr int QT = NBP / 16;  // query row tiles
  const int M = g.M, nb = g.nb;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int col = lane & 15, grp = lane >> 4;
  const long slice = blockIdx.x;
  const int h = (int)(slice % H);
  const bf16_t* Qs = Q + slice * (long)N * d;
  const bf16_t* Ks = K + slice * (long)N * d;
  const bf16_t* Vs = V + slice * (long)N * d;
  bf16_t* Ys = Y + slice * (long)N * d;

  // 0. Prefetch this wave's query rows in the readout's B-operand layout.
  uint2 qraw[QT][DS][2];
#pragma unroll
  for (int mt = 0; mt < QT; ++mt) {
    const int j = 16 * mt + col;
    const bool ok = j < nb;
    const long t = ok ? g.token(wave, j) : 0;
#pragma unroll
    for (int ks = 0; ks < DS; ++ks) {
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int k0 = 32 * ks + 16 * hh + 4 * grp;
        qraw[mt][ks][hh] = (ok && k0 < d) ? *reinterpret_cast<const uint2*>(Qs + t * d + k0)
                                          : make_uint2(0u, 0u);
      }
    }
  }

  // 1. Stage phi(K)^T and V^T of all blocks: KT[b][f][j], VT[b][f][j].  Pads
  //    (j >= nb or f >= d) are zero, which leaves S and z exact.
  bf16_t* KT = reinterpret_cast<bf16_t*>(smem);
  bf16_t* VT = KT + (size_t)M * DP * RS;
  {
    constexpr int F8 = DP / 8;
    const int total = M * NBP * F8;
    const int nf8 = d / 8;
    for (int e = threadIdx.x; e < total; e += blockDim.x) {
      const int f8 = e % F8;
      const int j = (e / F8) % NBP;
      const int b = e / (F8 * NBP);
      uint4 kr = make_uint4(0u, 0u, 0u, 0u), vr = kr;
      const bool ok = j < nb && f8 < nf8;
      if (ok) {
        const long t = g.token(b, j);
        kr = *reinterpret_cast<const uint4*>(Ks + t * d + 8 * f8);
        vr = *reinterpret_cast<const uint4*>(Vs + t * d + 8 * f8);
      }
      const uint32_t kw[4] = {kr.x, kr.y, kr.z, kr.w};
      const uint32_t vw[4] = {vr.x, vr.y, vr.z, vr.w};
      bf16_t* kdst = KT + ((size_t)b * DP + 8 * f8) * RS + j;
      bf16_t* vdst = VT + ((size_t)b * DP + 8 * f8) * RS + j;
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const bf16_t kb = (bf16_t)(kw[u >> 1] >> (16 * (u & 1)));
        const bf16_t vb = (bf16_t)(vw[u >> 1] >> (16 * (u & 1)));
        kdst[u * RS] = ok ? f32_to_bf16(phi_apply(phi, bf16_to_f32(kb))) : (bf16_t)0;
        vdst[u * RS] = vb;
      }
    }
  }
  __syncthreads();

  // 2. Summary of key block b = wave: acc[kt][ct] is the 16x16 tile
  //    S[16kt .. +15][16ct .. +15] with S[k][c] = sum_j phiK[j][k] V[j][c].
  f32x4_t acc[NT][NT];
#pragma unroll
  for (int kt = 0; kt < NT; ++kt)
#pragma unroll
    for (int ct = 0; ct < NT; ++ct) acc[kt][ct] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  {
    const bf16_t* KTb = KT + (size_t)wave * DP * RS;
    const bf16_t* VTb = VT + (size_t)wave * DP * RS;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u16x8_t a[NT], bv[NT];
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        a[t] = *reinterpret_cast<const u16x8_t*>(KTb + (16 * t + col) * RS + 32 * ks + 8 * grp);
        bv[t] = *reinterpret_cast<const u16x8_t*>(VTb + (16 * t + col) * RS + 32 * ks + 8 * grp);
      }
#pragma unroll
      for (int kt = 0; kt < NT; ++kt)
#pragma unroll
        for (int ct = 0; ct < NT; ++ct) acc[kt][ct] = mfma16x16x32(a[kt], bv[ct], acc[kt][ct]);
    }
  }
  // z_b[k] for k = lane, from the same rounded phi(K) the products used.
  float zb = 0.0f;
  if (lane < DP) {
    const bf16_t* row = KT + ((size_t)wave * DP + lane) * RS;
#pragma unroll
    for (int j8 = 0; j8 < NBP / 8; ++j8) {
      const u16x8_t v8 = *reinterpret_cast<const u16x8_t*>(row + 8 * j8);
#pragma unroll
      for (int u = 0; u < 8; ++u) zb += bf16_to_f32(v8[u]);
    }
  }
  __syncthreads();  // every wave is done with KT/VT; the region is reused below

  // 3. Exchange: SX[b][tile][lane][4] (fp32), ZX[b][k].
  float* SX = reinterpret_cast<float*>(smem);
  float* ZX = SX + (size_t)M * NT * NT * 256;
#pragma unroll
  for (int kt = 0; kt < NT; ++kt)
#pragma unroll
    for (int ct = 0; ct < NT; ++ct)
      *reinterpret_cast<f32x4_t*>(SX + (((size_t)wave * NT * NT + kt * NT + ct) * 64 + lane) * 4) =
          acc[kt][ct];
  if (lane < DP) ZX[wave * DP + lane] = zb;
  __syncthreads();

  // 4. Mixing for query block i = wave (row i of W).
  const float* Wi = W + ((size_t)h * M + wave) * M;
  f32x4_t zt[DS][2];
#pragma unroll
  for (int kt = 0; kt < NT; ++kt)
#pragma unroll
    for (int ct = 0; ct < NT; ++ct) acc[kt][ct] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < DS; ++ks) zt[ks][0] = zt[ks][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  for (int b = 0; b < M; ++b) {
    const float w = Wi[b];
#pragma unroll
    for (int kt = 0; kt < NT; ++kt)
#pragma unroll
      for (int ct = 0; ct < NT; ++ct)
        acc[kt][ct] += w * *reinterpret_cast<const f32x4_t*>(
                               SX + (((size_t)b * NT * NT + kt * NT + ct) * 64 + lane) * 4);
#pragma unroll
    for (int ks = 0; ks < DS; ++ks)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
        zt[ks][hh] += w * *reinterpret_cast<const f32x4_t*>(ZX + b * DP + 32 * ks + 16 * hh + 4 * grp);
  }

  // 5. Readout.  A operand: rows c of S~^T, i.e. S~[k][c] for the lane's
  //    contraction indices k = 32ks + {4g..4g+3, 16+4g..16+4g+3}.
  u16x8_t afr[NT][DS];
#pragma unroll
  for (int ct = 0; ct < NT; ++ct)
#pragma unroll
    for (int ks = 0; ks < DS; ++ks)
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        afr[ct][ks][u] = f32_to_bf16(acc[2 * ks][ct][u]);
        afr[ct][ks][u + 4] = f32_to_bf16(acc[2 * ks + 1][ct][u]);
      }
#pragma unroll
  for (int mt = 0; mt < QT; ++mt) {
    if (16 * mt >= nb) break;
    u16x8_t bq[DS];
    float den = 0.0f;
#pragma unroll
    for (int ks = 0; ks < DS; ++ks) {
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const uint32_t w2[2] = {qraw[mt][ks][hh].x, qraw[mt][ks][hh].y};
        const bool kin = 32 * ks + 16 * hh + 4 * grp < d;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const bf16_t qb = (bf16_t)(w2[u >> 1] >> (16 * (u & 1)));
          const bf16_t pq = kin ? f32_to_bf16(phi_apply(phi, bf16_to_f32(qb))) : (bf16_t)0;
          bq[ks][4 * hh + u] = pq;
          den += bf16_to_f32(pq) * zt[ks][hh][u];
        }
      }
    }
    den += __shfl_xor(den, 16);
    den += __shfl_xor(den, 32);
    const int j = 16 * mt + col;
    const bool ok = j < nb;
    const long t = ok ? g.token(wave, j) : 0;
#pragma unroll
    for (int ct = 0; ct < NT; ++ct) {
      f32x4_t o = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < DS; ++ks) o = mfma16x16x32(afr[ct][ks], bq[ks], o);
      const int c = 16 * ct + 4 * grp;
      if (ok && c < d) {
        // padded query rows (j >= nb) are computed but never stored
        uint32_t lo, hi;
        if (den == 0.0f) {
          lo = hi = 0u;
        } else {
          lo = (uint32_t)f32_to_bf16(o[0] / den) | ((uint32_t)f32_to_bf16(o[1] / den) << 16);
          hi = (uint32_t)f32_to_bf16(o[2] / den) | ((uint32_t)f32_to_bf16(o[3] / den) << 16);
        }
        *reinterpret_cast<uint2*>(Ys + t * d + c) = make_uint2(lo, hi);
      }
    }
  }
}

inline bool fused_supports(int dtype, int d, int M, int nb) {
  if (dtype != 1 || d % 8 != 0 || d > 64 || M < 1 || M > kFusedMaxM || nb > 64) return false;
  const int DP = d <= 32 ? 32 : 64;
  const int NBP = nb <= 32 ? 32 : 64;
  const size_t lds = (size_t)M * ((size_t)2 * DP * (NBP + 8) * 2 > (size_t)DP * DP * 4 + DP * 4
                                      ? (size_t)2 * DP * (NBP + 8) * 2
                                      : (size_t)DP * DP * 4 + DP * 4);
  return lds <= 160 * 1024;
}

template <int DP, int NBP>
int launch_fused_t(long slices, int H, int N, int d, const Geo& g, int phi, const bf16_t* Q,
                   const bf16_t* K, const bf16_t* V, const float* W, bf16_t* Y, hipStream_t st) {
  const size_t lds = fused_lds_bytes<DP, NBP>(g.M);
  static bool attr_set[64] = {false};
  int dev = 0;
  (void)hipGetDevice(&dev);
  if (dev >= 0 && dev < 64 && !attr_set[dev]) {
    if (hipFuncSetAttribute(reinterpret_cast<const void*>(&k_fused<DP, NBP>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024) != hipSuccess)
      return MHLA_ERR_HIP;
    attr_set[dev] = true;
  }
  k_fused<DP, NBP><<<dim3((unsigned)slices), dim3(64 * g.M), lds, st>>>(Q, K, V, W, Y, g, H, N, d,
                                                                       phi);
  return 0;
}

inline int launch_fused(long slices, int H, int N, int d, const Geo& g, int phi, const bf16_t* Q,
                        const bf16_t* K, const bf16_t* V, const float* W, bf16_t* Y,
                        hipStream_t st) {
  const bool d32 = d <= 32, n32 = g.nb <= 32;
  if (d32 && n32) return launch_fused_t<32, 32>(slices, H, N, d, g, phi, Q, K, V, W, Y, st);
  if (d32) return launch_fused_t<32, 64>(slices, H, N, d, g, phi, Q, K, V, W, Y, st);
  if (n32) return launch_fused_t<64, 32>(slices, H, N, d, g, phi, Q, K, V, W, Y, st);
  return launch_fused_t<64, 64>(slices, H, N, d, g, phi, Q, K, V, W, Y, st);
}

}  // namespace mhla
