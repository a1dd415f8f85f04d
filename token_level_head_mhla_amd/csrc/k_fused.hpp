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

constexpr int kFusedThreads = 512;
constexpr int kFusedWaves = kFusedThreads / 64;
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
  __host__ __device__ static size_t total(int N, int M) { return z_off(N, M) + (size_t)2 * M * DP * 4; }
};

// floor(a / b) for 0 <= a < 2^16 and 1 <= b <= 2^12 with inv = 1/b.
__device__ __forceinline__ int small_div(int a, float inv) {
  return (int)(((float)a + 0.5f) * inv);
}

template <int DP, int NBP, int MM, int PHI>
__global__ __launch_bounds__(kFusedThreads) void k_fused(
    const bf16_t* __restrict__ Q, const bf16_t* __restrict__ K, const bf16_t* __restrict__ V,
    const float* __restrict__ W, bf16_t* __restrict__ Y, Geo g, int H, int N, int d) {
  using L = FusedLayout<DP>;
  constexpr int RSQ = L::RSQ, RS = L::RS, NT = L::NT, DS = L::DS;
  constexpr int KS = NBP / 32;  // 32-token contraction steps per block
  constexpr int QT = NBP / 16;  // 16-query tiles per block
  constexpr int U = 4;          // 16-byte chunks per thread and tensor per batch
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

  // ---- A. loads: K and V first, then Q; stage phi(K) and V --------------------
  const int F8 = d >> 3;
  const int items = N * F8;
  const float inv8 = 1.0f / (float)F8;
  u32x4_t qr[U], kr[U], vr[U];
#define MHLA_LOAD(dst, src_ptr, base)                                                     \
  _Pragma("unroll") for (int u = 0; u < U; ++u) {                                          \
    /* clamped so that every lane loads: straight-line code, all loads in flight */       \
    const size_t o = off + (size_t)min((base) + u * kFusedThreads + tid, items - 1) * 8;  \
    dst[u] = *reinterpret_cast<const u32x4_t*>(src_ptr + o);                               \
  }
  MHLA_LOAD(kr, K, 0)
  MHLA_LOAD(vr, V, 0)
  MHLA_LOAD(qr, Q, 0)

  // zero row N (and every pad column when d < DP)
  if (d < DP) {
    const int chunks = (int)((L::q_bytes(N) + (size_t)2 * (N + 1) * RS * 2) / 16);
    for (int e = tid; e < chunks; e += kFusedThreads)
      reinterpret_cast<u32x4_t*>(smem)[e] = u32x4_t{0u, 0u, 0u, 0u};
    lds_barrier();
  } else if (tid < 3 * (DP / 8)) {
    const int m = tid / (DP / 8), f = tid - m * (DP / 8);
    bf16_t* row = m == 0 ? sQ + (size_t)N * RSQ : (m == 1 ? sK : sV) + (size_t)N * RS;
    *reinterpret_cast<u32x4_t*>(row + 8 * f) = u32x4_t{0u, 0u, 0u, 0u};
  }

  // N * d / 8 <= 8 * 64 * 64 / 8 = 2 * U * kFusedThreads chunks for every
  // shape this kernel accepts, so two batches cover the slice.
#pragma unroll
  for (int bt = 0; bt < 2; ++bt) {
    const int base = bt * U * kFusedThreads;
    if (base < items) {
      if (bt > 0) {
        MHLA_LOAD(kr, K, base)
        MHLA_LOAD(vr, V, base)
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int it = base + u * kFusedThreads + tid;
        if (it < items) {
          const int t = small_div(it, inv8);
          const int f = it - t * F8;
          *reinterpret_cast<u32x4_t*>(sK + t * RS + 8 * f) = phi8<PHI>(kr[u]);
          *reinterpret_cast<u32x4_t*>(sV + t * RS + 8 * f) = vr[u];
        }
      }
    }
  }

  auto tokoff = [&](int j) { return g.tokoff(j); };
  auto blockbase = [&](int b) { return g.blockbase(b); };
  lds_barrier();

  // ---- B. summaries and mixing ------------------------------------------------
  // Blocks b = M .. MM-1 (present when M is not a power of two) gather only the
  // zero row and have W = 0, so they add nothing; the loop is fully static.
  int bbase[MM];
  float wr[MM][MM];
#pragma unroll
  for (int b = 0; b < MM; ++b) {
    bbase[b] = b < M ? blockbase(b) : -1;
#pragma unroll
    for (int i = 0; i < MM; ++i) wr[i][b] = (i < M && b < M) ? Wh[i * M + b] : 0.0f;
  }
  const bool has_item = wave < NT * DS;
  const int ct = wave % NT, ksB = wave / NT;
  f32x4_t mix[MM][2];
#pragma unroll
  for (int i = 0; i < MM; ++i) mix[i][0] = mix[i][1] = zero4();
  if (has_item) {
    // this lane's tokens: member j = 32 st + 8 grp + 4 th + s / 4 of each block
    int toff[KS][2];
#pragma unroll
    for (int st = 0; st < KS; ++st)
#pragma unroll
      for (int th = 0; th < 2; ++th) {
        const int j = 32 * st + 8 * grp + 4 * th + (s >> 2);
        toff[st][th] = j < nb ? tokoff(j) : -1;
      }
    auto row = [&](int b, int st, int th) {
      return (bbase[b] >= 0 && toff[st][th] >= 0) ? bbase[b] + toff[st][th] : N;
    };
    const bf16_t* kb = sK + 4 * (s & 3) + 32 * ksB;
    const bf16_t* vb = sV + 4 * (s & 3) + 16 * ct;
#pragma unroll
    for (int b = 0; b < MM; ++b) {
      f32x4_t sb[2] = {zero4(), zero4()};
#pragma unroll
      for (int st = 0; st < KS; ++st) {
        const int r0 = row(b, st, 0), r1 = row(b, st, 1);
        const u16x8_t bv = lds_tr8_rows(vb, RS, r0, r1);
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
          sb[hh] = mfma_bf16(lds_tr8_rows(kb + 16 * hh, RS, r0, r1), bv, sb[hh]);
      }
#pragma unroll
      for (int i = 0; i < MM; ++i) {
        mix[i][0] += wr[i][b] * sb[0];
        mix[i][1] += wr[i][b] * sb[1];
      }
    }
    // z_b = sum_j phi(K_b)[j] for this item's 32 features, blocks b = ct, ct+NT, ..
    // (a ones B operand puts z_b in every column)
    const u16x8_t ones = {0x3f80, 0x3f80, 0x3f80, 0x3f80, 0x3f80, 0x3f80, 0x3f80, 0x3f80};
    for (int b = ct; b < M; b += NT) {
      const int bb = blockbase(b);
      f32x4_t zb[2] = {zero4(), zero4()};
#pragma unroll
      for (int st = 0; st < KS; ++st) {
        const int r0 = toff[st][0] >= 0 ? bb + toff[st][0] : N;
        const int r1 = toff[st][1] >= 0 ? bb + toff[st][1] : N;
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
          zb[hh] = mfma_bf16(lds_tr8_rows(kb + 16 * hh, RS, r0, r1), ones, zb[hh]);
      }
      if (s == 0) {
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
          *reinterpret_cast<f32x4_t*>(zraw + b * DP + 32 * ksB + 16 * hh + 4 * grp) = zb[hh];
      }
    }
  }

  // ---- stage phi(Q) (its loads were issued with K and V) -------------------
#pragma unroll
  for (int bt = 0; bt < 2; ++bt) {
    const int base = bt * U * kFusedThreads;
    if (base < items) {
      if (bt > 0) { MHLA_LOAD(qr, Q, base) }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int it = base + u * kFusedThreads + tid;
        if (it < items) {
          const int t = small_div(it, inv8);
          const int f = it - t * F8;
          *reinterpret_cast<u32x4_t*>(sQ + t * RSQ + 8 * f) = phi8<PHI>(qr[u]);
        }
      }
    }
  }
#undef MHLA_LOAD
  lds_barrier();  // phi(K) / V are no longer read; z_b and phi(Q) are complete

  // ---- C. exchange the mixed tiles; z~ ----------------------------------------
  if (has_item) {
#pragma unroll
    for (int i = 0; i < MM; ++i)
      if (i < M) frag[((i * NT + ct) * DS + ksB) * 64 + lane] = pack_acc8(mix[i][0], mix[i][1]);
  }
  for (int e = tid; e < M * DP; e += kFusedThreads) {
    const int i = e / DP, k = e - i * DP;
    float acc = 0.0f;
    for (int b = 0; b < M; ++b) acc += Wh[i * M + b] * zraw[b * DP + k];
    zmix[e] = acc;
  }
  lds_barrier();

  // ---- D. readout ------------------------------------------------------------
  // Wave w takes tiles w*tpw .. w*tpw+tpw-1 (16 queries each; consecutive tiles
  // share a block), so the S~_i fragments are read once per block and wave.
  const int ntile = M * QT;
  const int tpw = (ntile + kFusedWaves - 1) / kFusedWaves;
  int cur = -1, bb = 0;
  u16x8_t af[NT][DS], az[DS];
  for (int u = 0; u < tpw; ++u) {
    const int tile = wave * tpw + u;
    if (tile >= ntile) break;
    const int i = tile / QT, qt = tile - i * QT;
    if (qt * 16 >= nb) continue;
    if (i != cur) {
      cur = i;
      bb = blockbase(i);
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
    const int j = qt * 16 + s;
    const int t = j < nb ? bb + tokoff(j) : N;
    u16x8_t bq[DS];
#pragma unroll
    for (int ks = 0; ks < DS; ++ks) {
      const bf16_t* p = sQ + t * RSQ + 32 * ks + 4 * grp;
      bq[ks] = from_u2x2(*reinterpret_cast<const uint2*>(p),
                         *reinterpret_cast<const uint2*>(p + 16));
    }
    f32x4_t o[NT], oz = zero4();
#pragma unroll
    for (int c = 0; c < NT; ++c) {
      o[c] = zero4();
#pragma unroll
      for (int ks = 0; ks < DS; ++ks) o[c] = mfma_bf16(af[c][ks], bq[ks], o[c]);
    }
#pragma unroll
    for (int ks = 0; ks < DS; ++ks) oz = mfma_bf16(az[ks], bq[ks], oz);
    // row 0 of the z~ tile (lane s of group 0, element 0) is phi(q).z~_i
    const float den = __shfl(oz[0], s);
    const float rd = den == 0.0f ? 0.0f : 1.0f / den;
    if (j < nb) {
      bf16_t* yrow = Y + off + (size_t)t * d;
#pragma unroll
      for (int c = 0; c < NT; ++c) {
        const int cl = 16 * c + 4 * grp;
        if (cl < d)
          *reinterpret_cast<uint2*>(yrow + cl) =
              make_uint2(pack2(o[c][0] * rd, o[c][1] * rd), pack2(o[c][2] * rd, o[c][3] * rd));
      }
    }
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
