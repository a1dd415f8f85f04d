// k_causal.hpp -- readout of the chunkwise causal MHLA forward (bf16 in/out,
// gfx950 MFMA): "MHLA: Restoring Expressivity of Linear Attention via
// Token-Level Multi-Head" §4.2 ("Chunkwise parallel form of MHLA") and App. C.
//
// Blocks are consecutive chunks of nb tokens.  The summary kernel and the
// mixing GEMM of the blocked path run first, the mixing with W[i,b] = 0 for
// b >= i, so the workspace row of chunk i holds the prefix mixture
//   S^<_i = sum_{b<i} W[i,b] S_b,   z^<_i = sum_{b<i} W[i,b] z_b.
// This kernel adds the causal part of the query's own chunk:
//   num_q = phi(q) S^<_i + W[i,i] sum_{j in chunk i, j <= q} (phi(q).phi(k_j)) v_j
//   den_q = phi(q).z^<_i + W[i,i] sum_{j in chunk i, j <= q} phi(q).phi(k_j)
//   Y_q   = num_q / den_q   (or num_q with the normaliser off).
//
// One workgroup of 4 waves per (chunk, slice).  phi(K) and V of the chunk are
// staged in LDS (rows past nb are zero).  Wave w takes the 16-query tiles
// w, w + 4, ...; for each it computes Y^T in one set of accumulators: the
// prefix term from the workspace row (as in the plain readout), then, for
// every 32 keys up to the tile's last query, P^T = phi(K) phi(Q)^T on MFMA,
// masked (key > query -> 0) and scaled by W[i,i], packed to bf16 as the B
// operand of O^T += V^T P'^T (V^T from LDS transpose reads).  A ones row in
// the extra accumulator tile adds the chunk's part of the denominator to the
// prefix part phi(q).z^<_i.
#pragma once

#include "k_blocked.hpp"

namespace mhla {

constexpr int kCausalMaxNb = 256;

__host__ __device__ constexpr int causal_nbp(int nb) { return (nb + 31) / 32 * 32; }

template <int DP>
inline size_t causal_lds(int nb) {
  return 2 * (size_t)causal_nbp(nb) * BlockedDims<DP>::RS * sizeof(bf16_t);
}

// Static LDS of k_readout_causal: the per-wave output staging (d = 32, 64).
template <int DP>
constexpr size_t causal_stage_bytes() {
  return (DP == 64 || DP == 32) ? (size_t)kBlkWaves * 16 * (DP + 8) * sizeof(bf16_t) : 2;
}

template <int DP, int PHI>
__global__ __launch_bounds__(kBlkThreads) void k_readout_causal(
    const bf16_t* __restrict__ Q, const bf16_t* __restrict__ K, const bf16_t* __restrict__ V,
    const float* __restrict__ W, const bf16_t* __restrict__ St, bf16_t* __restrict__ Y, Geo g,
    int H, int N, int d) {
  using D = BlockedDims<DP>;
  constexpr int NT = D::NT, DS = D::DS, EP = D::EP, RS = D::RS;
  constexpr int F8P = DP / 8;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int nb = g.nb, M = g.M;
  const int NBP = causal_nbp(nb);
  bf16_t* sK = reinterpret_cast<bf16_t*>(smem);
  bf16_t* sV = sK + (size_t)NBP * RS;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int s = lane & 15, grp = lane >> 4;
  const long slice = blockIdx.y;
  const int i = blockIdx.x;
  const int h = (int)(slice % H);
  const size_t off = (size_t)slice * N * d;
  const int base = i * nb;  // first token of the chunk
  const int F8 = d >> 3;

  // ---- stage phi(K) and V of the chunk; rows >= nb and features >= d are 0 --
  // The loads of kStageU chunks per thread are issued together (clamped in
  // range, so that every load is issued), then written.
  constexpr int kStageU = 2;
  for (int it0 = 0; it0 < NBP * F8P; it0 += kStageU * kBlkThreads) {
    u32x4_t kr[kStageU], vr[kStageU];
#pragma unroll
    for (int u = 0; u < kStageU; ++u) {
      const int it = it0 + u * kBlkThreads + tid;
      const int j = it / F8P, f = it - (it / F8P) * F8P;
      const size_t src = off + (size_t)(base + min(j, nb - 1)) * d + 8 * min(f, F8 - 1);
      kr[u] = *reinterpret_cast<const u32x4_t*>(K + src);
      vr[u] = *reinterpret_cast<const u32x4_t*>(V + src);
    }
#pragma unroll
    for (int u = 0; u < kStageU; ++u) {
      const int it = it0 + u * kBlkThreads + tid;
      const int j = it / F8P, f = it - (it / F8P) * F8P;
      if (it < NBP * F8P) {
        const bool real = j < nb && f < F8;
        const u32x4_t zero = u32x4_t{0u, 0u, 0u, 0u};
        *reinterpret_cast<u32x4_t*>(sK + j * RS + 8 * f) = real ? phi8<PHI>(kr[u]) : zero;
        *reinterpret_cast<u32x4_t*>(sV + j * RS + 8 * f) = real ? vr[u] : zero;
      }
    }
  }

  // ---- prefix mixture S^<_i (transposed rows) and z^<_i from the workspace ----
  const bf16_t* row = St + ((size_t)slice * M + i) * EP;
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
  const float wii = W[((size_t)h * M + i) * M + i];
  const u16x8_t ones0 = s == 0 ? u16x8_t{0x3f80, 0x3f80, 0x3f80, 0x3f80, 0x3f80, 0x3f80, 0x3f80,
                                         0x3f80}
                               : u16x8_t{0, 0, 0, 0, 0, 0, 0, 0};
  lds_barrier();

  // rows of 128 or 64 bytes (d == DP = 64 or 32) are stored whole, through a
  // per-wave LDS staging area
  constexpr bool STAGED = DP == 64 || DP == 32;
  __shared__ __attribute__((aligned(16))) bf16_t stage_all[causal_stage_bytes<DP>() / 2];
  bf16_t* stage = stage_all + wave * 16 * (DP + 8);
  const bool whole_rows = STAGED && d == DP;
  const bf16_t* vbase = sV + 4 * (s & 3);
  const int vj = 4 * grp + (s >> 2);  // key row this lane addresses for the V^T reads
  for (int q0 = 16 * wave; q0 < nb; q0 += 16 * kBlkWaves) {
    const int qj = q0 + s;  // this lane's query (B-operand column)
    u16x8_t bq[DS];
#pragma unroll
    for (int ks = 0; ks < DS; ++ks) {
      const int k0 = 32 * ks + 8 * grp;
      u32x4_t v = u32x4_t{0u, 0u, 0u, 0u};
      if (qj < nb && k0 < d)
        // Q is read once (nontemporal); K and V are read twice per call (by the
        // summaries and by this kernel's own-chunk term), so they keep ordinary
        // loads (an LM-shaped A/B: 130.0-131.0 against 133.9-135.2 us per step)
        v = __builtin_nontemporal_load(
            reinterpret_cast<const u32x4_t*>(Q + off + (size_t)(base + qj) * d + k0));
      bq[ks] = __builtin_bit_cast(u16x8_t, phi8<PHI>(v));
    }
    f32x4_t o[NT], oz = zero4();
#pragma unroll
    for (int ct = 0; ct < NT; ++ct) {
      o[ct] = zero4();
#pragma unroll
      for (int ks = 0; ks < DS; ++ks) o[ct] = mfma_bf16(af[ct][ks], bq[ks], o[ct]);
    }
#pragma unroll
    for (int ks = 0; ks < DS; ++ks) oz = mfma_bf16(az[ks], bq[ks], oz);

    // own chunk, keys 32kp .. 32kp + 31 for every kp up to the tile's last query
    for (int k0 = 0; k0 <= q0 + 15; k0 += 32) {
      f32x4_t p[2];
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) {
        const bf16_t* krow = sK + (k0 + 16 * hb + s) * RS + 8 * grp;
        p[hb] = zero4();
#pragma unroll
        for (int ks = 0; ks < DS; ++ks)
          p[hb] = mfma_bf16(*reinterpret_cast<const u16x8_t*>(krow + 32 * ks), bq[ks], p[hb]);
        // element r: key k0 + 16hb + 4grp + r, query q0 + s
#pragma unroll
        for (int r = 0; r < 4; ++r)
          p[hb][r] = (k0 + 16 * hb + 4 * grp + r <= qj) ? p[hb][r] * wii : 0.0f;
      }
      const u16x8_t pb = pack_acc8(p[0], p[1]);
#pragma unroll
      for (int ct = 0; ct < NT; ++ct)
        o[ct] = mfma_bf16(lds_tr8_rows(vbase + 16 * ct, RS, k0 + vj, k0 + 16 + vj), pb, o[ct]);
      oz = mfma_bf16(ones0, pb, oz);
    }

    const float rd = out_scale(g, __shfl(oz[0], s));
    bf16_t* yrow = qj < nb ? Y + off + (size_t)(base + qj) * d : nullptr;
    if constexpr (STAGED) {
      if (whole_rows) {
        store_rows_staged<NT, true>(yrow, stage, o, rd, lane);
        continue;
      }
    }
    store_row_tiles<NT, true>(yrow, d, o, rd, grp);
  }
}

// Blocks are runs of consecutive tokens in block order: every block spans the
// full extent of each grid axis to the right of its first partial axis.
inline bool blocks_contiguous(const Geo& g) {
  if (g.bw < g.Wg) return g.bh == 1 && g.bt == 1;
  if (g.bh < g.Hg) return g.bt == 1;
  return true;
}

inline bool causal_supports(int dtype, int d, const Geo& g, long slices) {
  return blocks_contiguous(g) && g.nb <= kCausalMaxNb && blocked_supports(dtype, d, g.M, slices);
}

template <int DP, int PHI>
int launch_readout_causal(long slices, int H, int N, int d, const Geo& g, const bf16_t* Q,
                          const bf16_t* K, const bf16_t* V, const float* W, const bf16_t* St,
                          bf16_t* Y, hipStream_t st) {
  const size_t lds = causal_lds<DP>(g.nb);
  static std::atomic<bool> attr_set[64];
  // the dynamic part may use what the static staging leaves of the 160 KB
  if (lds > 64 * 1024 - causal_stage_bytes<DP>() &&
      lds_limit_once(reinterpret_cast<const void*>(&k_readout_causal<DP, PHI>), attr_set,
                     (int)(160 * 1024 - causal_stage_bytes<DP>())) != 0)
    return -1;
  k_readout_causal<DP, PHI><<<dim3((unsigned)g.M, (unsigned)slices), kBlkThreads, lds, st>>>(
      Q, K, V, W, St, Y, g, H, N, d);
  launch_mark(st, "k_readout_causal");
  return 0;
}

template <int DP, int PHI>
int launch_causal_t(long slices, int H, int N, int d, const Geo& g, const bf16_t* Q,
                    const bf16_t* K, const bf16_t* V, const float* W, bf16_t* Y, bf16_t* ws,
                    hipStream_t st) {
  const bf16_t* St = launch_summary_mix<DP, PHI>(slices, H, N, d, g, K, V, W, ws,
                                                 blocked_coef_scratch<DP>(ws, slices, g.M), 1, st);
  return launch_readout_causal<DP, PHI>(slices, H, N, d, g, Q, K, V, W, St, Y, st);
}

template <int PHI>
int launch_causal_p(long slices, int H, int N, int d, const Geo& g, const bf16_t* Q,
                    const bf16_t* K, const bf16_t* V, const float* W, bf16_t* Y, bf16_t* ws,
                    hipStream_t st) {
  switch (blocked_dp(d)) {
    case 32: return launch_causal_t<32, PHI>(slices, H, N, d, g, Q, K, V, W, Y, ws, st);
    case 64: return launch_causal_t<64, PHI>(slices, H, N, d, g, Q, K, V, W, Y, ws, st);
    default: return launch_causal_t<96, PHI>(slices, H, N, d, g, Q, K, V, W, Y, ws, st);
  }
}

// Chunkwise causal forward: summaries, prefix mixing, causal readout.  The
// workspace is the blocked path's (S, S~ and the mixing coefficients).
inline int launch_causal(long slices, int H, int N, int d, const Geo& g, int phi,
                         const bf16_t* Q, const bf16_t* K, const bf16_t* V, const float* W,
                         bf16_t* Y, bf16_t* ws, hipStream_t st) {
  if (phi == PHI_RELU)
    return launch_causal_p<PHI_RELU>(slices, H, N, d, g, Q, K, V, W, Y, ws, st);
  return launch_causal_p<PHI_ELU1>(slices, H, N, d, g, Q, K, V, W, Y, ws, st);
}

}  // namespace mhla
