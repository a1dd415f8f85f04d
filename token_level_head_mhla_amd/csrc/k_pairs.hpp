// k_pairs.hpp -- MHLA forward in the token-pair order of "MHLA: Restoring
// Expressivity of Linear Attention via Token-Level Multi-Head" §4.2 Eq. 5
// (bf16 in/out, gfx950 MFMA), for blocks of at most 16 tokens:
//
//   Y_q = sum_b W[i,b] sum_{j in b} (phi(q).phi(k_j)) v_j
//         / sum_b W[i,b] sum_{j in b} phi(q).phi(k_j),      q in block i.
//
// This is the same result as the summary order up to rounding (the
// summaries S_b are never formed), and it is the cheaper order when a block
// has fewer tokens than d, because it needs no d x d state per block and no
// workspace at all.
//
// One workgroup of 8 waves per (batch, head) slice; each wave owns query
// blocks i = wave, wave + 8, ...  K and V of the slice are staged in LDS
// (phi applied to K; V gets an extra column of ones at index d, so the
// denominator falls out of the same product as row d of O^T).  For every
// pair of key blocks (b0, b1):
//   P^T[j][q] = phi(K_b) phi(Q_i)^T          (16x16 per block, MFMA over d)
//   P'^T      = W[i,b] P^T, packed to bf16 -- already the B-operand layout
//               of the next product (contraction over the 32 keys)
//   O^T      += V_{b0,b1}^T P'^T             (MFMA 16x16x32, V^T from LDS
//                                             transpose reads)
// Finally Y_q = O^T[0..d-1][q] / O^T[d][q], with a zero row when O^T[d][q] = 0.
#pragma once

#include "mhla_mfma.hpp"

namespace mhla {

constexpr int kPairsThreads = 512;
constexpr int kPairsWaves = kPairsThreads / 64;
constexpr int kPairsMaxQB = 4;  // query blocks per wave (M <= 32)

// Feature operands of phi(K) phi(Q)^T in steps of 32 (lane group g holds
// features 32 ks + 8g .. +7).  When DK is not a multiple of 32 the last step
// (ks == ks_full) covers 16 features and groups 2 and 3 hold zeros, so that
// every product is a 16x16x32 MFMA.  (A 16x16x16 MFMA for the tail would
// accumulate onto the result of a 16x16x32 one; on gfx950 such a dependent
// pair of different shapes reads a wrong accumulator when it issues back to
// back, and the compiler inserts no wait states between them.)
//   feat_operand: from global row `tok` (phi applied; features past d and
//                 tok < 0 give 0)
//   feat_row:     from an LDS row of phi values (pad columns already 0)
// The load is unconditional (token and feature clamped in range) and masked
// afterwards: a load under a branch makes the compiler wait for it at the
// join, which would issue a wave's operand loads one round trip at a time.
template <int PHI>
__device__ __forceinline__ u16x8_t feat_operand(const bf16_t* base, int tok, int d, int ks,
                                                int ks_full, int grp) {
  const int k0 = 32 * ks + 8 * grp;
  const bool ok = tok >= 0 && k0 < d && (ks < ks_full || grp < 2);
  const u32x4_t v =
      *reinterpret_cast<const u32x4_t*>(base + (size_t)(tok > 0 ? tok : 0) * d + min(k0, d - 8));
  return __builtin_bit_cast(u16x8_t, ok ? phi8<PHI>(v) : u32x4_t{0u, 0u, 0u, 0u});
}

__device__ __forceinline__ u16x8_t feat_row(const bf16_t* lds, int row, int rs, int ks,
                                            int ks_full, int grp) {
  if (ks == ks_full && grp >= 2) return u16x8_t{0, 0, 0, 0, 0, 0, 0, 0};
  return *reinterpret_cast<const u16x8_t*>(lds + (size_t)row * rs + 32 * ks + 8 * grp);
}

// DK: contraction width over features (multiple of 16: 32-steps plus an
// optional 16-step tail).  DO: rows of O^T (multiple of 16, > d: the row d
// holds the denominator).
// LDS rows are in member order: row b * nb + m holds the token of member m of
// block b, so that the members of a block occupy consecutive rows (row N is
// all zero).  Row strides of 16 (mod 32) elements keep the 16-row transpose
// reads and the 16-byte row reads of one block free of bank conflicts.
__host__ __device__ constexpr int pairs_rs(int w) { return (w + 15) / 32 * 32 + 16; }

// Element offset of LDS row r at row stride rs: 8 more elements after every 8
// rows, so that rows r and r + 8 of a block do not share banks in the 8- and
// 16-byte row reads.
__host__ __device__ constexpr int prow(int r, int rs) { return r * rs + (r >> 3) * 8; }
// Elements of rows 0 .. N at stride rs.
__host__ __device__ constexpr size_t prow_elems(int N, int rs) { return (size_t)prow(N + 1, rs) + 8; }

template <int DK, int DO>
struct PairsLayout {
  static constexpr int RSK = pairs_rs(DK);  // LDS row stride of phi(K)
  static constexpr int RSV = pairs_rs(DO);  // LDS row stride of V (+ ones column)
  static constexpr int KS = DK / 32;   // full 32-feature steps
  static constexpr bool TAIL = (DK % 32) != 0;
  static constexpr int KSF = KS + (TAIL ? 1 : 0);  // steps, the last one maybe half empty
  static constexpr int CT = DO / 16;   // O^T row tiles
  __host__ __device__ static size_t k_bytes(int N) { return prow_elems(N, RSK) * 2; }
  __host__ __device__ static size_t v_bytes(int N) { return prow_elems(N, RSV) * 2; }
  __host__ __device__ static size_t total(int N, int M) {
    return k_bytes(N) + v_bytes(N) + (size_t)M * M * 4 + (size_t)kPairsMaxM * 4;
  }
  static constexpr int kPairsMaxM = 32;
};

template <int DK, int DO, int QB, int PHI>
__global__ __launch_bounds__(kPairsThreads) void k_pairs(
    const bf16_t* __restrict__ Q, const bf16_t* __restrict__ K, const bf16_t* __restrict__ V,
    const float* __restrict__ W, bf16_t* __restrict__ Y, Geo g, int H, int N, int d) {
  using L = PairsLayout<DK, DO>;
  constexpr int RSK = L::RSK, RSV = L::RSV, KS = L::KS, KSF = L::KSF, CT = L::CT;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int M = g.M, nb = g.nb;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int s = lane & 15, grp = lane >> 4;
  const long slice = blockIdx.x;
  const int h = (int)(slice % H);
  const size_t off = (size_t)slice * N * d;
  bf16_t* sK = reinterpret_cast<bf16_t*>(smem);
  bf16_t* sV = reinterpret_cast<bf16_t*>(smem + L::k_bytes(N));
  float* sW = reinterpret_cast<float*>(smem + L::k_bytes(N) + L::v_bytes(N));
  int* sB = reinterpret_cast<int*>(sW + M * M);  // first token of every block

  // ---- stage: zero pad columns and row N, then phi(K), V, ones column ------
  // The K and V loads of a batch of kStageU 16-byte chunks per thread are all
  // issued (clamped in range) before the LDS is zero-filled, so that they are
  // in flight together; the chunks are written once the fill is done.
  constexpr int kStageU = 6;
  const int F8 = d >> 3;
  const int items = N * F8;
  const float inv8 = 1.0f / (float)F8, invnb = 1.0f / (float)nb;
  u32x4_t kst[kStageU], vst[kStageU];
  int dst[kStageU];
  auto stage_load = [&](int base) {
#pragma unroll
    for (int u = 0; u < kStageU; ++u) {
      const int it = base + u * kPairsThreads + tid;
      const int itc = it < items ? it : items - 1;
      const int row = (int)(((float)itc + 0.5f) * inv8);
      const int f = itc - row * F8;
      const int b = (int)(((float)row + 0.5f) * invnb);
      const size_t src = off + (size_t)(g.blockbase(b) + g.tokoff(row - b * nb)) * d + 8 * f;
      kst[u] = *reinterpret_cast<const u32x4_t*>(K + src);
      vst[u] = *reinterpret_cast<const u32x4_t*>(V + src);
      dst[u] = it < items ? (row << 8) | f : -1;  // f < 16, row <= 512
    }
  };
  auto stage_store = [&]() {
#pragma unroll
    for (int u = 0; u < kStageU; ++u) {
      if (dst[u] >= 0) {
        const int row = dst[u] >> 8, f = dst[u] & 255;
        *reinterpret_cast<u32x4_t*>(sK + prow(row, RSK) + 8 * f) = phi8<PHI>(kst[u]);
        *reinterpret_cast<u32x4_t*>(sV + prow(row, RSV) + 8 * f) = vst[u];
      }
    }
  };
  // W (M * M <= 1024 entries: two per thread) is requested first, so that
  // waiting for it does not wait for the K / V loads behind it
  static_assert(2 * kPairsThreads >= 32 * 32, "W entries per thread");
  const float* Wh = W + (size_t)h * M * M;
  const float wv0 = tid < M * M ? Wh[tid] : 0.0f;
  const float wv1 = tid + kPairsThreads < M * M ? Wh[tid + kPairsThreads] : 0.0f;
  stage_load(0);
  for (int e = tid; e < (int)((L::k_bytes(N) + L::v_bytes(N)) / 16); e += kPairsThreads)
    reinterpret_cast<u32x4_t*>(smem)[e] = u32x4_t{0u, 0u, 0u, 0u};
  if (tid < M * M) sW[tid] = wv0;
  if (tid + kPairsThreads < M * M) sW[tid + kPairsThreads] = wv1;
  for (int b = tid; b < M; b += kPairsThreads) sB[b] = g.blockbase(b);
  lds_barrier();
  stage_store();
  for (int base = kStageU * kPairsThreads; base < items; base += kStageU * kPairsThreads) {
    stage_load(base);
    stage_store();
  }
  for (int t = tid; t < N; t += kPairsThreads) sV[prow(t, RSV) + d] = 0x3f80;  // bf16 1.0
  lds_barrier();

  // ---- this wave's query blocks: phi(Q) operands straight from global -------
  // B operand of P^T = phi(K) phi(Q)^T: lane (s, grp) holds query s of the
  // block, features 32ks + 8grp .. +7 (and 32KS + 4grp .. +3 for the tail).
  const int myq = (M - wave + kPairsWaves - 1) / kPairsWaves;  // query blocks of this wave
  int qtok[QB];
  u16x8_t qf[QB][KSF];
#pragma unroll
  for (int u = 0; u < QB; ++u) {
    const int i = wave + u * kPairsWaves;
    const bool real = u < myq && s < nb;
    qtok[u] = real ? sB[i] + g.tokoff(s) : -1;
#pragma unroll
    for (int ks = 0; ks < KSF; ++ks) qf[u][ks] = feat_operand<PHI>(Q + off, qtok[u], d, ks, KS, grp);
  }

  f32x4_t o[QB][CT];
#pragma unroll
  for (int u = 0; u < QB; ++u)
#pragma unroll
    for (int c = 0; c < CT; ++c) o[u][c] = zero4();

  // key member s of a block: row of this lane for the phi(K) A operand;
  // key member 4grp + s/4: row supplied to the V^T transpose reads
  const int vj = 4 * grp + (s >> 2);
  for (int b0 = 0; b0 < M; b0 += 2) {
    const int b1 = b0 + 1;
    int kr[2], vr[2];
    float wb[2][QB];
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      const int b = b0 + hb;
      const bool real = b < M;
      kr[hb] = (real && s < nb) ? b * nb + s : N;
      vr[hb] = (real && vj < nb) ? b * nb + vj : N;
#pragma unroll
      for (int u = 0; u < QB; ++u) {
        const int i = wave + u * kPairsWaves;
        wb[hb][u] = (real && u < myq) ? sW[i * M + b] : 0.0f;
      }
    }
    (void)b1;
    // phi(K) A operands of the two key blocks (row = key member s)
    u16x8_t ka[2][KSF];
#pragma unroll
    for (int hb = 0; hb < 2; ++hb)
#pragma unroll
      for (int ks = 0; ks < KSF; ++ks) ka[hb][ks] = feat_row(sK, prow(kr[hb], RSK), 1, ks, KS, grp);
    // V^T A operands: rows c = 16ct + s, keys {4grp..4grp+3} of b0 then of b1
    u16x8_t va[CT];
#pragma unroll
    for (int c = 0; c < CT; ++c)
      va[c] = lds_tr8_rows(sV + 16 * c + 4 * (s & 3), 1, prow(vr[0], RSV), prow(vr[1], RSV));
#pragma unroll
    for (int u = 0; u < QB; ++u) {
      if (u >= myq) break;
      f32x4_t p[2];
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) {
        p[hb] = zero4();
#pragma unroll
        for (int ks = 0; ks < KSF; ++ks) p[hb] = mfma_bf16(ka[hb][ks], qf[u][ks], p[hb]);
        p[hb] *= wb[hb][u];
      }
      // p[hb] lane (s, grp) element r = P'^T[key 4grp + r of block b0+hb][query s]
      const u16x8_t pb = pack_acc8(p[0], p[1]);
#pragma unroll
      for (int c = 0; c < CT; ++c) o[u][c] = mfma_bf16(va[c], pb, o[u][c]);
    }
  }

  // ---- epilogue: row d of O^T is the denominator ------------------------------
  const int dct = d >> 4, dg = (d & 15) >> 2, dr = d & 3;
#pragma unroll
  for (int u = 0; u < QB; ++u) {
    if (u >= myq) break;
    float dv = 0.0f;
#pragma unroll
    for (int c = 0; c < CT; ++c)
      if (c == dct) dv = o[u][c][dr];
    const float den = __shfl(dv, 16 * dg + s);
    const float rd = out_scale(g, den);
    store_row_tiles<CT>(qtok[u] >= 0 ? Y + off + (size_t)qtok[u] * d : nullptr, d, o[u], rd, grp);
  }
}

inline int pairs_dk(int d) { return (d + 15) / 16 * 16; }
inline int pairs_do(int d) { return (d + 1 + 15) / 16 * 16; }

template <int DK, int DO>
inline size_t pairs_lds_t(int N, int M) { return PairsLayout<DK, DO>::total(N, M); }

// (DK, DO) pairs compiled: d = 16 (16, 32), 32 (32, 48), 48 (48, 64), 64 (64, 80),
// 72 (80, 80), 80 (80, 96), 96 (96, 112).
inline bool pairs_dims(int d, int* dk, int* dout) {
  *dk = pairs_dk(d);
  *dout = pairs_do(d);
  switch (d) {
    case 16: case 32: case 48: case 64: case 72: case 80: case 96: return true;
    default: return false;
  }
}

inline size_t pairs_lds(int d, int N, int M) {
  switch (d) {
    case 16: return pairs_lds_t<16, 32>(N, M);
    case 32: return pairs_lds_t<32, 48>(N, M);
    case 48: return pairs_lds_t<48, 64>(N, M);
    case 64: return pairs_lds_t<64, 80>(N, M);
    case 72: return pairs_lds_t<80, 80>(N, M);
    case 80: return pairs_lds_t<80, 96>(N, M);
    default: return pairs_lds_t<96, 112>(N, M);
  }
}

inline bool pairs_supports(int dtype, int d, int M, int nb, int N) {
  int dk, dout;
  if (dtype != 1 || !pairs_dims(d, &dk, &dout)) return false;
  if (nb > 16 || M > kPairsWaves * kPairsMaxQB) return false;
  return pairs_lds(d, N, M) <= 160 * 1024;
}

template <int DK, int DO, int QB, int PHI>
int launch_pairs_t(long slices, int H, int N, int d, const Geo& g, const bf16_t* Q,
                   const bf16_t* K, const bf16_t* V, const float* W, bf16_t* Y, hipStream_t st) {
  const size_t lds = PairsLayout<DK, DO>::total(N, g.M);
  static std::atomic<bool> attr_set[64];
  if (lds_limit_once(reinterpret_cast<const void*>(&k_pairs<DK, DO, QB, PHI>), attr_set,
                     160 * 1024) != 0)
    return -1;
  k_pairs<DK, DO, QB, PHI><<<dim3((unsigned)slices), dim3(kPairsThreads), lds, st>>>(
      Q, K, V, W, Y, g, H, N, d);
  launch_mark(st, "k_pairs");
  return 0;
}

template <int DK, int DO, int PHI>
int launch_pairs_q(long slices, int H, int N, int d, const Geo& g, const bf16_t* Q,
                   const bf16_t* K, const bf16_t* V, const float* W, bf16_t* Y, hipStream_t st) {
  const int qb = (g.M + kPairsWaves - 1) / kPairsWaves;
  if (qb <= 1) return launch_pairs_t<DK, DO, 1, PHI>(slices, H, N, d, g, Q, K, V, W, Y, st);
  if (qb <= 2) return launch_pairs_t<DK, DO, 2, PHI>(slices, H, N, d, g, Q, K, V, W, Y, st);
  return launch_pairs_t<DK, DO, 4, PHI>(slices, H, N, d, g, Q, K, V, W, Y, st);
}

template <int PHI>
int launch_pairs_p(long slices, int H, int N, int d, const Geo& g, const bf16_t* Q,
                   const bf16_t* K, const bf16_t* V, const float* W, bf16_t* Y, hipStream_t st) {
  switch (d) {
    case 16: return launch_pairs_q<16, 32, PHI>(slices, H, N, d, g, Q, K, V, W, Y, st);
    case 32: return launch_pairs_q<32, 48, PHI>(slices, H, N, d, g, Q, K, V, W, Y, st);
    case 48: return launch_pairs_q<48, 64, PHI>(slices, H, N, d, g, Q, K, V, W, Y, st);
    case 64: return launch_pairs_q<64, 80, PHI>(slices, H, N, d, g, Q, K, V, W, Y, st);
    case 72: return launch_pairs_q<80, 80, PHI>(slices, H, N, d, g, Q, K, V, W, Y, st);
    case 80: return launch_pairs_q<80, 96, PHI>(slices, H, N, d, g, Q, K, V, W, Y, st);
    default: return launch_pairs_q<96, 112, PHI>(slices, H, N, d, g, Q, K, V, W, Y, st);
  }
}

inline int launch_pairs(long slices, int H, int N, int d, const Geo& g, int phi, const bf16_t* Q,
                        const bf16_t* K, const bf16_t* V, const float* W, bf16_t* Y,
                        hipStream_t st) {
  if (phi == PHI_RELU) return launch_pairs_p<PHI_RELU>(slices, H, N, d, g, Q, K, V, W, Y, st);
  return launch_pairs_p<PHI_ELU1>(slices, H, N, d, g, Q, K, V, W, Y, st);
}

}  // namespace mhla
