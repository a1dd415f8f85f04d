// k_generic.hpp -- three-kernel MHLA forward on the vector ALUs (fp32 math).
//
// Follows the three steps of "MHLA: Restoring Expressivity of Linear
// Attention via Token-Level Multi-Head" §4.1:
//   k_summary_valu : S_b = sum_{j in b} phi(K_j) V_j^T, z_b = sum_j phi(K_j)
//   k_mix_valu     : S~_i = sum_b W[i,b] S_b, z~_i = sum_b W[i,b] z_b
//   k_readout_valu : Y_q = phi(Q_q) S~_i / (phi(Q_q) . z~_i)
// Every input dtype (fp32, bf16) is widened to fp32; accumulation is fp32.
//
// Workspace rows: one row of L = d*d + d floats per (slice, block); the first
// d*d entries hold the summary transposed (entry c*d + k is S[k][c], i.e.
// value column c, key feature k), the last d hold z.  Mixing is elementwise
// along a row, so the same layout serves S and S~.
#pragma once

#include "mhla_common.hpp"

namespace mhla {

constexpr int kValuThreads = 256;
constexpr int kSumChunk = 32;   // tokens staged per pass in the summary kernel
constexpr int kMixRows = 16;    // query blocks per mixing workgroup
constexpr int kMixCols = 64;    // key blocks staged per pass in the mixing kernel
constexpr int kReadTok = 64;    // query tokens staged per pass in the readout
constexpr int kReadCols = 32;   // value columns staged per pass in the readout

// grid = (M, B*H); block = 256.  d <= 128 so d*d/256 <= 64 entries per thread.
template <typename T>
__global__ __launch_bounds__(kValuThreads) void k_summary_valu(
    const T* __restrict__ K, const T* __restrict__ V, float* __restrict__ S,
    Geo g, int N, int d, int phi) {
  __shared__ float sk[kSumChunk][129];
  __shared__ float sv[kSumChunk][129];
  const int b = blockIdx.x;
  const long bh = blockIdx.y;
  const int tid = threadIdx.x;
  const int dd = d * d;
  const T* Kb = K + bh * (long)N * d;
  const T* Vb = V + bh * (long)N * d;
  float acc[64];
#pragma unroll
  for (int r = 0; r < 64; ++r) acc[r] = 0.0f;
  float zacc = 0.0f;

  for (int j0 = 0; j0 < g.nb; j0 += kSumChunk) {
    const int nj = min(kSumChunk, g.nb - j0);
    for (int e = tid; e < nj * d; e += kValuThreads) {
      const int j = e / d, a = e - (e / d) * d;
      const long t = g.token(b, j0 + j);
      sk[j][a] = phi_apply(phi, Elt<T>::load(Kb + t * d + a));
      sv[j][a] = Elt<T>::load(Vb + t * d + a);
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < 64; ++r) {
      const int e = tid + r * kValuThreads;
      if (e < dd) {
        const int c = e / d, k = e - c * d;
        float s = acc[r];
        for (int j = 0; j < nj; ++j) s = fmaf(sk[j][k], sv[j][c], s);
        acc[r] = s;
      }
    }
    if (tid < d)
      for (int j = 0; j < nj; ++j) zacc += sk[j][tid];
    __syncthreads();
  }
  float* row = S + (bh * g.M + b) * (long)(dd + d);
#pragma unroll
  for (int r = 0; r < 64; ++r) {
    const int e = tid + r * kValuThreads;
    if (e < dd) row[e] = acc[r];
  }
  if (tid < d) row[dd + tid] = zacc;
}

// grid = (ceil(L/256), ceil(M/16), B*H); block = 256.
__global__ __launch_bounds__(kValuThreads) void k_mix_valu(
    const float* __restrict__ S, const float* __restrict__ W, float* __restrict__ St,
    int M, int L, int H) {
  __shared__ float sw[kMixRows][kMixCols];
  const long bh = blockIdx.z;
  const int h = (int)(bh % H);
  const int i0 = blockIdx.y * kMixRows;
  const int e = blockIdx.x * kValuThreads + threadIdx.x;
  const float* Sbh = S + bh * (long)M * L;
  const float* Wh = W + (long)h * M * M;
  float acc[kMixRows];
#pragma unroll
  for (int r = 0; r < kMixRows; ++r) acc[r] = 0.0f;
  for (int b0 = 0; b0 < M; b0 += kMixCols) {
    const int nbb = min(kMixCols, M - b0);
    for (int x = threadIdx.x; x < kMixRows * kMixCols; x += kValuThreads) {
      const int r = x / kMixCols, c = x % kMixCols;
      sw[r][c] = (i0 + r < M && c < nbb) ? Wh[(long)(i0 + r) * M + b0 + c] : 0.0f;
    }
    __syncthreads();
    if (e < L) {
      for (int bb = 0; bb < nbb; ++bb) {
        const float s = Sbh[(long)(b0 + bb) * L + e];
#pragma unroll
        for (int r = 0; r < kMixRows; ++r) acc[r] = fmaf(sw[r][bb], s, acc[r]);
      }
    }
    __syncthreads();
  }
  if (e < L) {
#pragma unroll
    for (int r = 0; r < kMixRows; ++r)
      if (i0 + r < M) St[(bh * M + i0 + r) * (long)L + e] = acc[r];
  }
}

// grid = (M, B*H); block = 256.
template <typename T>
__global__ __launch_bounds__(kValuThreads) void k_readout_valu(
    const T* __restrict__ Q, const float* __restrict__ St, T* __restrict__ Y,
    Geo g, int N, int d, int phi) {
  __shared__ float sq[kReadTok][129];
  __shared__ float ss[128][kReadCols + 1];
  __shared__ float sz[128];
  __shared__ float sden[kReadTok];
  const int i = blockIdx.x;
  const long bh = blockIdx.y;
  const int tid = threadIdx.x;
  const int dd = d * d;
  const float* row = St + (bh * g.M + i) * (long)(dd + d);
  const T* Qb = Q + bh * (long)N * d;
  T* Yb = Y + bh * (long)N * d;
  if (tid < d) sz[tid] = row[dd + tid];

  for (int j0 = 0; j0 < g.nb; j0 += kReadTok) {
    const int nj = min(kReadTok, g.nb - j0);
    __syncthreads();
    for (int e = tid; e < nj * d; e += kValuThreads) {
      const int j = e / d, a = e - (e / d) * d;
      const long t = g.token(i, j0 + j);
      sq[j][a] = phi_apply(phi, Elt<T>::load(Qb + t * d + a));
    }
    __syncthreads();
    if (tid < nj) {
      float den = 0.0f;
      for (int a = 0; a < d; ++a) den = fmaf(sq[tid][a], sz[a], den);
      sden[tid] = den;
    }
    for (int c0 = 0; c0 < d; c0 += kReadCols) {
      const int nc = min(kReadCols, d - c0);
      __syncthreads();
      for (int e = tid; e < nc * d; e += kValuThreads) {
        const int cc = e / d, k = e - (e / d) * d;
        ss[k][cc] = row[(long)(c0 + cc) * d + k];
      }
      __syncthreads();
      for (int e = tid; e < nj * kReadCols; e += kValuThreads) {
        const int j = e / kReadCols, cc = e % kReadCols;
        if (cc < nc) {
          float acc = 0.0f;
          for (int k = 0; k < d; ++k) acc = fmaf(sq[j][k], ss[k][cc], acc);
          const float den = sden[j];
          const long t = g.token(i, j0 + j);
          Elt<T>::store(Yb + t * d + c0 + cc, !g.norm ? acc : den == 0.0f ? 0.0f : acc / den);
        }
      }
    }
  }
}

// The three steps in one launch for problems whose slice fits in LDS (the
// launch, not the arithmetic, is what a small call costs): one workgroup per
// slice stages phi(Q), phi(K) and V with one round of loads, forms every
// block's summary, mixes every query block's S~, then every token's
// denominator and output.  Every sum is taken in the order the three kernels
// above take it (tokens of a block in order, key blocks in order, features in
// order, fma for fma).  LDS: generic_one_lds_bytes.  grid = B*H, block = 1024.
inline size_t generic_one_lds_bytes(int N, int d, int M) {
  const size_t C = (size_t)d + 1, L = (size_t)d * d + d;
  return (3 * (size_t)N * C + 2 * (size_t)M * L + (size_t)N) * sizeof(float);
}
constexpr size_t kGenericOneLds = 64 * 1024;  // the default dynamic LDS limit
constexpr int kGenericOneThreads = 1024;       // the whole slice's work in one workgroup

template <typename T>
__global__ __launch_bounds__(kGenericOneThreads) void k_generic_one(
    const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
    const float* __restrict__ W, T* __restrict__ Y, Geo g, int N, int d, int phi, int H) {
  extern __shared__ float sm1[];
  const int C = d + 1;  // LDS row stride (odd: no bank conflicts along a column)
  const int dd = d * d, L = dd + d, M = g.M, nb = g.nb;
  float* sQ = sm1;            // phi(Q) [N][C], token order of the slice
  float* sK = sQ + N * C;     // phi(K) [N][C]
  float* sV = sK + N * C;     // V [N][C]
  float* sS = sV + N * C;     // summaries [M][L] (entry c*d + k = S[k][c], then z)
  float* sT = sS + M * L;     // mixed summaries S~ [M][L]
  float* sden = sT + M * L;   // denominators [N]
  const int tid = threadIdx.x;
  const long bh = blockIdx.x;
  const int h = (int)(bh % H);
  const long off = bh * (long)N * d;
  const float* Wh = W + (long)h * M * M;

  for (int e = tid; e < N * d; e += kGenericOneThreads) {
    const int t = e / d, a = e - (e / d) * d;
    sQ[t * C + a] = phi_apply(phi, Elt<T>::load(Q + off + e));
    sK[t * C + a] = phi_apply(phi, Elt<T>::load(K + off + e));
    sV[t * C + a] = Elt<T>::load(V + off + e);
  }
  __syncthreads();
  for (int e = tid; e < M * L; e += kGenericOneThreads) {
    const int b = e / L, r = e - (e / L) * L;
    float s = 0.0f;
    if (r < dd) {
      const int c = r / d, k = r - (r / d) * d;
      for (int j = 0; j < nb; ++j) {
        const int t = g.token(b, j);
        s = fmaf(sK[t * C + k], sV[t * C + c], s);
      }
    } else {
      const int k = r - dd;
      for (int j = 0; j < nb; ++j) s += sK[g.token(b, j) * C + k];
    }
    sS[e] = s;
  }
  __syncthreads();
  for (int e = tid; e < M * L; e += kGenericOneThreads) {
    const int i = e / L, r = e - (e / L) * L;
    float a = 0.0f;
    for (int b = 0; b < M; ++b) a = fmaf(Wh[(long)i * M + b], sS[b * L + r], a);
    sT[e] = a;
  }
  __syncthreads();
  for (int e = tid; e < N; e += kGenericOneThreads) {  // e = (block i, member j)
    const int i = e / nb, j = e - (e / nb) * nb;
    const int t = g.token(i, j);
    const float* zt = sT + i * L + dd;
    float den = 0.0f;
    for (int a = 0; a < d; ++a) den = fmaf(sQ[t * C + a], zt[a], den);
    sden[t] = den;
  }
  __syncthreads();
  for (int e = tid; e < N * d; e += kGenericOneThreads) {  // e = (block i, member j, column c)
    const int ij = e / d, c = e - (e / d) * d;
    const int i = ij / nb, j = ij - (ij / nb) * nb;
    const int t = g.token(i, j);
    const float* st = sT + i * L + c * d;
    float acc = 0.0f;
    for (int k = 0; k < d; ++k) acc = fmaf(sQ[t * C + k], st[k], acc);
    const float den = sden[t];
    Elt<T>::store(Y + off + (long)t * d + c, !g.norm ? acc : den == 0.0f ? 0.0f : acc / den);
  }
}

}  // namespace mhla
