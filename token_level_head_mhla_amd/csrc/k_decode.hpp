// k_decode.hpp -- incremental (streaming) inference of the causal form, one
// token per (batch, head) slice per call: "MHLA: Restoring Expressivity of
// Linear Attention via Token-Level Multi-Head", App. C ("Causal inference").
//
// The sequence is cut into chunks of nb tokens; token t sits in chunk
// i = t / nb.  Per slice the state keeps, in fp32,
//   slots 0 .. M-1 : the chunk summaries [S_b | z_b] (rows f = key feature,
//                    columns c = value column, column d = z), finished for
//                    b < i and running for b = i;
//   slot M         : the prefix mixture [P_i | p_i] = sum_{b<i} W[i,b] [S_b | z_b],
//                    formed once when chunk i starts.
// One call:
//   t starts chunk i : P_i = sum_{b<i} W[i,b] S_b (the finished summaries are
//                      fixed from then on) and the running summary restarts;
//   every token      : S_i += phi(k_t) [v_t | 1]^T;
//   readout          : [n | den] = phi(q_t) (P_i + W[i,i] S_i),
//                      y_t = n / den (0 for den = 0), or n without the normaliser.
// This equals the chunkwise causal forward at position t.  The cost per token
// is O(d^2) (plus O(i d^2) once per chunk), independent of t.
#pragma once

#include "mhla_common.hpp"

namespace mhla {

constexpr int kDecThreads = 256;

inline size_t decode_state_elems(int d, int M) {
  return (size_t)(M + 1) * (size_t)d * (size_t)(d + 1);
}

inline size_t decode_lds_bytes(int d) {
  const size_t E = (size_t)d * (d + 1);
  return (E + 3 * (size_t)d + 2 * (size_t)(d + 1)) * sizeof(float);
}

// grid = B*H, block = 256.  q, k, v, y: [B*H, d]; W: [H, M, M]; state:
// [B*H][M+1][d][d+1] fp32.  Calls for t = 0, 1, 2, ... in order on one stream.
template <typename T, int PHI>
__global__ __launch_bounds__(kDecThreads) void k_decode_step(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const float* __restrict__ W, T* __restrict__ y, float* __restrict__ state, int H, int d, int M,
    int nb, int t, int norm) {
  extern __shared__ float smd[];
  const int C = d + 1;
  const int E = d * C;
  float* comb = smd;        // [d][C]: P_i + W[i,i] S_i after this token's update
  float* pq = comb + E;     // phi(q_t)
  float* pk = pq + d;       // phi(k_t)
  float* vv = pk + d;       // [v_t | 1]
  float* red = vv + C;      // [n | den]
  const int tid = threadIdx.x;
  const long slice = blockIdx.x;
  const int h = (int)(slice % H);
  const int i = t / nb, j = t - (t / nb) * nb;
  float* sums = state + (size_t)slice * (M + 1) * E;
  float* prefix = sums + (size_t)M * E;
  float* Si = sums + (size_t)i * E;
  const float* Wi = W + ((size_t)h * M + i) * M;
  const float wii = Wi[i];

  for (int f = tid; f < d; f += kDecThreads) {
    pq[f] = phi_apply(PHI, Elt<T>::load(q + slice * d + f));
    pk[f] = phi_apply(PHI, Elt<T>::load(k + slice * d + f));
    vv[f] = Elt<T>::load(v + slice * d + f);
  }
  if (tid == 0) vv[d] = 1.0f;
  __syncthreads();

  for (int e = tid; e < E; e += kDecThreads) {
    const int f = e / C, c = e - (e / C) * C;
    float P, s_old;
    if (j == 0) {  // chunk i starts: mix the finished chunks once, restart S_i
      P = 0.0f;
      for (int b = 0; b < i; ++b) P = fmaf(Wi[b], sums[(size_t)b * E + e], P);
      prefix[e] = P;
      s_old = 0.0f;
    } else {
      P = prefix[e];
      s_old = Si[e];
    }
    const float s_new = fmaf(pk[f], vv[c], s_old);
    Si[e] = s_new;
    comb[e] = fmaf(wii, s_new, P);
  }
  __syncthreads();

  for (int c = tid; c < C; c += kDecThreads) {
    float acc = 0.0f;
    for (int f = 0; f < d; ++f) acc = fmaf(pq[f], comb[f * C + c], acc);
    red[c] = acc;
  }
  __syncthreads();
  for (int c = tid; c < d; c += kDecThreads) {
    const float den = red[d];
    const float val = !norm ? red[c] : den == 0.0f ? 0.0f : red[c] / den;
    Elt<T>::store(y + slice * d + c, val);
  }
}

// Prefill: the state that T calls of k_decode_step (t = 0 .. T-1) leave, from
// the prompt's K and V in one pass.  k_decode_prefill_sums forms the summary
// of every chunk the prompt touches (the last one running when T is not a
// multiple of nb), adding the chunk's tokens in order with one fma each from
// zero, as the step does; k_decode_prefill_prefix then forms the prefix
// mixture of the last token's chunk i = (T - 1) / nb, over b < i in order.
// The state is therefore the same bits.  Slots of later chunks are not
// touched (the step restarts a chunk's summary when the chunk begins).
//
// grid = (ceil(T / nb), B*H), block = 256.  k, v: [B*H, T, d].
template <typename T, int PHI>
__global__ __launch_bounds__(kDecThreads) void k_decode_prefill_sums(
    const T* __restrict__ k, const T* __restrict__ v, float* __restrict__ state, int d, int M,
    int nb, int Tp) {
  constexpr int CHK = 32;   // tokens staged per pass
  constexpr int RS = 132;   // LDS row stride (floats): 16-byte aligned rows of up to 129
  __shared__ __attribute__((aligned(16))) float spk[CHK][RS];
  __shared__ __attribute__((aligned(16))) float svv[CHK][RS];
  const int C = d + 1;
  const int E = d * C;
  const int tid = threadIdx.x;
  const int b = blockIdx.x;
  const long slice = blockIdx.y;
  const T* kb = k + slice * (long)Tp * d;
  const T* vb = v + slice * (long)Tp * d;
  float* Sb = state + ((size_t)slice * (M + 1) + b) * E;
  const int t0 = b * nb, t1 = min(t0 + nb, Tp);
  // This thread's 4 x 4 tiles (features 4 ft .. +3, columns 4 ct .. +3) of the
  // chunk's [d][d+1] summary: tile x = tid + 256 u, ft = x / CT, ct = x % CT.
  // Each entry still adds the chunk's tokens in order, one fma each.
  const int FT = (d + 3) / 4, CT = (C + 3) / 4, NTL = FT * CT;
  constexpr int UMAX = (32 * 33 + kDecThreads - 1) / kDecThreads;  // d <= 128
  float acc[UMAX][4][4];
#pragma unroll
  for (int u = 0; u < UMAX; ++u)
#pragma unroll
    for (int x = 0; x < 4; ++x)
#pragma unroll
      for (int y = 0; y < 4; ++y) acc[u][x][y] = 0.0f;
  for (int c0 = t0; c0 < t1; c0 += CHK) {
    const int nt = min(CHK, t1 - c0);
    __syncthreads();
    // zero padding past d (features) and past d + 1 (columns) keeps the tiles' spare lanes at 0
    for (int e = tid; e < nt * RS; e += kDecThreads) {
      const int j = e / RS, f = e - (e / RS) * RS;
      spk[j][f] = f < d ? phi_apply(PHI, Elt<T>::load(kb + (long)(c0 + j) * d + f)) : 0.0f;
      svv[j][f] = f < d ? Elt<T>::load(vb + (long)(c0 + j) * d + f) : f == d ? 1.0f : 0.0f;
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < UMAX; ++u) {
      const int x = tid + kDecThreads * u;
      if (x < NTL) {
        const int ft = x / CT, ct = x - (x / CT) * CT;
        for (int j = 0; j < nt; ++j) {
          const float4 a = *reinterpret_cast<const float4*>(&spk[j][4 * ft]);
          const float4 w4 = *reinterpret_cast<const float4*>(&svv[j][4 * ct]);
          const float av[4] = {a.x, a.y, a.z, a.w}, bv[4] = {w4.x, w4.y, w4.z, w4.w};
#pragma unroll
          for (int p = 0; p < 4; ++p)
#pragma unroll
            for (int q = 0; q < 4; ++q) acc[u][p][q] = fmaf(av[p], bv[q], acc[u][p][q]);
        }
      }
    }
  }
#pragma unroll
  for (int u = 0; u < UMAX; ++u) {
    const int x = tid + kDecThreads * u;
    if (x < NTL) {
      const int ft = x / CT, ct = x - (x / CT) * CT;
#pragma unroll
      for (int p = 0; p < 4; ++p)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int f = 4 * ft + p, c = 4 * ct + q;
          if (f < d && c < C) Sb[f * C + c] = acc[u][p][q];
        }
    }
  }
}

// grid = (ceil(E / 256), B*H), block = 256.
__global__ __launch_bounds__(kDecThreads) void k_decode_prefill_prefix(
    const float* __restrict__ W, float* __restrict__ state, int H, int d, int M, int i) {
  const int E = d * (d + 1);
  const int e = blockIdx.x * kDecThreads + threadIdx.x;
  const long slice = blockIdx.y;
  if (e >= E) return;
  const float* sums = state + (size_t)slice * (M + 1) * E;
  const float* Wi = W + ((size_t)(slice % H) * M + i) * M;
  float P = 0.0f;
  for (int b = 0; b < i; ++b) P = fmaf(Wi[b], sums[(size_t)b * E + e], P);
  state[((size_t)slice * (M + 1) + M) * E + e] = P;
}

template <typename T>
int launch_decode_prefill_t(long slices, int H, int d, int M, int nb, int Tp, int phi,
                            const T* k, const T* v, const float* W, float* state,
                            hipStream_t st) {
  const unsigned nch = (unsigned)((Tp + nb - 1) / nb);
  if (phi == PHI_RELU)
    k_decode_prefill_sums<T, PHI_RELU><<<dim3(nch, (unsigned)slices), kDecThreads, 0, st>>>(
        k, v, state, d, M, nb, Tp);
  else
    k_decode_prefill_sums<T, PHI_ELU1><<<dim3(nch, (unsigned)slices), kDecThreads, 0, st>>>(
        k, v, state, d, M, nb, Tp);
  const int E = d * (d + 1);
  k_decode_prefill_prefix<<<dim3((unsigned)((E + kDecThreads - 1) / kDecThreads),
                                 (unsigned)slices), kDecThreads, 0, st>>>(W, state, H, d, M,
                                                                           (Tp - 1) / nb);
  return 0;
}

template <typename T>
int launch_decode_t(long slices, int H, int d, int M, int nb, int t, int phi, int norm,
                    const T* q, const T* k, const T* v, const float* W, T* y, float* state,
                    hipStream_t st) {
  const size_t lds = decode_lds_bytes(d);
  static std::atomic<bool> attr_set[2][64];
  const void* fn = phi == PHI_RELU ? reinterpret_cast<const void*>(&k_decode_step<T, PHI_RELU>)
                                   : reinterpret_cast<const void*>(&k_decode_step<T, PHI_ELU1>);
  if (lds > 64 * 1024 && lds_limit_once(fn, attr_set[phi == PHI_RELU ? 0 : 1], 160 * 1024) != 0)
    return -1;
  if (phi == PHI_RELU)
    k_decode_step<T, PHI_RELU><<<dim3((unsigned)slices), kDecThreads, lds, st>>>(
        q, k, v, W, y, state, H, d, M, nb, t, norm);
  else
    k_decode_step<T, PHI_ELU1><<<dim3((unsigned)slices), kDecThreads, lds, st>>>(
        q, k, v, W, y, state, H, d, M, nb, t, norm);
  return 0;
}

}  // namespace mhla
