// k_decode.hpp -- incremental (streaming) inference of the causal form, one
// or more tokens per (batch, head) slice per launch: "MHLA: Restoring Expressivity of
// Linear Attention via Token-Level Multi-Head", App. C ("Causal inference").
//
// The sequence is cut into chunks of nb tokens; token t sits in chunk
// i = t / nb.  Per slice the state keeps, in fp32,
//   slots 0 .. M-1 : the chunk summaries [S_b | z_b] (rows f = key feature,
//                    columns c = value column, column d = z), finished for
//                    b < i and running for b = i;
//   slot M         : the prefix mixture [P_i | p_i] = sum_{b<i} W[i,b] [S_b | z_b],
//                    formed once when chunk i starts.
// Per token t:
//   t starts chunk i : P_i = sum_{b<i} W[i,b] S_b (the finished summaries are
//                      fixed from then on) and the running summary restarts;
//   every token      : S_i += phi(k_t) [v_t | 1]^T;
//   readout          : [n | den] = phi(q_t) (P_i + W[i,i] S_i),
//                      y_t = n / den (0 for den = 0), or n without the normaliser.
// This equals the chunkwise causal forward at position t.  The cost per token
// is O(d^2) (plus O(i d^2) once per chunk), independent of t.
#pragma once

#include "mhla_common.hpp"
#include "mhla_mfma.hpp"

namespace mhla {

constexpr int kDecThreads = 256;

inline size_t decode_state_elems(int d, int M) {
  return (size_t)(M + 1) * (size_t)d * (size_t)(d + 1);
}

// LDS of the step kernel: TB tokens' phi(q), phi(k) [TB][d], [v | 1]
// [TB][d+1] and outputs [TB][d], the readout (up to 4 partial rows of d+1),
// and one (SREG) or two [d][d+1] tiles.
inline size_t decode_step_lds_bytes(int d, int tb, bool sreg) {
  const size_t C = (size_t)d + 1, E = (size_t)d * C;
  return ((size_t)tb * (3 * (size_t)d + C) + 4 * C + (sreg ? 1 : 2) * E) * sizeof(float);
}

// grid = B*H, block = NT.  q, k, v, y: [B*H, n, d] (token t0 + u of a slice
// at row u); W: [H, M, M]; state: [B*H][M+1][d][d+1] fp32.  A launch takes
// the n tokens t0 .. t0+n-1 of every slice in order, each with exactly the
// arithmetic of a launch for that token alone, so the outputs and the state
// do not depend on how a stream is split into launches.  Launches come for
// increasing t on one stream.
//
// Tokens go in groups of TB: the group's q, k, v are staged in LDS with one
// round of loads, its tokens run from LDS, and its outputs are written to
// y together when the group ends, so no global access waits inside a token.
// The running summary S_i and the prefix P_i of the current chunk stay on
// chip: they are read from the state when the launch starts inside a chunk,
// the prefix is formed (and written) when a chunk starts, and the summary is
// written when its chunk ends or the launch does.  With SREG thread tid
// keeps the entries e = tid + NT x (x < EPT) in registers and writes
// P_i + W[i,i] S_i to an LDS tile, whose readout the four waves share by
// features; otherwise S_i and P_i are LDS tiles and the readout forms that
// sum itself.  Entry e is only ever updated by one thread, and the finished
// summaries a chunk start mixes were written by that same thread, so the
// barriers order LDS only.
template <typename T, int PHI, int NT, int EPT, bool SREG, int TB>
__global__ __launch_bounds__(NT) void k_decode_step(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const float* __restrict__ W, T* __restrict__ y, float* __restrict__ state, int H, int d, int M,
    int nb, int t0, int n, int norm) {
  extern __shared__ float smd[];
  const int C = d + 1;
  const int E = d * C;
  float* sq = smd;              // [TB][d] phi(q_t)
  float* sk = sq + TB * d;      // [TB][d] phi(k_t)
  float* sv = sk + TB * d;      // [TB][C] [v_t | 1]
  float* sy = sv + TB * C;      // [TB][d] y_t
  float* red = sy + TB * d;     // [n | den]; SREG: [NT / 64][C] partial sums
  float* comb = red + 4 * C;        // SREG: [d][C] P_i + W[i,i] S_i after this token's update
  float* ls = comb;             // otherwise: [d][C] S_i,
  float* lp = ls + E;           //            [d][C] P_i
  const int tid = threadIdx.x;
  const long slice = blockIdx.x;
  const int h = (int)(slice % H);
  float* sums = state + (size_t)slice * (M + 1) * E;
  float* prefix = sums + (size_t)M * E;
  // feature and column of this thread's first entry, and the step to the next
  const int f0 = tid / C, c0 = tid - (tid / C) * C;
  const int fq = NT / C, cq = NT - (NT / C) * C;

  float s_reg[SREG ? EPT : 1], p_reg[SREG ? EPT : 1];
  if (t0 % nb != 0) {  // the launch starts inside a chunk: pick up its state
    const float* Si = sums + (size_t)(t0 / nb) * E;
    if constexpr (SREG) {
#pragma unroll
      for (int x = 0; x < EPT; ++x) {
        const int e = tid + NT * x;
        if (e < E) {
          s_reg[x] = Si[e];
          p_reg[x] = prefix[e];
        }
      }
    } else {
      for (int e = tid; e < E; e += NT) {
        ls[e] = Si[e];
        lp[e] = prefix[e];
      }
    }
  }
  const T* qs = q + slice * n * (long)d;
  const T* ks = k + slice * n * (long)d;
  const T* vs = v + slice * n * (long)d;
  T* ys = y + slice * n * (long)d;

  for (int g0 = 0; g0 < n; g0 += TB) {
    const int nt = min(TB, n - g0);
    // The readers of sq, sk, sv and sy of the previous group all passed a
    // barrier after their last read.
    for (int x = tid; x < nt * d; x += NT) {
      const int uu = x / d, f = x - (x / d) * d;
      const long r = (long)g0 * d + x;
      sq[x] = phi_apply(PHI, Elt<T>::load(qs + r));
      sk[x] = phi_apply(PHI, Elt<T>::load(ks + r));
      sv[uu * C + f] = Elt<T>::load(vs + r);
    }
    for (int uu = tid; uu < nt; uu += NT) sv[uu * C + d] = 1.0f;
    lds_barrier();

    for (int uu = 0; uu < nt; ++uu) {
      const int t = t0 + g0 + uu;
      const int i = t / nb, j = t - (t / nb) * nb;
      const float* Wi = W + ((size_t)h * M + i) * M;
      const float wii = Wi[i];
      float* Si = sums + (size_t)i * E;
      const bool keep = j == nb - 1 || g0 + uu == n - 1;   // the chunk or the launch ends
      const float* pq = sq + uu * d;
      const float* pk = sk + uu * d;
      const float* vv = sv + uu * C;

      if constexpr (SREG) {
        if (j == 0) {  // chunk i starts: mix the finished chunks once, restart S_i
          // P = sum over b < i in order, from 0; the loads of MB chunks are
          // issued before their fmas so that they are in flight together.
          constexpr int MB = 4;
#pragma unroll
          for (int x = 0; x < EPT; ++x) p_reg[x] = 0.0f;
          int b = 0;
          for (; b + MB <= i; b += MB) {
            float sv4[MB][EPT];
#pragma unroll
            for (int r = 0; r < MB; ++r)
#pragma unroll
              for (int x = 0; x < EPT; ++x) {
                const int e = tid + NT * x;
                sv4[r][x] = e < E ? sums[(size_t)(b + r) * E + e] : 0.0f;
              }
#pragma unroll
            for (int r = 0; r < MB; ++r) {
              const float wb = Wi[b + r];
#pragma unroll
              for (int x = 0; x < EPT; ++x) p_reg[x] = fmaf(wb, sv4[r][x], p_reg[x]);
            }
          }
          for (; b < i; ++b) {
            const float wb = Wi[b];
#pragma unroll
            for (int x = 0; x < EPT; ++x) {
              const int e = tid + NT * x;
              if (e < E) p_reg[x] = fmaf(wb, sums[(size_t)b * E + e], p_reg[x]);
            }
          }
#pragma unroll
          for (int x = 0; x < EPT; ++x) {
            const int e = tid + NT * x;
            if (e < E) prefix[e] = p_reg[x];
            s_reg[x] = 0.0f;
          }
        }
        int f = f0, c = c0;
#pragma unroll
        for (int x = 0; x < EPT; ++x) {
          const int e = tid + NT * x;
          if (e < E) {
            const float s_new = fmaf(pk[f], vv[c], s_reg[x]);
            s_reg[x] = s_new;
            comb[e] = fmaf(wii, s_new, p_reg[x]);
          }
          f += fq;
          c += cq;
          if (c >= C) {
            c -= C;
            ++f;
          }
        }
        if (keep) {
#pragma unroll
          for (int x = 0; x < EPT; ++x) {
            const int e = tid + NT * x;
            if (e < E) Si[e] = s_reg[x];
          }
        }
      } else {
        if (j == 0) {  // chunk i starts: P over b < i in order, chunk by chunk
          for (int e = tid; e < E; e += NT) lp[e] = 0.0f;
          for (int b = 0; b < i; ++b) {
            const float wb = Wi[b];
            const float* Sb = sums + (size_t)b * E;
#pragma unroll 4
            for (int e = tid; e < E; e += NT) lp[e] = fmaf(wb, Sb[e], lp[e]);
          }
          for (int e = tid; e < E; e += NT) prefix[e] = lp[e];
        }
        int f = f0, c = c0;
        for (int e = tid; e < E; e += NT) {
          const float s_old = j == 0 ? 0.0f : ls[e];
          const float s_new = fmaf(pk[f], vv[c], s_old);
          ls[e] = s_new;
          if (keep) Si[e] = s_new;
          f += fq;
          c += cq;
          if (c >= C) {
            c -= C;
            ++f;
          }
        }
      }
      lds_barrier();

      if constexpr (SREG) {
        // Wave w sums the features of its quarter of [0, d) in order, for every
        // column; the four partials are added in wave order when y is formed.
        // The operands of RU terms are loaded before their fmas.
        constexpr int NW = NT / 64, RU = 16;
        static_assert(NW <= 4, "partial rows of the readout");
        const int w = tid >> 6, lane = tid & 63;
        const int fw = (d + NW - 1) / NW, fb = w * fw, fe = min(d, fb + fw);
        for (int c = lane; c < C; c += 64) {
          float acc = 0.0f;
          int f = fb;
          for (; f + RU <= fe; f += RU) {
            float a[RU], cw[RU];
#pragma unroll
            for (int r = 0; r < RU; ++r) {
              a[r] = pq[f + r];
              cw[r] = comb[(f + r) * C + c];
            }
#pragma unroll
            for (int r = 0; r < RU; ++r) acc = fmaf(a[r], cw[r], acc);
          }
          for (; f < fe; ++f) acc = fmaf(pq[f], comb[f * C + c], acc);
          red[w * C + c] = acc;
        }
        lds_barrier();
        // red is written again only after the next token's first barrier,
        // which every reader here reaches after these reads
        for (int c = tid; c < d; c += NT) {
          float num = red[c], den = red[d];
#pragma unroll
          for (int r = 1; r < NW; ++r) {
            num += red[r * C + c];
            den += red[r * C + d];
          }
          sy[uu * d + c] = !norm ? num : den == 0.0f ? 0.0f : num / den;
        }
      } else {
        for (int c = tid; c < C; c += NT) {
          float acc = 0.0f;
          constexpr int RU = 8;
          int f = 0;
          for (; f + RU <= d; f += RU) {
            float a[RU], sw[RU], pw[RU];
#pragma unroll
            for (int r = 0; r < RU; ++r) {
              a[r] = pq[f + r];
              sw[r] = ls[(f + r) * C + c];
              pw[r] = lp[(f + r) * C + c];
            }
#pragma unroll
            for (int r = 0; r < RU; ++r) acc = fmaf(a[r], fmaf(wii, sw[r], pw[r]), acc);
          }
          for (; f < d; ++f) acc = fmaf(pq[f], fmaf(wii, ls[f * C + c], lp[f * C + c]), acc);
          red[c] = acc;
        }
        lds_barrier();
        for (int c = tid; c < d; c += NT) {
          const float den = red[d];
          sy[uu * d + c] = !norm ? red[c] : den == 0.0f ? 0.0f : red[c] / den;
        }
      }
    }
    lds_barrier();
    for (int x = tid; x < nt * d; x += NT) Elt<T>::store(ys + (long)g0 * d + x, sy[x]);
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
  // in order over b from 0, as the step mixes; the loads of PB chunks are
  // issued before their fmas so that they are in flight together
  constexpr int PB = 8;
  float P = 0.0f;
  int b = 0;
  for (; b + PB <= i; b += PB) {
    float sv[PB];
#pragma unroll
    for (int r = 0; r < PB; ++r) sv[r] = sums[(size_t)(b + r) * E + e];
#pragma unroll
    for (int r = 0; r < PB; ++r) P = fmaf(Wi[b + r], sv[r], P);
  }
  for (; b < i; ++b) P = fmaf(Wi[b], sums[(size_t)b * E + e], P);
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

// NT threads of EPT entries each hold the state of one slice, d (d + 1) fp32.
template <typename T, int NT, int EPT, bool SREG, int TB>
int launch_decode_ept(long slices, int H, int d, int M, int nb, int t0, int n, int phi,
                      int norm, const T* q, const T* k, const T* v, const float* W, T* y,
                      float* state, hipStream_t st) {
  const size_t lds = decode_step_lds_bytes(d, TB, SREG);
  static std::atomic<bool> attr_set[2][64];
  const void* fn =
      phi == PHI_RELU ? reinterpret_cast<const void*>(&k_decode_step<T, PHI_RELU, NT, EPT, SREG, TB>)
                      : reinterpret_cast<const void*>(&k_decode_step<T, PHI_ELU1, NT, EPT, SREG, TB>);
  if (lds > 64 * 1024 && lds_limit_once(fn, attr_set[phi == PHI_RELU ? 0 : 1], 160 * 1024) != 0)
    return -1;
  if (phi == PHI_RELU)
    k_decode_step<T, PHI_RELU, NT, EPT, SREG, TB><<<dim3((unsigned)slices), NT, lds, st>>>(
        q, k, v, W, y, state, H, d, M, nb, t0, n, norm);
  else
    k_decode_step<T, PHI_ELU1, NT, EPT, SREG, TB><<<dim3((unsigned)slices), NT, lds, st>>>(
        q, k, v, W, y, state, H, d, M, nb, t0, n, norm);
  return 0;
}

// Up to d = 65: 256 threads of 17 entries, summary and prefix in registers
// (4 waves: one a SIMD at one slice a CU), groups of 16 tokens.  Beyond,
// larger per-thread shares would spill: 512 threads with both tiles in LDS
// and groups of 8 tokens (149 KB at d = 128).
template <typename T>
int launch_decode_t(long slices, int H, int d, int M, int nb, int t0, int n, int phi, int norm,
                    const T* q, const T* k, const T* v, const float* W, T* y, float* state,
                    hipStream_t st) {
  const long E = (long)d * (d + 1);
  if (E <= 17 * 256)
    return launch_decode_ept<T, 256, 17, true, 16>(slices, H, d, M, nb, t0, n, phi, norm, q, k,
                                                   v, W, y, state, st);
  return launch_decode_ept<T, 512, 1, false, 8>(slices, H, d, M, nb, t0, n, phi, norm, q, k, v,
                                                W, y, state, st);
}

}  // namespace mhla
