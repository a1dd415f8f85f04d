// k_pairs_bwd.hpp -- backward pass in the token-pair order of "MHLA:
// Restoring Expressivity of Linear Attention via Token-Level Multi-Head"
// §4.2 Eq. 5, for blocks of at most 16 tokens (the shapes of the pairs
// forward).  With P[q][j] = phi(q).phi(k_j), A = W[blk q][blk j] P,
// num = A V, den = A 1 and Y = num / den, the chain rule gives (G = dY):
//
//   dnum_q = G_q / den_q,   dden_q = -(G_q . Y_q) / den_q   (G_q and 0 without
//                                                          the normaliser)
//   dA[q][j] = dnum_q . v_j + dden_q
//   dW[i][b] = sum_{q in i, j in b} dA[q][j] P[q][j]
//   dphi(q)  = sum_j W dA[q][j] phi(k_j),   dphi(k_j) = sum_q W dA[q][j] phi(q)
//   dv_j     = sum_q A[q][j] dnum_q
//   dQ = dphi(Q) * phi'(Q),   dK = dphi(K) * phi'(K)
//
// A zero denominator (ReLU with phi(q) = 0) makes Y_q a constant 0, so that
// row passes no gradient.  No d x d state is formed and nothing of size N^2
// leaves the chip.  Two kernels, one workgroup of 8 waves per slice each:
//   k_pbwd_q (query side): phi(K) and [V | 1] staged in LDS as in the
//     forward; wave w owns query blocks w, w + 8, ...  Pass 1 forms O^T =
//     [num | den]^T exactly like the forward, then dnum and dden; pass 2 runs
//     over the key blocks again, forms P^T and dA^T (MFMA over d), the dW
//     partial of every block pair (a wave-wide sum), and accumulates dphi(Q)^T
//     += phi(K)^T (W dA^T).  Writes dQ, and dnum (two bf16 parts), dden and
//     the dW partials to the workspace.
//   k_pbwd_k (key side): phi(Q), dnum and dden staged in LDS; wave w owns key
//     blocks.  Per query block pair it forms P and dA again (keys in the
//     columns), and accumulates dV^T += dnum^T (W P) and dphi(K)^T +=
//     phi(Q)^T (W dA).
// The dW partials ([slices][M][M]) are summed over the batch by k_dw_reduce.
#pragma once

#include "k_backward.hpp"
#include "k_pairs.hpp"

namespace mhla {

// Contraction over the value columns c in steps of 32, in the "acc8" order of
// two adjacent accumulator tiles: lane group g, elements 0..3 hold c = 32m +
// 4g + 0..3 and elements 4..7 hold c = 32m + 16 + 4g + 0..3.  Reads the two
// 8-byte halves of row `row` (bf16, stride rs) for step m; the second half is
// zero when tile 2m+1 does not exist (CT odd).
template <int CT>
__device__ __forceinline__ u16x8_t acc8_row(const bf16_t* base, int row, int rs, int m, int grp) {
  const bf16_t* p = base + (size_t)row * rs + 32 * m + 4 * grp;
  const uint2 lo = *reinterpret_cast<const uint2*>(p);
  const uint2 hi = 2 * m + 1 < CT ? *reinterpret_cast<const uint2*>(p + 16) : make_uint2(0u, 0u);
  return from_u2x2(lo, hi);
}

// LDS of the key side: phi(Q), dnum as two bf16 parts (hi, lo), dden, W,
// block bases.
template <int DK, int DO>
struct PairsBwdLayout {
  static constexpr int RSQ = pairs_rs(DK);  // phi(Q) rows (member order, as the forward's)
  static constexpr int RSD = pairs_rs(DO);  // dnum rows (columns d .. DO-1 zero)
  __host__ __device__ static size_t q_bytes(int N) { return prow_elems(N, RSQ) * 2; }
  __host__ __device__ static size_t d_bytes(int N) { return prow_elems(N, RSD) * 2; }
  __host__ __device__ static size_t total(int N, int M) {
    return q_bytes(N) + 2 * d_bytes(N) + (size_t)(N + 1) * 4 + (size_t)M * M * 4 +
           (size_t)32 * 4;
  }
};

// Two accumulator tiles (rows 4g..4g+3 each) as the acc8 operands of their
// bf16 value (hi) and of the rounding remainder (lo): hi + lo carries about
// 16 bits of the fp32 value.
__device__ __forceinline__ void split_acc8(const f32x4_t& a, const f32x4_t& b, u16x8_t& hi,
                                           u16x8_t& lo) {
  hi = pack_acc8(a, b);
  const u32x4_t h = __builtin_bit_cast(u32x4_t, hi);
  const f32x4_t ra = f32x4_t{a[0] - lo_f32(h[0]), a[1] - hi_f32(h[0]), a[2] - lo_f32(h[1]),
                             a[3] - hi_f32(h[1])};
  const f32x4_t rb = f32x4_t{b[0] - lo_f32(h[2]), b[1] - hi_f32(h[2]), b[2] - lo_f32(h[3]),
                             b[3] - hi_f32(h[3])};
  lo = pack_acc8(ra, rb);
}

template <int DK, int DO, int QB, int PHI>
__global__ __launch_bounds__(kPairsThreads) void k_pbwd_q(
    const bf16_t* __restrict__ Q, const bf16_t* __restrict__ K, const bf16_t* __restrict__ V,
    const float* __restrict__ W, const bf16_t* __restrict__ G, bf16_t* __restrict__ dQ,
    bf16_t* __restrict__ dN, bf16_t* __restrict__ dNlo, float* __restrict__ dden,
    float* __restrict__ Pw, Geo g, int H, int N, int d) {
  using L = PairsLayout<DK, DO>;
  constexpr int RSK = L::RSK, RSV = L::RSV, KS = L::KS, CT = L::CT;
  constexpr bool TAIL = L::TAIL;
  constexpr int CS = (CT + 1) / 2;   // 32-wide steps over the value columns
  constexpr int FT = DK / 16;        // 16-wide feature tiles of dphi(Q)^T
  constexpr int KSF = KS + (TAIL ? 1 : 0);  // 32-wide feature steps, the last one half empty
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
  int* sB = reinterpret_cast<int*>(sW + M * M);

  // ---- stage phi(K), [V | 1] (zero pad columns and row N), W, block bases ----
  for (int e = tid; e < (int)((L::k_bytes(N) + L::v_bytes(N)) / 16); e += kPairsThreads)
    reinterpret_cast<u32x4_t*>(smem)[e] = u32x4_t{0u, 0u, 0u, 0u};
  for (int e = tid; e < M * M; e += kPairsThreads) sW[e] = W[(size_t)h * M * M + e];
  for (int b = tid; b < M; b += kPairsThreads) sB[b] = g.blockbase(b);
  lds_barrier();
  {  // rows in member order (see PairsLayout)
    const int F8 = d >> 3;
    const float inv8 = 1.0f / (float)F8, invnb = 1.0f / (float)nb;
    for (int it = tid; it < N * F8; it += kPairsThreads) {
      const int row = (int)(((float)it + 0.5f) * inv8);
      const int f = it - row * F8;
      const int b = (int)(((float)row + 0.5f) * invnb);
      const size_t src = off + (size_t)(sB[b] + g.tokoff(row - b * nb)) * d + 8 * f;
      const u32x4_t kr = *reinterpret_cast<const u32x4_t*>(K + src);
      const u32x4_t vr = *reinterpret_cast<const u32x4_t*>(V + src);
      *reinterpret_cast<u32x4_t*>(sK + prow(row, RSK) + 8 * f) = phi8<PHI>(kr);
      *reinterpret_cast<u32x4_t*>(sV + prow(row, RSV) + 8 * f) = vr;
    }
    for (int t = tid; t < N; t += kPairsThreads) sV[prow(t, RSV) + d] = 0x3f80;  // bf16 1.0
  }
  lds_barrier();

  // ---- this wave's query blocks: phi(Q) B operands (query s, features) ------
  const int myq = (M - wave + kPairsWaves - 1) / kPairsWaves;
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
  // G of this lane's query and value columns 16c + 4grp .. +3, requested now
  // (unconditional, clamped; masked where it is used) so that it is in flight
  // during pass 1
  uint2 gx[QB][CT];
#pragma unroll
  for (int u = 0; u < QB; ++u)
#pragma unroll
    for (int c = 0; c < CT; ++c)
      gx[u][c] = *reinterpret_cast<const uint2*>(G + off + (size_t)(qtok[u] > 0 ? qtok[u] : 0) * d +
                                                 min(16 * c + 4 * grp, d - 4));

  // key member s of a block: row of this lane for the row-operand reads; key
  // member 4grp + s/4: row supplied to the transpose reads
  const int vj = 4 * grp + (s >> 2);
  auto pair_rows = [&](int b0, int (&kr)[2], int (&vr)[2]) {
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      const int b = b0 + hb;
      const bool real = b < M;
      kr[hb] = (real && s < nb) ? b * nb + s : N;
      vr[hb] = (real && vj < nb) ? b * nb + vj : N;
    }
  };

  // ---- pass 1: O^T = [num | den]^T, as in the forward ------------------------
  f32x4_t o[QB][CT];
#pragma unroll
  for (int u = 0; u < QB; ++u)
#pragma unroll
    for (int c = 0; c < CT; ++c) o[u][c] = zero4();
  for (int b0 = 0; b0 < M; b0 += 2) {
    int kr[2], vr[2];
    pair_rows(b0, kr, vr);
    u16x8_t ka[2][KSF];
#pragma unroll
    for (int hb = 0; hb < 2; ++hb)
#pragma unroll
      for (int ks = 0; ks < KSF; ++ks) ka[hb][ks] = feat_row(sK, prow(kr[hb], RSK), 1, ks, KS, grp);
    u16x8_t va[CT];
#pragma unroll
    for (int c = 0; c < CT; ++c)
      va[c] = lds_tr8_rows(sV + 16 * c + 4 * (s & 3), 1, prow(vr[0], RSV), prow(vr[1], RSV));
#pragma unroll
    for (int u = 0; u < QB; ++u) {
      if (u >= myq) break;
      const int i = wave + u * kPairsWaves;
      f32x4_t p[2];
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) {
        p[hb] = zero4();
#pragma unroll
        for (int ks = 0; ks < KSF; ++ks) p[hb] = mfma_bf16(ka[hb][ks], qf[u][ks], p[hb]);
        p[hb] *= b0 + hb < M ? sW[i * M + b0 + hb] : 0.0f;
      }
      const u16x8_t pb = pack_acc8(p[0], p[1]);
#pragma unroll
      for (int c = 0; c < CT; ++c) o[u][c] = mfma_bf16(va[c], pb, o[u][c]);
    }
  }

  // ---- dnum, dden ------------------------------------------------------------
  // o[u][c] lane (s, grp) element r = O^T[16c + 4grp + r][query s]
  const int dct = d >> 4, dg = (d & 15) >> 2, dr = d & 3;
  // dnum^T as B operands (query s, value columns in acc8 order), in two bf16
  // parts: dA = dnum . v + dden cancels when v_j is close to Y_q, so dnum
  // enters with about 16 bits
  u16x8_t dnb[QB][CS], dnl[QB][CS];
  float ddn[QB];
#pragma unroll
  for (int u = 0; u < QB; ++u) {
    ddn[u] = 0.0f;
#pragma unroll
    for (int m = 0; m < CS; ++m) dnb[u][m] = dnl[u][m] = u16x8_t{0, 0, 0, 0, 0, 0, 0, 0};
    if (u >= myq) continue;
    float dv = 0.0f;
#pragma unroll
    for (int c = 0; c < CT; ++c)
      if (c == dct) dv = o[u][c][dr];
    const float den = __shfl(dv, 16 * dg + s);
    const float rd = out_scale(g, den);
    f32x4_t dn[CT];
    float part = 0.0f;
#pragma unroll
    for (int c = 0; c < CT; ++c) {
      const int c0 = 16 * c + 4 * grp;
      f32x4_t gv = zero4();
      if (qtok[u] >= 0 && c0 < d) {
        const uint2 x = gx[u][c];
        gv = f32x4_t{lo_f32(x.x), hi_f32(x.x), lo_f32(x.y), hi_f32(x.y)};
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        dn[c][r] = gv[r] * rd;
        part += gv[r] * (o[u][c][r] * rd);  // G . Y over the real columns (gv = 0 past d)
      }
    }
    part += __shfl_xor(part, 16);
    part += __shfl_xor(part, 32);
    ddn[u] = g.norm ? -rd * part : 0.0f;
#pragma unroll
    for (int m = 0; m < CS; ++m)
      split_acc8(dn[2 * m], 2 * m + 1 < CT ? dn[2 * m + 1] : zero4(), dnb[u][m], dnl[u][m]);
    // dnum's two parts (exactly the operands used here) and dden for the key side
    f32x4_t dr[CT];
#pragma unroll
    for (int c = 0; c < CT; ++c) {
#pragma unroll
      for (int r = 0; r < 4; ++r) dr[c][r] = dn[c][r] - bf16_to_f32(f32_to_bf16(dn[c][r]));
    }
    bf16_t* nrow = qtok[u] >= 0 ? dN + off + (size_t)qtok[u] * d : nullptr;
    bf16_t* lrow = qtok[u] >= 0 ? dNlo + off + (size_t)qtok[u] * d : nullptr;
    store_row_tiles<CT>(nrow, d, dn, 1.0f, grp);
    store_row_tiles<CT>(lrow, d, dr, 1.0f, grp);
    if (grp == 0 && qtok[u] >= 0) dden[(size_t)slice * N + qtok[u]] = ddn[u];
  }

  // ---- pass 2: dA^T, dW partials, dphi(Q)^T ----------------------------------
  f32x4_t dq[QB][FT];
#pragma unroll
  for (int u = 0; u < QB; ++u)
#pragma unroll
    for (int f = 0; f < FT; ++f) dq[u][f] = zero4();
  float* Ph = Pw + (size_t)slice * M * M;
  for (int b0 = 0; b0 < M; b0 += 2) {
    int kr[2], vr[2];
    pair_rows(b0, kr, vr);
    u16x8_t ka[2][KSF], vb[2][CS];
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
#pragma unroll
      for (int ks = 0; ks < KSF; ++ks) ka[hb][ks] = feat_row(sK, prow(kr[hb], RSK), 1, ks, KS, grp);
#pragma unroll
      for (int m = 0; m < CS; ++m) vb[hb][m] = acc8_row<CT>(sV, prow(kr[hb], RSV), 1, m, grp);
    }
    // phi(K)^T A operands: rows f = 16ft + s, keys {4grp..4grp+3} of b0 then b1
    u16x8_t kT[FT];
#pragma unroll
    for (int f = 0; f < FT; ++f)
      kT[f] = lds_tr8_rows(sK + 16 * f + 4 * (s & 3), 1, prow(vr[0], RSK), prow(vr[1], RSK));
#pragma unroll
    for (int u = 0; u < QB; ++u) {
      if (u >= myq) break;
      const int i = wave + u * kPairsWaves;
      f32x4_t dp[2];
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) {
        f32x4_t p = zero4(), da = zero4();
#pragma unroll
        for (int ks = 0; ks < KSF; ++ks) p = mfma_bf16(ka[hb][ks], qf[u][ks], p);
#pragma unroll
        for (int m = 0; m < CS; ++m) {
          da = mfma_bf16(vb[hb][m], dnb[u][m], da);
          da = mfma_bf16(vb[hb][m], dnl[u][m], da);
        }
        // p, da lane (s, grp) element r: key 4grp + r of block b0 + hb, query s
        float x = 0.0f;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          da[r] += ddn[u];
          x += da[r] * p[r];
        }
#pragma unroll
        for (int o2 = 32; o2 >= 1; o2 >>= 1) x += __shfl_xor(x, o2);
        const int b = b0 + hb;
        if (b < M && lane == 0) Ph[i * M + b] = x;
        dp[hb] = da * (b < M ? sW[i * M + b] : 0.0f);
      }
      const u16x8_t dpb = pack_acc8(dp[0], dp[1]);
#pragma unroll
      for (int f = 0; f < FT; ++f) dq[u][f] = mfma_bf16(kT[f], dpb, dq[u][f]);
    }
  }

  // ---- dQ = dphi(Q) * phi'(Q) --------------------------------------------------
  // dq[u][f] lane (s, grp) element r = dphi(Q)^T[16f + 4grp + r][query s]
#pragma unroll
  for (int u = 0; u < QB; ++u) {
    if (u >= myq) break;
#pragma unroll
    for (int f = 0; f < FT; ++f) {
      const int f0 = 16 * f + 4 * grp;
      if (qtok[u] >= 0 && f0 < d) {
        const uint2 x = *reinterpret_cast<const uint2*>(Q + off + (size_t)qtok[u] * d + f0);
        const float xv[4] = {lo_f32(x.x), hi_f32(x.x), lo_f32(x.y), hi_f32(x.y)};
#pragma unroll
        for (int r = 0; r < 4; ++r) dq[u][f][r] *= dphi_apply<PHI>(xv[r]);
      }
    }
    store_row_tiles<FT>(qtok[u] >= 0 ? dQ + off + (size_t)qtok[u] * d : nullptr, d, dq[u], 1.0f,
                        grp);
  }
}

template <int DK, int DO, int QB, int PHI>
__global__ __launch_bounds__(kPairsThreads) void k_pbwd_k(
    const bf16_t* __restrict__ Q, const bf16_t* __restrict__ K, const bf16_t* __restrict__ V,
    const float* __restrict__ W, const bf16_t* __restrict__ dN, const bf16_t* __restrict__ dNlo,
    const float* __restrict__ dden, bf16_t* __restrict__ dK, bf16_t* __restrict__ dV, Geo g,
    int H, int N, int d) {
  using L = PairsBwdLayout<DK, DO>;
  constexpr int RSQ = L::RSQ, RSD = L::RSD;
  constexpr int KS = DK / 32;
  constexpr bool TAIL = (DK % 32) != 0;
  constexpr int KSF = KS + (TAIL ? 1 : 0);
  constexpr int CT = DO / 16, CS = (CT + 1) / 2, FT = DK / 16;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int M = g.M, nb = g.nb;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int s = lane & 15, grp = lane >> 4;
  const long slice = blockIdx.x;
  const int h = (int)(slice % H);
  const size_t off = (size_t)slice * N * d;
  bf16_t* sQ = reinterpret_cast<bf16_t*>(smem);
  bf16_t* sD = reinterpret_cast<bf16_t*>(smem + L::q_bytes(N));
  bf16_t* sDl = reinterpret_cast<bf16_t*>(smem + L::q_bytes(N) + L::d_bytes(N));
  float* sdd = reinterpret_cast<float*>(smem + L::q_bytes(N) + 2 * L::d_bytes(N));
  float* sW = sdd + (N + 1);
  int* sB = reinterpret_cast<int*>(sW + M * M);

  // ---- stage phi(Q), dnum (zero pad columns and row N), dden, W, bases -------
  for (int e = tid; e < (int)((L::q_bytes(N) + 2 * L::d_bytes(N)) / 16); e += kPairsThreads)
    reinterpret_cast<u32x4_t*>(smem)[e] = u32x4_t{0u, 0u, 0u, 0u};
  for (int e = tid; e < M * M; e += kPairsThreads) sW[e] = W[(size_t)h * M * M + e];
  for (int b = tid; b < M; b += kPairsThreads) sB[b] = g.blockbase(b);
  lds_barrier();
  {  // rows in member order (see PairsLayout)
    const float invnb = 1.0f / (float)nb;
    for (int row = tid; row <= N; row += kPairsThreads) {
      float v = 0.0f;
      if (row < N) {
        const int b = (int)(((float)row + 0.5f) * invnb);
        v = dden[(size_t)slice * N + sB[b] + g.tokoff(row - b * nb)];
      }
      sdd[row] = v;
    }
    const int F8 = d >> 3;
    const float inv8 = 1.0f / (float)F8;
    for (int it = tid; it < N * F8; it += kPairsThreads) {
      const int row = (int)(((float)it + 0.5f) * inv8);
      const int f = it - row * F8;
      const int b = (int)(((float)row + 0.5f) * invnb);
      const size_t src = off + (size_t)(sB[b] + g.tokoff(row - b * nb)) * d + 8 * f;
      const u32x4_t qr = *reinterpret_cast<const u32x4_t*>(Q + src);
      const u32x4_t nr = *reinterpret_cast<const u32x4_t*>(dN + src);
      const u32x4_t lr = *reinterpret_cast<const u32x4_t*>(dNlo + src);
      *reinterpret_cast<u32x4_t*>(sQ + prow(row, RSQ) + 8 * f) = phi8<PHI>(qr);
      *reinterpret_cast<u32x4_t*>(sD + prow(row, RSD) + 8 * f) = nr;
      *reinterpret_cast<u32x4_t*>(sDl + prow(row, RSD) + 8 * f) = lr;
    }
  }
  lds_barrier();

  // ---- this wave's key blocks, one after another: each block's phi(K) and V
  // operands and dV, dK accumulators are live only while its queries are
  // swept (two blocks at once took more than 256 registers and spilled)
  const int myk = (M - wave + kPairsWaves - 1) / kPairsWaves;
  const int vj = 4 * grp + (s >> 2);
#pragma unroll 1
  for (int u = 0; u < QB; ++u) {
    if (u >= myk) break;
    const int b = wave + u * kPairsWaves;
    const bool kreal = s < nb;
    const int ktok = kreal ? sB[b] + g.tokoff(s) : -1;
    u16x8_t kf[KSF], vf[CS];
#pragma unroll
    for (int ks = 0; ks < KSF; ++ks) kf[ks] = feat_operand<PHI>(K + off, ktok, d, ks, KS, grp);
    // V in the acc8 order of the value columns; columns past d are 0
#pragma unroll
    for (int m = 0; m < CS; ++m) {
      // unconditional loads at clamped addresses, masked after
      const int c0 = 32 * m + 4 * grp, c1 = c0 + 16;
      const bf16_t* vrow = V + off + (size_t)(kreal ? ktok : 0) * d;
      const uint2 lo = *reinterpret_cast<const uint2*>(vrow + min(c0, d - 4));
      const uint2 hi = *reinterpret_cast<const uint2*>(vrow + min(c1, d - 4));
      const uint2 z = make_uint2(0u, 0u);
      vf[m] = from_u2x2(kreal && c0 < d ? lo : z, kreal && c1 < d ? hi : z);
    }
    f32x4_t dv[FT], dk[FT];
#pragma unroll
    for (int f = 0; f < FT; ++f) dv[f] = dk[f] = zero4();
    for (int i0 = 0; i0 < M; i0 += 2) {
      int qr[2], qv[2];
      float dd[2][4];
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) {
        const int i = i0 + hb;
        const bool real = i < M;
        qr[hb] = (real && s < nb) ? i * nb + s : N;
        qv[hb] = (real && vj < nb) ? i * nb + vj : N;
        // this lane's output rows of P and dA: query members 4grp + r
#pragma unroll
        for (int r = 0; r < 4; ++r)
          dd[hb][r] = (real && 4 * grp + r < nb) ? sdd[i * nb + 4 * grp + r] : 0.0f;
      }
      // row operands (query member s): phi(Q) over features, dnum over values
      u16x8_t qa[2][KSF], na[2][CS], nl[2][CS];
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) {
#pragma unroll
        for (int ks = 0; ks < KSF; ++ks) qa[hb][ks] = feat_row(sQ, prow(qr[hb], RSQ), 1, ks, KS, grp);
#pragma unroll
        for (int m = 0; m < CS; ++m) {
          na[hb][m] = acc8_row<CT>(sD, prow(qr[hb], RSD), 1, m, grp);
          nl[hb][m] = acc8_row<CT>(sDl, prow(qr[hb], RSD), 1, m, grp);
        }
      }
      // transposed operands: rows c (dnum^T) and f (phi(Q)^T) = 16t + s,
      // queries {4grp..4grp+3} of i0 then of i0 + 1
      u16x8_t nT[FT], qT[FT];
#pragma unroll
      for (int f = 0; f < FT; ++f) {
        nT[f] = lds_tr8_rows(sD + 16 * f + 4 * (s & 3), 1, prow(qv[0], RSD), prow(qv[1], RSD));
        qT[f] = lds_tr8_rows(sQ + 16 * f + 4 * (s & 3), 1, prow(qv[0], RSQ), prow(qv[1], RSQ));
      }
      f32x4_t a[2], dp[2];
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) {
        f32x4_t p = zero4(), da = zero4();
#pragma unroll
        for (int ks = 0; ks < KSF; ++ks) p = mfma_bf16(qa[hb][ks], kf[ks], p);
#pragma unroll
        for (int m = 0; m < CS; ++m) {
          da = mfma_bf16(na[hb][m], vf[m], da);
          da = mfma_bf16(nl[hb][m], vf[m], da);
        }
        // lane (s, grp) element r: query 4grp + r of block i0 + hb, key s
#pragma unroll
        for (int r = 0; r < 4; ++r) da[r] += dd[hb][r];
        const float w = i0 + hb < M ? sW[(i0 + hb) * M + b] : 0.0f;
        a[hb] = p * w;
        dp[hb] = da * w;
      }
      const u16x8_t ab = pack_acc8(a[0], a[1]), dpb = pack_acc8(dp[0], dp[1]);
#pragma unroll
      for (int f = 0; f < FT; ++f) {
        dv[f] = mfma_bf16(nT[f], ab, dv[f]);
        dk[f] = mfma_bf16(qT[f], dpb, dk[f]);
      }
    }

    // ---- dV, dK = dphi(K) * phi'(K) ----------------------------------------------
    // dv[f] / dk[f] lane (s, grp) element r = dV^T / dphi(K)^T[16f + 4grp + r][key s]
#pragma unroll
    for (int f = 0; f < FT; ++f) {
      const int f0 = 16 * f + 4 * grp;
      if (ktok >= 0 && f0 < d) {
        const uint2 x = *reinterpret_cast<const uint2*>(K + off + (size_t)ktok * d + f0);
        const float xv[4] = {lo_f32(x.x), hi_f32(x.x), lo_f32(x.y), hi_f32(x.y)};
#pragma unroll
        for (int r = 0; r < 4; ++r) dk[f][r] *= dphi_apply<PHI>(xv[r]);
      }
    }
    store_row_tiles<FT>(ktok >= 0 ? dV + off + (size_t)ktok * d : nullptr, d, dv, 1.0f, grp);
    store_row_tiles<FT>(ktok >= 0 ? dK + off + (size_t)ktok * d : nullptr, d, dk, 1.0f, grp);
  }
}

// ---------------------------------------------------------------------------
inline bool pairs_bwd_lds_ok(int d, int N, int M) {
  int dk, dout;
  if (!pairs_dims(d, &dk, &dout)) return false;
  const size_t kq = pairs_lds(d, N, M);
  size_t kk = 0;
  switch (d) {
    case 16: kk = PairsBwdLayout<16, 32>::total(N, M); break;
    case 32: kk = PairsBwdLayout<32, 48>::total(N, M); break;
    case 48: kk = PairsBwdLayout<48, 64>::total(N, M); break;
    case 64: kk = PairsBwdLayout<64, 80>::total(N, M); break;
    case 72: kk = PairsBwdLayout<80, 80>::total(N, M); break;
    case 80: kk = PairsBwdLayout<80, 96>::total(N, M); break;
    default: kk = PairsBwdLayout<96, 112>::total(N, M); break;
  }
  return kq <= 160 * 1024 && kk <= 160 * 1024;
}

// Query (key) blocks per wave the token-pair backward compiles for d: four
// blocks (M <= 32) only up to d = 48 and two (M <= 16) up to d = 80, so that
// both kernels stay within 256 registers without spilling.
inline int pairs_bwd_max_m(int d) { return d <= 48 ? 4 * kPairsWaves : (d <= 80 ? 2 * kPairsWaves : kPairsWaves); }

// The token-pair backward covers the pairs forward's shapes whose two
// kernels fit in LDS and in registers.
inline bool pairs_bwd_supports(int dtype, int d, int M, int nb, int N) {
  return pairs_supports(dtype, d, M, nb, N) && M <= pairs_bwd_max_m(d) &&
         pairs_bwd_lds_ok(d, N, M);
}

// Workspace: dnum in two bf16 parts ([slices][N][d] each), dden ([slices][N]
// fp32), the dW partials ([slices][M][M] fp32).
inline size_t pairs_bwd_workspace(long slices, int M, int N, int d) {
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  return 2 * up((size_t)slices * N * d * sizeof(bf16_t)) +
         up((size_t)slices * N * sizeof(float)) + up((size_t)slices * M * M * sizeof(float));
}

template <int DK, int DO, int QB, int PHI>
int launch_pairs_bwd_t(long slices, int B, int H, int N, int d, const Geo& g, const bf16_t* Q,
                       const bf16_t* K, const bf16_t* V, const float* W, const bf16_t* dY,
                       bf16_t* dQ, bf16_t* dK, bf16_t* dV, float* dW, void* ws, hipStream_t st) {
  const int M = g.M;
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  char* p = static_cast<char*>(ws);
  bf16_t* dN = reinterpret_cast<bf16_t*>(p);
  p += up((size_t)slices * N * d * sizeof(bf16_t));
  bf16_t* dNlo = reinterpret_cast<bf16_t*>(p);
  p += up((size_t)slices * N * d * sizeof(bf16_t));
  float* dd = reinterpret_cast<float*>(p);
  p += up((size_t)slices * N * sizeof(float));
  float* Pw = reinterpret_cast<float*>(p);
  const size_t lq = PairsLayout<DK, DO>::total(N, M), lk = PairsBwdLayout<DK, DO>::total(N, M);
  static std::atomic<bool> set_q[64], set_k[64];
  if (lds_limit_once(reinterpret_cast<const void*>(&k_pbwd_q<DK, DO, QB, PHI>), set_q,
                     160 * 1024) != 0 ||
      lds_limit_once(reinterpret_cast<const void*>(&k_pbwd_k<DK, DO, QB, PHI>), set_k,
                     160 * 1024) != 0)
    return -1;
  // with one batch item the per-slice dW partials are dW itself
  float* Pd = B == 1 ? dW : Pw;
  k_pbwd_q<DK, DO, QB, PHI><<<dim3((unsigned)slices), dim3(kPairsThreads), lq, st>>>(
      Q, K, V, W, dY, dQ, dN, dNlo, dd, Pd, g, H, N, d);
  k_pbwd_k<DK, DO, QB, PHI><<<dim3((unsigned)slices), dim3(kPairsThreads), lk, st>>>(
      Q, K, V, W, dN, dNlo, dd, dK, dV, g, H, N, d);
  if (B > 1) {
    const long nw = (long)H * M * M;
    k_dw_reduce<<<dim3((unsigned)((nw + 255) / 256)), 256, 0, st>>>(Pw, dW, B, H, M, 1, 0);
  }
  return 0;
}

template <int DK, int DO, int PHI>
int launch_pairs_bwd_q(long slices, int B, int H, int N, int d, const Geo& g, const bf16_t* Q,
                       const bf16_t* K, const bf16_t* V, const float* W, const bf16_t* dY,
                       bf16_t* dQ, bf16_t* dK, bf16_t* dV, float* dW, void* ws, hipStream_t st) {
  if (g.M <= kPairsWaves)
    return launch_pairs_bwd_t<DK, DO, 1, PHI>(slices, B, H, N, d, g, Q, K, V, W, dY, dQ, dK, dV,
                                              dW, ws, st);
  if constexpr (DK <= 80) {
    if (g.M <= 2 * kPairsWaves)
      return launch_pairs_bwd_t<DK, DO, 2, PHI>(slices, B, H, N, d, g, Q, K, V, W, dY, dQ, dK, dV,
                                                dW, ws, st);
  }
  if constexpr (DK <= 48) {
    return launch_pairs_bwd_t<DK, DO, 4, PHI>(slices, B, H, N, d, g, Q, K, V, W, dY, dQ, dK, dV,
                                              dW, ws, st);
  }
  return -1;  // excluded by pairs_bwd_supports
}

template <int PHI>
int launch_pairs_bwd_p(long slices, int B, int H, int N, int d, const Geo& g, const bf16_t* Q,
                       const bf16_t* K, const bf16_t* V, const float* W, const bf16_t* dY,
                       bf16_t* dQ, bf16_t* dK, bf16_t* dV, float* dW, void* ws, hipStream_t st) {
#define MHLA_PB(DKV, DOV) \
  launch_pairs_bwd_q<DKV, DOV, PHI>(slices, B, H, N, d, g, Q, K, V, W, dY, dQ, dK, dV, dW, ws, st)
  switch (d) {
    case 16: return MHLA_PB(16, 32);
    case 32: return MHLA_PB(32, 48);
    case 48: return MHLA_PB(48, 64);
    case 64: return MHLA_PB(64, 80);
    case 72: return MHLA_PB(80, 80);
    case 80: return MHLA_PB(80, 96);
    default: return MHLA_PB(96, 112);
  }
#undef MHLA_PB
}

inline int launch_pairs_backward(long slices, int B, int H, int N, int d, const Geo& g, int phi,
                                 const bf16_t* Q, const bf16_t* K, const bf16_t* V, const float* W,
                                 const bf16_t* dY, bf16_t* dQ, bf16_t* dK, bf16_t* dV, float* dW,
                                 void* ws, hipStream_t st) {
  if (phi == PHI_RELU)
    return launch_pairs_bwd_p<PHI_RELU>(slices, B, H, N, d, g, Q, K, V, W, dY, dQ, dK, dV, dW, ws,
                                        st);
  return launch_pairs_bwd_p<PHI_ELU1>(slices, B, H, N, d, g, Q, K, V, W, dY, dQ, dK, dV, dW, ws,
                                      st);
}

}  // namespace mhla
