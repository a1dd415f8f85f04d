/*
 * mhla_oracle.c -- plain fp64 CPU oracle for the MHLA forward.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call, link or
 * load this file; only the tests, the smoke check and the benchmark's CPU
 * baseline leg use it.  It shares no source with the HIP library.
 *
 * What it computes (MHLA paper = "MHLA: Restoring Expressivity of Linear
 * Attention via Token-Level Multi-Head", arXiv 2601.07832):
 *
 *   phi            feature map applied elementwise: ReLU(x) = max(x, 0), or
 *                  elu(x)+1 with alpha = 1, i.e. x+1 for x > 0 and exp(x)
 *                  otherwise (the two choices named in the tutorial page
 *                  "Attention 变体：从 Sliding Window 到 MLA", section
 *                  "Linear Attention 与 Gated Delta Net").
 *   geometry       the N tokens are a (T, Hg, Wg) grid in raster order
 *                  (x fastest); blocks are (bt, bh, bw) tiles of that grid,
 *                  numbered in raster order of the block grid (MHLA paper
 *                  §1 and §4.1; blog review §2.1 stresses spatial tiles,
 *                  not cuts of the flattened sequence).
 *   summary        S_b = sum_{j in b} phi(K_j) V_j^T (d x d) and
 *                  z_b = sum_{j in b} phi(K_j)            (MHLA paper §4.1)
 *   mixing         S~_i = sum_b W[i,b] S_b, z~_i = sum_b W[i,b] z_b, with
 *                  row i = query block, column b = key block (§4.1-§4.2)
 *   readout        Y_q = phi(Q_q) S~_i / (phi(Q_q) . z~_i), q in block i
 *                  (§4.1, the output equation).
 *
 * Readings taken where the pages leave a step open: no 1/sqrt(d) scaling
 * (that belongs to softmax only, §3.1); V is used raw (no phi on V); W is per
 * channel head [H,M,M] and shared across the batch; equal blocks only; when
 * the denominator is exactly 0 the output row is 0.
 *
 * Two routines:
 *   oracle_mhla_blockwise  -- the three steps above, in that order.
 *   oracle_mhla_rows       -- brute force on rows of the explicit N x N
 *                             matrix A[q,j] = W[blk(q),blk(j)] phi(q).phi(k_j)
 *                             (the token-expanded form, §4.2 Eq. 5):
 *                             Y_q = sum_j A[q,j] V_j / sum_j A[q,j].
 *
 * Option bits (`flags`):
 *   1  no normaliser: Y_q is the numerator alone (the MHLA paper drops the
 *      denominator for language modelling and very long video; the blog
 *      review §2.2 stresses that the switch is part of the method).
 *   2  causal: the blocks must be consecutive runs of tokens (chunks, in
 *      sequence order).  Query chunk i mixes only the summaries of earlier
 *      chunks, S^<_i = sum_{b<i} W[i,b] S_b, and adds the causal part of its
 *      own chunk weighted by W[i,i] (MHLA paper §4.2 "Chunkwise parallel form
 *      of MHLA" and App. C; the appendix formula is garbled, so this is the
 *      token form of Eq. 5 with the mask j <= q, split at the chunk border).
 *      In brute force: A[q,j] = 0 for j > q.  Entries W[i,b] with b > i are
 *      never used.
 */
#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int oracle_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

static int geom_ok(int N, const int grid[3], const int block[3]) {
  long n = 1;
  for (int a = 0; a < 3; ++a) {
    if (grid[a] <= 0 || block[a] <= 0 || grid[a] % block[a] != 0) return 0;
    n *= grid[a];
  }
  return n == N;
}

int oracle_num_blocks(const int grid[3], const int block[3]) {
  return (grid[0] / block[0]) * (grid[1] / block[1]) * (grid[2] / block[2]);
}

/* Block index of token t: split t into grid coordinates (x fastest), divide by
 * the block dims, and number the block coordinates in raster order. */
int oracle_block_of_token(const int grid[3], const int block[3], long t) {
  long x = t % grid[2];
  long y = (t / grid[2]) % grid[1];
  long z = t / ((long)grid[2] * grid[1]);
  long bx = x / block[2], by = y / block[1], bz = z / block[0];
  long nbx = grid[2] / block[2], nby = grid[1] / block[1];
  return (int)((bz * nby + by) * nbx + bx);
}

double oracle_phi(int kind, double x) {
  if (kind == 0) return x > 0.0 ? x : 0.0;
  return x > 0.0 ? x + 1.0 : exp(x);
}

enum { ORACLE_NO_NORM = 1, ORACLE_CAUSAL = 2 };

/* Output row from numerator and denominator: divide (0 when the denominator is
 * exactly 0), or the numerator alone when the normaliser is switched off. */
static void finish_row(double* y, const double* num, double den, int d, int flags) {
  if (flags & ORACLE_NO_NORM) {
    for (int c = 0; c < d; ++c) y[c] = num[c];
    return;
  }
  for (int c = 0; c < d; ++c) y[c] = den == 0.0 ? 0.0 : num[c] / den;
}

/* One (batch, head) slice: q,k,v,y point at [N,d]; w at [M,M]. */
static void blockwise_slice(const double* q, const double* k, const double* v,
                            const double* w, double* y, int N, int d, int M,
                            const int* blk, int phi, int flags) {
  size_t dd = (size_t)d * d;
  double* S = (double*)calloc((size_t)M * dd, sizeof(double));
  double* z = (double*)calloc((size_t)M * d, sizeof(double));
  double* St = (double*)malloc(dd * sizeof(double));
  double* zt = (double*)malloc((size_t)d * sizeof(double));
  double* pk = (double*)malloc((size_t)d * sizeof(double));
  double* num = (double*)malloc((size_t)d * sizeof(double));

  /* Step 1: per-block key/value summary and normaliser. */
  for (int t = 0; t < N; ++t) {
    int b = blk[t];
    for (int a = 0; a < d; ++a) pk[a] = oracle_phi(phi, k[(size_t)t * d + a]);
    double* Sb = S + (size_t)b * dd;
    for (int a = 0; a < d; ++a) {
      z[(size_t)b * d + a] += pk[a];
      for (int c = 0; c < d; ++c) Sb[(size_t)a * d + c] += pk[a] * v[(size_t)t * d + c];
    }
  }
  /* Steps 2 and 3 per query block i: mix, then read out its queries.  In the
   * causal form only the earlier chunks b < i are mixed here. */
  const int causal = (flags & ORACLE_CAUSAL) != 0;
  for (int i = 0; i < M; ++i) {
    memset(St, 0, dd * sizeof(double));
    memset(zt, 0, (size_t)d * sizeof(double));
    for (int b = 0; b < (causal ? i : M); ++b) {
      double m = w[(size_t)i * M + b];
      const double* Sb = S + (size_t)b * dd;
      for (size_t e = 0; e < dd; ++e) St[e] += m * Sb[e];
      for (int a = 0; a < d; ++a) zt[a] += m * z[(size_t)b * d + a];
    }
    for (int t = 0; t < N; ++t) {
      if (blk[t] != i) continue;
      double den = 0.0;
      for (int c = 0; c < d; ++c) num[c] = 0.0;
      for (int a = 0; a < d; ++a) {
        double pq = oracle_phi(phi, q[(size_t)t * d + a]);
        den += pq * zt[a];
        for (int c = 0; c < d; ++c) num[c] += pq * St[(size_t)a * d + c];
      }
      if (causal) {
        /* own chunk: keys t2 <= t of block i, weight W[i,i] */
        double mii = w[(size_t)i * M + i];
        for (int t2 = 0; t2 <= t; ++t2) {
          if (blk[t2] != i) continue;
          double dot = 0.0;
          for (int a = 0; a < d; ++a)
            dot += oracle_phi(phi, q[(size_t)t * d + a]) * oracle_phi(phi, k[(size_t)t2 * d + a]);
          den += mii * dot;
          for (int c = 0; c < d; ++c) num[c] += mii * dot * v[(size_t)t2 * d + c];
        }
      }
      finish_row(y + (size_t)t * d, num, den, d, flags);
    }
  }
  free(S); free(z); free(St); free(zt); free(pk); free(num);
}

/* Causal form needs every block to be one run of consecutive tokens, in block
 * order: block b = tokens [b*nb, (b+1)*nb). */
static int chunks_contiguous(const int* blk, int N, int M) {
  int nb = N / M;
  for (int t = 0; t < N; ++t)
    if (blk[t] != t / nb) return 0;
  return 1;
}

/* Q,K,V,Y: [B,H,N,d] fp64 row-major.  W: [H,M,M] fp64.  Returns 0, or -1 on a
 * bad shape.  nthreads <= 0 means all available threads. */
int oracle_mhla_blockwise(const double* Q, const double* K, const double* V,
                          const double* W, double* Y, int B, int H, int N, int d,
                          const int grid[3], const int block[3], int phi, int flags,
                          int nthreads) {
  if (B <= 0 || H <= 0 || N <= 0 || d <= 0 || (phi != 0 && phi != 1)) return -1;
  if (flags & ~(ORACLE_NO_NORM | ORACLE_CAUSAL)) return -1;
  if (!geom_ok(N, grid, block)) return -1;
  int M = oracle_num_blocks(grid, block);
  int* blk = (int*)malloc((size_t)N * sizeof(int));
  for (int t = 0; t < N; ++t) {
    blk[t] = oracle_block_of_token(grid, block, t);
    if (blk[t] < 0 || blk[t] >= M) { free(blk); return -1; }
  }
  if ((flags & ORACLE_CAUSAL) && !chunks_contiguous(blk, N, M)) { free(blk); return -1; }
  long nslices = (long)B * H;
  size_t sl = (size_t)N * d;
#ifdef _OPENMP
  int nt = nthreads > 0 ? nthreads : omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(nt)
#endif
  for (long s = 0; s < nslices; ++s) {
    int h = (int)(s % H);
    blockwise_slice(Q + s * sl, K + s * sl, V + s * sl, W + (size_t)h * M * M,
                    Y + s * sl, N, d, M, blk, phi, flags);
  }
  (void)nthreads;
  free(blk);
  return 0;
}

/* Brute force on explicit rows of A.  rows[r] = slice * N + q with slice =
 * b*H + h.  Yrows: [nrows, d].  Returns 0 or -1. */
int oracle_mhla_rows(const double* Q, const double* K, const double* V,
                     const double* W, double* Yrows, int B, int H, int N, int d,
                     const int grid[3], const int block[3], int phi, int flags,
                     const long* rows, int nrows) {
  if (B <= 0 || H <= 0 || N <= 0 || d <= 0 || (phi != 0 && phi != 1)) return -1;
  if (flags & ~(ORACLE_NO_NORM | ORACLE_CAUSAL)) return -1;
  if (!geom_ok(N, grid, block)) return -1;
  int M = oracle_num_blocks(grid, block);
  /* the causal mask is on token order; it is the chunkwise form only when the
   * blocks are consecutive runs, which the caller checks with blockwise */
  const int jmax_causal = (flags & ORACLE_CAUSAL) != 0;
  size_t sl = (size_t)N * d;
  if (nrows < 0 || (nrows > 0 && rows == NULL)) return -1;
  for (int r = 0; r < nrows; ++r)
    if (rows[r] < 0 || rows[r] >= (long)B * H * N) return -1;
#ifdef _OPENMP
#pragma omp parallel for schedule(dynamic, 1)
#endif
  for (int r = 0; r < nrows; ++r) {
    long s = rows[r] / N;
    int qi = (int)(rows[r] % N);
    int h = (int)(s % H);
    const double* q = Q + s * sl + (size_t)qi * d;
    const double* k = K + s * sl;
    const double* v = V + s * sl;
    const double* w = W + (size_t)h * M * M;
    int iq = oracle_block_of_token(grid, block, qi);
    if (iq < 0 || iq >= M) { Yrows[(size_t)r * d] = NAN; continue; }
    double* out = Yrows + (size_t)r * d;
    double den = 0.0;
    for (int c = 0; c < d; ++c) out[c] = 0.0;
    for (int j = 0; j < (jmax_causal ? qi + 1 : N); ++j) {
      double dot = 0.0;
      for (int a = 0; a < d; ++a)
        dot += oracle_phi(phi, q[a]) * oracle_phi(phi, k[(size_t)j * d + a]);
      int jb = oracle_block_of_token(grid, block, j);
      if (jb < 0 || jb >= M) { den = NAN; break; }
      double A = w[(size_t)iq * M + jb] * dot;
      den += A;
      for (int c = 0; c < d; ++c) out[c] += A * v[(size_t)j * d + c];
    }
    if (!(flags & ORACLE_NO_NORM))
      for (int c = 0; c < d; ++c) out[c] = den == 0.0 ? 0.0 : out[c] / den;
  }
  return 0;
}
