/* Runs the fp64 oracle under the address and undefined-behaviour sanitizers
 * (built without OpenMP): the blockwise routine and the brute-force rows on a
 * few small geometries and both option bits must agree, and bad arguments
 * must be rejected without touching memory out of bounds.  Exit status 0 on
 * success. */
#include <math.h>
#include <stdio.h>
#include <stdlib.h>

int oracle_mhla_blockwise(const double* Q, const double* K, const double* V, const double* W,
                          double* Y, int B, int H, int N, int d, const int grid[3],
                          const int block[3], int phi, int flags, int nthreads);
int oracle_mhla_rows(const double* Q, const double* K, const double* V, const double* W,
                     double* Yrows, int B, int H, int N, int d, const int grid[3],
                     const int block[3], int phi, int flags, const long* rows, int nrows);
int oracle_num_blocks(const int grid[3], const int block[3]);

static unsigned long long rng_state = 0x9E3779B97F4A7C15ull;
static double uniform(void) { /* splitmix64 -> [-1, 1) */
  unsigned long long z = (rng_state += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  z ^= z >> 31;
  return (double)(z >> 11) / 9007199254740992.0 * 2.0 - 1.0;
}

static int run_case(int B, int H, int d, const int grid[3], const int block[3], int phi,
                    int flags) {
  const int N = grid[0] * grid[1] * grid[2];
  const int M = oracle_num_blocks(grid, block);
  const size_t n = (size_t)B * H * N * d;
  double* Q = malloc(n * sizeof(double));
  double* K = malloc(n * sizeof(double));
  double* V = malloc(n * sizeof(double));
  double* Y = malloc(n * sizeof(double));
  double* W = malloc((size_t)H * M * M * sizeof(double));
  long* rows = malloc((size_t)B * H * N * sizeof(long));
  double* R = malloc(n * sizeof(double));
  for (size_t i = 0; i < n; ++i) { Q[i] = uniform(); K[i] = uniform(); V[i] = uniform(); }
  for (size_t i = 0; i < (size_t)H * M * M; ++i) W[i] = 0.5 + 0.5 * uniform();
  for (long r = 0; r < (long)B * H * N; ++r) rows[r] = r;
  int bad = 0;
  if (oracle_mhla_blockwise(Q, K, V, W, Y, B, H, N, d, grid, block, phi, flags, 1) != 0) bad = 1;
  if (oracle_mhla_rows(Q, K, V, W, R, B, H, N, d, grid, block, phi, flags, rows, B * H * N) != 0)
    bad = 1;
  double err = 0.0, mx = 0.0;
  for (size_t i = 0; i < n; ++i) {
    err = fmax(err, fabs(Y[i] - R[i]));
    mx = fmax(mx, fabs(R[i]));
  }
  if (!(err <= 1e-12 * (mx > 1.0 ? mx : 1.0))) bad = 1;
  printf("case B%d H%d N%d d%d M%d phi%d flags%d: max|blockwise - rows| = %.3e%s\n", B, H, N, d,
         M, phi, flags, err, bad ? "  FAIL" : "");
  free(Q); free(K); free(V); free(Y); free(W); free(rows); free(R);
  return bad;
}

int main(void) {
  int fails = 0;
  const int g1[3] = {1, 8, 8}, b1[3] = {1, 4, 4};
  const int g2[3] = {2, 4, 6}, b2[3] = {1, 2, 3};
  const int g3[3] = {1, 1, 24}, b3[3] = {1, 1, 6};
  const int g4[3] = {1, 6, 10}, b4[3] = {1, 3, 5};
  for (int phi = 0; phi < 2; ++phi)
    for (int flags = 0; flags < 2; ++flags) {
      fails += run_case(2, 3, 16, g1, b1, phi, flags);
      fails += run_case(1, 2, 5, g2, b2, phi, flags);
      fails += run_case(1, 1, 7, g4, b4, phi, flags);
    }
  for (int flags = 2; flags < 4; ++flags) fails += run_case(2, 2, 8, g3, b3, 1, flags);
  /* bad arguments: rejected, nothing written */
  double x[64] = {0}, y[64];
  const int gbad[3] = {1, 8, 8}, bbad[3] = {1, 3, 4};
  long r_out = 64, r_neg = -1;
  if (oracle_mhla_blockwise(x, x, x, x, y, 1, 1, 64, 1, gbad, bbad, 0, 0, 1) != -1) ++fails;
  if (oracle_mhla_blockwise(x, x, x, x, y, 1, 1, 63, 1, g1, b1, 0, 0, 1) != -1) ++fails;
  if (oracle_mhla_blockwise(x, x, x, x, y, 1, 1, 64, 1, g1, b1, 2, 0, 1) != -1) ++fails;
  if (oracle_mhla_blockwise(x, x, x, x, y, 1, 1, 64, 1, g1, b1, 0, 4, 1) != -1) ++fails;
  if (oracle_mhla_blockwise(x, x, x, x, y, 1, 1, 64, 1, g1, b1, 0, 2, 1) != -1) ++fails;
  if (oracle_mhla_rows(x, x, x, x, y, 1, 1, 64, 1, g1, b1, 0, 0, &r_out, 1) != -1) ++fails;
  if (oracle_mhla_rows(x, x, x, x, y, 1, 1, 64, 1, g1, b1, 0, 0, &r_neg, 1) != -1) ++fails;
  if (oracle_mhla_rows(x, x, x, x, y, 1, 1, 64, 1, g1, b1, 0, 0, NULL, 1) != -1) ++fails;
  printf("%s\n", fails ? "FAILED" : "ok");
  return fails ? 1 : 0;
}
