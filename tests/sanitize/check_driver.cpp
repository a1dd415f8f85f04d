// Runs the library's host-side argument checks (mhla_check.hpp, the code
// behind mhla_validate, mhla_num_blocks, mhla_lb_init and the checks of every
// entry point) under the address and undefined-behaviour sanitizers: valid
// shapes, every rejection, extreme sizes near the int limits, and the
// locality-biased initial matrix on many block grids.  Exit status 0 on
// success.
#include <climits>
#include <cmath>
#include <cstdio>
#include <vector>

#include "mhla_check.hpp"

using namespace mhla;

static int fails = 0;

static void expect(int got, int want, const char* what) {
  if (got != want) {
    std::printf("FAIL %s: got %d want %d (%s)\n", what, got, want, g_last_error.c_str());
    ++fails;
  }
}

static mhla_block_shape bs(int ndim, int T, int Hg, int Wg, int bt, int bh, int bw) {
  mhla_block_shape s;
  s.ndim = ndim;
  s.grid[0] = T; s.grid[1] = Hg; s.grid[2] = Wg;
  s.block[0] = bt; s.block[1] = bh; s.block[2] = bw;
  return s;
}

int main() {
  Shape p;
  const mhla_block_shape video = bs(3, 8, 64, 64, 1, 8, 8);
  expect(check_shape(1, 24, 32768, 64, &video, 1, 1, &p), MHLA_OK, "video");
  expect(p.M, 512, "video M");
  expect(p.nb, 64, "video nb");
  const mhla_block_shape deit = bs(2, 1, 14, 14, 1, 7, 7);
  expect(check_shape(64, 3, 196, 64, &deit, 1, 1, &p), MHLA_OK, "deit");
  expect(p.M, 4, "deit M");
  expect(check_flags(MHLA_FLAG_CAUSAL, &p), MHLA_ERR_SHAPE, "deit causal");
  expect(check_flags(8, &p), MHLA_ERR_INVALID_ARG, "unknown flag");
  const mhla_block_shape lm = bs(1, 1, 1, 2048, 1, 1, 64);
  expect(check_shape(16, 16, 2048, 64, &lm, 1, 1, &p), MHLA_OK, "lm");
  expect(check_flags(MHLA_FLAG_CAUSAL | MHLA_FLAG_NO_NORM, &p), MHLA_OK, "lm causal");

  // rejections
  expect(check_shape(1, 1, 64, 16, nullptr, 0, 0, &p), MHLA_ERR_INVALID_ARG, "null shape");
  const mhla_block_shape g8 = bs(2, 1, 8, 8, 1, 4, 4);
  expect(check_shape(0, 1, 64, 16, &g8, 0, 0, &p), MHLA_ERR_INVALID_ARG, "B=0");
  expect(check_shape(1, INT_MIN, 64, 16, &g8, 0, 0, &p), MHLA_ERR_INVALID_ARG, "H<0");
  expect(check_shape(1, 1, 64, 16, &g8, 5, 0, &p), MHLA_ERR_INVALID_ARG, "phi");
  expect(check_shape(1, 1, 64, 16, &g8, 0, -3, &p), MHLA_ERR_INVALID_ARG, "dtype");
  expect(check_shape(1, 1, 65, 16, &g8, 0, 0, &p), MHLA_ERR_SHAPE, "N");
  expect(check_shape(1, 1, 64, 129, &g8, 0, 0, &p), MHLA_ERR_UNSUPPORTED, "d");
  expect(check_shape(1, 1, 64, 12, &g8, 0, 1, &p), MHLA_ERR_UNSUPPORTED, "bf16 d");
  mhla_block_shape s = bs(0, 1, 8, 8, 1, 4, 4);
  expect(check_shape(1, 1, 64, 16, &s, 0, 0, &p), MHLA_ERR_SHAPE, "ndim 0");
  s = bs(2, 2, 8, 4, 1, 4, 4);
  expect(check_shape(1, 1, 64, 16, &s, 0, 0, &p), MHLA_ERR_SHAPE, "unused axis");
  s = bs(2, 1, 8, 8, 1, 3, 4);
  expect(check_shape(1, 1, 64, 16, &s, 0, 0, &p), MHLA_ERR_SHAPE, "divide");
  s = bs(2, 1, 8, 8, 1, 0, 4);
  expect(check_shape(1, 1, 64, 16, &s, 0, 0, &p), MHLA_ERR_SHAPE, "zero block");
  // extreme sizes: products near and past the int limits must not overflow
  s = bs(3, INT_MAX, INT_MAX, INT_MAX, 1, 1, 1);
  expect(check_shape(1, 1, INT_MAX, 8, &s, 0, 0, &p), MHLA_ERR_SHAPE, "huge grid");
  s = bs(3, 65536, 65536, 1, 1, 1, 1);
  expect(check_shape(1, 1, 0, 8, &s, 0, 0, &p), MHLA_ERR_INVALID_ARG, "N=0");
  s = bs(1, 1, 1, INT_MAX, 1, 1, 1);
  expect(check_shape(1, 1, INT_MAX, 8, &s, 0, 0, &p), MHLA_ERR_UNSUPPORTED, "M*M*H");
  s = bs(1, 1, 1, 1 << 24, 1, 1, 1 << 23);
  expect(check_shape(1, 1, 1 << 24, 8, &s, 0, 0, &p), MHLA_ERR_UNSUPPORTED, "block size");
  s = bs(1, 1, 1, 4096, 1, 1, 64);
  expect(check_shape(INT_MAX, INT_MAX, 4096, 8, &s, 0, 0, &p), MHLA_ERR_UNSUPPORTED, "slices");
  expect(check_shape(65536, 65536, 4096, 128, &s, 0, 0, &p), MHLA_ERR_UNSUPPORTED, "elements");

  // decode arguments
  expect(check_decode(1, 1, 16, 4, 8, 31, 0, 1, 0), MHLA_OK, "decode");
  expect(check_decode(1, 1, 16, 4, 8, 32, 0, 1, 0), MHLA_ERR_INVALID_ARG, "decode t");
  expect(check_decode(1, 1, 16, INT_MAX, INT_MAX, 0, 0, 1, 0), MHLA_ERR_INVALID_ARG,
         "decode M*nb");
  expect(check_decode(1, 1, 12, 4, 8, 0, 0, 1, 0), MHLA_ERR_UNSUPPORTED, "decode d");
  expect(check_decode(INT_MAX, INT_MAX, 16, 4, 8, 0, 0, 1, 0), MHLA_ERR_UNSUPPORTED,
         "decode slices");

  // locality-biased initial matrix: rows sum to 1, the diagonal is the row
  // maximum, the farthest block gets 0, entries are in [0, 1]
  const int shapes[][6] = {{1, 1, 3, 1, 1, 1},  {1, 4, 4, 1, 2, 2},  {1, 14, 14, 1, 7, 7},
                           {8, 64, 64, 1, 8, 8}, {2, 3, 4, 1, 1, 1},  {1, 8, 8, 1, 8, 8},
                           {4, 16, 16, 2, 4, 4}, {1, 1, 64, 1, 1, 2}, {3, 5, 7, 1, 1, 1}};
  for (const auto& sh : shapes) {
    s = bs(3, sh[0], sh[1], sh[2], sh[3], sh[4], sh[5]);
    const int M = (sh[0] / sh[3]) * (sh[1] / sh[4]) * (sh[2] / sh[5]);
    std::vector<float> W((size_t)M * M + 1, -1.0f);
    expect(lb_init_checked(&s, W.data(), (size_t)M * M - 1), MHLA_ERR_INVALID_ARG, "capacity");
    expect(lb_init_checked(&s, W.data(), (size_t)M * M), MHLA_OK, "lb_init");
    if (W[(size_t)M * M] != -1.0f) { std::printf("FAIL lb_init wrote past M*M\n"); ++fails; }
    for (int i = 0; i < M; ++i) {
      double sum = 0.0, mx = 0.0, mn = 2.0;
      for (int j = 0; j < M; ++j) {
        const float w = W[(size_t)i * M + j];
        sum += w;
        mx = std::fmax(mx, w);
        mn = std::fmin(mn, w);
      }
      if (std::fabs(sum - 1.0) > 1e-5 || W[(size_t)i * M + i] != (float)mx || mn < 0.0 ||
          (M > 1 && mn != 0.0)) {
        std::printf("FAIL lb_init row %d of M=%d\n", i, M);
        ++fails;
        break;
      }
    }
  }
  s = bs(1, 1, 1, 8, 1, 1, 3);
  float w1[64];
  expect(lb_init_checked(&s, w1, 64), MHLA_ERR_SHAPE, "lb_init shape");
  expect(lb_init_checked(nullptr, w1, 64), MHLA_ERR_INVALID_ARG, "lb_init null");

  // overlap test on adjacent and distant ranges
  char buf[64];
  if (overlaps(buf, 16, buf + 16, 16) || !overlaps(buf, 17, buf + 16, 16) ||
      !overlaps(buf + 8, 1, buf, 64)) {
    std::printf("FAIL overlaps\n");
    ++fails;
  }
  std::printf("%s\n", fails ? "FAILED" : "ok");
  return fails ? 1 : 0;
}
