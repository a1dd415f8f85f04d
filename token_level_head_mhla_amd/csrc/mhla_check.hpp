// mhla_check.hpp -- host-side argument checks of libmhla, in plain C++17 (no
// HIP header), so that they also build for the CPU with the address and
// undefined-behaviour sanitizers.
//
// The checks follow the statement of the problem in "MHLA: Restoring
// Expressivity of Linear Attention via Token-Level Multi-Head": the N tokens
// of a slice are a (T, Hg, Wg) grid in raster order, cut into M equal,
// non-overlapping (bt, bh, bw) tiles (§1 and §4.1; blocks are numbered in
// raster order of the block grid, Fig. 4b).  Blocks must divide the grid
// (§5.1 pads 224 to 256 for this).  The locality-biased initial mixing matrix
// is the one of §4.2.
#pragma once

#include <cmath>
#include <cstdarg>
#include <cstddef>
#include <cstdint>
#include <cstdio>
#include <string>

#include "mhla.h"

namespace mhla {

// The calling thread's most recent failure message (mhla_last_error).
inline thread_local std::string g_last_error;

inline int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

// A checked shape: the token grid, the block dims, the block grid and the
// option bits.
struct Shape {
  int B = 0, H = 0, N = 0, d = 0, phi = 0, dtype = 0;
  int flags = 0;
  int T = 1, Hg = 1, Wg = 1;     // token grid
  int bt = 1, bh = 1, bw = 1;    // block dims
  int nbz = 1, nby = 1, nbx = 1; // block grid
  int M = 1;                     // number of blocks
  int nb = 1;                    // tokens per block
  bool causal() const { return (flags & MHLA_FLAG_CAUSAL) != 0; }
  bool norm() const { return (flags & MHLA_FLAG_NO_NORM) == 0; }
  long slices() const { return (long)B * H; }
  size_t elt() const { return dtype == MHLA_DTYPE_F32 ? 4 : 2; }
  size_t tensor_bytes() const { return (size_t)B * H * N * d * elt(); }
  size_t w_bytes() const { return (size_t)H * M * M * sizeof(float); }
};

// Sizes, enums and the block shape.  Clears the thread's last error first.
inline int check_shape(int B, int H, int N, int d, const mhla_block_shape* s, int phi, int dtype,
                       Shape* p) {
  g_last_error.clear();
  if (s == nullptr) return fail(MHLA_ERR_INVALID_ARG, "block_shape is NULL");
  if (B <= 0 || H <= 0 || N <= 0 || d <= 0)
    return fail(MHLA_ERR_INVALID_ARG, "B=%d H=%d N=%d d=%d: all must be positive", B, H, N, d);
  if (phi != MHLA_PHI_RELU && phi != MHLA_PHI_ELU1)
    return fail(MHLA_ERR_INVALID_ARG, "unknown phi_kind %d", phi);
  if (dtype != MHLA_DTYPE_F32 && dtype != MHLA_DTYPE_BF16)
    return fail(MHLA_ERR_INVALID_ARG, "unknown dtype %d", dtype);
  if (s->ndim < 1 || s->ndim > 3)
    return fail(MHLA_ERR_SHAPE, "block_shape.ndim=%d must be 1, 2 or 3", s->ndim);
  long n = 1;
  for (int a = 0; a < 3; ++a) {
    const int gd = s->grid[a], bd = s->block[a];
    if (gd <= 0 || bd <= 0)
      return fail(MHLA_ERR_SHAPE, "grid[%d]=%d block[%d]=%d must be positive", a, gd, a, bd);
    if (a < 3 - s->ndim && (gd != 1 || bd != 1))
      return fail(MHLA_ERR_SHAPE, "axis %d is unused for ndim=%d but grid/block are %d/%d", a,
                  s->ndim, gd, bd);
    if (gd % bd != 0)
      return fail(MHLA_ERR_SHAPE, "block[%d]=%d does not divide grid[%d]=%d", a, bd, a, gd);
    n *= gd;  // each factor < 2^31, so the running product never passes 2^62 before the check
    if (n > 0x7fffffffL)
      return fail(MHLA_ERR_SHAPE, "grid %dx%dx%d has more than 2^31-1 tokens", s->grid[0],
                  s->grid[1], s->grid[2]);
  }
  if (n != N)
    return fail(MHLA_ERR_SHAPE, "grid %dx%dx%d has %ld tokens but N=%d", s->grid[0], s->grid[1],
                s->grid[2], n, N);
  if (d > 128) return fail(MHLA_ERR_UNSUPPORTED, "d=%d > 128 is not supported", d);
  if (dtype == MHLA_DTYPE_BF16 && d % 8 != 0)
    return fail(MHLA_ERR_UNSUPPORTED, "bf16 needs d to be a multiple of 8 (d=%d)", d);
  if ((long)B * H > 0x7fffffffL) return fail(MHLA_ERR_UNSUPPORTED, "too many slices");
  if ((long)B * H * N > (1L << 40) / d)
    return fail(MHLA_ERR_UNSUPPORTED, "B*H*N*d = %ld elements is too large",
                (long)B * H * N * d);
  Shape q;
  q.B = B; q.H = H; q.N = N; q.d = d; q.phi = phi; q.dtype = dtype;
  q.T = s->grid[0]; q.Hg = s->grid[1]; q.Wg = s->grid[2];
  q.bt = s->block[0]; q.bh = s->block[1]; q.bw = s->block[2];
  q.nbz = q.T / q.bt; q.nby = q.Hg / q.bh; q.nbx = q.Wg / q.bw;
  q.M = q.nbz * q.nby * q.nbx;          // <= N < 2^31
  q.nb = N / q.M;
  if (q.nb >= (1 << 22))
    return fail(MHLA_ERR_UNSUPPORTED, "blocks of %d tokens are too large (limit 2^22)", q.nb);
  if ((long)q.M * q.M * H > 0x7fffffffL)
    return fail(MHLA_ERR_UNSUPPORTED, "M=%d is too large", q.M);
  if (p) *p = q;
  return MHLA_OK;
}

// Blocks are runs of consecutive tokens when every grid axis to the right of
// the first axis that a block does not span in full is spanned in full.
inline bool contiguous_blocks(const Shape& s) {
  if (s.bw < s.Wg) return s.bh == 1 && s.bt == 1;
  if (s.bh < s.Hg) return s.bt == 1;
  return true;
}

// Option bits: reject unknown ones and causal calls whose blocks are not runs
// of consecutive tokens.
inline int check_flags(int flags, Shape* p) {
  if (flags & ~(MHLA_FLAG_NO_NORM | MHLA_FLAG_CAUSAL))
    return fail(MHLA_ERR_INVALID_ARG, "unknown option bits 0x%x", flags);
  p->flags = flags;
  if (p->causal() && !contiguous_blocks(*p))
    return fail(MHLA_ERR_SHAPE,
                "the causal form needs blocks that are runs of consecutive tokens (block "
                "%dx%dx%d in grid %dx%dx%d is not)",
                p->bt, p->bh, p->bw, p->T, p->Hg, p->Wg);
  return MHLA_OK;
}

inline bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t pa = reinterpret_cast<uintptr_t>(a), pb = reinterpret_cast<uintptr_t>(b);
  return pa < pb + nb && pb < pa + na;
}

// Locality-biased initial mixing matrix (§4.2): blocks at their integer
// coordinates (bz, by, bx) on the block grid, Euclidean distance between
// them, m0[i][j] = (1 - dist(i,j) / max_k dist(i,k)) / (row sum).  With one
// block m0 = [[1]].  W holds M*M floats.
inline void lb_init(const Shape& g, float* W) {
  const size_t M = (size_t)g.M;
  if (M == 1) {
    W[0] = 1.0f;
    return;
  }
  auto coord = [&](size_t b, double* c) {
    const size_t nyx = (size_t)g.nby * g.nbx;
    c[0] = (double)(b / nyx);
    c[1] = (double)((b % nyx) / g.nbx);
    c[2] = (double)(b % g.nbx);
  };
  auto dist = [](const double* a, const double* b) {
    return std::sqrt((a[0] - b[0]) * (a[0] - b[0]) + (a[1] - b[1]) * (a[1] - b[1]) +
                     (a[2] - b[2]) * (a[2] - b[2]));
  };
  for (size_t i = 0; i < M; ++i) {
    double ci[3];
    coord(i, ci);
    // the farthest block from i is a corner of the block grid
    double far = 0.0;
    for (int corner = 0; corner < 8; ++corner) {
      const double c[3] = {(corner & 4) ? g.nbz - 1.0 : 0.0, (corner & 2) ? g.nby - 1.0 : 0.0,
                           (corner & 1) ? g.nbx - 1.0 : 0.0};
      far = std::fmax(far, dist(ci, c));
    }
    double sum = 0.0;
    for (size_t j = 0; j < M; ++j) {
      double cj[3];
      coord(j, cj);
      sum += 1.0 - dist(ci, cj) / far;
    }
    for (size_t j = 0; j < M; ++j) {
      double cj[3];
      coord(j, cj);
      W[i * M + j] = (float)((1.0 - dist(ci, cj) / far) / sum);
    }
  }
}

// mhla_lb_init's checks and fill (host only).
inline int lb_init_checked(const mhla_block_shape* s, float* W, size_t capacity) {
  g_last_error.clear();
  if (s == nullptr) return fail(MHLA_ERR_INVALID_ARG, "block_shape is NULL");
  long n = 1;
  for (int a = 0; a < 3; ++a) {
    if (s->grid[a] <= 0)
      return fail(MHLA_ERR_SHAPE, "grid[%d]=%d must be positive", a, s->grid[a]);
    n *= s->grid[a];
    if (n > 0x7fffffffL)
      return fail(MHLA_ERR_SHAPE, "grid %dx%dx%d is too large", s->grid[0], s->grid[1],
                  s->grid[2]);
  }
  Shape g;
  const int rc = check_shape(1, 1, (int)n, 8, s, MHLA_PHI_RELU, MHLA_DTYPE_F32, &g);
  if (rc != MHLA_OK) return rc;
  const size_t M = (size_t)g.M;
  if (W == nullptr || capacity < M * M)
    return fail(MHLA_ERR_INVALID_ARG, "W needs room for %zu floats (M=%zu)", M * M, M);
  lb_init(g, W);
  return MHLA_OK;
}

// Checks of mhla_decode_step's scalar arguments (the pointers are checked by
// the caller).
inline int check_decode(int B, int H, int d, int M, int nb, int t, int phi, int dtype, int flags) {
  g_last_error.clear();
  if (B <= 0 || H <= 0 || d <= 0 || M <= 0 || nb <= 0)
    return fail(MHLA_ERR_INVALID_ARG, "B=%d H=%d d=%d M=%d nb=%d: all must be positive", B, H, d,
                M, nb);
  if ((long)M * nb > 0x7fffffffL || t < 0 || (long)t >= (long)M * nb)
    return fail(MHLA_ERR_INVALID_ARG, "t=%d is outside [0, M*nb) with M=%d nb=%d", t, M, nb);
  if (phi != MHLA_PHI_RELU && phi != MHLA_PHI_ELU1)
    return fail(MHLA_ERR_INVALID_ARG, "unknown phi_kind %d", phi);
  if (dtype != MHLA_DTYPE_F32 && dtype != MHLA_DTYPE_BF16)
    return fail(MHLA_ERR_INVALID_ARG, "unknown dtype %d", dtype);
  if (flags & ~(MHLA_FLAG_NO_NORM | MHLA_FLAG_CAUSAL))
    return fail(MHLA_ERR_INVALID_ARG, "unknown option bits 0x%x", flags);
  if (d > 128) return fail(MHLA_ERR_UNSUPPORTED, "d=%d > 128 is not supported", d);
  if (dtype == MHLA_DTYPE_BF16 && d % 8 != 0)
    return fail(MHLA_ERR_UNSUPPORTED, "bf16 needs d to be a multiple of 8 (d=%d)", d);
  if ((long)B * H > 0x7fffffffL || (long)M * M * H > 0x7fffffffL)
    return fail(MHLA_ERR_UNSUPPORTED, "too many slices or blocks");
  return MHLA_OK;
}

}  // namespace mhla
