// mhla_common.hpp -- device helpers shared by the MHLA kernels (gfx950).
//
// Geometry follows "MHLA: Restoring Expressivity of Linear Attention via
// Token-Level Multi-Head" §1/§4.1: the N tokens of a slice are a (T, Hg, Wg)
// grid in raster order (x fastest), cut into M equal (bt, bh, bw) tiles that
// are numbered in raster order of the block grid (Fig. 4b puts block 1 at the
// top-left).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mhla {

typedef uint16_t bf16_t;  // raw bfloat16 bits

struct Geo {
  int T, Hg, Wg;        // token grid
  int bt, bh, bw;       // block dims
  int nbz, nby, nbx;    // block grid
  int M;                // number of blocks
  int nb;               // tokens per block

  // Token index of member j (raster order inside the tile) of block b.
  __host__ __device__ __forceinline__ int token(int b, int j) const {
    const int bx = b % nbx;
    const int by = (b / nbx) % nby;
    const int bz = b / (nbx * nby);
    const int jx = j % bw;
    const int jy = (j / bw) % bh;
    const int jz = j / (bw * bh);
    return ((bz * bt + jz) * Hg + by * bh + jy) * Wg + bx * bw + jx;
  }
};

enum { PHI_RELU = 0, PHI_ELU1 = 1 };

// Feature maps named in the attention-variants tutorial (linear attention
// section): ReLU, and elu(x)+1 with alpha = 1.
__device__ __forceinline__ float phi_apply(int kind, float x) {
  if (kind == PHI_RELU) return fmaxf(x, 0.0f);
  return x > 0.0f ? x + 1.0f : expf(x);
}

__device__ __forceinline__ float bf16_to_f32(bf16_t u) {
  return __uint_as_float(static_cast<uint32_t>(u) << 16);
}

// Round to nearest, ties to even (finite inputs; NaN maps to a quiet NaN).
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<bf16_t>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<bf16_t>(u >> 16);
}

template <typename T> struct Elt;
template <> struct Elt<float> {
  static __device__ __forceinline__ float load(const float* p) { return *p; }
  static __device__ __forceinline__ void store(float* p, float v) { *p = v; }
};
template <> struct Elt<bf16_t> {
  static __device__ __forceinline__ float load(const bf16_t* p) { return bf16_to_f32(*p); }
  static __device__ __forceinline__ void store(bf16_t* p, float v) { *p = f32_to_bf16(v); }
};

}  // namespace mhla
