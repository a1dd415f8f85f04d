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

#include <atomic>

namespace mhla {

typedef uint16_t bf16_t;  // raw bfloat16 bits

struct Geo {
  int T, Hg, Wg;        // token grid
  int bt, bh, bw;       // block dims
  int nbz, nby, nbx;    // block grid
  int M;                // number of blocks
  int nb;               // tokens per block
  float inv_bw, inv_bhw;  // 1/bw and 1/(bh*bw), for exact small-integer division
  int norm;             // 1: divide by the denominator; 0: numerator only (the
                        // normaliser switch of the MHLA paper, used for language
                        // modelling and very long video)

  // Token index of member j (raster order inside the tile) of block b.
  __host__ __device__ __forceinline__ int token(int b, int j) const {
    return blockbase(b) + tokoff(j);
  }
  // First token of block b (blocks in raster order of the block grid).
  __host__ __device__ __forceinline__ int blockbase(int b) const {
    const int nyx = nby * nbx;
    const int bz = b / nyx, r = b - bz * nyx;
    const int by = r / nbx, bx = r - by * nbx;
    return ((bz * bt) * Hg + by * bh) * Wg + bx * bw;
  }
  // Offset of member j from the block's first token.  floor(a / b) is taken
  // as (int)((a + 0.5) * fl(1/b)): the true quotient is at least 0.5/b away
  // from an integer and the rounding error is below 2^-23 (a + 0.5)/b, so the
  // result is exact for 0 <= a < 2^22 (the library rejects larger blocks).
  __host__ __device__ __forceinline__ int tokoff(int j) const {
    const int bhw = bh * bw;
    const int jz = (int)(((float)j + 0.5f) * inv_bhw);
    const int r = j - jz * bhw;
    const int jy = (int)(((float)r + 0.5f) * inv_bw);
    return (jz * Hg + jy) * Wg + (r - jy * bw);
  }
};

enum { PHI_RELU = 0, PHI_ELU1 = 1 };

// Factor applied to a numerator row: 1/den, 0 for a zero denominator (a
// ReLU query whose features are all zero), or 1 with the normaliser off.
__device__ __forceinline__ float out_scale(const Geo& g, float den) {
  return g.norm ? (den == 0.0f ? 0.0f : 1.0f / den) : 1.0f;
}

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

// Per-launch event recording (mhla_forward_profiled).  While a recorder is
// installed for the calling thread, every forward launch site calls
// launch_mark(stream, name) right after its kernel launch: the next event is
// recorded on that stream and the kernel's name kept.  With no recorder the
// call does nothing.
struct LaunchRecorder {
  void* const* events;  // hipEvent_t handles; events[0] precedes the first launch
  int cap;              // launches that have an event (max_events - 1)
  int n = 0;            // launches seen
  const char** names;   // may be null
  bool failed = false;  // a hipEventRecord failed
};
inline thread_local LaunchRecorder* g_launch_rec = nullptr;

inline void launch_mark(hipStream_t st, const char* name) {
  LaunchRecorder* r = g_launch_rec;
  if (r == nullptr) return;
  if (r->n < r->cap) {
    if (hipEventRecord(static_cast<hipEvent_t>(r->events[r->n + 1]), st) != hipSuccess)
      r->failed = true;
    if (r->names != nullptr) r->names[r->n] = name;
  }
  ++r->n;
}

// Raises a kernel's dynamic LDS limit to `bytes` once per device (the
// attribute belongs to the function on each device).  `done` is the caller's
// per-kernel flag array; threads that race here only repeat the call.
// Returns 0, or -1 when the runtime refuses.
inline int lds_limit_once(const void* fn, std::atomic<bool> (&done)[64], int bytes) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return -1;
  const bool tracked = dev >= 0 && dev < 64;
  if (tracked && done[dev].load(std::memory_order_acquire)) return 0;
  if (hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, bytes) != hipSuccess)
    return -1;
  if (tracked) done[dev].store(true, std::memory_order_release);
  return 0;
}

}  // namespace mhla
