// mhla_api.hip -- C ABI of libmhla: argument checks, path choice, workspace
// cache and kernel launches for the MHLA forward (gfx950).
//
// The operation is the forward pass of "MHLA: Restoring Expressivity of
// Linear Attention via Token-Level Multi-Head" §4.1 (summaries, multi-head
// mixing, readout); the entry points are declared and documented in mhla.h.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <utility>

#include "mhla.h"
#include "mhla_common.hpp"
#include "k_generic.hpp"
#include "k_fused.hpp"
#include "k_cols.hpp"
#include "k_blocked.hpp"
#include "k_pairs.hpp"
#include "k_causal.hpp"
#include "k_backward.hpp"
#include "k_pairs_bwd.hpp"
#include "k_decode.hpp"

namespace mhla {
namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

struct Problem {
  int B, H, N, d, phi, dtype;
  int flags = 0;
  bool causal() const { return (flags & MHLA_FLAG_CAUSAL) != 0; }
  Geo g;
  long slices() const { return (long)B * H; }
  size_t elt() const { return dtype == MHLA_DTYPE_F32 ? 4 : 2; }
  size_t tensor_bytes() const { return (size_t)B * H * N * d * elt(); }
};

int check(int B, int H, int N, int d, const mhla_block_shape* s, int phi, int dtype,
          Problem* p) {
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
    n *= gd;
  }
  if (n != N)
    return fail(MHLA_ERR_SHAPE, "grid %dx%dx%d has %ld tokens but N=%d", s->grid[0], s->grid[1],
                s->grid[2], n, N);
  if (d > 128) return fail(MHLA_ERR_UNSUPPORTED, "d=%d > 128 is not supported", d);
  if (dtype == MHLA_DTYPE_BF16 && d % 8 != 0)
    return fail(MHLA_ERR_UNSUPPORTED, "bf16 needs d to be a multiple of 8 (d=%d)", d);
  if ((long)B * H > 0x7fffffffL) return fail(MHLA_ERR_UNSUPPORTED, "too many slices");
  if (p) {
    Geo& g = p->g;
    g.T = s->grid[0]; g.Hg = s->grid[1]; g.Wg = s->grid[2];
    g.bt = s->block[0]; g.bh = s->block[1]; g.bw = s->block[2];
    g.nbz = g.T / g.bt; g.nby = g.Hg / g.bh; g.nbx = g.Wg / g.bw;
    g.M = g.nbz * g.nby * g.nbx;
    g.nb = g.bt * g.bh * g.bw;
    g.inv_bw = 1.0f / (float)g.bw;
    g.inv_bhw = 1.0f / (float)(g.bh * g.bw);
    g.norm = 1;
    p->B = B; p->H = H; p->N = N; p->d = d; p->phi = phi; p->dtype = dtype;
    if (g.nb >= (1 << 22))
      return fail(MHLA_ERR_UNSUPPORTED, "blocks of %d tokens are too large (limit 2^22)", g.nb);
    if ((long)g.M * g.M * H > 0x7fffffffL)
      return fail(MHLA_ERR_UNSUPPORTED, "M=%d is too large", g.M);
  }
  return MHLA_OK;
}

// Option bits: reject unknown ones and causal calls whose blocks are not runs
// of consecutive tokens.
int check_flags(int flags, Problem* p) {
  if (flags & ~(MHLA_FLAG_NO_NORM | MHLA_FLAG_CAUSAL))
    return fail(MHLA_ERR_INVALID_ARG, "unknown option bits 0x%x", flags);
  p->flags = flags;
  p->g.norm = (flags & MHLA_FLAG_NO_NORM) ? 0 : 1;
  if (p->causal() && !blocks_contiguous(p->g))
    return fail(MHLA_ERR_SHAPE,
                "the causal form needs blocks that are runs of consecutive tokens (block "
                "%dx%dx%d in grid %dx%dx%d is not)",
                p->g.bt, p->g.bh, p->g.bw, p->g.T, p->g.Hg, p->g.Wg);
  return MHLA_OK;
}

bool path_supports(int path, const Problem& p) {
  if (p.causal())
    return path == MHLA_PATH_BLOCKED && causal_supports(p.dtype, p.d, p.g, p.slices());
  switch (path) {
    case MHLA_PATH_GENERIC: return p.slices() <= 65535;  // slices run along grid y/z
    case MHLA_PATH_FUSED: return fused_supports(p.dtype, p.d, p.g.M, p.g.nb);
    case MHLA_PATH_BLOCKED: return blocked_supports(p.dtype, p.d, p.g.M, p.slices());
    case MHLA_PATH_PAIRS: return pairs_supports(p.dtype, p.d, p.g.M, p.g.nb, p.N);
    case MHLA_PATH_COLUMNS: return cols_supports(p.dtype, p.d, p.g.M, p.g.nb, p.slices());
    default: return false;
  }
}

int choose_path(const Problem& p) {
  if (p.causal())
    return path_supports(MHLA_PATH_BLOCKED, p) ? MHLA_PATH_BLOCKED : -MHLA_ERR_UNSUPPORTED;
  if (path_supports(MHLA_PATH_FUSED, p)) return MHLA_PATH_FUSED;
  if (path_supports(MHLA_PATH_PAIRS, p)) return MHLA_PATH_PAIRS;
  // MHLA_PATH_COLUMNS is never chosen here: every column chunk re-reads the
  // slice's K and Q through L2, and on the 4096-token image shape it took
  // 64 us against 54 us for the blocked path.
  if (path_supports(MHLA_PATH_BLOCKED, p)) return MHLA_PATH_BLOCKED;
  if (path_supports(MHLA_PATH_GENERIC, p)) return MHLA_PATH_GENERIC;
  return -MHLA_ERR_UNSUPPORTED;
}

size_t workspace_for(const Problem& p, int path) {
  if (path == MHLA_PATH_GENERIC) {
    const size_t L = (size_t)p.d * p.d + p.d;
    return 2 * (size_t)p.slices() * p.g.M * L * sizeof(float);
  }
  if (path == MHLA_PATH_BLOCKED) return blocked_workspace(p.slices(), p.H, p.g.M, p.d);
  return 0;
}

// Library-owned workspaces, one per (device, stream): calls on one stream are
// ordered, so reuse across calls is safe; different streams never share.
struct Buf {
  void* ptr = nullptr;
  size_t bytes = 0;
};
std::mutex g_ws_mutex;
std::map<std::pair<int, void*>, Buf> g_ws;

int get_workspace(size_t need, hipStream_t stream, void** out) {
  *out = nullptr;
  if (need == 0) return MHLA_OK;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(MHLA_ERR_HIP, "hipGetDevice failed");
  std::lock_guard<std::mutex> lock(g_ws_mutex);
  Buf& b = g_ws[std::make_pair(dev, (void*)stream)];
  if (b.bytes < need) {
    if (b.ptr) {
      // The previous buffer may still be read by work queued on this stream.
      if (hipStreamSynchronize(stream) != hipSuccess)
        return fail(MHLA_ERR_HIP, "hipStreamSynchronize failed while growing the workspace");
      (void)hipFree(b.ptr);
      b.ptr = nullptr;
      b.bytes = 0;
    }
    size_t want = need + need / 8;
    hipError_t e = hipMalloc(&b.ptr, want);
    if (e != hipSuccess) {
      b.ptr = nullptr;
      return fail(MHLA_ERR_HIP, "hipMalloc(%zu) for the workspace failed: %s", want,
                  hipGetErrorString(e));
    }
    b.bytes = want;
  }
  *out = b.ptr;
  return MHLA_OK;
}

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const char* pa = static_cast<const char*>(a);
  const char* pb = static_cast<const char*>(b);
  return pa < pb + nb && pb < pa + na;
}

template <typename T>
int launch_generic(const Problem& p, const T* Q, const T* K, const T* V, const float* W,
                   T* Y, float* ws, hipStream_t st) {
  const int M = p.g.M, d = p.d;
  const int L = d * d + d;
  float* S = ws;
  float* St = ws + (size_t)p.slices() * M * L;
  const unsigned nsl = (unsigned)p.slices();
  k_summary_valu<T><<<dim3(M, nsl), kValuThreads, 0, st>>>(K, V, S, p.g, p.N, d, p.phi);
  k_mix_valu<<<dim3((L + kValuThreads - 1) / kValuThreads, (M + kMixRows - 1) / kMixRows, nsl),
               kValuThreads, 0, st>>>(S, W, St, M, L, p.H);
  k_readout_valu<T><<<dim3(M, nsl), kValuThreads, 0, st>>>(Q, St, Y, p.g, p.N, d, p.phi);
  return MHLA_OK;
}

int run(const void* Q, const void* K, const void* V, const float* W, void* out, int B, int H,
        int N, int d, const mhla_block_shape* shape, int phi, int dtype, int flags, int path,
        void* stream) {
  Problem p;
  int rc = check(B, H, N, d, shape, phi, dtype, &p);
  if (rc != MHLA_OK) return rc;
  rc = check_flags(flags, &p);
  if (rc != MHLA_OK) return rc;
  if (!Q || !K || !V || !W || !out)
    return fail(MHLA_ERR_INVALID_ARG, "a tensor pointer is NULL");
  const void* ptrs[5] = {Q, K, V, W, out};
  for (const void* q : ptrs)
    if (reinterpret_cast<uintptr_t>(q) % 16 != 0)
      return fail(MHLA_ERR_INVALID_ARG, "tensor pointers must be 16-byte aligned");
  const size_t tb = p.tensor_bytes();
  if (overlaps(out, tb, Q, tb) || overlaps(out, tb, K, tb) || overlaps(out, tb, V, tb))
    return fail(MHLA_ERR_ALIAS, "out overlaps Q, K or V");
  if (overlaps(out, tb, W, (size_t)H * p.g.M * p.g.M * sizeof(float)))
    return fail(MHLA_ERR_ALIAS, "out overlaps Wmix");
  if (path == MHLA_PATH_AUTO) path = choose_path(p);
  if (path < 0 || !path_supports(path, p))
    return fail(MHLA_ERR_UNSUPPORTED, "path %d does not support this shape/dtype/options", path);

  hipStream_t st = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();  // clear a stale error so the check below is ours
  void* ws = nullptr;
  rc = get_workspace(workspace_for(p, path), st, &ws);
  if (rc != MHLA_OK) return rc;

  if (path == MHLA_PATH_GENERIC) {
    if (dtype == MHLA_DTYPE_F32)
      rc = launch_generic<float>(p, (const float*)Q, (const float*)K, (const float*)V, W,
                                 (float*)out, (float*)ws, st);
    else
      rc = launch_generic<bf16_t>(p, (const bf16_t*)Q, (const bf16_t*)K, (const bf16_t*)V, W,
                                  (bf16_t*)out, (float*)ws, st);
  } else if (path == MHLA_PATH_FUSED) {
    rc = launch_fused(p.slices(), p.H, p.N, p.d, p.g, p.phi, (const bf16_t*)Q,
                      (const bf16_t*)K, (const bf16_t*)V, W, (bf16_t*)out, st);
  } else if (path == MHLA_PATH_PAIRS) {
    rc = launch_pairs(p.slices(), p.H, p.N, p.d, p.g, p.phi, (const bf16_t*)Q, (const bf16_t*)K,
                      (const bf16_t*)V, W, (bf16_t*)out, st);
  } else if (path == MHLA_PATH_COLUMNS) {
    rc = launch_cols(p.slices(), p.H, p.N, p.d, p.g, p.phi, (const bf16_t*)Q, (const bf16_t*)K,
                     (const bf16_t*)V, W, (bf16_t*)out, st);
  } else if (path == MHLA_PATH_BLOCKED && p.causal()) {
    rc = launch_causal(p.slices(), p.H, p.N, p.d, p.g, p.phi, (const bf16_t*)Q, (const bf16_t*)K,
                       (const bf16_t*)V, W, (bf16_t*)out, (bf16_t*)ws, st);
  } else if (path == MHLA_PATH_BLOCKED) {
    rc = launch_blocked(p.slices(), p.H, p.N, p.d, p.g, p.phi, (const bf16_t*)Q,
                        (const bf16_t*)K, (const bf16_t*)V, W, (bf16_t*)out, (bf16_t*)ws, st);
  }
  if (rc != MHLA_OK) return fail(MHLA_ERR_HIP, "kernel set-up failed (hipFuncSetAttribute)");
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(MHLA_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return MHLA_OK;
}

int run_backward(const void* Q, const void* K, const void* V, const float* W, const void* dY,
                 void* dQ, void* dK, void* dV, float* dW, int B, int H, int N, int d,
                 const mhla_block_shape* shape, int phi, int dtype, int flags, void* stream) {
  Problem p;
  int rc = check(B, H, N, d, shape, phi, dtype, &p);
  if (rc != MHLA_OK) return rc;
  rc = check_flags(flags, &p);
  if (rc != MHLA_OK) return rc;
  if (p.causal()) return fail(MHLA_ERR_UNSUPPORTED, "the causal form has no backward pass here");
  // blocks of at most 16 tokens: the token-pair order; otherwise the blocked one
  const bool pairs = pairs_bwd_supports(dtype, d, p.g.M, p.g.nb, N);
  if (!pairs && !backward_supports(dtype, d, p.g.M, p.slices()))
    return fail(MHLA_ERR_UNSUPPORTED, "the backward pass needs bf16 and d <= 96 (d=%d dtype=%d)",
                d, dtype);
  const void* in[5] = {Q, K, V, W, dY};
  void* outp[4] = {dQ, dK, dV, dW};
  for (const void* q : in)
    if (!q) return fail(MHLA_ERR_INVALID_ARG, "an input pointer is NULL");
  for (const void* q : outp)
    if (!q) return fail(MHLA_ERR_INVALID_ARG, "an output pointer is NULL");
  for (const void* q : in)
    if (reinterpret_cast<uintptr_t>(q) % 16 != 0)
      return fail(MHLA_ERR_INVALID_ARG, "tensor pointers must be 16-byte aligned");
  for (const void* q : outp)
    if (reinterpret_cast<uintptr_t>(q) % 16 != 0)
      return fail(MHLA_ERR_INVALID_ARG, "tensor pointers must be 16-byte aligned");
  const size_t tb = p.tensor_bytes(), wb = (size_t)H * p.g.M * p.g.M * sizeof(float);
  const size_t in_b[5] = {tb, tb, tb, wb, tb};
  const size_t out_b[4] = {tb, tb, tb, wb};
  for (int a = 0; a < 4; ++a) {
    for (int b = 0; b < 5; ++b)
      if (overlaps(outp[a], out_b[a], in[b], in_b[b]))
        return fail(MHLA_ERR_ALIAS, "gradient %d overlaps input %d", a, b);
    for (int b = a + 1; b < 4; ++b)
      if (overlaps(outp[a], out_b[a], outp[b], out_b[b]))
        return fail(MHLA_ERR_ALIAS, "gradients %d and %d overlap", a, b);
  }
  hipStream_t st = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  void* ws = nullptr;
  rc = get_workspace(pairs ? pairs_bwd_workspace(p.slices(), p.g.M, N, d)
                           : backward_workspace(p.slices(), H, p.g.M, N, d),
                     st, &ws);
  if (rc != MHLA_OK) return rc;
  if (pairs)
    rc = launch_pairs_backward(p.slices(), B, H, N, d, p.g, phi, (const bf16_t*)Q,
                               (const bf16_t*)K, (const bf16_t*)V, W, (const bf16_t*)dY,
                               (bf16_t*)dQ, (bf16_t*)dK, (bf16_t*)dV, dW, ws, st);
  else
    rc = launch_backward(p.slices(), B, H, N, d, p.g, phi, (const bf16_t*)Q, (const bf16_t*)K,
                       (const bf16_t*)V, W, (const bf16_t*)dY, (bf16_t*)dQ, (bf16_t*)dK,
                       (bf16_t*)dV, dW, ws, st);
  if (rc != MHLA_OK) return fail(MHLA_ERR_HIP, "backward set-up failed");
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(MHLA_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return MHLA_OK;
}

}  // namespace
}  // namespace mhla

using namespace mhla;

extern "C" {

int mhla_forward(const void* Q, const void* K, const void* V, const float* Wmix, void* out,
                 int B, int H, int N, int d, const mhla_block_shape* block_shape, int phi_kind,
                 int dtype, void* stream) {
  return run(Q, K, V, Wmix, out, B, H, N, d, block_shape, phi_kind, dtype, 0, MHLA_PATH_AUTO,
             stream);
}

int mhla_forward_path(const void* Q, const void* K, const void* V, const float* Wmix,
                      void* out, int B, int H, int N, int d,
                      const mhla_block_shape* block_shape, int phi_kind, int dtype, int path,
                      void* stream) {
  if (path < MHLA_PATH_AUTO || path > MHLA_PATH_COLUMNS)
    return fail(MHLA_ERR_INVALID_ARG, "unknown path %d", path);
  return run(Q, K, V, Wmix, out, B, H, N, d, block_shape, phi_kind, dtype, 0, path, stream);
}

int mhla_forward_ex(const void* Q, const void* K, const void* V, const float* Wmix, void* out,
                    int B, int H, int N, int d, const mhla_block_shape* block_shape,
                    int phi_kind, int dtype, int flags, int path, void* stream) {
  if (path < MHLA_PATH_AUTO || path > MHLA_PATH_COLUMNS)
    return fail(MHLA_ERR_INVALID_ARG, "unknown path %d", path);
  return run(Q, K, V, Wmix, out, B, H, N, d, block_shape, phi_kind, dtype, flags, path, stream);
}

int mhla_backward(const void* Q, const void* K, const void* V, const float* Wmix, const void* dY,
                  void* dQ, void* dK, void* dV, float* dWmix, int B, int H, int N, int d,
                  const mhla_block_shape* block_shape, int phi_kind, int dtype, int flags,
                  void* stream) {
  return run_backward(Q, K, V, Wmix, dY, dQ, dK, dV, dWmix, B, H, N, d, block_shape, phi_kind,
                      dtype, flags, stream);
}

size_t mhla_decode_state_bytes(int B, int H, int d, int M) {
  if (B <= 0 || H <= 0 || d <= 0 || M <= 0 || d > 128) return 0;
  return (size_t)B * H * decode_state_elems(d, M) * sizeof(float);
}

int mhla_decode_step(const void* q, const void* k, const void* v, const float* Wmix, void* y,
                     void* state, int B, int H, int d, int M, int nb, int t, int phi_kind,
                     int dtype, int flags, void* stream) {
  g_last_error.clear();
  if (B <= 0 || H <= 0 || d <= 0 || M <= 0 || nb <= 0)
    return fail(MHLA_ERR_INVALID_ARG, "B=%d H=%d d=%d M=%d nb=%d: all must be positive", B, H, d,
                M, nb);
  if ((long)M * nb > 0x7fffffffL || t < 0 || (long)t >= (long)M * nb)
    return fail(MHLA_ERR_INVALID_ARG, "t=%d is outside [0, M*nb) with M=%d nb=%d", t, M, nb);
  if (phi_kind != MHLA_PHI_RELU && phi_kind != MHLA_PHI_ELU1)
    return fail(MHLA_ERR_INVALID_ARG, "unknown phi_kind %d", phi_kind);
  if (dtype != MHLA_DTYPE_F32 && dtype != MHLA_DTYPE_BF16)
    return fail(MHLA_ERR_INVALID_ARG, "unknown dtype %d", dtype);
  if (flags & ~(MHLA_FLAG_NO_NORM | MHLA_FLAG_CAUSAL))
    return fail(MHLA_ERR_INVALID_ARG, "unknown option bits 0x%x", flags);
  if (d > 128) return fail(MHLA_ERR_UNSUPPORTED, "d=%d > 128 is not supported", d);
  if (dtype == MHLA_DTYPE_BF16 && d % 8 != 0)
    return fail(MHLA_ERR_UNSUPPORTED, "bf16 needs d to be a multiple of 8 (d=%d)", d);
  if ((long)B * H > 0x7fffffffL || (long)M * M * H > 0x7fffffffL)
    return fail(MHLA_ERR_UNSUPPORTED, "too many slices or blocks");
  if (!q || !k || !v || !Wmix || !y || !state)
    return fail(MHLA_ERR_INVALID_ARG, "a pointer is NULL");
  const void* ptrs[6] = {q, k, v, Wmix, y, state};
  for (const void* p : ptrs)
    if (reinterpret_cast<uintptr_t>(p) % 4 != 0)
      return fail(MHLA_ERR_INVALID_ARG, "pointers must be 4-byte aligned");
  const size_t eb = dtype == MHLA_DTYPE_F32 ? 4 : 2;
  const size_t tb = (size_t)B * H * d * eb;
  const size_t sb = mhla_decode_state_bytes(B, H, d, M);
  if (overlaps(y, tb, q, tb) || overlaps(y, tb, k, tb) || overlaps(y, tb, v, tb) ||
      overlaps(y, tb, state, sb))
    return fail(MHLA_ERR_ALIAS, "y overlaps q, k, v or the state");
  hipStream_t st = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  const int norm = (flags & MHLA_FLAG_NO_NORM) ? 0 : 1;
  const long slices = (long)B * H;
  int rc;
  if (dtype == MHLA_DTYPE_F32)
    rc = launch_decode_t<float>(slices, H, d, M, nb, t, phi_kind, norm, (const float*)q,
                                (const float*)k, (const float*)v, Wmix, (float*)y, (float*)state,
                                st);
  else
    rc = launch_decode_t<bf16_t>(slices, H, d, M, nb, t, phi_kind, norm, (const bf16_t*)q,
                                 (const bf16_t*)k, (const bf16_t*)v, Wmix, (bf16_t*)y,
                                 (float*)state, st);
  if (rc != 0) return fail(MHLA_ERR_HIP, "decode set-up failed (hipFuncSetAttribute)");
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(MHLA_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return MHLA_OK;
}

int mhla_plan_ex(int B, int H, int N, int d, const mhla_block_shape* block_shape, int phi_kind,
                 int dtype, int flags) {
  Problem p;
  int rc = check(B, H, N, d, block_shape, phi_kind, dtype, &p);
  if (rc != MHLA_OK) return -rc;
  rc = check_flags(flags, &p);
  if (rc != MHLA_OK) return -rc;
  return choose_path(p);
}

int mhla_lb_init(const mhla_block_shape* block_shape, float* W, size_t capacity) {
  Problem p;
  if (block_shape == nullptr) return fail(MHLA_ERR_INVALID_ARG, "block_shape is NULL");
  const long n = (long)block_shape->grid[0] * block_shape->grid[1] * block_shape->grid[2];
  if (n <= 0 || n > 0x7fffffffL)
    return fail(MHLA_ERR_SHAPE, "grid %dx%dx%d is empty or too large", block_shape->grid[0],
                block_shape->grid[1], block_shape->grid[2]);
  int rc = check(1, 1, (int)n, 8, block_shape, MHLA_PHI_RELU, MHLA_DTYPE_F32, &p);
  if (rc != MHLA_OK) return rc;
  const Geo& g = p.g;
  const size_t M = (size_t)g.M;
  if (W == nullptr || capacity < M * M)
    return fail(MHLA_ERR_INVALID_ARG, "W needs room for %zu floats (M=%zu)", M * M, M);
  if (M == 1) {
    W[0] = 1.0f;
    return MHLA_OK;
  }
  // block coordinates in raster order of the block grid (x fastest)
  auto coord = [&](size_t b, double* c) {
    const size_t nyx = (size_t)g.nby * g.nbx;
    c[0] = (double)(b / nyx);
    c[1] = (double)((b % nyx) / g.nbx);
    c[2] = (double)(b % g.nbx);
  };
  for (size_t i = 0; i < M; ++i) {
    double ci[3];
    coord(i, ci);
    // the farthest block from i is a corner of the block grid
    double far = 0.0;
    for (int corner = 0; corner < 8; ++corner) {
      const double cz = (corner & 4) ? g.nbz - 1 : 0, cy = (corner & 2) ? g.nby - 1 : 0,
                   cx = (corner & 1) ? g.nbx - 1 : 0;
      far = std::fmax(far, std::sqrt((ci[0] - cz) * (ci[0] - cz) + (ci[1] - cy) * (ci[1] - cy) +
                                     (ci[2] - cx) * (ci[2] - cx)));
    }
    double sum = 0.0;
    for (size_t j = 0; j < M; ++j) {
      double cj[3];
      coord(j, cj);
      const double dist = std::sqrt((ci[0] - cj[0]) * (ci[0] - cj[0]) +
                                    (ci[1] - cj[1]) * (ci[1] - cj[1]) +
                                    (ci[2] - cj[2]) * (ci[2] - cj[2]));
      sum += 1.0 - dist / far;
    }
    for (size_t j = 0; j < M; ++j) {
      double cj[3];
      coord(j, cj);
      const double dist = std::sqrt((ci[0] - cj[0]) * (ci[0] - cj[0]) +
                                    (ci[1] - cj[1]) * (ci[1] - cj[1]) +
                                    (ci[2] - cj[2]) * (ci[2] - cj[2]));
      W[i * M + j] = (float)((1.0 - dist / far) / sum);
    }
  }
  return MHLA_OK;
}

int mhla_validate(int B, int H, int N, int d, const mhla_block_shape* block_shape, int phi_kind,
                  int dtype) {
  Problem p;
  return check(B, H, N, d, block_shape, phi_kind, dtype, &p);
}

int mhla_plan(int B, int H, int N, int d, const mhla_block_shape* block_shape, int phi_kind,
              int dtype) {
  Problem p;
  int rc = check(B, H, N, d, block_shape, phi_kind, dtype, &p);
  if (rc != MHLA_OK) return -rc;
  return choose_path(p);
}

int mhla_num_blocks(int N, const mhla_block_shape* block_shape) {
  Problem p;
  int rc = check(1, 1, N, 8, block_shape, MHLA_PHI_RELU, MHLA_DTYPE_F32, &p);
  if (rc != MHLA_OK) return -rc;
  return p.g.M;
}

size_t mhla_workspace_bytes(int B, int H, int N, int d, const mhla_block_shape* block_shape,
                            int dtype, int path) {
  Problem p;
  if (check(B, H, N, d, block_shape, MHLA_PHI_RELU, dtype, &p) != MHLA_OK) return 0;
  if (path == MHLA_PATH_AUTO) path = choose_path(p);
  if (path < 0 || !path_supports(path, p)) return 0;
  return workspace_for(p, path);
}

const char* mhla_error_string(int code) {
  switch (code) {
    case MHLA_OK: return "ok";
    case MHLA_ERR_INVALID_ARG: return "invalid argument";
    case MHLA_ERR_SHAPE: return "invalid block shape";
    case MHLA_ERR_UNSUPPORTED: return "unsupported size or dtype";
    case MHLA_ERR_HIP: return "HIP runtime error";
    case MHLA_ERR_ALIAS: return "output aliases an input";
    default: return "unknown error code";
  }
}

const char* mhla_last_error(void) { return g_last_error.c_str(); }

void mhla_release(void) {
  std::lock_guard<std::mutex> lock(g_ws_mutex);
  int cur = 0;
  const bool have_dev = hipGetDevice(&cur) == hipSuccess;
  for (auto& kv : g_ws) {
    if (!kv.second.ptr) continue;
    if (hipSetDevice(kv.first.first) == hipSuccess) {
      (void)hipDeviceSynchronize();
      (void)hipFree(kv.second.ptr);
    }
  }
  g_ws.clear();
  if (have_dev) (void)hipSetDevice(cur);
}

}  // extern "C"
