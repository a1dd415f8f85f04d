// mhla_api.hip -- C ABI of libmhla: argument checks, path choice, workspace
// cache and kernel launches for the MHLA forward (gfx950).
//
// The operation is the forward pass of "MHLA: Restoring Expressivity of
// Linear Attention via Token-Level Multi-Head" §4.1 (summaries, multi-head
// mixing, readout); the entry points are declared and documented in mhla.h.
#include <hip/hip_runtime.h>

#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <utility>

#include "mhla.h"
#include "mhla_check.hpp"
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

// A checked call: the host-side shape and the device-side geometry.
struct Problem : Shape {
  Geo g;
};

Geo make_geo(const Shape& s) {
  Geo g;
  g.T = s.T; g.Hg = s.Hg; g.Wg = s.Wg;
  g.bt = s.bt; g.bh = s.bh; g.bw = s.bw;
  g.nbz = s.nbz; g.nby = s.nby; g.nbx = s.nbx;
  g.M = s.M;
  g.nb = s.nb;
  g.inv_bw = 1.0f / (float)g.bw;
  g.inv_bhw = 1.0f / (float)(g.bh * g.bw);
  g.norm = s.norm() ? 1 : 0;
  return g;
}

int check(int B, int H, int N, int d, const mhla_block_shape* s, int phi, int dtype, int flags,
          Problem* p) {
  int rc = check_shape(B, H, N, d, s, phi, dtype, p);
  if (rc != MHLA_OK) return rc;
  rc = check_flags(flags, p);
  if (rc != MHLA_OK) return rc;
  p->g = make_geo(*p);
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

// The generic path's single-launch form (k_generic_one) when a slice fits in LDS.
bool generic_one(const Problem& p) {
  return generic_one_lds_bytes(p.N, p.d, p.g.M) <= kGenericOneLds;
}

size_t workspace_for(const Problem& p, int path) {
  if (path == MHLA_PATH_GENERIC) {
    if (generic_one(p)) return 0;
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

template <typename T>
int launch_generic(const Problem& p, const T* Q, const T* K, const T* V, const float* W,
                   T* Y, float* ws, hipStream_t st) {
  const int M = p.g.M, d = p.d;
  if (generic_one(p)) {
    const size_t lds = generic_one_lds_bytes(p.N, d, M);
    k_generic_one<T><<<dim3((unsigned)p.slices()), kGenericOneThreads, lds, st>>>(
        Q, K, V, W, Y, p.g, p.N, d, p.phi, p.H);
    launch_mark(st, "k_generic_one");
    return MHLA_OK;
  }
  const int L = d * d + d;
  float* S = ws;
  float* St = ws + (size_t)p.slices() * M * L;
  const unsigned nsl = (unsigned)p.slices();
  k_summary_valu<T><<<dim3(M, nsl), kValuThreads, 0, st>>>(K, V, S, p.g, p.N, d, p.phi);
  launch_mark(st, "k_summary_valu");
  k_mix_valu<<<dim3((L + kValuThreads - 1) / kValuThreads, (M + kMixRows - 1) / kMixRows, nsl),
               kValuThreads, 0, st>>>(S, W, St, M, L, p.H);
  launch_mark(st, "k_mix_valu");
  k_readout_valu<T><<<dim3(M, nsl), kValuThreads, 0, st>>>(Q, St, Y, p.g, p.N, d, p.phi);
  launch_mark(st, "k_readout_valu");
  return MHLA_OK;
}

// Scratch of mhla_forward_noalloc, for callers that cannot allocate device
// memory: a fixed array in the library's code object, so that each device the
// library runs on holds its own copy from the first launch until the process
// ends.  256 MiB holds the workspace of every forward workload the library is
// measured on (the largest, the video-latent shape, needs 211 MiB); larger
// calls are rejected.  Host code never uses the array's name as an address:
// it takes the device address from hipGetSymbolAddress (scratch_address).
constexpr size_t kNoAllocScratchBytes = (size_t)256 << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's address of `scratch`, looked up once per device.
int scratch_address(void** out) {
  *out = nullptr;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(MHLA_ERR_HIP, "hipGetDevice failed");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(MHLA_ERR_UNSUPPORTED, "device %d is beyond the scratch table", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
      return fail(MHLA_ERR_HIP, "hipGetSymbolAddress(scratch) failed: %s", hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MHLA_OK;
}

// Where a forward call's workspace comes from: the library's cache (one
// growing buffer per device and stream), or a caller-supplied fixed region
// (`fixed`, `fixed_bytes`) that is never grown.
struct WsSource {
  void* fixed = nullptr;
  size_t fixed_bytes = 0;
};

int run(const void* Q, const void* K, const void* V, const float* W, void* out, int B, int H,
        int N, int d, const mhla_block_shape* shape, int phi, int dtype, int flags, int path,
        hipStream_t st, LaunchRecorder* rec = nullptr, const WsSource* src = nullptr) {
  Problem p;
  int rc = check(B, H, N, d, shape, phi, dtype, flags, &p);
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
  if (overlaps(out, tb, W, p.w_bytes())) return fail(MHLA_ERR_ALIAS, "out overlaps Wmix");
  if (path == MHLA_PATH_AUTO) path = choose_path(p);
  if (path < 0 || !path_supports(path, p))
    return fail(MHLA_ERR_UNSUPPORTED, "path %d does not support this shape/dtype/options", path);

  (void)hipGetLastError();  // clear a stale error so the check below is ours
  void* ws = nullptr;
  const size_t need = workspace_for(p, path);
  if (src != nullptr) {
    if (need > src->fixed_bytes)
      return fail(MHLA_ERR_UNSUPPORTED,
                  "this call needs %zu bytes of scratch; the fixed scratch holds %zu", need,
                  src->fixed_bytes);
    ws = need ? src->fixed : nullptr;
  } else {
    rc = get_workspace(need, st, &ws);
    if (rc != MHLA_OK) return rc;
  }
  if (rec != nullptr) {
    if (hipEventRecord(static_cast<hipEvent_t>(rec->events[0]), st) != hipSuccess)
      return fail(MHLA_ERR_HIP, "hipEventRecord failed");
    g_launch_rec = rec;
  }

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
  g_launch_rec = nullptr;
  if (rc != MHLA_OK) return fail(MHLA_ERR_HIP, "kernel set-up failed (hipFuncSetAttribute)");
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(MHLA_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  if (rec != nullptr && rec->failed) return fail(MHLA_ERR_HIP, "hipEventRecord failed");
  return MHLA_OK;
}

int run_backward(const void* Q, const void* K, const void* V, const float* W, const void* dY,
                 void* dQ, void* dK, void* dV, float* dW, int B, int H, int N, int d,
                 const mhla_block_shape* shape, int phi, int dtype, int flags, hipStream_t st) {
  Problem p;
  int rc = check(B, H, N, d, shape, phi, dtype, flags, &p);
  if (rc != MHLA_OK) return rc;
  if (p.causal()) return fail(MHLA_ERR_UNSUPPORTED, "the causal form has no backward pass here");
  // blocks of at most 16 tokens: the token-pair order; otherwise the blocked one
  const bool pairs = pairs_bwd_supports(dtype, d, p.M, p.nb, N);
  if (!pairs && !backward_supports(dtype, d, p.M, p.slices()))
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
  const size_t tb = p.tensor_bytes(), wb = p.w_bytes();
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
  (void)hipGetLastError();
  void* ws = nullptr;
  rc = get_workspace(pairs ? pairs_bwd_workspace(p.slices(), p.M, N, d)
                           : backward_workspace(p.slices(), H, p.M, N, d),
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
                 int dtype, mhla_stream_t stream) {
  return run(Q, K, V, Wmix, out, B, H, N, d, block_shape, phi_kind, dtype, 0, MHLA_PATH_AUTO,
             stream);
}

int mhla_forward_path(const void* Q, const void* K, const void* V, const float* Wmix,
                      void* out, int B, int H, int N, int d,
                      const mhla_block_shape* block_shape, int phi_kind, int dtype, int path,
                      mhla_stream_t stream) {
  g_last_error.clear();
  if (path < MHLA_PATH_AUTO || path > MHLA_PATH_COLUMNS)
    return fail(MHLA_ERR_INVALID_ARG, "unknown path %d", path);
  return run(Q, K, V, Wmix, out, B, H, N, d, block_shape, phi_kind, dtype, 0, path, stream);
}

int mhla_forward_ex(const void* Q, const void* K, const void* V, const float* Wmix, void* out,
                    int B, int H, int N, int d, const mhla_block_shape* block_shape,
                    int phi_kind, int dtype, int flags, int path, mhla_stream_t stream) {
  g_last_error.clear();
  if (path < MHLA_PATH_AUTO || path > MHLA_PATH_COLUMNS)
    return fail(MHLA_ERR_INVALID_ARG, "unknown path %d", path);
  return run(Q, K, V, Wmix, out, B, H, N, d, block_shape, phi_kind, dtype, flags, path, stream);
}

int mhla_forward_noalloc(const void* Q, const void* K, const void* V, const float* Wmix,
                         void* out, int B, int H, int N, int d,
                         const mhla_block_shape* block_shape, int phi_kind, int dtype, int flags,
                         int path, mhla_stream_t stream) {
  g_last_error.clear();
  if (path < MHLA_PATH_AUTO || path > MHLA_PATH_COLUMNS)
    return fail(MHLA_ERR_INVALID_ARG, "unknown path %d", path);
  WsSource src;
  const int rc = scratch_address(&src.fixed);
  if (rc != MHLA_OK) return rc;
  src.fixed_bytes = kNoAllocScratchBytes;
  return run(Q, K, V, Wmix, out, B, H, N, d, block_shape, phi_kind, dtype, flags, path, stream,
             nullptr, &src);
}

int mhla_forward_profiled(const void* Q, const void* K, const void* V, const float* Wmix,
                          void* out, int B, int H, int N, int d,
                          const mhla_block_shape* block_shape, int phi_kind, int dtype, int flags,
                          int path, void* const* events, int max_events, int* n_launches,
                          const char** names, mhla_stream_t stream) {
  g_last_error.clear();
  if (path < MHLA_PATH_AUTO || path > MHLA_PATH_COLUMNS)
    return fail(MHLA_ERR_INVALID_ARG, "unknown path %d", path);
  if (events == nullptr || n_launches == nullptr || max_events < MHLA_MAX_LAUNCHES + 1)
    return fail(MHLA_ERR_INVALID_ARG,
                "events (at least %d handles) and n_launches must be given (max_events=%d)",
                MHLA_MAX_LAUNCHES + 1, max_events);
  for (int k = 0; k < MHLA_MAX_LAUNCHES + 1; ++k)
    if (events[k] == nullptr) return fail(MHLA_ERR_INVALID_ARG, "events[%d] is NULL", k);
  LaunchRecorder rec;
  rec.events = events;
  rec.cap = max_events - 1;
  rec.names = names;
  const int rc = run(Q, K, V, Wmix, out, B, H, N, d, block_shape, phi_kind, dtype, flags, path,
                     stream, &rec);
  if (rc == MHLA_OK) *n_launches = rec.n;
  return rc;
}

int mhla_backward(const void* Q, const void* K, const void* V, const float* Wmix, const void* dY,
                  void* dQ, void* dK, void* dV, float* dWmix, int B, int H, int N, int d,
                  const mhla_block_shape* block_shape, int phi_kind, int dtype, int flags,
                  mhla_stream_t stream) {
  return run_backward(Q, K, V, Wmix, dY, dQ, dK, dV, dWmix, B, H, N, d, block_shape, phi_kind,
                      dtype, flags, stream);
}

size_t mhla_decode_state_bytes(int B, int H, int d, int M) {
  if (B <= 0 || H <= 0 || d <= 0 || M <= 0 || d > 128) return 0;
  return (size_t)B * H * decode_state_elems(d, M) * sizeof(float);
}

namespace {

// Tokens t0 .. t0+n-1 of every slice; q, k, v, y: [B*H, n, d].
int decode_tokens(const void* q, const void* k, const void* v, const float* Wmix, void* y,
                  void* state, int B, int H, int d, int M, int nb, int t0, int n, int phi_kind,
                  int dtype, int flags, hipStream_t st) {
  if (n <= 0) return fail(MHLA_ERR_INVALID_ARG, "n=%d: at least one token per call", n);
  int rc = check_decode(B, H, d, M, nb, t0, phi_kind, dtype, flags);
  if (rc != MHLA_OK) return rc;
  if ((long)t0 + n > (long)M * nb)
    return fail(MHLA_ERR_INVALID_ARG, "tokens %d..%ld run past the %ld positions of M*nb", t0,
                (long)t0 + n - 1, (long)M * nb);
  if (!q || !k || !v || !Wmix || !y || !state)
    return fail(MHLA_ERR_INVALID_ARG, "a pointer is NULL");
  const void* ptrs[6] = {q, k, v, Wmix, y, state};
  for (const void* p : ptrs)
    if (reinterpret_cast<uintptr_t>(p) % 4 != 0)
      return fail(MHLA_ERR_INVALID_ARG, "pointers must be 4-byte aligned");
  const size_t eb = dtype == MHLA_DTYPE_F32 ? 4 : 2;
  const size_t tb = (size_t)B * H * n * d * eb;
  const size_t sb = mhla_decode_state_bytes(B, H, d, M);
  const size_t wb = (size_t)H * M * M * sizeof(float);
  if (overlaps(y, tb, q, tb) || overlaps(y, tb, k, tb) || overlaps(y, tb, v, tb) ||
      overlaps(y, tb, state, sb) || overlaps(y, tb, Wmix, wb))
    return fail(MHLA_ERR_ALIAS, "y overlaps q, k, v, Wmix or the state");
  if (overlaps(state, sb, q, tb) || overlaps(state, sb, k, tb) || overlaps(state, sb, v, tb) ||
      overlaps(state, sb, Wmix, wb))
    return fail(MHLA_ERR_ALIAS, "the state overlaps q, k, v or Wmix");
  (void)hipGetLastError();
  const int norm = (flags & MHLA_FLAG_NO_NORM) ? 0 : 1;
  const long slices = (long)B * H;
  if (dtype == MHLA_DTYPE_F32)
    rc = launch_decode_t<float>(slices, H, d, M, nb, t0, n, phi_kind, norm, (const float*)q,
                                (const float*)k, (const float*)v, Wmix, (float*)y, (float*)state,
                                st);
  else
    rc = launch_decode_t<bf16_t>(slices, H, d, M, nb, t0, n, phi_kind, norm, (const bf16_t*)q,
                                 (const bf16_t*)k, (const bf16_t*)v, Wmix, (bf16_t*)y,
                                 (float*)state, st);
  if (rc != 0) return fail(MHLA_ERR_HIP, "decode set-up failed (hipFuncSetAttribute)");
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(MHLA_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return MHLA_OK;
}

}  // namespace

int mhla_decode_step(const void* q, const void* k, const void* v, const float* Wmix, void* y,
                     void* state, int B, int H, int d, int M, int nb, int t, int phi_kind,
                     int dtype, int flags, mhla_stream_t stream) {
  g_last_error.clear();
  return decode_tokens(q, k, v, Wmix, y, state, B, H, d, M, nb, t, 1, phi_kind, dtype, flags,
                       stream);
}

int mhla_decode_steps(const void* q, const void* k, const void* v, const float* Wmix, void* y,
                      void* state, int B, int H, int d, int M, int nb, int t0, int n,
                      int phi_kind, int dtype, int flags, mhla_stream_t stream) {
  g_last_error.clear();
  return decode_tokens(q, k, v, Wmix, y, state, B, H, d, M, nb, t0, n, phi_kind, dtype, flags,
                       stream);
}

int mhla_decode_prefill(const void* k, const void* v, const float* Wmix, void* state, int B,
                        int H, int d, int M, int nb, int T, int phi_kind, int dtype, int flags,
                        mhla_stream_t stream) {
  if (T <= 0) return fail(MHLA_ERR_INVALID_ARG, "T=%d: the prompt must hold a token", T);
  int rc = check_decode(B, H, d, M, nb, T - 1, phi_kind, dtype, flags);
  if (rc != MHLA_OK) return rc;
  if (!k || !v || !Wmix || !state) return fail(MHLA_ERR_INVALID_ARG, "a pointer is NULL");
  const void* ptrs[4] = {k, v, Wmix, state};
  for (const void* p : ptrs)
    if (reinterpret_cast<uintptr_t>(p) % 4 != 0)
      return fail(MHLA_ERR_INVALID_ARG, "pointers must be 4-byte aligned");
  const size_t eb = dtype == MHLA_DTYPE_F32 ? 4 : 2;
  const size_t tb = (size_t)B * H * T * d * eb;
  const size_t sb = mhla_decode_state_bytes(B, H, d, M);
  if (overlaps(state, sb, k, tb) || overlaps(state, sb, v, tb) ||
      overlaps(state, sb, Wmix, (size_t)H * M * M * sizeof(float)))
    return fail(MHLA_ERR_ALIAS, "the state overlaps k, v or Wmix");
  hipStream_t st = stream;
  (void)hipGetLastError();
  const long slices = (long)B * H;
  if (dtype == MHLA_DTYPE_F32)
    launch_decode_prefill_t<float>(slices, H, d, M, nb, T, phi_kind, (const float*)k,
                                   (const float*)v, Wmix, (float*)state, st);
  else
    launch_decode_prefill_t<bf16_t>(slices, H, d, M, nb, T, phi_kind, (const bf16_t*)k,
                                    (const bf16_t*)v, Wmix, (float*)state, st);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(MHLA_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return MHLA_OK;
}

int mhla_plan_ex(int B, int H, int N, int d, const mhla_block_shape* block_shape, int phi_kind,
                 int dtype, int flags) {
  Problem p;
  const int rc = check(B, H, N, d, block_shape, phi_kind, dtype, flags, &p);
  if (rc != MHLA_OK) return -rc;
  return choose_path(p);
}

int mhla_lb_init(const mhla_block_shape* block_shape, float* W, size_t capacity) {
  return lb_init_checked(block_shape, W, capacity);
}

int mhla_validate(int B, int H, int N, int d, const mhla_block_shape* block_shape, int phi_kind,
                  int dtype) {
  Problem p;
  return check(B, H, N, d, block_shape, phi_kind, dtype, 0, &p);
}

int mhla_plan(int B, int H, int N, int d, const mhla_block_shape* block_shape, int phi_kind,
              int dtype) {
  return mhla_plan_ex(B, H, N, d, block_shape, phi_kind, dtype, 0);
}

int mhla_num_blocks(int N, const mhla_block_shape* block_shape) {
  Problem p;
  const int rc = check(1, 1, N, 8, block_shape, MHLA_PHI_RELU, MHLA_DTYPE_F32, 0, &p);
  if (rc != MHLA_OK) return -rc;
  return p.M;
}

size_t mhla_workspace_bytes_ex(int B, int H, int N, int d, const mhla_block_shape* block_shape,
                               int dtype, int flags, int path) {
  Problem p;
  if (check(B, H, N, d, block_shape, MHLA_PHI_RELU, dtype, flags, &p) != MHLA_OK) return 0;
  if (path == MHLA_PATH_AUTO) path = choose_path(p);
  if (path < 0 || !path_supports(path, p)) return 0;
  return workspace_for(p, path);
}

size_t mhla_workspace_bytes(int B, int H, int N, int d, const mhla_block_shape* block_shape,
                            int dtype) {
  return mhla_workspace_bytes_ex(B, H, N, d, block_shape, dtype, 0, MHLA_PATH_AUTO);
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
