/*
 * mhla.h -- C ABI of libmhla, the MI355X (gfx950) forward pass of MHLA
 * (Multi-Head Linear Attention with token-level heads).
 *
 * Operation (MHLA paper = "MHLA: Restoring Expressivity of Linear Attention
 * via Token-Level Multi-Head", arXiv 2601.07832):
 *   For every (batch b, channel head h) slice with Q, K, V in R^{N x d}
 *   (§4.1, the projected queries, keys and values), the N tokens form a
 *   (T, Hg, Wg) grid that is cut into M equal, non-overlapping (bt, bh, bw)
 *   tiles (§1 and §4.1; blocks are numbered in raster order of the block grid,
 *   Fig. 4b).  With phi the feature map (ReLU, or elu+1 -- the two choices of
 *   the tutorial "Attention 变体：从 Sliding Window 到 MLA", linear attention
 *   section):
 *     S_b  = sum_{j in b} phi(K_j) V_j^T,   z_b = sum_{j in b} phi(K_j)   (§4.1)
 *     S~_i = sum_b W[h][i][b] S_b,          z~_i = sum_b W[h][i][b] z_b   (§4.1-§4.2)
 *     Y_q  = phi(Q_q) S~_i / (phi(Q_q) . z~_i)   for q in query block i   (§4.1)
 *   The result equals the token-pair form of §4.2 Eq. 5 up to rounding order.
 *   No 1/sqrt(d) scale is applied and V is used as given.  A row whose
 *   denominator is exactly 0 (possible only with ReLU) is written as zeros.
 *
 * Conventions shared by every entry point:
 *   - Q, K, V, out: device pointers to [B, H, N, d] contiguous row-major
 *     tensors of element type `dtype` (fp32 or bf16), tokens in raster order
 *     of the grid (x fastest, then y, then t).  `out` must not overlap Q, K or V.
 *   - Wmix: device pointer to [H, M, M] fp32 row-major; Wmix[h][i][b] is the
 *     weight of key block b in query block i's mixture.  It is shared over B.
 *     Any values are accepted (no sign or normalisation check); a positive
 *     per-row scale cancels in the output.
 *   - All pointers are caller-owned; the library never frees them.  Device
 *     pointers must be 16-byte aligned.
 *   - stream: a hipStream_t (mhla_stream_t below is the same type; NULL = the
 *     null stream).  Work is enqueued asynchronously; no host or device-wide
 *     synchronisation happens (except when the library's workspace for that
 *     (device, stream) has to grow, which synchronises the stream once).
 *   - Argument and shape errors are detected on the host before anything is
 *     enqueued; the return code says which (MHLA_ERR_*), and
 *     mhla_last_error() gives a message for the calling thread.
 *   - Supported: d a multiple of 8 in [8, 128] (bf16) or any d in [1, 128]
 *     (fp32); n_b = N / M >= 1; B*H <= 2^31-1 slices.
 */
#ifndef MHLA_H
#define MHLA_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The HIP runtime's stream handle: hip_runtime_api.h defines hipStream_t as
 * a pointer to this opaque struct, so a hipStream_t converts to mhla_stream_t
 * without a cast, and this header needs no HIP include. */
struct ihipStream_t;
typedef struct ihipStream_t* mhla_stream_t;

typedef struct mhla_block_shape {
  int ndim;      /* 1, 2 or 3: how many trailing grid axes are in use        */
  int grid[3];   /* (T, Hg, Wg) token grid; unused leading entries are 1     */
  int block[3];  /* (bt, bh, bw) block dims; each divides its grid dimension */
} mhla_block_shape;

enum { MHLA_PHI_RELU = 0, MHLA_PHI_ELU1 = 1 };
enum { MHLA_DTYPE_F32 = 0, MHLA_DTYPE_BF16 = 1 };
enum {
  MHLA_OK = 0,
  MHLA_ERR_INVALID_ARG = 1, /* null pointer, bad enum, non-positive size    */
  MHLA_ERR_SHAPE = 2,       /* grid product != N, block does not divide grid */
  MHLA_ERR_UNSUPPORTED = 3, /* d or dtype outside the supported set          */
  MHLA_ERR_HIP = 4,         /* a HIP runtime call or kernel launch failed    */
  MHLA_ERR_ALIAS = 5        /* out overlaps Q, K or V                        */
};

/* Kernel path selection for mhla_forward_path (testing and tuning). */
enum {
  MHLA_PATH_AUTO = 0,       /* the library's choice for the shape            */
  MHLA_PATH_GENERIC = 1,    /* summary -> mixing -> readout, three kernels   */
  MHLA_PATH_FUSED = 2,      /* one workgroup per slice, summaries kept in LDS */
  MHLA_PATH_PAIRS = 3,      /* token-pair form of Eq. 5, no summaries        */
  MHLA_PATH_BLOCKED = 4,    /* summary, mixing GEMM, readout on bf16 MFMA     */
  MHLA_PATH_COLUMNS = 5     /* one workgroup per (slice, 16 value columns):
                               summaries, mixing and readout on chip; bf16,
                               d <= 64, M <= 64, blocks of <= 256 tokens
                               (output column c needs only column c of every
                               S_b, plus z_b).  Never picked by AUTO.       */
};

/* Option bits for mhla_forward_ex (any combination). */
enum {
  /* Y_q = phi(Q_q) S~_i: the denominator is dropped.  The MHLA paper runs its
   * language-modelling and very long video models this way (blog review
   * §2.2: the normaliser switch is part of the method). */
  MHLA_FLAG_NO_NORM = 1,
  /* Chunkwise causal form (MHLA paper §4.2 "Chunkwise parallel form of MHLA",
   * App. C).  Every block must be a run of consecutive tokens (for a grid:
   * full rows of the x axis, or full frames), so blocks are chunks in
   * sequence order.  Query chunk i mixes only earlier chunks,
   *   S^<_i = sum_{b<i} W[h][i][b] S_b,  z^<_i likewise,
   * and adds its own chunk causally with weight W[h][i][i]:
   *   Y_q = (phi(Q_q) S^<_i + W_ii sum_{j<=q in chunk i} (phi(Q_q).phi(K_j)) V_j)
   *       / (phi(Q_q).z^<_i + W_ii sum_{j<=q in chunk i}  phi(Q_q).phi(K_j)),
   * i.e. the token form of Eq. 5 with the mask j <= q.  Entries W[h][i][b]
   * with b > i are ignored.  Supported for bf16, d a multiple of 8 up to 96,
   * chunks of at most 256 tokens (MHLA_PATH_BLOCKED). */
  MHLA_FLAG_CAUSAL = 2
};

/* Forward pass (MHLA paper §4.1).  Returns MHLA_OK or an MHLA_ERR_* code. */
int mhla_forward(const void* Q, const void* K, const void* V, const float* Wmix,
                 void* out, int B, int H, int N, int d,
                 const mhla_block_shape* block_shape, int phi_kind, int dtype,
                 mhla_stream_t stream);

/* Same as mhla_forward with an explicit kernel path.  A path that does not
 * support the shape returns MHLA_ERR_UNSUPPORTED without enqueuing work. */
int mhla_forward_path(const void* Q, const void* K, const void* V,
                      const float* Wmix, void* out, int B, int H, int N, int d,
                      const mhla_block_shape* block_shape, int phi_kind,
                      int dtype, int path, mhla_stream_t stream);

/* mhla_forward_path with option bits (MHLA_FLAG_*; 0 = mhla_forward_path).
 * Unknown bits return MHLA_ERR_INVALID_ARG; a causal call whose blocks are not
 * runs of consecutive tokens returns MHLA_ERR_SHAPE; a path that cannot run
 * the options returns MHLA_ERR_UNSUPPORTED.  Nothing is enqueued on error. */
int mhla_forward_ex(const void* Q, const void* K, const void* V, const float* Wmix,
                    void* out, int B, int H, int N, int d,
                    const mhla_block_shape* block_shape, int phi_kind, int dtype,
                    int flags, int path, mhla_stream_t stream);

/* mhla_forward_ex for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the call's scratch (the blocked path's S / S~ tables and mixing
 * coefficients, the generic path's fp32 tables) lives in a fixed array of
 * MHLA_NOALLOC_SCRATCH_BYTES that the library's code object holds on every
 * device it runs on, until the process ends; nothing is allocated or freed.
 * The caller still passes Q, K, V, Wmix and out.  A call whose scratch need
 * (mhla_workspace_bytes_ex) exceeds the array returns MHLA_ERR_UNSUPPORTED
 * before any launch; other errors are those of mhla_forward_ex.  Every call
 * on one device shares that device's array (it keeps the last call's
 * contents; no call depends on them): calls that overlap in time on one
 * device -- on different streams or host threads -- race and give undefined
 * results, so serialise them. */
#define MHLA_NOALLOC_SCRATCH_BYTES ((size_t)256 << 20)
int mhla_forward_noalloc(const void* Q, const void* K, const void* V,
                         const float* Wmix, void* out, int B, int H, int N,
                         int d, const mhla_block_shape* block_shape,
                         int phi_kind, int dtype, int flags, int path,
                         mhla_stream_t stream);

/* Upper bound on the kernel launches of one forward call (any path and
 * options). */
#define MHLA_MAX_LAUNCHES 8

/* mhla_forward_ex that also records HIP events around its kernel launches,
 * for measuring each kernel of a call (timing only; the results are those of
 * mhla_forward_ex).  events: max_events caller-created hipEvent_t handles
 * (passed as void*), max_events >= MHLA_MAX_LAUNCHES + 1.  events[0] is
 * recorded on `stream` before the first launch and events[k] right after the
 * k-th launch, so hipEventElapsedTime(events[k-1], events[k]) spans launch k
 * (plus any gap before it).  On success *n_launches = the number of launches
 * and, when names is not NULL (MHLA_MAX_LAUNCHES entries), names[k-1] points
 * at the static name of launch k's kernel.  Errors are those of
 * mhla_forward_ex, plus MHLA_ERR_INVALID_ARG for a NULL events array or
 * n_launches, or max_events below the bound; nothing is enqueued or recorded
 * on error. */
int mhla_forward_profiled(const void* Q, const void* K, const void* V,
                          const float* Wmix, void* out, int B, int H, int N,
                          int d, const mhla_block_shape* block_shape,
                          int phi_kind, int dtype, int flags, int path,
                          void* const* events, int max_events, int* n_launches,
                          const char** names, mhla_stream_t stream);

/* The path MHLA_PATH_AUTO picks for these sizes and option bits (host only),
 * or -code for the error mhla_forward_ex would return before any launch. */
int mhla_plan_ex(int B, int H, int N, int d, const mhla_block_shape* block_shape,
                 int phi_kind, int dtype, int flags);

/* Locality-biased initial mixing matrix m0 of the MHLA paper (§4.2; Fig. 4b
 * shows it): blocks sit at their integer coordinates (bz, by, bx) on the
 * block grid, dist is the Euclidean distance between those coordinates, and
 * m0[i][j] = (1 - dist(i,j) / max_k dist(i,k)) / (sum over j of the same),
 * so every row sums to 1, the block itself has the largest weight and the
 * farthest block gets 0.  With one block, m0 = [[1]].  Host-only: writes
 * M*M floats row-major into the caller's host buffer W (M = number of blocks;
 * replicate it per head for Wmix).  Returns MHLA_OK, MHLA_ERR_SHAPE for an
 * invalid block shape, or MHLA_ERR_INVALID_ARG when W is NULL or `capacity`
 * (in floats) is below M*M. */
int mhla_lb_init(const mhla_block_shape* block_shape, float* W, size_t capacity);

/* Backward pass of the non-causal forward: given dY = dL/dY, writes dQ, dK,
 * dV ([B, H, N, d], dtype) and dWmix ([H, M, M] fp32, summed over the batch,
 * overwritten).  The pages print no backward; it is the chain rule through
 * the three forward steps of the MHLA paper §4.1 (readout, mixing,
 * summaries, in reverse order), with phi'(x) = [x > 0] for ReLU and 1 or
 * exp(x) for elu+1.  A row whose denominator is exactly 0 is the constant 0
 * and passes no gradient.  flags may hold MHLA_FLAG_NO_NORM; the causal form
 * has no backward here (MHLA_ERR_UNSUPPORTED).  Supported: bf16, d a multiple
 * of 8 up to 96.  All pointers are device pointers with the conventions
 * above; the outputs must not overlap any input or each other
 * (MHLA_ERR_ALIAS).  Uses the library's workspace (4 [B,H,M,d*d+d] bf16
 * tables plus per-token and per-slice scratch). */
int mhla_backward(const void* Q, const void* K, const void* V, const float* Wmix,
                  const void* dY, void* dQ, void* dK, void* dV, float* dWmix,
                  int B, int H, int N, int d, const mhla_block_shape* block_shape,
                  int phi_kind, int dtype, int flags, mhla_stream_t stream);

/* Incremental (streaming) inference of the causal form (MHLA paper App. C,
 * "Causal inference"): one new token per (batch, head) slice per call.  The
 * sequence is cut into chunks of nb tokens (at most M chunks); token t lies
 * in chunk i = t / nb.  The caller owns a device state buffer of
 * mhla_decode_state_bytes(B, H, d, M) bytes, holding per slice, in fp32, the
 * M chunk summaries [S_b | z_b] and the current chunk's prefix mixture
 * sum_{b<i} W[h][i][b] [S_b | z_b].  A call:
 *   - when t starts chunk i, forms that prefix mixture once and restarts the
 *     running summary of chunk i;
 *   - adds phi(k_t) [v_t | 1]^T to the running summary;
 *   - writes y_t = phi(q_t)(P_i + W[h][i][i] S_i) / phi(q_t).(p_i + W[h][i][i] z_i)
 *     (the numerator alone with MHLA_FLAG_NO_NORM; 0 for a zero denominator),
 *     which equals mhla_forward_ex(..., MHLA_FLAG_CAUSAL, ...) at position t
 *     of a 1-D sequence with chunks of nb tokens.
 * q, k, v, y: [B, H, d] device tensors of `dtype` (the token at position t of
 * every slice); Wmix: [H, M, M] fp32.  Calls must come for t = 0, 1, 2, ...
 * in order on one stream (t = 0 starts a new sequence; no separate
 * initialisation is needed).  Cost per call: O(B H d^2), plus O(B H i d^2)
 * when a chunk starts.  flags: 0 or MHLA_FLAG_NO_NORM (MHLA_FLAG_CAUSAL is
 * implied and accepted).  Errors: MHLA_ERR_INVALID_ARG (bad sizes, t outside
 * [0, M*nb), NULL pointers, unknown flags), MHLA_ERR_UNSUPPORTED (d > 128, or
 * bf16 with d not a multiple of 8), MHLA_ERR_ALIAS (y overlaps q, k, v, Wmix or
 * the state, or the state overlaps q, k, v or Wmix). */
size_t mhla_decode_state_bytes(int B, int H, int d, int M);
int mhla_decode_step(const void* q, const void* k, const void* v, const float* Wmix,
                     void* y, void* state, int B, int H, int d, int M, int nb, int t,
                     int phi_kind, int dtype, int flags, mhla_stream_t stream);

/* Several tokens per slice in one call (MHLA paper App. C, "Causal
 * inference"): the n tokens t0 .. t0+n-1 of every slice, taken in order, each
 * exactly as one mhla_decode_step call for it would take it, so y and the
 * state are the same bits as those n calls leave; one launch instead of n
 * (for a block of tokens known ahead, such as candidate tokens to check, or
 * a prompt whose outputs are wanted as well).  q, k, v, y: [B, H, n, d]
 * device tensors of `dtype`, token t0 + u of every slice at row u; the other
 * arguments, the ordering rule and the errors are those of mhla_decode_step,
 * with t0 + n - 1 in place of t (n >= 1, t0 >= 0, t0 + n <= M*nb). */
int mhla_decode_steps(const void* q, const void* k, const void* v, const float* Wmix,
                      void* y, void* state, int B, int H, int d, int M, int nb, int t0, int n,
                      int phi_kind, int dtype, int flags, mhla_stream_t stream);

/* Prefill for incremental inference (MHLA paper App. C, "Causal inference"):
 * builds, from the first T tokens of every slice, the decode state that T
 * calls of mhla_decode_step (t = 0 .. T-1) would leave, so that the stream
 * continues with mhla_decode_step at t = T.  k, v: [B, H, T, d] device
 * tensors of `dtype` (the prompt's keys and values; no query is needed);
 * Wmix: [H, M, M] fp32; state: the caller's buffer of
 * mhla_decode_state_bytes(B, H, d, M) bytes.  It writes the summaries of the
 * ceil(T / nb) chunks the prompt touches (the last one running when T is not
 * a multiple of nb) and the prefix mixture of chunk (T - 1) / nb, each sum
 * taken in the order the decode step takes it, so the state is the same
 * bits; the slots of later chunks are left as they are.  The prompt's outputs
 * are those of mhla_forward_ex(..., MHLA_FLAG_CAUSAL, ...) on its first T
 * tokens.  Errors: MHLA_ERR_INVALID_ARG (bad sizes, T outside [1, M*nb], NULL
 * pointers, unknown flags), MHLA_ERR_UNSUPPORTED (as mhla_decode_step),
 * MHLA_ERR_ALIAS (the state overlaps k, v or Wmix). */
int mhla_decode_prefill(const void* k, const void* v, const float* Wmix, void* state, int B,
                        int H, int d, int M, int nb, int T, int phi_kind, int dtype, int flags,
                        mhla_stream_t stream);

/* Host-only argument check (no HIP call): MHLA_OK or the code mhla_forward
 * would return for these sizes. */
int mhla_validate(int B, int H, int N, int d, const mhla_block_shape* block_shape,
                  int phi_kind, int dtype);

/* The path MHLA_PATH_AUTO picks for these sizes (host only), or -code. */
int mhla_plan(int B, int H, int N, int d, const mhla_block_shape* block_shape,
              int phi_kind, int dtype);

/* Number of blocks M for a valid shape, or -code. */
int mhla_num_blocks(int N, const mhla_block_shape* block_shape);

/* Device workspace in bytes that mhla_forward needs for these sizes (the
 * path MHLA_PATH_AUTO picks, no option bits; 0 when that path keeps its
 * intermediates on chip).  Returns 0 for invalid sizes.  Host only.  The
 * library allocates and caches this workspace itself (one buffer per device
 * and stream, freed by mhla_release); the query tells a caller how much
 * device memory a call will hold. */
size_t mhla_workspace_bytes(int B, int H, int N, int d,
                            const mhla_block_shape* block_shape, int dtype);

/* mhla_workspace_bytes for mhla_forward_ex's option bits and kernel path.
 * Returns 0 for invalid sizes or options, and for a path that does not take
 * the shape. */
size_t mhla_workspace_bytes_ex(int B, int H, int N, int d,
                               const mhla_block_shape* block_shape, int dtype,
                               int flags, int path);

/* Static description of a code; never NULL. */
const char* mhla_error_string(int code);

/* Message describing the calling thread's most recent failure ("" if none). */
const char* mhla_last_error(void);

/* Frees the library-owned workspaces on every device (synchronises each
 * device that has one).  Safe to call at any time outside a forward call. */
void mhla_release(void);

#ifdef __cplusplus
}
#endif

#endif /* MHLA_H */
