/*
 * flashbob.h - C ABI of the MI355X (gfx950) library for exact
 * backward-over-backward (BoB) through softmax attention.
 *
 * The operation (FlashBoB pages: the arXiv abstract page; the evolve.pub review
 * page, Summary, Key claims under review and Report preview / Scope & Claims):
 * for one attention head with inputs Q, K, V in R^{N x d}, scale tau and
 * upstream gradient dO,
 *     S = tau Q K^T,  P = softmax_rows(S),  O = P V,
 *     g(Q, K, V, dO) = (dQ, dK, dV)            (the first backward),
 * BoB applies the transposed Jacobian of g to upstream cotangents
 * (UQ, UK, UV) placed on (dQ, dK, dV) and returns the cotangents of the four
 * inputs, written here gQ, gK, gV, gdO (the pages write them with a "partial"
 * sign). The result is exact up to floating-point rounding (review page,
 * FAQ on whether the method approximates).
 *
 * Schedule (review page, Summary and Key claims: Prop. 4.1, Algorithm 1): a
 * statistics kernel (row LSE L, O and D = rowsum(dO * O)), then two passes.
 * Pass 1 is query-tile parallel and produces gQ, gdO and the two row scalars
 * alpha, E; pass 2 is key-tile parallel and produces gK, gV. Only alpha and E
 * cross the pass boundary besides L and D; no N x N matrix is ever written to
 * device memory.
 *
 * Conventions for every entry point:
 *  - Tensors are contiguous [B][H][N][d] arrays in `dtype`, in device memory
 *    owned by the caller. Row vectors (L, D, alpha, E) are contiguous
 *    [B][H][N] float32 arrays in device memory. L is the natural-log LSE of
 *    row i of tau Q K^T.
 *  - d must be 64 or 128; B, H, N >= 1; B*H <= 65535 and B*H*N <= 2^31 - 256
 *    (else FB_ERR_SHAPE); tau finite. `causal` != 0 masks key j
 *    for query i when j > i (square, top-left aligned).
 *  - Outputs are fully overwritten (never accumulated), are written in `dtype`
 *    (round to nearest even from float32 accumulators), and must not alias any
 *    input (checked for equal pointers).
 *  - Arguments are checked synchronously before any launch; a non-zero status
 *    is returned and nothing is launched. After the checks all work is
 *    asynchronous on `stream` (0 = the null stream); the caller synchronises.
 *    No entry point aborts or throws. fb_last_error() gives a message for the
 *    last non-OK status on the calling thread.
 *  - float32 inputs use float32 matrix-core arithmetic (for exactness checks);
 *    bf16/fp16 inputs use bf16/fp16 matrix-core operands with float32
 *    accumulation and float32 element-wise arithmetic.
 */
#ifndef FLASHBOB_H
#define FLASHBOB_H

#include <stddef.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { FB_F32 = 0, FB_F16 = 1, FB_BF16 = 2 } fb_dtype_t;

typedef enum {
  FB_OK = 0,
  FB_ERR_NULL = -1,      /* a required pointer is NULL                      */
  FB_ERR_SHAPE = -2,     /* B, H or N < 1, B*H > 65535 or B*H*N > 2^31-256  */
  FB_ERR_DTYPE = -3,     /* unknown dtype                                    */
  FB_ERR_HEADDIM = -4,   /* d not in {64, 128}                               */
  FB_ERR_WORKSPACE = -5, /* workspace NULL or smaller than required          */
  FB_ERR_OOM = -6,       /* device allocation failed                         */
  FB_ERR_HIP = -7,       /* a HIP runtime call failed (message has details)  */
  FB_ERR_ARG = -8        /* other invalid argument (tau, aliasing, options)  */
} fb_status_t;

/* Message for the last non-OK status returned on this thread ("" if none).
 * The string is owned by the library and valid until the next call. */
const char* fb_last_error(void);

/*
 * bob_attention: the whole BoB call (statistics kernel + pass 1 + pass 2).
 * In:  Q, K, V, dO, UQ, UK, UV  [B][H][N][d] dtype, device.
 * Out: gQ, gK, gV, gdO          [B][H][N][d] dtype, device, overwritten.
 * Allocates its workspace with hipMallocAsync on `stream` and frees it with
 * hipFreeAsync on the same stream. Returns FB_ERR_OOM, with nothing launched,
 * when the workspace exceeds the limit set by fb_set_alloc_limit or the free
 * memory of the current device, or when hipMallocAsync fails.
 */
fb_status_t bob_attention(const void* Q, const void* K, const void* V, const void* dO,
                          const void* UQ, const void* UK, const void* UV,
                          float tau, int causal, int B, int H, int N, int d, fb_dtype_t dtype,
                          void* gQ, void* gK, void* gV, void* gdO, hipStream_t stream);

/*
 * bob_workspace_bytes: device workspace bytes that bob_attention_ws and
 * bob_attention_with_stats need for this shape under the current tuning
 * (fb_set_tuning). Linear in B*H*N*d: no N^2 term. Returns 0 for invalid
 * arguments.
 */
size_t bob_workspace_bytes(int B, int H, int N, int d, fb_dtype_t dtype);

/*
 * bob_attention_ws: as bob_attention, with a caller-provided device workspace
 * `ws` of at least bob_workspace_bytes(...) bytes, 256-byte aligned. Allocates
 * nothing. The workspace contents on entry are ignored.
 */
fb_status_t bob_attention_ws(const void* Q, const void* K, const void* V, const void* dO,
                             const void* UQ, const void* UK, const void* UV,
                             float tau, int causal, int B, int H, int N, int d, fb_dtype_t dtype,
                             void* gQ, void* gK, void* gV, void* gdO,
                             void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * bob_attention_noalloc: as bob_attention, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc). It calls no hipMalloc, hipFree or allocating routine:
 * its workspace is a fixed 64 MiB device array inside the library, one copy per
 * GPU, held from the library's load until the process ends. Shapes whose
 * workspace (bob_workspace_bytes) exceeds 64 MiB return FB_ERR_WORKSPACE with
 * nothing launched. Every call on one GPU uses that GPU's array: calls that
 * overlap on one GPU (different streams, or host threads) race and must be
 * ordered by the caller. The array's contents on entry are ignored.
 */
fb_status_t bob_attention_noalloc(const void* Q, const void* K, const void* V, const void* dO,
                                  const void* UQ, const void* UK, const void* UV,
                                  float tau, int causal, int B, int H, int N, int d, fb_dtype_t dtype,
                                  void* gQ, void* gK, void* gV, void* gdO, hipStream_t stream);

/*
 * bob_attention_fourpass_ws: the same result as bob_attention_ws through the
 * natural four-pass schedule that the method's affine structure collapses to
 * two (review page, Summary; Strengths on Prop. 4.1): after the statistics
 * kernel, one key sweep per query tile for alpha, a second for E (alpha
 * known), a third for gQ and gdO (alpha and E known), then pass 2. It exists to
 * measure what the collapse saves (an ablation). bf16/fp16 inputs only
 * (FB_ERR_DTYPE for float32); same arguments, workspace and errors as
 * bob_attention_ws.
 */
fb_status_t bob_attention_fourpass_ws(const void* Q, const void* K, const void* V, const void* dO,
                                      const void* UQ, const void* UK, const void* UV,
                                      float tau, int causal, int B, int H, int N, int d, fb_dtype_t dtype,
                                      void* gQ, void* gK, void* gV, void* gdO,
                                      void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * bob_attention_with_stats: pass 1 + pass 2 only, from saved statistics: the
 * forward output O ([B][H][N][d] dtype), the row LSE L and the row scalar
 * D = rowsum(dO * O) ([B][H][N] float32). This is the path whose device-memory
 * traffic the review page's Theorem 4.3 ledger counts (Strengths).
 * alpha_out, E_out: optional [B][H][N] float32 outputs of the two row scalars
 * (NULL to skip; then they live in the workspace).
 * alpha_i = sum_j P_ij * Gbar_ij with Gbar = tau (UQ K^T + Q UK^T) the cotangent
 * of dS; E_i = sum_j P_ij * Pbar_ij with Pbar the cotangent of P.
 */
fb_status_t bob_attention_with_stats(const void* Q, const void* K, const void* V, const void* dO,
                                     const void* UQ, const void* UK, const void* UV,
                                     const void* O, const float* L, const float* D,
                                     float tau, int causal, int B, int H, int N, int d,
                                     fb_dtype_t dtype, void* gQ, void* gK, void* gV, void* gdO,
                                     float* alpha_out, float* E_out,
                                     void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * attn_fwd: forward attention with the statistics BoB recomputes from
 * (the score-recomputation model, review page, Strengths: Theorem 4.5).
 * Out: O [B][H][N][d] dtype; L [B][H][N] float32 (natural-log row LSE of
 * tau Q K^T); D_out optional (NULL to skip): rowsum(dO * O) [B][H][N] float32,
 * formed from the float32 O before rounding, in which case dO must be given
 * (dO may be NULL when D_out is NULL).
 */
fb_status_t attn_fwd(const void* Q, const void* K, const void* V, const void* dO,
                     float tau, int causal, int B, int H, int N, int d, fb_dtype_t dtype,
                     void* O, float* L, float* D_out, hipStream_t stream);

/*
 * attn_bwd: the first backward g (the map BoB differentiates).
 * In: Q, K, V, O, dO [B][H][N][d] dtype; L [B][H][N] float32 from attn_fwd.
 * Out: dQ, dK, dV [B][H][N][d] dtype; D_out optional [B][H][N] float32
 * (rowsum(dO * O)). Scratch (a B*H*N float32 vector when D_out is NULL, and for
 * bf16/fp16 inputs the partial sums of a split streamed range, sized like
 * bob_workspace_bytes' split records) is allocated with hipMallocAsync and freed
 * with hipFreeAsync on `stream`; FB_ERR_OOM (nothing launched) under the same
 * conditions as bob_attention. bf16/fp16 inputs run
 * the staged kernels of pass 1 and pass 2 restricted to S and dP; float32 inputs
 * run single-buffered kernels.
 */
fb_status_t attn_bwd(const void* Q, const void* K, const void* V, const void* O, const void* dO,
                     const float* L, float tau, int causal, int B, int H, int N, int d,
                     fb_dtype_t dtype, void* dQ, void* dK, void* dV, float* D_out,
                     hipStream_t stream);

/*
 * fb_set_tuning: number of splits of the streamed dimension in pass 1 (keys)
 * and pass 2 (queries); 0 = automatic (the default). Values must be 0..64.
 * Process-wide; affects bob_workspace_bytes. Partial results of the splits
 * are written to workspace buffers and summed in a fixed order by a separate
 * kernel, so results do not depend on scheduling.
 */
fb_status_t fb_set_tuning(int pass1_splits, int pass2_splits);

/*
 * fb_set_reduction: how pass 2 combines the partial gK, gV of a split query range
 * (bf16/fp16 inputs; see fb_set_tuning for when the range is split). Process-wide;
 * affects bob_workspace_bytes. Returns FB_ERR_ARG for other values.
 *   0 (default): each split writes a record and a separate kernel sums the
 *      records in split order (deterministic);
 *   1: each split adds its sums into float32 buffers with hardware atomics, then a
 *      conversion kernel writes gK, gV (order of additions not fixed, so results
 *      may differ in the last bits between runs);
 *   2: records as in 0, summed in split order by the last workgroup of each key
 *      tile to finish (deterministic, bitwise equal to 0, no separate kernel).
 */
fb_status_t fb_set_reduction(int mode);

/*
 * fb_probe_gq_atomics: a measurement probe, not part of the BoB path. It issues the
 * float32 atomic additions that a schedule forming gQ in pass 2 (instead of pass 1,
 * the alternative to the review page's two-pass design, Summary) needs at the least:
 * for every pair of a 128-key tile and a 32-query tile, one 32 x d tile of additions
 * into gq (the four waves of the key tile having summed theirs first), each adding
 * 1.0f, with pass 2's grid (key tiles x B*H x `splits`, split s taking its share of
 * the query tiles in order) and no other arithmetic. Its time bounds from below what
 * the atomics alone would cost that schedule.
 * gq: device, [B][H][N][d] float32, 16-byte aligned, caller-owned; on completion
 * (stream-ordered) every element has grown by ceil(N / 128).
 * Errors: FB_ERR_SHAPE / FB_ERR_HEADDIM as bob_attention; FB_ERR_ARG for splits
 * outside [1, 64]; FB_ERR_NULL for a NULL gq; FB_ERR_HIP for launch errors.
 */
fb_status_t fb_probe_gq_atomics(float* gq, int B, int H, int N, int d, int splits, hipStream_t stream);

/*
 * fb_set_alloc_limit: process-wide cap, in bytes, on each device allocation the
 * library makes itself (bob_attention's workspace, attn_bwd's scratch); 0 (the
 * default) means no cap. A larger request returns FB_ERR_OOM before any HIP
 * call, which lets a caller hold the library to a memory budget. The _ws entry
 * points allocate nothing and ignore it. Always returns FB_OK.
 */
fb_status_t fb_set_alloc_limit(size_t bytes);

/*
 * Kernel timing: fb_profile_start(only) makes every later launch of the
 * kernel named `only` (every launch when `only` is NULL or "") record a pair
 * of HIP events on the stream it is launched on; the string is copied.
 * Restricting the events to one kernel keeps the timing of the others
 * undisturbed. fb_profile_stop() waits for them, writes up to `max` entries
 * (kernel name, launches, total ms) and turns recording off. Returns the
 * number of distinct kernels (may exceed max), or a negative status.
 */
typedef struct {
  char name[48];
  int launches;
  double total_ms;
} fb_kernel_time_t;

void fb_profile_start(const char* only);
int fb_profile_stop(fb_kernel_time_t* out, int max);

#ifdef __cplusplus
}
#endif

#endif /* FLASHBOB_H */
