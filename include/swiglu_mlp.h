/*
 * swiglu_mlp.h -- C ABI of the fused SwiGLU MLP library for MI355X (gfx950).
 *
 * The operation (page "[RFC] Full-pipeline SwiGLU MLP with forward/backward
 * co-optimization", Liger-Kernel issue #1347, section "Summary"):
 *
 *   forward   G = X Wg, U = X Wu, A = SiLU(G) * U, Y = A Wd
 *   backward  dA = dY Wd^T (never stored), dU = dA * SiLU(G),
 *             dG = dA * U * SiLU'(G), dWd = A^T dY,
 *             [dWg | dWu] = X^T [dG | dU]   (one GEMM),
 *             dI = [dG | dU] [Wg | Wu]^T    (one accumulator over 2H)
 *   no-grad   the forward without keeping G and U.
 *
 * Shapes and layouts. All matrices are dense and row-major (last index
 * contiguous): X, Y, dY, dX are [T, D]; Wg, Wu, dWg, dWu are [D, H];
 * Wd, dWd are [H, D]. All tensors of one call share one dtype. T >= 0 is any
 * value below 2^31; D and H must be positive multiples of 8, at most 4194296
 * for bf16/fp16 and 2097144 for fp32 (the kernels address a 256-row tile of
 * any operand with 32-bit byte offsets), and every launch's tile count must
 * fit in 32 bits. Every pointer must be 16-byte aligned; pointers to buffers
 * of zero bytes (T = 0) may be NULL.
 *
 * Numerics. bf16/fp16 storage with fp32 accumulation; every stored value is
 * rounded once (round to nearest even) from fp32. The SwiGLU epilogue is the
 * one-round program of "Scope one-round FP32 SwiGLU to the exact Qwen3.5
 * contract" (xorl PR #51, review thread): A = rnd(SiLU(g) * u), evaluated in
 * fp32 from the stored (rounded) g and u (the _ex entry points can select
 * the historical two-round program instead). SWIGLU_FP32 is true IEEE fp32:
 * fp32 operands enter the matrix cores unrounded (the TF32 issue described
 * in "[RFC] Testing Methodology for FP32 Convergence Tests on Fused
 * SwiGLU/dSwiGLU Kernels", Liger-Kernel issue #1383, section "Root Cause").
 *
 * Saved buffer. One allocation of swiglu_mlp_saved_bytes() bytes holding three
 * [T, H] planes in the order A, G, U ("store A, G, and U in one contiguous
 * buffer", issue #1347, section "Summary"). swiglu_mlp_bwd overwrites the G
 * and U planes with dG and dU ("overwrite expired G/U storage with dG/dU",
 * same section), so a saved buffer supports exactly one backward (same page,
 * section "Known limitations and validation gaps"). The A plane is left
 * unchanged.
 *
 * Ownership and streams. The caller owns every buffer; the library keeps no
 * per-call state and allocates no device memory in these calls. Work is
 * enqueued on `stream` (a hipStream_t; NULL = the default stream) and the
 * calls return before it finishes. Arguments are validated on the host
 * before anything is launched: a nonzero status means nothing was enqueued,
 * except SWIGLU_ERR_LAUNCH (a launch failed after validation). NaN and Inf
 * propagate through the arithmetic; there are no device-side traps.
 * Gradients are written (beta = 0), not accumulated.
 */
#ifndef SWIGLU_MLP_H
#define SWIGLU_MLP_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SWIGLU_BF16 = 0, /* bfloat16 storage, fp32 accumulation */
  SWIGLU_FP16 = 1, /* float16 storage, fp32 accumulation (issue #1347, "Validation environment") */
  SWIGLU_FP32 = 2  /* IEEE fp32 storage and products */
} swiglu_dtype_t;

typedef enum {
  SWIGLU_OK = 0,
  SWIGLU_ERR_NULL = 1,      /* a required pointer is NULL */
  SWIGLU_ERR_SHAPE = 2,     /* T < 0, D or H <= 0, not a multiple of 8 or above the limit, or a size overflows */
  SWIGLU_ERR_DTYPE = 3,     /* unknown dtype */
  SWIGLU_ERR_ALIGN = 4,     /* a pointer is not 16-byte aligned */
  SWIGLU_ERR_ALIAS = 5,     /* an output overlaps an input or another output */
  SWIGLU_ERR_WORKSPACE = 6, /* workspace NULL or smaller than required */
  SWIGLU_ERR_DEVICE = 7,    /* current device is not gfx950, or a HIP query failed */
  SWIGLU_ERR_LAUNCH = 8,    /* a kernel launch failed (work may be partially enqueued) */
  SWIGLU_ERR_FLAGS = 9,     /* unknown bits in the flags of an _ex entry point */
  SWIGLU_ERR_SCRATCH = 10   /* swiglu_mlp_infer_noalloc: the call needs more than its fixed scratch */
} swiglu_status_t;

/* Flags of the _ex entry points (swiglu_mlp_fwd_ex, swiglu_mlp_bwd_ex,
 * swiglu_mlp_infer_ex, swiglu_mlp_infer_noalloc).
 *
 * SWIGLU_FLAG_TWO_ROUND selects the historical two-round SwiGLU program of
 * "Scope one-round FP32 SwiGLU to the exact Qwen3.5 contract" (xorl PR #51,
 * review thread): A = rnd(rnd(SiLU(g)) * u), SiLU(g) rounded to the storage
 * dtype before the product. This gives byte compatibility with unfused
 * pipelines that store SiLU(g) first. The page reports that about 27% of
 * bf16 outputs differ from the one-round program. Only A changes: G, U and
 * the backward are as without the flag, and the backward's dWd uses the A it
 * finds in the saved buffer (the backward ignores the flag). In SWIGLU_FP32
 * the two programs coincide.
 *
 * SWIGLU_FLAG_LINEAR_WEIGHTS: the weights (and the weight gradients the
 * backward writes) are in the layout of the nn.Linear layers of the
 * transformers MLP modules ("an interchangeable layer which has identical
 * __init__ and forward signatures as hf/transformers xxxMLP", maintainers'
 * thread on the mirror of issue #1347, "Three levels of APIs"):
 * Wg = gate_proj.weight and Wu = up_proj.weight are [H, D], Wd =
 * down_proj.weight is [D, H], all row-major; dWg, dWu are then [H, D] and
 * dWd is [D, H]. The kernels read this layout directly (no transposed
 * copy). The forward, backward and no-grad call of one computation must
 * all pass the same layout flag. */
#define SWIGLU_FLAG_TWO_ROUND 1u
#define SWIGLU_FLAG_LINEAR_WEIGHTS 2u
#define SWIGLU_FLAGS_ALL 3u

/* Bytes of the saved A|G|U buffer: 3 * T * H * sizeof(dtype). 0 on bad args. */
size_t swiglu_mlp_saved_bytes(int64_t T, int64_t H, int dtype);

/* Bytes of the no-grad workspace: the A plane, T * H * sizeof(dtype) ("a
 * dedicated no-grad path that does not save G/U", issue #1347, "Summary";
 * the page's table "Inference, BF16, B=1" equals A + Y at S = 256). For
 * bf16/fp16 with 1 <= T <= 128 (weight streaming) it also holds, after A and
 * 256-byte aligned, one arrival counter per 64 columns of the down
 * projection and the fp32 partial sums of its K splits, capped so that
 * workspace + Y stays within 3 (A + Y) (D = 4096, H = 11008, T = 128:
 * 10.2 MB against A + Y = 3.9 MB). The size covers both weight layouts
 * (with SWIGLU_FLAG_LINEAR_WEIGHTS only the A plane is used). 0 on bad
 * args. */
size_t swiglu_mlp_infer_workspace_bytes(int64_t T, int64_t D, int64_t H, int dtype);

/* Bytes of the backward workspace: fp32 partial tiles (256 x 256, 256 KiB
 * each) of the weight-gradient GEMMs (K = T; bf16/fp16, T > 512). Their
 * 256 x 256 output tiles run whole in rounds of one per CU of the current
 * device; the tiles of a partly filled last round are split over K when
 * that is modelled to be faster (for example D = 4096, H = 11008: 176 tiles
 * of dWd in 4 pieces, 176 MiB). 0 when no tile is split (whole
 * rounds, as at D = 4096, H = 8192) and for fp32. 0 on bad args. */
size_t swiglu_mlp_bwd_workspace_bytes(int64_t T, int64_t D, int64_t H, int dtype);

/* Forward for training. Reads X, Wg, Wu, Wd; writes Y [T, D] and the saved
 * A|G|U buffer (swiglu_mlp_saved_bytes bytes). Y and saved must not overlap
 * each other or any input. Kernels: gate/up GEMM with the fused SwiGLU
 * epilogue, then the down projection. */
int swiglu_mlp_fwd(const void* X, const void* Wg, const void* Wu, const void* Wd,
                   void* Y, void* saved, int64_t T, int64_t D, int64_t H,
                   int dtype, hipStream_t stream);

/* swiglu_mlp_fwd with epilogue flags (SWIGLU_FLAG_*); flags = 0 is
 * swiglu_mlp_fwd. Unknown bits: SWIGLU_ERR_FLAGS, nothing launched. */
int swiglu_mlp_fwd_ex(const void* X, const void* Wg, const void* Wu, const void* Wd,
                      void* Y, void* saved, int64_t T, int64_t D, int64_t H,
                      int dtype, unsigned flags, hipStream_t stream);

/* Full backward. Reads dY, X, Wg, Wu, Wd and the saved buffer written by
 * swiglu_mlp_fwd with the same inputs; writes dX [T, D] (the page's dI),
 * dWg, dWu [D, H], dWd [H, D]. Consumes the saved buffer: its G and U planes
 * hold dG and dU afterwards, and a second call on it computes garbage.
 * workspace (>= swiglu_mlp_bwd_workspace_bytes() bytes, contents on entry
 * irrelevant) may be NULL when that size is 0. Outputs and workspace must
 * not overlap each other, the inputs, or the saved buffer. */
int swiglu_mlp_bwd(const void* dY, const void* X, const void* Wg, const void* Wu,
                   const void* Wd, void* saved, void* dX, void* dWg, void* dWu,
                   void* dWd, void* workspace, size_t workspace_bytes,
                   int64_t T, int64_t D, int64_t H, int dtype, hipStream_t stream);

/* swiglu_mlp_bwd with flags (SWIGLU_FLAG_*); flags = 0 is swiglu_mlp_bwd.
 * With SWIGLU_FLAG_LINEAR_WEIGHTS the weights are read, and dWg, dWu, dWd
 * written, in the nn.Linear layout. Unknown bits: SWIGLU_ERR_FLAGS, nothing
 * launched. */
int swiglu_mlp_bwd_ex(const void* dY, const void* X, const void* Wg, const void* Wu,
                      const void* Wd, void* saved, void* dX, void* dWg, void* dWu,
                      void* dWd, void* workspace, size_t workspace_bytes,
                      int64_t T, int64_t D, int64_t H, int dtype, unsigned flags,
                      hipStream_t stream);

/* No-grad forward: Y [T, D] from X and the weights; G and U are never
 * stored. workspace (>= swiglu_mlp_infer_workspace_bytes bytes) holds A and,
 * for T <= 128, counters and partial sums; its contents on entry do not
 * matter (the call clears what it counts on). Two launches. Calls that use
 * one workspace must not overlap (stream order them). Y must not overlap
 * the inputs or the workspace. */
int swiglu_mlp_infer(const void* X, const void* Wg, const void* Wu, const void* Wd,
                     void* Y, void* workspace, size_t workspace_bytes,
                     int64_t T, int64_t D, int64_t H, int dtype, hipStream_t stream);

/* swiglu_mlp_infer with epilogue flags (SWIGLU_FLAG_*); flags = 0 is
 * swiglu_mlp_infer. Unknown bits: SWIGLU_ERR_FLAGS, nothing launched. */
int swiglu_mlp_infer_ex(const void* X, const void* Wg, const void* Wu, const void* Wd,
                        void* Y, void* workspace, size_t workspace_bytes,
                        int64_t T, int64_t D, int64_t H, int dtype, unsigned flags,
                        hipStream_t stream);

/* Allocation-free no-grad forward, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc). Same computation, kernels and results as
 * swiglu_mlp_infer_ex with the same flags, but the workspace is a fixed
 * array of SWIGLU_NOALLOC_SCRATCH_BYTES inside the library: one copy per
 * device, held from the library's first call on that device until the
 * process ends. Calls allocate nothing (no hipMalloc, hipFree or allocating
 * library routine). A call whose swiglu_mlp_infer_workspace_bytes exceeds
 * the scratch returns SWIGLU_ERR_SCRATCH with nothing launched (bf16 at
 * D = 4096, H = 11008: every T <= 128, and T <= 1524 above that). The
 * caller passes the inputs and Y as for swiglu_mlp_infer. Every call on one
 * device shares that device's scratch, which keeps the last call's
 * contents (the call clears what it counts on): calls that overlap on one
 * device race and must be ordered (one stream, or events). */
#define SWIGLU_NOALLOC_SCRATCH_BYTES (32u << 20)
int swiglu_mlp_infer_noalloc(const void* X, const void* Wg, const void* Wu, const void* Wd,
                             void* Y, int64_t T, int64_t D, int64_t H, int dtype,
                             unsigned flags, hipStream_t stream);

/* Static description of a status code (never NULL). */
const char* swiglu_mlp_status_string(int status);

/* ---- Profiling aid (not part of the computation) -------------------------
 * Stage ids, one per kernel of the path:
 *   0 gate/up GEMM + SwiGLU (fwd)      1 down projection (fwd)
 *   2 dA GEMM + in-place dSwiGLU       3 dWd = A^T dY
 *   4 [dWg | dWu] = X^T [dG | dU]      5 dI single accumulator
 *   6 no-grad gate/up (A only)         7 no-grad down projection
 *   8 stages 3 + 2 in one launch       9 stages 4 + 5 in one launch
 * (bf16/fp16 run every stage as its own launch; in fp32 with T > 512 the
 * backward runs as launches 8 and 9, where the long-K weight-gradient tiles
 * are dispatched first and the short tiles of the other stage fill in
 * behind them.)
 * swiglu_mlp_timer_start(capacity) makes every later launch of a stage record
 * a HIP event pair around it on the launch stream, up to `capacity` launches
 * per stage (events are created here; returns a status). swiglu_mlp_timer_stop
 * waits for the recorded events and writes, for each of the first `n` stages,
 * the summed milliseconds to ms[s] and the launch count to count[s], then
 * disables recording. Not thread-safe; meant for a benchmark's timed loop. */
#define SWIGLU_NUM_STAGES 10
int swiglu_mlp_timer_start(int capacity);
int swiglu_mlp_timer_stop(double* ms, int* count, int n);

#ifdef __cplusplus
}
#endif
#endif /* SWIGLU_MLP_H */
