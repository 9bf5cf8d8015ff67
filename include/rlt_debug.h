/*
 * rlt_debug.h -- test-only entry point for kernel-level parity checks of the
 * library's matrix-product kernel (the kernel behind every projection of
 * "Recurrent Looped Transformer" §2.5 eqs. (2.9)-(2.16) and the readout of
 * §2.3 eq. (2.6)). Not part of the method's interface.
 */
#ifndef RLT_DEBUG_H
#define RLT_DEBUG_H

#include <stdint.h>

#include "rlt.h"

#ifdef __cplusplus
extern "C" {
#endif

/* out[m][n] = sum_k A[m][k] * W[n][k] for m < M, n < N (float32 output),
 * computed by the same kernel, K split and reduction order the decoder step
 * uses for an M-row call. A [M][K] and W [N][K] are device buffers of the
 * context's dtype; out is a device [M][N] float32 buffer. Requires
 * 1 <= M <= max_rows, N and K multiples of 32, K <= max(2 * d_model, d_ffn).
 * Enqueued on `stream`; returns RLT_ESHAPE / RLT_EINVAL on bad sizes. */
int rlt_dbg_gemm(rlt_ctx* ctx, const void* A, const void* W, int32_t M, int32_t N, int32_t K, float* out,
                 void* stream);

/* The same product through the operand-order path that bf16 decoder calls
 * take: W and A are first rearranged into the order of the 32x32x16 matrix
 * instruction (into buffers this call allocates and frees; it waits for
 * `stream`), then multiplied with the tile shape an M-row call would use.
 * Requires a bf16 context, 1 <= M <= max_rows, N a multiple of 32, K a
 * multiple of 64, K <= max(2 * d_model, d_ffn). */
int rlt_dbg_gemm_packed(rlt_ctx* ctx, const void* A, const void* W, int32_t M, int32_t N, int32_t K, float* out,
                        void* stream);

/* Kernel classes for the timing hook below. */
enum {
  RLT_PROF_XATTN = 0,     /* prefix cross-attention partials (eq. 2.15) */
  RLT_PROF_XCOMBINE = 1,  /* ordered merge of the cross-attention partials */
  RLT_PROF_SWA = 2,       /* SWA over the ring cache + insert (eq. 2.14) */
  RLT_PROF_GEMM = 3,      /* every matrix product incl. its split reduction */
  RLT_PROF_NORM = 4,      /* RMSNorms, merge preparation, state write-back */
  RLT_PROF_READOUT = 5,   /* log-sum-exp / argmax / sampling */
  RLT_PROF_FUSED = 6,     /* persistent step kernel (small calls: every class above
                             except the readout, in one launch) */
  RLT_PROF_NCLASS = 7
};

/* Timing hook for benchmarks: while enabled, every launch of a kernel class
 * made by non-captured calls is bracketed by two HIP events recorded on the
 * launch stream. enable != 0 also clears previous records. */
int rlt_dbg_profile(rlt_ctx* ctx, int32_t enable);

/* HOST, synchronising: total milliseconds and number of bracketed launches of
 * one kernel class since profiling was enabled. */
int rlt_dbg_profile_read(rlt_ctx* ctx, int32_t kernel_class, double* total_ms, int64_t* launches);

#ifdef __cplusplus
}
#endif
#endif /* RLT_DEBUG_H */
