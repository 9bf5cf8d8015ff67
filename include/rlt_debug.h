/*
 * rlt_debug.h -- test and benchmark hooks: kernel-level parity checks of the
 * library's matrix-product kernel (the kernel behind every projection of
 * "Recurrent Looped Transformer" §2.5 eqs. (2.9)-(2.16) and the readout of
 * §2.3 eq. (2.6)), launch options, per-class timing. Not part of the
 * method's interface.
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

/* Launch options of a context, for tests and tuning sweeps. A field left 0
 * keeps the library's choice, which depends on the config and the context's
 * capacities (max_rows, max_ctx) only. Fields that change a reduction order
 * (the attention fields) change the low bits of results. */
typedef struct rlt_dbg_launch {
  int32_t xattn_chunk;  /* memory positions per cross-attention partial, 16 .. 4096
                           (more than one chunk per row: partials merged by a combine kernel) */
  int32_t swa_hpw;      /* attention heads per SWA workgroup (ignored if invalid) */
  int32_t xattn_hpw;    /* attention heads per cross-attention workgroup (ignored if invalid) */
  int32_t fused_rows;   /* bf16: calls of at most this many rows (<= 32) run the persistent
                           step kernel (one launch, grid barriers between phases) */
  int32_t no_packed;    /* 1: no operand-order weight copy (bf16 products on the other tiles) */
  int32_t one_term;     /* 1: the operand-order products take their activations as one bf16
                           term (the other tiles always do) instead of two (value rounded,
                           then its rounding remainder): lower precision, for comparisons */
  int32_t replay_graph_min; /* rlt_replay_sequence: runs of at least this many ticks with one
                           active set are captured as a graph and replayed (0: 4; -1: never) */
  int32_t no_big_tile;  /* 1: the memory construction's K/V product on the 128 x 128 LDS tile
                           instead of the 256 x 256 one (same summation order, same results) */
  int32_t xattn_combine_kernel; /* where several cross-attention chunks of a row are merged
                           (same results): 0 by call size (inside the cross-attention launch, by
                           the last of the row's chunk workgroups, for calls of at most 256
                           workgroups; else a separate combine kernel), 1 always the combine
                           kernel, 2 always inside the launch */
  int32_t one_row_pf;   /* weight chunks in flight per wave in one-row products, 2 .. 4
                           (other values: the default; timing only, same results) */
  int32_t no_lt_dma;    /* 1: the staged product tile of 64 x 128 stages its chunks through
                           registers (three LDS buffers) instead of copying them from memory
                           straight into LDS (four buffers; same summation order, same results) */
  int32_t bwd_activations; /* rlt_replay_backward: 0 keep every step's activations when they
                           fit a quarter of the free device memory, else recompute them per step;
                           1 always recompute; 2 always keep (same results) */
} rlt_dbg_launch;

/* rlt_create with launch options (opt must not be NULL). */
int rlt_dbg_create(const rlt_config* cfg, const rlt_weights* w, int32_t max_rows, int32_t max_ctx,
                   const rlt_dbg_launch* opt, rlt_ctx** out);

/* Tuning sweeps: force the shape of the operand-order products of later
 * calls. lt > 0: the staged tile split over lt workgroups per tile
 * (1, 2, 4 or 8), of 128 rows x 2 column pairs, or of 64 rows x 4 column
 * pairs when cb = 4 (rb, pf, pre ignored). lt = 0: the register tile of
 * 32 * rb rows and cb column pairs with pf chunks in flight per wave, the
 * epilogue's values loaded before (pre = 1) or after (0) the K loop, or by
 * epilogue kind (-1). rb = 0 restores the library's choice. Shapes change
 * timing only, never results; shapes without a compiled kernel fall back to
 * the default register tile. */
int rlt_dbg_product_shape(rlt_ctx* ctx, int32_t rb, int32_t cb, int32_t lt, int32_t pf, int32_t pre);

/* Host-side walk of the narrow product tile's index math (the functions the
 * kernel itself uses) over every workgroup and lane of an n-row product with
 * npairs column pairs, K inputs, a weight of nseg segments of seg_rows rows
 * (pairing: 0 plain, 1 rotary halves of dh-wide heads, 2 two segments side
 * by side), activations of M_pad rows, and the launcher's own choice of K
 * split, row blocks and K slice (narrow_rows = min(max_rows, 32), target: 0
 * for a stand-alone launch, else the persistent step's workgroup count,
 * partial_cap: partial-buffer floats). Runs on the CPU: no device needed.
 * Fills *out with the plan and the largest index of each access. */
typedef struct rlt_narrow_report {
  int32_t S, mb, kslice;      /* the plan: K splits, 16-row blocks per tile, K per (split, wave) */
  int32_t w_seg_max, w_row_max; /* largest weight segment and row read */
  int32_t pad_;
  int64_t a_row_max;          /* largest activation row read (must be < M_pad) */
  int64_t a_col_end;          /* largest activation / weight column read + 8 (must be <= K) */
  int64_t partial_end;        /* largest partial index written + 1 (0: no split) */
  int64_t ssq_end;            /* largest row-statistics index written + 1 */
  int64_t steps_missing;      /* 32-wide K steps of a tile no wave multiplies */
  int64_t steps_repeated;     /* 32-wide K steps multiplied more than once */
} rlt_narrow_report;
int rlt_dbg_narrow_bounds(int32_t n, int32_t npairs, int32_t K, int32_t pairing, int32_t dh, int32_t nseg,
                          int32_t seg_rows, int32_t M_pad, int32_t narrow_rows, int32_t target, int64_t partial_cap,
                          rlt_narrow_report* out);

/* Counter calibration: read `bytes` (a multiple of 16) at device pointer
 * src once, in 16-byte pieces, with non-temporal loads (the load instruction
 * of the attention kernels' key and value streams; nontemporal = 1) or plain
 * ones, on `stream`; sink is a device word written only if the xor of all
 * data equals a fixed value (it keeps the loads). A rocprofv3 counter of
 * this launch against `bytes` gives the counter's bytes-per-unit factor. */
int rlt_dbg_stream_read(const void* src, int64_t bytes, int32_t nontemporal, uint32_t* sink, void* stream);

/* Peak calibration of the matrix cores: `blocks` workgroups of 256 threads,
 * each wave running 4 independent chains of the bf16 32x32x16 matrix
 * instruction (32768 flops each) for `iters` steps on register operands, on
 * `stream`: 4 * 4 * 32768 * iters * blocks flops per launch, timed by the
 * caller. sink: a device word written only if the results' xor equals a
 * fixed value (it keeps the work). Errors: RLT_EINVAL (null sink),
 * RLT_ESHAPE (blocks outside 1..2^20 or iters < 1). */
int rlt_dbg_mfma_loop(int32_t blocks, int32_t iters, uint32_t* sink, void* stream);

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
