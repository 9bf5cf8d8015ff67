/*
 * rlt.h -- C ABI of the MI355X (gfx950) implementation of the Recurrent
 * Looped Transformer's batched recurrent decoder state transition.
 *
 * Source of the operations: "Recurrent Looped Transformer" (Y. Zhang,
 * technical report, 2026), cited as [RLT §x, eq. (y)].
 *
 *   H_t = (s_t, C_t^D) = D(Merge(e_t, s_{t-1}); M_{<=t}, C_{t-1}^D, t)
 *                                                  [RLT §2.3, eqs. (2.4)-(2.5)]
 *   p(x_{t+1} | x_{1:t}) = softmax(W_o RMSNorm_o(s_t))_{x_{t+1}}   [eq. (2.6)]
 *
 * Conventions for every entry point:
 *  - Pointers are DEVICE pointers unless a field says HOST.
 *  - The caller owns every buffer it passes; the library keeps the weight
 *    pointers given to rlt_create (they must outlive the context) and owns
 *    only its internal workspace (for bf16 contexts with max_rows > 32 this
 *    includes a copy of the decoder's matrix weights, see rlt_create).
 *  - Calls enqueue work on `stream` (a hipStream_t passed as void*; NULL is
 *    the default stream) and return without waiting for it, except where
 *    a call says otherwise.
 *  - Return value: RLT_OK (0) or a negative status below. Host-checkable
 *    errors are returned before anything is enqueued. Errors the device
 *    detects (a row whose memory is too short, a pending-token mismatch)
 *    skip that row's update (its state is left unchanged), are recorded in
 *    the context, and are returned by the first call made after the
 *    detecting kernel completed (or by rlt_sync_error). No C++ exception
 *    crosses this interface. rlt_last_error() gives a message.
 *  - Element types: dtype RLT_BF16 means bfloat16 for weight matrices,
 *    the SWA cache, encoder memory and e; RLT_F32 means float32 for all of
 *    them. Gains, biases, s_star, the state s and all scores/log-probs are
 *    always float32.
 *  - Matrices use the natural [out][in] row-major layout (y = W x).
 */
#ifndef RLT_H
#define RLT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  RLT_OK = 0,
  RLT_EINVAL = -1,       /* null pointer or out-of-range argument */
  RLT_ESHAPE = -2,       /* sizes inconsistent with the config or capacities */
  RLT_EPREFIX = -3,      /* memory shorter than the position being consumed */
  RLT_ESTALE = -4,       /* state version differs from the weights version */
  RLT_EPENDING = -5,     /* consumed token differs from the pending token */
  RLT_EHIP = -6,         /* HIP runtime failure */
  RLT_ENOMEM = -7,       /* device allocation failed */
  RLT_EUNSUPPORTED = -8  /* shape or option the kernels do not implement */
};

enum { RLT_F32 = 0, RLT_BF16 = 1 };
enum { RLT_MERGE_GATED = 0, RLT_MERGE_CONVEX = 1 };
enum { RLT_POS_NONE = 0, RLT_POS_ROPE = 1 };
/* merge gate [RLT §2.5, text after eq. (2.11)]: one gate per channel
 * (eq. (2.10)) or one scalar gate per token, sigmoid(w_g . [e; r] + b_g) */
enum { RLT_GATE_VECTOR = 0, RLT_GATE_SCALAR = 1 };
/* sublayer order of every block [RLT §2.5, text after eq. (2.16)]: S = SWA,
 * X = cross-attention, F = FFN, each a pre-norm residual update with its own
 * RMSNorm; SXF is eqs. (2.14)-(2.16) */
enum { RLT_ORDER_SXF = 0, RLT_ORDER_SFX = 1, RLT_ORDER_XSF = 2, RLT_ORDER_XFS = 3, RLT_ORDER_FSX = 4,
       RLT_ORDER_FXS = 5 };

/* Model configuration.
 * merge_kind GATED:  r = RMSNorm_s(s_{t-1}); g = sigmoid(W_g [e; r] + b_g);
 *                    u = e + alpha * g (.) W_s r         [RLT §2.5, eqs. (2.9)-(2.11)]
 * merge_kind CONVEX: g = sigmoid(W_g [e; s] + b_g); u = g (.) e + (1 - g) (.) s
 * pos_kind ROPE: rotary transform (rotate-half pairing (i, i+dh/2), angle
 *   t * rope_theta^(-2i/dh), t the 1-based position) inside the SWA query
 *   and key maps and the cross-attention query map [RLT §2.5, text after
 *   eq. (2.16): query/key maps include positional transformations].
 * Supported shapes: d = n_heads * d_head; d_head in {16, 32, 64, 128}
 * (16 only with RLT_F32); d, d_ffn, vocab multiples of 32; window >= 1;
 * n_groups = 1 or n_layers (layer l reads group floor(l * G / L_D)). */
typedef struct rlt_config {
  int32_t n_layers;    /* L_D */
  int32_t d_model;     /* d */
  int32_t n_heads;     /* H */
  int32_t d_head;      /* dh */
  int32_t window;      /* W, includes the current token; cache keeps W-1 */
  int32_t n_groups;    /* G */
  int32_t d_ffn;       /* SwiGLU hidden width F */
  int32_t vocab;       /* V */
  int32_t merge_kind;  /* RLT_MERGE_* */
  int32_t pos_kind;    /* RLT_POS_* */
  int32_t dtype;       /* RLT_F32 | RLT_BF16 */
  float alpha;         /* feedback scale of the gated merge */
  float rms_eps;       /* RMSNorm: x / sqrt(mean(x^2) + eps) * gain */
  float rope_theta;
  uint64_t weights_version; /* states must carry the same version */
  int32_t merge_gate;  /* RLT_GATE_* (SCALAR: gated merge only) */
  int32_t merge_rank;  /* 0: full W_s; k > 0 (multiple of 32, <= d_ffn): W_s = U V of rank k */
  int32_t block_order; /* RLT_ORDER_* */
} rlt_config;

/* Parameters (device pointers, natural layout). Per-layer fields are HOST
 * arrays of n_layers device pointers. */
typedef struct rlt_weights {
  const float* s_star;      /* [d]     learned initial state [RLT §2.3, eq. (2.3)] */
  const float* merge_norm;  /* [d]     gain of RMSNorm_s (gated only) */
  const void* merge_wg;     /* [d][2d] W_g, input [e; r] (gated) or [e; s] (convex) */
  const float* merge_bg;    /* [d]     b_g */
  const void* merge_ws;     /* [d][d]  W_s (gated only) */
  const float* const* norm_s;  /* [d] gain of RMSNorm_{S,l}, feeds SWA q, k, v */
  const void* const* wq;       /* [d][d] SWA query  [RLT §2.5, eq. (2.12)] */
  const void* const* wk;       /* [d][d] SWA key    [eq. (2.13)] */
  const void* const* wv;       /* [d][d] SWA value  [eq. (2.13)] */
  const void* const* wo;       /* [d][d] SWA output projection [eq. (2.14)] */
  const float* const* norm_m;  /* [d] gain of RMSNorm_{M,l} (cross query) */
  const void* const* wqm;      /* [d][d] cross-attention query [eq. (2.15)] */
  const void* const* wom;      /* [d][d] cross-attention output projection */
  const float* const* norm_d;  /* [d] gain of RMSNorm_{D,l} [eq. (2.16)] */
  const void* const* w_gate;   /* [F][d] */
  const void* const* w_up;     /* [F][d] */
  const void* const* w_down;   /* [d][F]: FFN(h) = W_down(silu(W_gate h) (.) W_up h) */
  const float* out_norm;       /* [d]    gain of RMSNorm_o [eq. (2.6)] */
  const void* w_out;           /* [V][d] W_o */
  const void* merge_ws_u;      /* [d][k] U of a rank-k W_s (merge_rank = k > 0) */
  const void* merge_ws_v;      /* [k][d] V of a rank-k W_s; merge_ws is unused then.
                                  A scalar gate uses merge_wg [1][2d], merge_bg [1]. */
} rlt_weights;

/* Decoder state of B_cap independent rows [RLT §2.1: H_t = (s_t, C_t^D)].
 * Sizes from rlt_state_layout. Row r after consuming t tokens:
 *   s[r][0..d)                         s_t (float32)
 *   pos[r] = t                         number of consumed tokens
 *   pending[r]                         a sampled token recorded but not yet
 *                                      consumed, or -1 [RLT App. A.2]
 *   ring_k/ring_v[l][r][slot][0..d)    layer-l SWA keys/values of the
 *                                      retained positions j = max(1,t-W+2)..t
 *                                      at slot (j-1) mod (W-1); W-1 slots,
 *                                      none when W = 1 [RLT §2.5]. */
typedef struct rlt_state {
  float* s;
  void* ring_k;
  void* ring_v;
  int32_t* pos;
  int32_t* pending;
  int32_t B_cap;
  uint64_t version;   /* must equal rlt_config.weights_version [RLT §5.4, §6] */
} rlt_state;

/* Encoder memory M_{<=t} [RLT §2.2, eq. (2.2)]: read by the decoder calls,
 * written by rlt_memory_append / rlt_memory_prefill. Key of group g,
 * state row r, position j (1-based) starts at element
 *   k[g * stride_g + r * stride_b + (j - 1) * stride_t]   (likewise v)
 * and holds d contiguous elements of the config dtype. Only positions
 * j <= t are read at step t [RLT §4.2]; mem_len[r] (device) is the number
 * of valid positions of row r; a step needing t > mem_len[r] is a
 * device-detected RLT_EPREFIX. Strides are in elements. The decoder calls
 * (rlt_decoder_step, rlt_replay_sequence) read entries in 16-byte runs: k and
 * v must be 16-byte aligned and the strides multiples of 16 bytes' worth of
 * elements (8 bf16, 4 fp32), else RLT_EINVAL; the memory writers accept any
 * element-aligned layout (16-byte stores where it allows them). */
typedef struct rlt_memory {
  const void* k;
  const void* v;
  int64_t stride_g, stride_b, stride_t;
  const int32_t* mem_len;
} rlt_memory;

/* One transition for a ready set of rows [RLT §4.1]. */
enum { RLT_STEP_GRAPH = 1,  /* capture the step in a hipGraph on the first
                               call with these exact arguments and replay it
                               on later identical calls */
       RLT_STEP_DEFER = 2   /* record the sampled (or argmax) token as the
                               row's pending token [RLT App. A.2] */ };
typedef struct rlt_step_io {
  int32_t n;                 /* rows in this call, 0 < n <= max_rows */
  const int32_t* rows;       /* [n] distinct state rows; a row outside 0..B_cap-1 or
                                named by more than one slot is a device-detected
                                RLT_EINVAL and those slots are skipped */
  const void* e;             /* [n][d] e_t of the token each row consumes */
  rlt_memory mem;
  const int32_t* consume_tok;  /* [n] id of the consumed token, or NULL; must
                                  equal pending[row] when that is >= 0 */
  /* optional outputs (NULL = not produced) */
  float* s_out;              /* [n][d]   s_t */
  float* logits;             /* [n][V]   W_o RMSNorm_o(s_t) */
  int32_t* argmax;           /* [n]      lowest id among the largest logits */
  const int32_t* score_tok;  /* [n]      tokens to score ... */
  float* logp;               /* [n]      ... log p(score_tok | x_{1:t}) */
  /* behaviour sampler: tau, top-k truncation, renormalisation [RLT §5.3];
     draw = first id in (logit desc, id asc) order whose cumulative weight
     exp((z - z_max)/tau) exceeds u * total */
  const float* uniform;      /* [n] u in [0,1), or NULL = no sampling */
  float temperature;         /* tau > 0 */
  int32_t top_k;             /* 1 .. 1024 */
  int32_t* sample_tok;       /* [n] */
  float* sample_logmu;       /* [n] log mu(sample_tok) */
  float* z_trace;            /* [L_D][n][d] z after each block (debug), or NULL */
  int32_t flags;             /* RLT_STEP_* */
  float top_p;               /* nucleus of the behaviour distribution applied after
                                top-k (needs top_k >= 1); outside (0, 1): none */
} rlt_step_io;

/* Current-policy replay from H_0 [RLT App. A.4, eq. (2.7)]: for each
 * sequence b, re-initialise its row, consume x_1 .. x_{len_b - 1} in order
 * and, for split_b <= t <= len_b - 1, read log p(x_{t+1} | x_{1:t}) from s_t
 * before x_{t+1} is consumed. x_{len_b} is left as the row's pending token.
 * Sequences are advanced together; at tick t the active set is every b with
 * len_b - 1 >= t. */
typedef struct rlt_replay_io {
  int32_t B;                   /* sequences */
  const int32_t* rows_host;    /* HOST [B] state row of each sequence, or NULL = b */
  const int32_t* len_host;     /* HOST [B] tokens x_1..x_len, 2 <= len */
  const int32_t* split_host;   /* HOST [B] first scored position, 1 <= split */
  const void* e;               /* e_t of sequence b at e[b*e_stride_b + (t-1)*e_stride_t] */
  int64_t e_stride_b, e_stride_t;
  rlt_memory mem;              /* indexed by state row */
  const int32_t* tokens;       /* x_t of sequence b at tokens[b*tok_stride_b + t-1] */
  int64_t tok_stride_b;
  float* logp;                 /* logp[b*logp_stride_b + t] = log p(x_{t+1}|x_{1:t}) */
  int64_t logp_stride_b;
  float* s_trace;              /* optional: s_t at s_trace[(b*s_stride_b) + (t-1)*d] */
  int64_t s_stride_b;
} rlt_replay_io;

/* Scoring of given states [RLT §5.3, eq. (5.5)]: raw log-probabilities of
 * given tokens and, optionally, their behaviour log-probabilities under
 * (tau, top-k) and the ratios exp(log p - log mu_behaviour). */
typedef struct rlt_score_io {
  int32_t n;
  const float* s;            /* [n][d] states s_t */
  const int32_t* tokens;     /* [n] */
  float* logp;               /* [n] log p_Theta(token) */
  float temperature;         /* used when logmu != NULL */
  int32_t top_k;             /* 0 = no truncation; else 1 .. 1024 */
  float* logmu;              /* [n] log mu(token) under (tau, top_k), -inf off-support; or NULL */
  const float* logmu_behaviour; /* [n] recorded behaviour log-probs, or NULL */
  float* ratio;              /* [n] exp(logp - logmu_behaviour), or NULL */
  float top_p;               /* nucleus after top-k as in rlt_step_io; outside (0, 1): none */
} rlt_score_io;

typedef struct rlt_ctx rlt_ctx;

/* Create a context on the current HIP device. Validates the config,
 * precomputes position tables and allocates workspace for up to max_rows
 * rows per call and memory prefixes up to max_ctx positions.
 * bf16 with max_rows > 32 (and d_model, d_ffn multiples of 64, weights
 * 16-byte aligned): the context also holds a copy of the decoder's matrix
 * weights (wq/wk/wv, wo, wqm, wom, w_gate/w_up, w_down, w_out; as much device
 * memory again as those) in the operand order of the gfx950 32x32x16 bf16
 * matrix instruction, read by calls of more than 32 rows. The copy is made
 * here: after changing those weights in place, call rlt_refresh_weights
 * before the next call. Returns RLT_ENOMEM if it does not fit. The workspace
 * (activations, partial sums, arrival counters that kernels reset for the
 * next launch) is shared by every call on the context: calls on one context
 * must not overlap (issue them on one stream, or order the streams). */
int rlt_create(const rlt_config* cfg, const rlt_weights* w, int32_t max_rows, int32_t max_ctx,
               rlt_ctx** out);
void rlt_destroy(rlt_ctx* ctx);

/* HOST: bytes of the five state buffers for B_cap rows, in the order
 * s, ring_k, ring_v, pos, pending. */
int rlt_state_layout(const rlt_config* cfg, int32_t B_cap, size_t bytes_out[5]);

/* Message of the last error on the calling thread (static storage). */
const char* rlt_last_error(void);

/* H_0 = (s_star, empty) for the given rows [RLT §2.3, eq. (2.3)]: s = s_star,
 * pos = 0, pending = -1. rows: device [n]. flags bit 1 (RLT_INIT_POISON)
 * fills the rows' cache slots with NaN (any read of a slot outside the
 * window then shows in the outputs). */
enum { RLT_INIT_POISON = 1 };
int rlt_init_state(rlt_ctx* ctx, rlt_state* st, const int32_t* rows, int32_t n, int32_t flags,
                   void* stream);

/* One transition F_t for each listed row, t = pos[row] + 1, then the
 * readout and optional scoring/sampling from s_t. Advances pos[row].
 * A row's results do not depend on the other rows of the call or their
 * order (bit for bit within one context: every reduction order is fixed by
 * the config and the context's capacities, not by n) [RLT §3.1 Prop. 3.1,
 * §4.1]. For bf16 contexts without the operand-order weight copy this holds
 * among calls of at most 32 rows and among calls of more than 32 rows. */
int rlt_decoder_step(rlt_ctx* ctx, rlt_state* st, const rlt_step_io* io, void* stream);

/* rlt_decoder_step for callers that cannot allocate device memory (code
 * under their own HIP graph capture, tight serving loops, harnesses that
 * forbid allocation): the same transition, kernels and results bit for bit,
 * but the call allocates nothing. The duplicate-row counters, which
 * rlt_decoder_step allocates on its first call for a state, live here in a
 * fixed device array of the library (RLT_NOALLOC_MAX_ROWS int32 per device,
 * held until the process ends); everything else is the context's workspace
 * from rlt_create. Limits: st->B_cap <= RLT_NOALLOC_MAX_ROWS (else
 * RLT_ESHAPE); RLT_STEP_GRAPH is refused (RLT_EINVAL: instantiating a graph
 * allocates) and the opt-in persistent step is not used. The counters are
 * shared by every such call on one device and cleared by each call for its
 * own rows: calls of this entry point that overlap on one device (other
 * streams, other contexts) race and must be ordered by the caller. */
#define RLT_NOALLOC_MAX_ROWS 65536
int rlt_decoder_step_noalloc(rlt_ctx* ctx, rlt_state* st, const rlt_step_io* io, void* stream);

/* See rlt_replay_io. Synchronises the stream once at the start (upload of
 * the schedule). On a non-default stream that is not being captured, each
 * run of ticks with the same active set (the sequences still running) is
 * captured once as a graph and replayed for the run's ticks (the launches
 * of a tick depend on the set's size only; the position is kept on the
 * device); the call then also waits for the stream at its end, when it
 * releases those graphs. Results are the same either way. */
int rlt_replay_sequence(rlt_ctx* ctx, rlt_state* st, const rlt_replay_io* io, void* stream);

int rlt_score_logprobs(rlt_ctx* ctx, const rlt_score_io* io, void* stream);

/* Wait for `stream`, then return (and clear) any device-detected error. */
int rlt_sync_error(rlt_ctx* ctx, void* stream);

/* The caller changed weight values in place (an optimiser step on the
 * gradients of rlt_replay_backward): states computed under the old values no
 * longer hold the model's state [RLT §5.4; App. A.4 replays under the current
 * parameters]. This rebuilds the context's operand-order copy of the matrix
 * weights (see rlt_create) from the caller's weights, on `stream` (nothing to
 * rebuild for contexts without the copy), and makes weights_version the
 * context's version: states and snapshots carrying any other version are then
 * refused with RLT_ESTALE until re-initialised under the new version. The
 * pointers themselves are fixed at rlt_create. weights_version must differ
 * from the context's current version (else RLT_EINVAL, nothing done). */
int rlt_refresh_weights(rlt_ctx* ctx, uint64_t weights_version, void* stream);

/* Log of the trajectory importance weight prod_i r_i [RLT §5.3, text after
 * eq. (5.5)] of B sequences: out[b] = sum over t = split_host[b] ..
 * len_host[b] - 1 of logp[b * logp_stride_b + t] - logmu[b * logmu_stride_b + t]
 * (the positions a replay scores), summed in t order. HOST len/split arrays,
 * device logp / logmu / out (float32). */
int rlt_trajectory_log_ratio(rlt_ctx* ctx, int32_t B, const int32_t* len_host, const int32_t* split_host,
                             const float* logp, int64_t logp_stride_b, const float* logmu,
                             int64_t logmu_stride_b, float* out, void* stream);

/* Exact prefix snapshot of decoder rows [RLT §6]: the complete decoder
 * state H_t = (s_t, C_t^D) of a row with its position metadata and the model
 * version, so that a restored row continues bit for bit as if it had never
 * been saved (the encoder memory M_{<=t} is the caller's buffer and is kept
 * by the caller). One row's snapshot is the header below followed by
 *   s [d] float32, ring_k [L_D][W-1][d], ring_v [L_D][W-1][d] (config dtype),
 * slots as in rlt_state (slot (j-1) mod (W-1) holds position j). */
#define RLT_SNAPSHOT_MAGIC 0x53544c52u /* "RLTS" */
typedef struct rlt_snapshot_header {
  uint32_t magic;            /* RLT_SNAPSHOT_MAGIC */
  uint32_t layout;           /* 1 */
  uint64_t weights_version;  /* rlt_config.weights_version of the saving context */
  int32_t n_layers, d_model, window, dtype;
  int32_t pos;               /* consumed tokens t */
  int32_t pending;           /* pending token or -1 [RLT App. A.2] */
  int32_t reserved[6];
} rlt_snapshot_header;

/* HOST: bytes of one row's snapshot for this config. */
int rlt_snapshot_bytes(const rlt_config* cfg, size_t* bytes_per_row);

/* Copy rows rows_host[i] (HOST array) of `st` into the HOST buffer dst,
 * row i at dst + i * rlt_snapshot_bytes. Waits for `stream` (the copies
 * follow the work already enqueued on it) and returns when dst is complete. */
int rlt_state_snapshot(rlt_ctx* ctx, const rlt_state* st, const int32_t* rows_host, int32_t n, void* dst,
                       void* stream);

/* Restore snapshot i of the HOST buffer src into row rows_host[i] of `st`
 * (s, cache, pos, pending). Every header is checked before anything is
 * written: bad magic/layout RLT_EINVAL, another config RLT_ESHAPE, another
 * weights version (or a state of another version) RLT_ESTALE. Waits for
 * `stream`. */
int rlt_state_restore(rlt_ctx* ctx, rlt_state* st, const int32_t* rows_host, int32_t n, const void* src,
                      void* stream);

/* Parameters of the encoder-memory maps [RLT §2.2, eq. (2.2)], one set per
 * group g < G; arrays of G device pointers, caller-owned, valid during the
 * call: RMSNorm_E gain [d] fp32, W_K^g and W_V^g [d][d] of the config dtype
 * (natural [out][in] layout). The key map is RoPE(W_K^g RMSNorm_E(e_t), t)
 * with the decoder's rotary convention (pos_kind, rope_theta); the value
 * map is W_V^g RMSNorm_E(e_t). */
typedef struct rlt_memory_weights {
  const float* const* norm_e;
  const void* const* wk;
  const void* const* wv;
} rlt_memory_weights;

/* Memory append, the step before a transition [RLT §2.2 eq. (2.2), §2.3
 * eq. (2.8), App. A.2]: slot i < n writes, for every group, the entry of
 * memory row rows[i] (device [n], distinct) at position
 * t = mem_len[rows[i]] + 1 from e[i] (device [n][d], config dtype), then
 * sets mem_len[rows[i]] = t. The buffers of `mem` are written (k, v) and
 * updated (mem_len); B_cap and T_cap are their row and position
 * capacities. A row outside 0..B_cap-1 raises a device-detected
 * RLT_EINVAL, a row already holding T_cap entries RLT_EPREFIX; such slots
 * are skipped. Enqueued on `stream`. */
int rlt_memory_append(rlt_ctx* ctx, const rlt_memory_weights* mw, const rlt_memory* mem, int32_t B_cap,
                      int32_t T_cap, const int32_t* rows, int32_t n, const void* e, void* stream);

/* Token-parallel memory prefill [RLT §2.2 eq. (2.2), §4.1]: for sequences
 * b < B (memory row b) every entry t = 1 .. len_host[b] (HOST array, each
 * 1 <= len <= T_cap) from e[b * e_stride_b + (t - 1) * e_stride_t] (device,
 * strides in elements), then mem_len[b] = len_host[b]. Enqueued on
 * `stream` after one synchronous upload of the schedule. */
int rlt_memory_prefill(rlt_ctx* ctx, const rlt_memory_weights* mw, const rlt_memory* mem, int32_t T_cap,
                       int32_t B, const int32_t* len_host, const void* e, int64_t e_stride_b, int64_t e_stride_t,
                       void* stream);

/* Replay backward: full backpropagation through time of a replayed loss
 * [RLT §5.4; App. B, eqs. (B.1)-(B.5)]. The loss is linear in the replayed
 * log-probabilities,
 *   L = sum_b sum_{t = split_b}^{len_b - 1} w[b][t] * log p(x_{t+1} | x_{1:t}),
 * (w = -1: next-token likelihood; w = advantages: the score-function
 * surrogate of eq. (5.4)), each sequence replayed from H_0 as in
 * rlt_replay_sequence. Its gradient flows through s_t, through every decoder
 * SWA key/value to the steps that read it (also after eviction) and through
 * the encoder memory; nothing is detached.
 *
 * Gradients are float32 device buffers shaped as the matching rlt_weights
 * fields, ACCUMULATED into (zero them first); per-layer fields are HOST
 * arrays of n_layers device pointers. Any field (or per-layer array, or
 * entry of one) may be NULL: that gradient is not formed.
 *
 * Arithmetic is float32 throughout, on the given parameter values (bf16
 * parameters, e and memory are widened): the call differentiates the float32
 * transition, which for a float32 configuration is the one the forward calls
 * compute (up to summation order). A forward pass keeps s_t and the decoder
 * keys/values of every step; it also keeps every step's activations when they
 * fit in a quarter of the device memory free at the call, and otherwise
 * (per-step checkpointing) the backward pass recomputes each step's
 * activations before differentiating it, with the same results. Covers the vector merge gate, full-rank W_s and sublayer order SXF
 * (others: RLT_EUNSUPPORTED); len - 1 <= 8192 - d_head. Work buffers are
 * allocated for the call (RLT_ENOMEM if they do not fit). */
typedef struct rlt_grads {
  float* s_star;
  float* merge_norm;
  float* merge_wg;
  float* merge_bg;
  float* merge_ws;
  float* const* norm_s;
  float* const* wq;
  float* const* wk;
  float* const* wv;
  float* const* wo;
  float* const* norm_m;
  float* const* wqm;
  float* const* wom;
  float* const* norm_d;
  float* const* w_gate;
  float* const* w_up;
  float* const* w_down;
  float* out_norm;
  float* w_out;
} rlt_grads;

typedef struct rlt_backward_io {
  int32_t B;                   /* sequences */
  const int32_t* len_host;     /* HOST [B] tokens x_1..x_len, 2 <= len */
  const int32_t* split_host;   /* HOST [B] first scored position, 1 <= split <= len - 1 */
  const void* e;               /* e_t of sequence b at e[b*e_stride_b + (t-1)*e_stride_t] (config dtype) */
  int64_t e_stride_b, e_stride_t;
  rlt_memory mem;              /* memory of sequence b (config dtype), >= len_b - 1 positions; mem_len unused */
  const int32_t* tokens;       /* x_t of sequence b at tokens[b*tok_stride_b + t-1] */
  int64_t tok_stride_b;
  const float* w;              /* w[b*w_stride_b + t]: weight of log p(x_{t+1} | x_{1:t}) */
  int64_t w_stride_b;
  float* logp;                 /* optional: logp[b*logp_stride_b + t] of the replay */
  int64_t logp_stride_b;
  float* de;                   /* optional: dL/de_t at de[b*de_stride_b + (t-1)*de_stride_t] (accumulated) */
  int64_t de_stride_b, de_stride_t;
  float* dmem_k;               /* optional (both or none): dL/dM at [g*stride_g + b*stride_b + (t-1)*stride_t] */
  float* dmem_v;
  int64_t dmem_stride_g, dmem_stride_b, dmem_stride_t;
} rlt_backward_io;

int rlt_replay_backward(rlt_ctx* ctx, const rlt_backward_io* io, const rlt_grads* grads, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* RLT_H */
