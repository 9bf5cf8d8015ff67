// Kernels of the replay backward (full BPTT through the decoder recurrence,
// "Recurrent Looped Transformer" §5.4 and App. B). Every kernel computes in
// float32; parameters, e_t and memory arrive in the configuration's element
// type (dt 0 = float32, 1 = bf16). Activations and gradients are float32,
// row-major, rows = the active sequences of a step. All reductions run in a
// fixed order, so results do not depend on scheduling.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <string>
#include <vector>

#include "../../include/rlt.h"

namespace rlt {
namespace bwd {

// C[i][j] (+)= sum_k A(i,k) B(k,j), A(i,k) = a[i*a_si + k*a_sk] (float32),
// B(k,j) = b[k*b_sk + j*b_sj] (element type bdt), C[i][j] at c[i*c_si + j].
void mm(int M, int N, int K, const float* a, int64_t a_si, int64_t a_sk, const void* b, int bdt, int64_t b_sk,
        int64_t b_sj, float* c, int64_t c_si, bool accumulate, hipStream_t s);
// C = base + A B (base with C's row stride): the bits of copying base to C
// and then accumulating
void mm_base(int M, int N, int K, const float* a, int64_t a_si, int64_t a_sk, const void* b, int bdt, int64_t b_sk,
             int64_t b_sj, const float* base, float* c, int64_t c_si, hipStream_t s);
// nseg (<= 3) products of one launch, each the same bits as its own mm call:
// one A, B and C per segment (mm_outputs), or A and B per segment added into
// one C in segment order (mm_summed: C (+)= A_0 B_0, then += A_1 B_1, ...)
void mm_outputs(int nseg, int M, int N, int K, const float* a, int64_t a_si, int64_t a_sk, const void* const* b,
                int bdt, int64_t b_sk, int64_t b_sj, float* const* c, int64_t c_si, bool accumulate, hipStream_t s);
void mm_summed(int nseg, int M, int N, int K, const float* const* a, int64_t a_si, int64_t a_sk,
               const void* const* b, int bdt, int64_t b_sk, int64_t b_sj, float* c, int64_t c_si, bool accumulate,
               hipStream_t s);

// y = RMSNorm(x) * gain (rows of width d, leading dimensions ld), rstd[r] saved
void rms_fwd(const float* x, int64_t ldx, const float* gain, float* y, int64_t ldy, float* rstd, int n, int d,
             float eps, hipStream_t s);
// dx (+)= d RMSNorm(x)*gain / dx applied to dy; with base: dx = base + that
void rms_bwd(const float* x, int64_t ldx, const float* gain, const float* rstd, const float* dy, int64_t ldy,
             float* dx, int64_t lddx, int n, int d, bool accumulate, hipStream_t s, const float* base = nullptr,
             int64_t ldb = 0);
// dst[c] += sum_r a[r][c] * (b ? b[r][c] : 1) * (rs ? rs[r] : 1), rows in order
void colsum(float* dst, const float* a, int64_t lda, const float* b, int64_t ldb, const float* rs, int n, int d,
            hipStream_t s);
// the same sums over many rows (16 row lanes per column, lanes added in order)
void colsum_rows(float* dst, const float* a, int64_t lda, const float* b, int64_t ldb, const float* rs, int64_t n,
                 int d, hipStream_t s);
// rotary transform of every head of n rows at position t (sign -1: inverse)
void rope(float* x, int64_t ld, int n, int d, int dh, int t, const double* inv_freq, int sign, hipStream_t s);
// the same on two distinct arrays of the same shape and position, one launch
void rope2(float* x, float* x2, int64_t ld, int n, int d, int dh, int t, const double* inv_freq, int sign,
           hipStream_t s);

// Keys / values of one row over positions lo..hi (1-based): row r reads
// base + row_off(r) + (j-1)*s_pos, row_off(r) = (map ? map[r] : r) * s_row.
struct KV {
  const void* k;
  const void* v;
  int dt;  // element type of k/v
  int64_t s_row, s_pos;
  const int* map;
};
struct DKV {
  float* k;
  float* v;
  int64_t s_row, s_pos;
  const int* map;
};
// o[r][h*dh..] = softmax_j(q_h . k_j / sqrt(dh)) v_j, j = lo..hi
void attn_fwd(const float* q, int64_t ldq, KV kv, int lo, int hi, float* o, int64_t ldo, int n, int H, int dh,
              hipStream_t s);
// dq (written), dK/dV (accumulated; skipped when dkv.k is null) of attn_fwd
void attn_bwd(const float* q, int64_t ldq, KV kv, int lo, int hi, const float* dout, int64_t lddo, float* dq,
              int64_t lddq, DKV dkv, int n, int H, int dh, hipStream_t s);

// e_t rows (element type dt) of sequences map[r] into x[r][0..d)
void gather_e(float* x, int64_t ldx, const void* e, int dt, int64_t sb, int64_t st, const int* map, int t, int n,
              int d, hipStream_t s);
// de[map[r]][t] += g[r][0..d)
void scatter_add_e(float* de, int64_t sb, int64_t st, const float* g, int64_t ldg, const int* map, int t, int n,
                   int d, hipStream_t s);
// g = sigmoid(pre + bias) in place
void sigmoid_bias(float* g, int64_t ld, const float* bias, int n, int d, hipStream_t s);
// gated merge u = e + alpha * g * wsr; convex u = g * e + (1 - g) * sp
void merge_fwd(int gated, float* u, const float* e, int64_t lde, const float* g, const float* wsr_or_s,
               int64_t ldw, float alpha, int n, int d, hipStream_t s);
// gated: dpre = alpha du*wsr*g(1-g), dw = alpha g du, de = du
// convex: dpre = du*(e-s)*g(1-g), dw(=ds) = du*(1-g), de = du*g
void merge_bwd(int gated, const float* du, const float* e, int64_t lde, const float* g, const float* wsr_or_s,
               int64_t ldw, float alpha, float* dpre, float* dw, float* de, int64_t ldde, int n, int d,
               hipStream_t s);
void swiglu_fwd(const float* a, const float* u, float* act, int n, int F, hipStream_t s);
void swiglu_bwd(const float* a, const float* u, const float* dact, float* da, float* du, int n, int F,
                hipStream_t s);
// log p of token x_{t+1} of sequence map[r] (rows with t >= split[r]): logp
// written (if non-null) and dlogits = w[t] * (onehot - softmax); zero rows
// otherwise
void logsoftmax_bwd(const float* logits, int V, const int* tokens, int64_t tok_sb, const float* w,
                    int64_t w_sb, const int* map, const int* split, int t, float* logp, int64_t logp_sb,
                    float* dlogits, int n, hipStream_t s);
// y = a + b (elementwise rows), or y = a when b is null
void add(float* y, int64_t ldy, const float* a, int64_t lda, const float* b, int64_t ldb, int n, int d,
         hipStream_t s);

// Parameters of a context (caller-owned device memory) as the backward sees them.
struct Model {
  rlt_config cfg;
  int dt;  // 0 = float32, 1 = bf16
  const float *s_star, *merge_norm, *merge_bg, *out_norm;
  const void *merge_wg, *merge_ws, *w_out;
  std::vector<const float*> norm_s, norm_m, norm_d;
  std::vector<const void*> wq, wk, wv, wo, wqm, wom, w_gate, w_up, w_down;
  const double* inv_freq;  // [d_head / 2] rotary frequencies
  int keep_acts;  // 0: keep every step's activations when they fit a quarter of the free device
                  // memory, else recompute them per step; 1: always recompute; 2: always keep
};

// The replay backward of rlt_replay_backward (validated arguments); returns
// an RLT_* code and, on failure, a message in err.
int replay_backward(const Model& m, const rlt_backward_io* io, const rlt_grads* gr, hipStream_t s, std::string& err);

}  // namespace bwd
}  // namespace rlt
