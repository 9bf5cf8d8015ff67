// Device-side bodies of the per-slot merge preparation and state
// write-back (one 256-thread block per slot); included by their stand-alone
// kernels and by the persistent step kernel.
#pragma once
#include "rlt_internal.h"

namespace rlt {

// gated: X = [e ; RMSNorm_s(s_{t-1})]  (eq. 2.10 input); convex: X = [e ; s].
// With a.pk (operand-order merge products) X is written in fragment order
// ([n][2d]) and, for the gated merge, RMSNorm_s(s_{t-1}) once more alone
// ([n][d], fragment order) to a.out2, the W_s product's input.
// A slot whose state row is named by more than one slot of the call
// (a.claim[row] > 1, counted by the pre-step) is skipped from here on:
// its t becomes 0 and the error word is set.
template <typename T>
__device__ __forceinline__ void merge_prep_body(const MiscArgs& a, int slot, float* scratch /* 16 */) {
  int t = a.rows.t_row[slot];
  if (t > 0 && a.claim && a.claim[a.rows.rows[slot]] > 1) {
    t = 0;
    __syncthreads();  // every thread has read t_row before it changes
    if (threadIdx.x == 0) {
      ((int*)a.rows.t_row)[slot] = 0;
      *(volatile int*)a.err = -1;  // RLT_EINVAL
    }
  }
  T* X = (T*)a.out + (a.pk ? 0 : (int64_t)slot * a.ld_out);
  T* X2 = (T*)a.out2;
  const int d = a.d, nc2 = (2 * d) >> 6, nc1 = d >> 6;
  // element c of the slot's X row (and of its r row)
  auto xi = [&](int c) -> int64_t { return a.pk ? pk_off(slot, c, nc2) : (int64_t)c; };
  auto ri = [&](int c) -> int64_t { return pk_off(slot, c, nc1); };
  const bool gated = a.merge_kind == 0;
  if (t <= 0) {
    for (int c = threadIdx.x; c < 2 * d; c += 256) store_op(X, xi(c), a.lo, 0.f);
    if (a.pk && gated)
      for (int c = threadIdx.x; c < d; c += 256) store_op(X2, ri(c), a.lo2, 0.f);
    return;
  }
  const float* s = a.s_state + (int64_t)a.rows.rows[slot] * d;
  const T* e = (const T*)a.e.p + (int64_t)a.rows.src[slot] * a.e.sb + (int64_t)(t - 1) * a.e.st;
  for (int c = threadIdx.x; c < d; c += 256) store_op(X, xi(c), a.lo, to_f<T>(e[c]));  // e is exact: no remainder
  if (gated) {
    float ss = 0.f;
    for (int c = threadIdx.x; c < d; c += 256) ss = fmaf(s[c], s[c], ss);
    ss = block_sum(ss, scratch);
    const float r = 1.0f / sqrtf(ss / (float)d + a.eps);
    for (int c = threadIdx.x; c < d; c += 256) {
      const float v = s[c] * r * a.gain[c];
      store_op(X, xi(d + c), a.lo, v);
      if (a.pk) store_op(X2, ri(c), a.lo2, v);
    }
    if (a.wg) {
      // scalar gate [text after eq. (2.11)]: g = sigmoid(w_g . [e; r] + b_g)
      // over the product input as the products see it (one rounded term, or
      // the float32 value the two terms carry), one value for every channel
      const T* wg = (const T*)a.wg;
      float dot = 0.f;
      for (int c = threadIdx.x; c < 2 * d; c += 256) {
        const float rv = c < d ? 0.f : s[c - d] * r * a.gain[c - d];
        const float x = c < d ? to_f<T>(e[c]) : (a.lo ? rv : to_f<T>(from_f<T>(rv)));
        dot = fmaf(to_f<T>(wg[c]), x, dot);
      }
      dot = block_sum(dot, scratch);
      const float g = 1.0f / (1.0f + __expf(-(dot + a.bg[0])));
      float* gb = a.gbuf + (int64_t)slot * d;
      for (int c = threadIdx.x; c < d; c += 256) gb[c] = g;
    }
  } else {
    for (int c = threadIdx.x; c < d; c += 256) store_op(X, xi(d + c), a.lo, s[c]);
  }
}

// s_t write-back to the state and the optional outputs (the readout's
// RMSNorm_o input was produced by the last block's down projection)
template <typename T>
__device__ __forceinline__ void final_body(const MiscArgs& a, int slot) {
  const int t = a.rows.t_row[slot];
  const float* z = a.z + (int64_t)slot * a.d;
  if (t <= 0) return;
  float* s = a.s_state + (int64_t)a.rows.rows[slot] * a.d;
  for (int c = threadIdx.x; c < a.d; c += 256) s[c] = z[c];
  if (a.s_out)
    for (int c = threadIdx.x; c < a.d; c += 256) a.s_out[(int64_t)slot * a.d + c] = z[c];
  if (a.s_trace) {
    float* st = a.s_trace + (int64_t)a.rows.src[slot] * a.s_trace_sb + (int64_t)(t - 1) * a.d;
    for (int c = threadIdx.x; c < a.d; c += 256) st[c] = z[c];
  }
}

}  // namespace rlt
