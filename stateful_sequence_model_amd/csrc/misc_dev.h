// Device-side bodies of the per-slot merge preparation and state
// write-back (one 256-thread block per slot); included by their stand-alone
// kernels and by the persistent step kernel.
#pragma once
#include "rlt_internal.h"

namespace rlt {

// gated: X = [e ; RMSNorm_s(s_{t-1})]  (eq. 2.10 input); convex: X = [e ; s]
template <typename T>
__device__ __forceinline__ void merge_prep_body(const MiscArgs& a, int slot, float* scratch /* 16 */) {
  const int t = a.rows.t_row[slot];
  T* X = (T*)a.out + (int64_t)slot * a.ld_out;
  if (t <= 0) {
    for (int c = threadIdx.x; c < 2 * a.d; c += 256) X[c] = from_f<T>(0.f);
    return;
  }
  const float* s = a.s_state + (int64_t)a.rows.rows[slot] * a.d;
  const T* e = (const T*)a.e.p + (int64_t)a.rows.src[slot] * a.e.sb + (int64_t)(t - 1) * a.e.st;
  for (int c = threadIdx.x; c < a.d; c += 256) X[c] = e[c];
  if (a.merge_kind == 0) {
    float ss = 0.f;
    for (int c = threadIdx.x; c < a.d; c += 256) ss = fmaf(s[c], s[c], ss);
    ss = block_sum(ss, scratch);
    const float r = 1.0f / sqrtf(ss / (float)a.d + a.eps);
    for (int c = threadIdx.x; c < a.d; c += 256) X[a.d + c] = from_f<T>(s[c] * r * a.gain[c]);
    if (a.wg) {
      // scalar gate [text after eq. (2.11)]: g = sigmoid(w_g . [e; r] + b_g)
      // over the product input as stored, one value for every channel
      const T* wg = (const T*)a.wg;
      float dot = 0.f;
      for (int c = threadIdx.x; c < 2 * a.d; c += 256) {
        const float x = c < a.d ? to_f<T>(e[c]) : to_f<T>(from_f<T>(s[c - a.d] * r * a.gain[c - a.d]));
        dot = fmaf(to_f<T>(wg[c]), x, dot);
      }
      dot = block_sum(dot, scratch);
      const float g = 1.0f / (1.0f + __expf(-(dot + a.bg[0])));
      float* gb = a.gbuf + (int64_t)slot * a.d;
      for (int c = threadIdx.x; c < a.d; c += 256) gb[c] = g;
    }
  } else {
    for (int c = threadIdx.x; c < a.d; c += 256) X[a.d + c] = from_f<T>(s[c]);
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
