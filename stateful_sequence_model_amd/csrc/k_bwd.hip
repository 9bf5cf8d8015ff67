// Kernels of the replay backward: the float32 transition with its
// activations kept, and the derivative of each of its operations
// ("Recurrent Looped Transformer" §2.5 eqs. (2.9)-(2.16), §2.3 eq. (2.6);
// full BPTT per §5.4 and App. B). Plain float32 arithmetic throughout; every
// sum runs in a fixed order (deterministic results).
#include <math.h>

#include "bwd.h"
#include "rlt_internal.h"

namespace rlt {
namespace bwd {
namespace {

template <typename T>
__device__ __forceinline__ float ld_f(const void* p, int64_t i) {
  return to_f<T>(((const T*)p)[i]);
}

__device__ __forceinline__ float ld_any(const void* p, int dt, int64_t i) {
  return dt ? ld_f<uint16_t>(p, i) : ld_f<float>(p, i);
}

// fixed-order tree sum over a 256-thread block (every thread gets the sum)
__device__ __forceinline__ float block_sum(float v, float* red) {
  red[threadIdx.x] = v;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  const float r = red[0];
  __syncthreads();
  return r;
}

__device__ __forceinline__ float block_max(float v, float* red) {
  red[threadIdx.x] = v;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] = fmaxf(red[threadIdx.x], red[threadIdx.x + w]);
    __syncthreads();
  }
  const float r = red[0];
  __syncthreads();
  return r;
}

__device__ __forceinline__ float sigm(float x) { return 1.0f / (1.0f + expf(-x)); }

// 16x16 output tile per 1024-thread block: 8 groups of 128 threads take the
// 16-wide K steps round-robin (group q: steps q, q + 8, ...), each thread
// summing two outputs over its group's steps in k order; the 8 partial sums
// are then added in group order. The unit-stride dimension of each operand
// runs along the fastest thread index when its tile is loaded; the next
// step's elements are loaded into registers while the current step is
// multiplied.
// Up to three products in one launch (MmSeg): segments with their own B
// operand and either their own output (sum = 0: blockIdx.z picks the
// segment) or their own A operand and one shared output that they are added
// into in segment order (sum = 1). Each segment's product is the k_mm sum
// above, so the results equal separate launches bit for bit.
struct MmSeg {
  const float* a[3];
  const void* b[3];
  float* c[3];
  int nseg, sum;
  const float* base;  // if set: the first segment starts from base (row stride c_si) instead of C or zero
};

template <typename TB>
__global__ __launch_bounds__(1024) void k_mm(int M, int N, int K, MmSeg sg, int64_t a_si, int64_t a_sk,
                                            int64_t b_sk, int64_t b_sj, int64_t c_si, int accumulate) {
  constexpr int KG = 8;
  __shared__ float As[KG][16][17], Bs[KG][16][17];
  __shared__ float red[KG - 1][256];
  const int q = threadIdx.x >> 7, t = threadIdx.x & 127;
  const int tx = t & 7, ty = t >> 3;  // outputs (ty, 2 tx) and (ty, 2 tx + 1)
  const int i0 = blockIdx.y * 16, j0 = blockIdx.x * 16;
  const bool a_k_fast = a_sk == 1, b_j_fast = b_sj == 1;
  const int seg0 = sg.sum ? 0 : blockIdx.z, seg1 = sg.sum ? sg.nseg : blockIdx.z + 1;
  float* c = sg.c[sg.sum ? 0 : blockIdx.z];
  float out0 = 0.f, out1 = 0.f;  // running output of the summed segments
  for (int sgi = seg0; sgi < seg1; ++sgi) {
    const float* a = sg.a[sgi];
    const TB* b = (const TB*)sg.b[sgi];
    // tile loads: element e = t + 128 h (h < 2) of a 16 x 16 tile, fastest index e % 16
    auto lda = [&](int k0, int h) {
      const int e = t + 128 * h, f = e & 15, o = e >> 4;
      const int i = i0 + (a_k_fast ? o : f), k = k0 + (a_k_fast ? f : o);
      return (i < M && k < K) ? a[(int64_t)i * a_si + (int64_t)k * a_sk] : 0.f;
    };
    auto ldb = [&](int k0, int h) {
      const int e = t + 128 * h, f = e & 15, o = e >> 4;
      const int k = k0 + (b_j_fast ? o : f), j = j0 + (b_j_fast ? f : o);
      return (k < K && j < N) ? to_f<TB>(b[(int64_t)k * b_sk + (int64_t)j * b_sj]) : 0.f;
    };
    auto sta = [&](int h, float v) {
      const int e = t + 128 * h, f = e & 15, o = e >> 4;
      if (a_k_fast) As[q][o][f] = v;
      else As[q][f][o] = v;
    };
    auto stb = [&](int h, float v) {
      const int e = t + 128 * h, f = e & 15, o = e >> 4;
      if (b_j_fast) Bs[q][o][f] = v;
      else Bs[q][f][o] = v;
    };
    const int nst = (K + 15) / 16;
    const int steps = (nst + KG - 1) / KG;  // the same trip count in every group (barriers)
    float acc0 = 0.f, acc1 = 0.f;
    float an0 = lda(16 * q, 0), an1 = lda(16 * q, 1), bn0 = ldb(16 * q, 0), bn1 = ldb(16 * q, 1);
    for (int s = 0; s < steps; ++s) {
      const int k0 = 16 * (q + KG * s);
      sta(0, an0);
      sta(1, an1);
      stb(0, bn0);
      stb(1, bn1);
      __syncthreads();
      if (s + 1 < steps) {
        an0 = lda(k0 + 16 * KG, 0);
        an1 = lda(k0 + 16 * KG, 1);
        bn0 = ldb(k0 + 16 * KG, 0);
        bn1 = ldb(k0 + 16 * KG, 1);
      }
      if (k0 < K) {
#pragma unroll
        for (int kk = 0; kk < 16; ++kk) {
          const float av = As[q][ty][kk];
          acc0 = fmaf(av, Bs[q][kk][2 * tx], acc0);
          acc1 = fmaf(av, Bs[q][kk][2 * tx + 1], acc1);
        }
      }
      __syncthreads();
    }
    if (q > 0) {
      red[q - 1][2 * t] = acc0;
      red[q - 1][2 * t + 1] = acc1;
    }
    __syncthreads();
    if (q == 0) {
#pragma unroll
      for (int g = 0; g < KG - 1; ++g) {
        acc0 += red[g][2 * t];
        acc1 += red[g][2 * t + 1];
      }
      const int i = i0 + ty, j = j0 + 2 * tx;
      if (i < M) {
        const float* p = (sg.base ? sg.base : c) + (int64_t)i * c_si + j;
        const bool first = sgi == seg0, from = accumulate || sg.base;
        // the first segment starts from the output (accumulate), the base or
        // zero; later ones add to the running value
        if (j < N) out0 = first ? (from ? p[0] + acc0 : acc0) : out0 + acc0;
        if (j + 1 < N) out1 = first ? (from ? p[1] + acc1 : acc1) : out1 + acc1;
      }
    }
    __syncthreads();  // red is reused by the next segment
  }
  if (q == 0) {
    const int i = i0 + ty, j = j0 + 2 * tx;
    if (i < M) {
      float* p = c + (int64_t)i * c_si + j;
      if (j < N) p[0] = out0;
      if (j + 1 < N) p[1] = out1;
    }
  }
}

// block per row
__global__ __launch_bounds__(256) void k_rms_fwd(const float* x, int64_t ldx, const float* gain, float* y,
                                                int64_t ldy, float* rstd, int d, float eps) {
  __shared__ float red[256];
  const int r = blockIdx.x;
  const float* xr = x + (int64_t)r * ldx;
  float ss = 0.f;
  for (int c = threadIdx.x; c < d; c += 256) ss += xr[c] * xr[c];
  const float rs = 1.0f / sqrtf(block_sum(ss, red) / (float)d + eps);
  for (int c = threadIdx.x; c < d; c += 256) y[(int64_t)r * ldy + c] = xr[c] * rs * gain[c];
  if (threadIdx.x == 0) rstd[r] = rs;
}

// y = x * rs * g: dx_c = rs g_c dy_c - x_c rs^3 (1/d) sum_j x_j g_j dy_j,
// stored as v, dx + v (accumulate) or base + v (base given)
__global__ __launch_bounds__(256) void k_rms_bwd(const float* x, int64_t ldx, const float* gain, const float* rstd,
                                                const float* dy, int64_t ldy, float* dx, int64_t lddx, int d,
                                                int accumulate, const float* base, int64_t ldb) {
  __shared__ float red[256];
  const int r = blockIdx.x;
  const float* xr = x + (int64_t)r * ldx;
  const float* dyr = dy + (int64_t)r * ldy;
  float dot = 0.f;
  for (int c = threadIdx.x; c < d; c += 256) dot += xr[c] * gain[c] * dyr[c];
  dot = block_sum(dot, red);
  const float rs = rstd[r];
  const float k = rs * rs * rs * dot / (float)d;
  for (int c = threadIdx.x; c < d; c += 256) {
    const float v = rs * gain[c] * dyr[c] - xr[c] * k;
    float* p = dx + (int64_t)r * lddx + c;
    *p = base ? base[(int64_t)r * ldb + c] + v : accumulate ? *p + v : v;
  }
}

// thread per column, rows in order
__global__ __launch_bounds__(256) void k_colsum(float* dst, const float* a, int64_t lda, const float* b, int64_t ldb,
                                               const float* rs, int n, int d) {
  const int c = blockIdx.x * 256 + threadIdx.x;
  if (c >= d) return;
  float acc = 0.f;
  for (int r = 0; r < n; ++r) {
    float v = a[(int64_t)r * lda + c];
    if (b) v *= b[(int64_t)r * ldb + c];
    if (rs) v *= rs[r];
    acc += v;
  }
  dst[c] += acc;
}

// thread per (row, head, i < dh/2): rotate (x_i, x_{i+dh/2}) by sign * t * w_i
// blockIdx.y selects x (0) or x2 (1): two arrays of one position in one launch
__global__ __launch_bounds__(256) void k_rope(float* x, float* x2, int64_t ld, int n, int d, int dh, int t,
                                             const double* inv_freq, int sign) {
  if (blockIdx.y) x = x2;
  const int half = dh / 2;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (int64_t)n * (d / 2)) return;
  const int r = (int)(idx / (d / 2)), q = (int)(idx % (d / 2));
  const int h = q / half, i = q % half;
  double sn, cs;
  sincos((double)t * inv_freq[i], &sn, &cs);
  const float c = (float)cs, s = (float)sn * (float)sign;
  float* p = x + (int64_t)r * ld + h * dh;
  const float a = p[i], b = p[i + half];
  p[i] = a * c - b * s;
  p[i + half] = b * c + a * s;
}

// block per (row, head); scores of all keys in dynamic LDS
// sum over keys j < nk of w[j] * x_j[c] for c < dh (dh divides 256), by all
// 256 threads: 256 / dh groups take keys round-robin, the group partials are
// then added in group order; the result is returned on threads c < dh.
// Contains one barrier (part: 256 floats of LDS).
template <typename TK>
__device__ __forceinline__ float key_wsum(const float* w, const void* x, int64_t row_off, int lo, int nk, int64_t s_pos,
                                          int dh, float* part) {
  const int G = 256 / dh, c = threadIdx.x % dh, g = threadIdx.x / dh;
  float acc = 0.f;
  for (int j = g; j < nk; j += G) acc = fmaf(w[j], ld_f<TK>(x, row_off + (int64_t)(lo + j - 1) * s_pos + c), acc);
  part[threadIdx.x] = acc;
  __syncthreads();
  float sum = 0.f;
  if (threadIdx.x < dh)
    for (int q = 0; q < G; ++q) sum += part[q * dh + c];
  return sum;
}

template <typename TK>
__global__ __launch_bounds__(256) void k_attn_fwd(const float* q, int64_t ldq, KV kv, int lo, int hi, float* o,
                                                 int64_t ldo, int H, int dh) {
  extern __shared__ float sc[];  // [nk] scores, then [dh] query
  __shared__ float red[256];
  const int r = blockIdx.x / H, h = blockIdx.x % H;
  const int nk = hi - lo + 1;
  float* qs = sc + nk;
  const float scale = 1.0f / sqrtf((float)dh);
  for (int c = threadIdx.x; c < dh; c += 256) qs[c] = q[(int64_t)r * ldq + h * dh + c];
  __syncthreads();
  const int64_t row_off = (int64_t)(kv.map ? kv.map[r] : r) * kv.s_row + h * dh;
  float mx = -INFINITY;
  for (int j = threadIdx.x; j < nk; j += 256) {
    const int64_t base = row_off + (int64_t)(lo + j - 1) * kv.s_pos;
    float acc = 0.f;
    for (int c = 0; c < dh; ++c) acc = fmaf(qs[c], ld_f<TK>(kv.k, base + c), acc);
    sc[j] = acc * scale;
    mx = fmaxf(mx, sc[j]);
  }
  mx = block_max(mx, red);
  float sum = 0.f;
  for (int j = threadIdx.x; j < nk; j += 256) {
    sc[j] = expf(sc[j] - mx);
    sum += sc[j];
  }
  sum = block_sum(sum, red);  // contains barriers: scores are visible below
  const float inv = 1.0f / sum;
  __shared__ float part[256];
  const float acc = key_wsum<TK>(sc, kv.v, row_off, lo, nk, kv.s_pos, dh, part);
  if (threadIdx.x < dh) o[(int64_t)r * ldo + h * dh + threadIdx.x] = acc * inv;
}

// p_j = softmax(s)_j; dv_j = p_j do; dp_j = do . v_j; ds_j = p_j (dp_j - sum_i p_i dp_i);
// dq = scale sum_j ds_j k_j; dk_j = scale ds_j q
template <typename TK>
__global__ __launch_bounds__(256) void k_attn_bwd(const float* q, int64_t ldq, KV kv, int lo, int hi,
                                                 const float* dout, int64_t lddo, float* dq, int64_t lddq, DKV dkv,
                                                 int H, int dh) {
  extern __shared__ float sc[];  // [nk] p, [nk] ds, [dh] q, [dh] do
  __shared__ float red[256];
  const int r = blockIdx.x / H, h = blockIdx.x % H;
  const int nk = hi - lo + 1;
  float* ds = sc + nk;
  float* qs = ds + nk;
  float* dos = qs + dh;
  const float scale = 1.0f / sqrtf((float)dh);
  for (int c = threadIdx.x; c < dh; c += 256) {
    qs[c] = q[(int64_t)r * ldq + h * dh + c];
    dos[c] = dout[(int64_t)r * lddo + h * dh + c];
  }
  __syncthreads();
  const int64_t row_off = (int64_t)(kv.map ? kv.map[r] : r) * kv.s_row + h * dh;
  float mx = -INFINITY;
  for (int j = threadIdx.x; j < nk; j += 256) {
    const int64_t base = row_off + (int64_t)(lo + j - 1) * kv.s_pos;
    float acc = 0.f;
    for (int c = 0; c < dh; ++c) acc = fmaf(qs[c], ld_f<TK>(kv.k, base + c), acc);
    sc[j] = acc * scale;
    mx = fmaxf(mx, sc[j]);
  }
  mx = block_max(mx, red);
  float sum = 0.f;
  for (int j = threadIdx.x; j < nk; j += 256) {
    sc[j] = expf(sc[j] - mx);
    sum += sc[j];
  }
  sum = block_sum(sum, red);
  const float inv = 1.0f / sum;
  float dsum = 0.f;
  for (int j = threadIdx.x; j < nk; j += 256) {
    const int64_t base = row_off + (int64_t)(lo + j - 1) * kv.s_pos;
    sc[j] *= inv;
    float dp = 0.f;
    for (int c = 0; c < dh; ++c) dp = fmaf(dos[c], ld_f<TK>(kv.v, base + c), dp);
    ds[j] = dp;
    dsum += sc[j] * dp;
  }
  dsum = block_sum(dsum, red);
  for (int j = threadIdx.x; j < nk; j += 256) ds[j] = sc[j] * (ds[j] - dsum);
  __syncthreads();
  __shared__ float part[256];
  const float acc = key_wsum<TK>(ds, kv.k, row_off, lo, nk, kv.s_pos, dh, part);
  if (threadIdx.x < dh) dq[(int64_t)r * lddq + h * dh + threadIdx.x] = acc * scale;
  if (!dkv.k) return;
  const int64_t drow = (int64_t)(dkv.map ? dkv.map[r] : r) * dkv.s_row + h * dh;
  for (int64_t idx = threadIdx.x; idx < (int64_t)nk * dh; idx += 256) {
    const int j = (int)(idx / dh), c = (int)(idx % dh);
    const int64_t o = drow + (int64_t)(lo + j - 1) * dkv.s_pos + c;
    dkv.k[o] += scale * ds[j] * qs[c];
    dkv.v[o] += sc[j] * dos[c];
  }
}

template <typename T>
__global__ __launch_bounds__(256) void k_gather_e(float* x, int64_t ldx, const T* e, int64_t sb, int64_t st,
                                                 const int* map, int t, int n, int d) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (int64_t)n * d) return;
  const int r = (int)(idx / d), c = (int)(idx % d);
  x[(int64_t)r * ldx + c] = to_f<T>(e[(int64_t)map[r] * sb + (int64_t)(t - 1) * st + c]);
}

__global__ __launch_bounds__(256) void k_scatter_add_e(float* de, int64_t sb, int64_t st, const float* g, int64_t ldg,
                                                      const int* map, int t, int n, int d) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (int64_t)n * d) return;
  const int r = (int)(idx / d), c = (int)(idx % d);
  de[(int64_t)map[r] * sb + (int64_t)(t - 1) * st + c] += g[(int64_t)r * ldg + c];
}

__global__ __launch_bounds__(256) void k_sigmoid_bias(float* g, int64_t ld, const float* bias, int n, int d) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (int64_t)n * d) return;
  const int r = (int)(idx / d), c = (int)(idx % d);
  float* p = g + (int64_t)r * ld + c;
  *p = sigm(*p + bias[c]);
}

__global__ __launch_bounds__(256) void k_merge_fwd(int gated, float* u, const float* e, int64_t lde, const float* g,
                                                  const float* w, int64_t ldw, float alpha, int n, int d) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (int64_t)n * d) return;
  const int r = (int)(idx / d), c = (int)(idx % d);
  const float ev = e[(int64_t)r * lde + c], gv = g[idx], wv = w[(int64_t)r * ldw + c];
  u[idx] = gated ? ev + alpha * gv * wv : gv * ev + (1.0f - gv) * wv;
}

__global__ __launch_bounds__(256) void k_merge_bwd(int gated, const float* du, const float* e, int64_t lde,
                                                  const float* g, const float* w, int64_t ldw, float alpha, float* dpre,
                                                  float* dw, float* de, int64_t ldde, int n, int d) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (int64_t)n * d) return;
  const int r = (int)(idx / d), c = (int)(idx % d);
  const float duv = du[idx], ev = e[(int64_t)r * lde + c], gv = g[idx], wv = w[(int64_t)r * ldw + c];
  const float gp = gv * (1.0f - gv);
  if (gated) {
    dpre[idx] = alpha * duv * wv * gp;
    dw[idx] = alpha * gv * duv;
    de[(int64_t)r * ldde + c] = duv;
  } else {
    dpre[idx] = duv * (ev - wv) * gp;
    dw[idx] = duv * (1.0f - gv);
    de[(int64_t)r * ldde + c] = duv * gv;
  }
}

__global__ __launch_bounds__(256) void k_swiglu_fwd(const float* a, const float* u, float* act, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  act[i] = a[i] * sigm(a[i]) * u[i];
}

__global__ __launch_bounds__(256) void k_swiglu_bwd(const float* a, const float* u, const float* dact, float* da,
                                                   float* du, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  const float s = sigm(a[i]);
  da[i] = dact[i] * u[i] * s * (1.0f + a[i] * (1.0f - s));
  du[i] = dact[i] * a[i] * s;
}

// block per row
__global__ __launch_bounds__(256) void k_logsoftmax_bwd(const float* logits, int V, const int* tokens, int64_t tok_sb,
                                                       const float* w, int64_t w_sb, const int* map, const int* split,
                                                       int t, float* logp, int64_t logp_sb, float* dlogits) {
  __shared__ float red[256];
  const int r = blockIdx.x;
  const int b = map[r];
  const float* z = logits + (int64_t)r * V;
  float* dz = dlogits + (int64_t)r * V;
  if (t < split[r]) {
    for (int c = threadIdx.x; c < V; c += 256) dz[c] = 0.f;
    return;
  }
  float mx = -INFINITY;
  for (int c = threadIdx.x; c < V; c += 256) mx = fmaxf(mx, z[c]);
  mx = block_max(mx, red);
  float s = 0.f;
  for (int c = threadIdx.x; c < V; c += 256) s += expf(z[c] - mx);
  s = block_sum(s, red);
  const float lse = mx + logf(s);
  const int tok = tokens[(int64_t)b * tok_sb + t];
  const float wt = w[(int64_t)b * w_sb + t];
  for (int c = threadIdx.x; c < V; c += 256) dz[c] = wt * ((c == tok ? 1.0f : 0.0f) - expf(z[c] - lse));
  if (threadIdx.x == 0 && logp) logp[(int64_t)b * logp_sb + t] = z[tok] - lse;
}

__global__ __launch_bounds__(256) void k_add(float* y, int64_t ldy, const float* a, int64_t lda, const float* b,
                                            int64_t ldb, int n, int d) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (int64_t)n * d) return;
  const int r = (int)(idx / d), c = (int)(idx % d);
  y[(int64_t)r * ldy + c] = a[(int64_t)r * lda + c] + (b ? b[(int64_t)r * ldb + c] : 0.f);
}

// the column sums of k_colsum over many rows: 16 columns per block, row lane
// q (of 16) sums rows q, q + 16, ... in order, then the lanes' sums are
// added in lane order
__global__ __launch_bounds__(256) void k_colsum_rows(float* dst, const float* a, int64_t lda, const float* b,
                                                    int64_t ldb, const float* rs, int64_t n, int d) {
  __shared__ float part[16][17];
  const int cx = threadIdx.x & 15, q = threadIdx.x >> 4;
  const int c = blockIdx.x * 16 + cx;
  float acc = 0.f;
  if (c < d) {
    for (int64_t r = q; r < n; r += 16) {
      float v = a[r * lda + c];
      if (b) v *= b[r * ldb + c];
      if (rs) v *= rs[r];
      acc += v;
    }
  }
  part[q][cx] = acc;
  __syncthreads();
  if (q == 0 && c < d) {
    float sum = part[0][cx];
    for (int k = 1; k < 16; ++k) sum += part[k][cx];
    dst[c] += sum;
  }
}

inline unsigned nblk(int64_t n) { return (unsigned)((n + 255) / 256); }

}  // namespace

static void mm_launch(int M, int N, int K, const MmSeg& sg, int64_t a_si, int64_t a_sk, int bdt, int64_t b_sk,
                      int64_t b_sj, int64_t c_si, bool accumulate, hipStream_t s) {
  if (M <= 0 || N <= 0 || sg.nseg <= 0) return;
  dim3 grid((N + 15) / 16, (M + 15) / 16, sg.sum ? 1 : sg.nseg);
  if (bdt)
    hipLaunchKernelGGL(k_mm<uint16_t>, grid, dim3(1024), 0, s, M, N, K, sg, a_si, a_sk, b_sk, b_sj, c_si,
                       (int)accumulate);
  else
    hipLaunchKernelGGL(k_mm<float>, grid, dim3(1024), 0, s, M, N, K, sg, a_si, a_sk, b_sk, b_sj, c_si,
                       (int)accumulate);
}

void mm(int M, int N, int K, const float* a, int64_t a_si, int64_t a_sk, const void* b, int bdt, int64_t b_sk,
        int64_t b_sj, float* c, int64_t c_si, bool accumulate, hipStream_t s) {
  MmSeg sg{};
  sg.a[0] = a;
  sg.b[0] = b;
  sg.c[0] = c;
  sg.nseg = 1;
  mm_launch(M, N, K, sg, a_si, a_sk, bdt, b_sk, b_sj, c_si, accumulate, s);
}

void mm_base(int M, int N, int K, const float* a, int64_t a_si, int64_t a_sk, const void* b, int bdt, int64_t b_sk,
             int64_t b_sj, const float* base, float* c, int64_t c_si, hipStream_t s) {
  MmSeg sg{};
  sg.a[0] = a;
  sg.b[0] = b;
  sg.c[0] = c;
  sg.nseg = 1;
  sg.base = base;
  mm_launch(M, N, K, sg, a_si, a_sk, bdt, b_sk, b_sj, c_si, false, s);
}

void mm_outputs(int nseg, int M, int N, int K, const float* a, int64_t a_si, int64_t a_sk, const void* const* b,
                int bdt, int64_t b_sk, int64_t b_sj, float* const* c, int64_t c_si, bool accumulate, hipStream_t s) {
  MmSeg sg{};
  for (int i = 0; i < nseg && i < 3; ++i) {
    sg.a[i] = a;
    sg.b[i] = b[i];
    sg.c[i] = c[i];
  }
  sg.nseg = nseg < 3 ? nseg : 3;
  mm_launch(M, N, K, sg, a_si, a_sk, bdt, b_sk, b_sj, c_si, accumulate, s);
}

void mm_summed(int nseg, int M, int N, int K, const float* const* a, int64_t a_si, int64_t a_sk,
               const void* const* b, int bdt, int64_t b_sk, int64_t b_sj, float* c, int64_t c_si, bool accumulate,
               hipStream_t s) {
  MmSeg sg{};
  for (int i = 0; i < nseg && i < 3; ++i) {
    sg.a[i] = a[i];
    sg.b[i] = b[i];
  }
  sg.c[0] = c;
  sg.nseg = nseg < 3 ? nseg : 3;
  sg.sum = 1;
  mm_launch(M, N, K, sg, a_si, a_sk, bdt, b_sk, b_sj, c_si, accumulate, s);
}

void rms_fwd(const float* x, int64_t ldx, const float* gain, float* y, int64_t ldy, float* rstd, int n, int d,
             float eps, hipStream_t s) {
  if (n > 0) hipLaunchKernelGGL(k_rms_fwd, dim3(n), dim3(256), 0, s, x, ldx, gain, y, ldy, rstd, d, eps);
}

void rms_bwd(const float* x, int64_t ldx, const float* gain, const float* rstd, const float* dy, int64_t ldy,
             float* dx, int64_t lddx, int n, int d, bool accumulate, hipStream_t s, const float* base, int64_t ldb) {
  if (n > 0)
    hipLaunchKernelGGL(k_rms_bwd, dim3(n), dim3(256), 0, s, x, ldx, gain, rstd, dy, ldy, dx, lddx, d, (int)accumulate,
                       base, ldb);
}

void colsum(float* dst, const float* a, int64_t lda, const float* b, int64_t ldb, const float* rs, int n, int d,
            hipStream_t s) {
  if (n > 0 && dst) hipLaunchKernelGGL(k_colsum, dim3(nblk(d)), dim3(256), 0, s, dst, a, lda, b, ldb, rs, n, d);
}

void colsum_rows(float* dst, const float* a, int64_t lda, const float* b, int64_t ldb, const float* rs, int64_t n,
                 int d, hipStream_t s) {
  if (n > 0 && dst)
    hipLaunchKernelGGL(k_colsum_rows, dim3((d + 15) / 16), dim3(256), 0, s, dst, a, lda, b, ldb, rs, n, d);
}

void rope(float* x, int64_t ld, int n, int d, int dh, int t, const double* inv_freq, int sign, hipStream_t s) {
  if (n > 0)
    hipLaunchKernelGGL(k_rope, dim3(nblk((int64_t)n * (d / 2))), dim3(256), 0, s, x, x, ld, n, d, dh, t, inv_freq, sign);
}

void rope2(float* x, float* x2, int64_t ld, int n, int d, int dh, int t, const double* inv_freq, int sign,
           hipStream_t s) {
  if (n > 0)
    hipLaunchKernelGGL(k_rope, dim3(nblk((int64_t)n * (d / 2)), 2), dim3(256), 0, s, x, x2, ld, n, d, dh, t, inv_freq,
                       sign);
}

void attn_fwd(const float* q, int64_t ldq, KV kv, int lo, int hi, float* o, int64_t ldo, int n, int H, int dh,
              hipStream_t s) {
  if (n <= 0) return;
  const size_t lds = (size_t)(hi - lo + 1 + dh) * sizeof(float);
  if (kv.dt)
    hipLaunchKernelGGL(k_attn_fwd<uint16_t>, dim3(n * H), dim3(256), lds, s, q, ldq, kv, lo, hi, o, ldo, H, dh);
  else
    hipLaunchKernelGGL(k_attn_fwd<float>, dim3(n * H), dim3(256), lds, s, q, ldq, kv, lo, hi, o, ldo, H, dh);
}

void attn_bwd(const float* q, int64_t ldq, KV kv, int lo, int hi, const float* dout, int64_t lddo, float* dq,
              int64_t lddq, DKV dkv, int n, int H, int dh, hipStream_t s) {
  if (n <= 0) return;
  const size_t lds = (size_t)(2 * (hi - lo + 1) + 2 * dh) * sizeof(float);
  if (kv.dt)
    hipLaunchKernelGGL(k_attn_bwd<uint16_t>, dim3(n * H), dim3(256), lds, s, q, ldq, kv, lo, hi, dout, lddo, dq, lddq,
                       dkv, H, dh);
  else
    hipLaunchKernelGGL(k_attn_bwd<float>, dim3(n * H), dim3(256), lds, s, q, ldq, kv, lo, hi, dout, lddo, dq, lddq,
                       dkv, H, dh);
}

void gather_e(float* x, int64_t ldx, const void* e, int dt, int64_t sb, int64_t st, const int* map, int t, int n,
              int d, hipStream_t s) {
  if (n <= 0) return;
  if (dt)
    hipLaunchKernelGGL(k_gather_e<uint16_t>, dim3(nblk((int64_t)n * d)), dim3(256), 0, s, x, ldx, (const uint16_t*)e,
                       sb, st, map, t, n, d);
  else
    hipLaunchKernelGGL(k_gather_e<float>, dim3(nblk((int64_t)n * d)), dim3(256), 0, s, x, ldx, (const float*)e, sb,
                       st, map, t, n, d);
}

void scatter_add_e(float* de, int64_t sb, int64_t st, const float* g, int64_t ldg, const int* map, int t, int n,
                   int d, hipStream_t s) {
  if (n > 0 && de)
    hipLaunchKernelGGL(k_scatter_add_e, dim3(nblk((int64_t)n * d)), dim3(256), 0, s, de, sb, st, g, ldg, map, t, n, d);
}

void sigmoid_bias(float* g, int64_t ld, const float* bias, int n, int d, hipStream_t s) {
  if (n > 0) hipLaunchKernelGGL(k_sigmoid_bias, dim3(nblk((int64_t)n * d)), dim3(256), 0, s, g, ld, bias, n, d);
}

void merge_fwd(int gated, float* u, const float* e, int64_t lde, const float* g, const float* w, int64_t ldw,
               float alpha, int n, int d, hipStream_t s) {
  if (n > 0)
    hipLaunchKernelGGL(k_merge_fwd, dim3(nblk((int64_t)n * d)), dim3(256), 0, s, gated, u, e, lde, g, w, ldw, alpha, n, d);
}

void merge_bwd(int gated, const float* du, const float* e, int64_t lde, const float* g, const float* w, int64_t ldw,
               float alpha, float* dpre, float* dw, float* de, int64_t ldde, int n, int d, hipStream_t s) {
  if (n > 0)
    hipLaunchKernelGGL(k_merge_bwd, dim3(nblk((int64_t)n * d)), dim3(256), 0, s, gated, du, e, lde, g, w, ldw, alpha,
                       dpre, dw, de, ldde, n, d);
}

void swiglu_fwd(const float* a, const float* u, float* act, int n, int F, hipStream_t s) {
  const int64_t m = (int64_t)n * F;
  if (m > 0) hipLaunchKernelGGL(k_swiglu_fwd, dim3(nblk(m)), dim3(256), 0, s, a, u, act, m);
}

void swiglu_bwd(const float* a, const float* u, const float* dact, float* da, float* du, int n, int F,
                hipStream_t s) {
  const int64_t m = (int64_t)n * F;
  if (m > 0) hipLaunchKernelGGL(k_swiglu_bwd, dim3(nblk(m)), dim3(256), 0, s, a, u, dact, da, du, m);
}

void logsoftmax_bwd(const float* logits, int V, const int* tokens, int64_t tok_sb, const float* w, int64_t w_sb,
                    const int* map, const int* split, int t, float* logp, int64_t logp_sb, float* dlogits, int n,
                    hipStream_t s) {
  if (n > 0)
    hipLaunchKernelGGL(k_logsoftmax_bwd, dim3(n), dim3(256), 0, s, logits, V, tokens, tok_sb, w, w_sb, map, split, t,
                       logp, logp_sb, dlogits);
}

void add(float* y, int64_t ldy, const float* a, int64_t lda, const float* b, int64_t ldb, int n, int d,
         hipStream_t s) {
  if (n > 0) hipLaunchKernelGGL(k_add, dim3(nblk((int64_t)n * d)), dim3(256), 0, s, y, ldy, a, lda, b, ldb, n, d);
}

}  // namespace bwd
}  // namespace rlt
