// Row bookkeeping, normalisation, merge preparation, state write-back and
// readout ("Recurrent Looped Transformer", §2.3 eqs. (2.3)-(2.6), §2.5
// eqs. (2.9)-(2.11), §5.3, App. A.2).
#include "misc_dev.h"

namespace rlt {

static constexpr int ERR_PREFIX = -3;   // RLT_EPREFIX
static constexpr int ERR_PENDING = -5;  // RLT_EPENDING
static constexpr int ERR_INVAL = -1;    // RLT_EINVAL

// ---------------------------------------------------------------------------
// bookkeeping
// ---------------------------------------------------------------------------

// t = pos + 1 per slot; rows whose memory is shorter than t, or whose
// consumed token differs from a recorded pending token, get t = 0 (skipped)
// and raise the error word. Each slot also counts its row in a.claim (zero
// between calls): the merge preparation skips rows counted more than once.
__global__ void k_prestep(MiscArgs a) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= a.n) return;
  const int row = a.rows.rows[i];
  if (row < 0 || row >= a.B_cap) {
    a.t_row_out[i] = 0;
    *(volatile int*)a.err = ERR_INVAL;
    return;
  }
  if (a.claim) atomicAdd(a.claim + row, 1);
  const int t = a.pos[row] + 1;
  int code = 0;
  if (t > a.max_t || (a.mem_len && t > a.mem_len[row])) code = ERR_PREFIX;
  if (a.consume_tok && a.pending[row] >= 0 && a.consume_tok[i] != a.pending[row]) code = ERR_PENDING;
  a.t_row_out[i] = code ? 0 : t;
  if (code) *(volatile int*)a.err = code;
}

// replay tick: every active slot is at position `tick`
// tick: the replay's current position, on the device (advanced by the
// post-step of each tick), so that the launches of a tick do not depend on it
__global__ void k_replay_rows(const int* rows, int n, const int* tick_dev, int* t_row, const int* pos,
                              const int* mem_len, int* err) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const int tick = *tick_dev;
  const int row = rows[i];
  int code = 0;
  if (pos[row] + 1 != tick) code = ERR_PENDING;
  if (mem_len && tick > mem_len[row]) code = ERR_PREFIX;
  t_row[i] = code ? 0 : tick;
  if (code) *(volatile int*)err = code;
}

__global__ void k_poststep(PostArgs a) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (a.tick && i == 0) *a.tick += 1;  // replay: the next tick (read by the next tick's kernels only)
  if (i >= a.n) return;
  const int row = a.rows.rows[i];
  if (a.claim && row >= 0 && row < a.B_cap) a.claim[row] = 0;  // ready for the next call
  const int t = a.rows.t_row[i];
  if (t <= 0) return;
  a.pos[row] = t;
  a.pending[row] = a.next_tok ? a.next_tok[i] : -1;
}

template <typename T>
__global__ void k_init(const int* rows, int n, const float* s_star, float* s, int* pos, int* pending,
                       T* ring_k, T* ring_v, int L, int B_cap, int W1, int d, int poison) {
  const int i = blockIdx.x;
  if (i >= n) return;
  const int row = rows[i];
  if (row < 0 || row >= B_cap) return;
  for (int c = threadIdx.x; c < d; c += blockDim.x) s[(int64_t)row * d + c] = s_star[c];
  if (threadIdx.x == 0) {
    pos[row] = 0;
    pending[row] = -1;
  }
  if (poison && W1 > 0) {
    const T nanv = from_f<T>(__uint_as_float(0x7fc00000u));
    for (int l = 0; l < L; ++l) {
      const int64_t base = ((int64_t)l * B_cap + row) * W1 * d;
      for (int64_t c = threadIdx.x; c < (int64_t)W1 * d; c += blockDim.x) {
        ring_k[base + c] = nanv;
        ring_v[base + c] = nanv;
      }
    }
  }
}

// pending[row] = x_len after a replay (the scored but unconsumed token)
__global__ void k_set_pending(const int* rows, const int* src, int n, const int* tokens, int64_t tok_sb,
                              const int* last_index, int* pending) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const int b = src[i];
  pending[rows[i]] = tokens[(int64_t)b * tok_sb + last_index[b]];
}

// ---------------------------------------------------------------------------
// normalisation and merge preparation (one workgroup per slot)
// ---------------------------------------------------------------------------

// RMSNorm(x) = x / sqrt(mean(x^2) + eps) * gain
template <typename T>
__global__ __launch_bounds__(256) void k_rmsnorm(MiscArgs a) {
  __shared__ float scratch[16];
  const int slot = blockIdx.x;
  const float* z = a.z + (int64_t)slot * a.d;
  float ss = 0.f;
  for (int c = threadIdx.x; c < a.d; c += 256) ss = fmaf(z[c], z[c], ss);
  ss = block_sum(ss, scratch);
  const float r = 1.0f / sqrtf(ss / (float)a.d + a.eps);
  T* out = (T*)a.out + (int64_t)slot * a.ld_out;
  for (int c = threadIdx.x; c < a.d; c += 256) out[c] = from_f<T>(z[c] * r * a.gain[c]);
}

template <typename T>
__global__ __launch_bounds__(256) void k_merge_prep(MiscArgs a) {
  __shared__ float scratch[16];
  merge_prep_body<T>(a, blockIdx.x, scratch);
}

template <typename T>
__global__ __launch_bounds__(256) void k_final(MiscArgs a) {
  final_body<T>(a, blockIdx.x);
}

__global__ void k_copy_f32(const float* src, float* dst, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) dst[i] = src[i];
}

// ---------------------------------------------------------------------------
// encoder memory entries [RLT §2.2, eq. (2.2)]
// ---------------------------------------------------------------------------

// append: slot i writes position mem_len[rows[i]] + 1 (0 = skip: bad row or full)
__global__ void k_mem_slots(const int* rows, int n, const int* mem_len, int B_cap, int T_cap, int* t_out, int* err) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const int row = rows[i];
  if (row < 0 || row >= B_cap) {
    t_out[i] = 0;
    *(volatile int*)err = ERR_INVAL;
    return;
  }
  const int t = mem_len[row] + 1;
  if (t > T_cap) {
    t_out[i] = 0;
    *(volatile int*)err = ERR_PREFIX;
    return;
  }
  t_out[i] = t;
}

// prefill: flattened entry r0 + i -> (sequence b, position t) with
// offs[b] <= r0 + i < offs[b + 1] (offs: prefix sums of the lengths)
__global__ void k_mem_rows(const int* offs, int B, int64_t r0, int n, int* src_out, int* t_out) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const int64_t g = r0 + i;
  int lo = 0, hi = B;  // largest b with offs[b] <= g
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (offs[mid] <= g) lo = mid;
    else hi = mid;
  }
  src_out[i] = lo;
  t_out[i] = (int)(g - offs[lo]) + 1;
}

// one workgroup per slot: the product input e * gain (the consumer applies
// 1/sqrt(mean(e^2) + eps)) and the sum of squares of e
template <typename T>
__global__ __launch_bounds__(256) void k_mem_prep(Rows rows, EIn e, int d, const float* gain, T* A, float* ssq) {
  __shared__ float scratch[16];
  const int slot = blockIdx.x;
  const int t = rows.t_row[slot];
  T* out = A + (int64_t)slot * d;
  if (t <= 0) {
    for (int c = threadIdx.x; c < d; c += 256) out[c] = from_f<T>(0.f);
    if (threadIdx.x == 0) ssq[slot] = (float)d;
    return;
  }
  const T* x = (const T*)e.p + (int64_t)rows.src[slot] * e.sb + (int64_t)(t - 1) * e.st;
  float ss = 0.f;
  for (int c = threadIdx.x; c < d; c += 256) {
    const float v = to_f<T>(x[c]);
    ss = fmaf(v, v, ss);
    out[c] = from_f<T>(v * gain[c]);
  }
  ss = block_sum(ss, scratch);
  if (threadIdx.x == 0) ssq[slot] = ss;
}

// bf16 with every row of e and of A in 16-byte runs: thread i takes the 8
// consecutive elements 8 i, 8 i + 2048, ... (one 16-byte load and store each)
__global__ __launch_bounds__(256) void k_mem_prep_v8(Rows rows, EIn e, int d, const float* gain, uint16_t* A,
                                                     float* ssq) {
  __shared__ float scratch[16];
  const int slot = blockIdx.x;
  const int t = rows.t_row[slot];
  uint16_t* out = A + (int64_t)slot * d;
  if (t <= 0) {
    for (int c = threadIdx.x * 8; c < d; c += 2048) *(uint4*)(out + c) = make_uint4(0, 0, 0, 0);
    if (threadIdx.x == 0) ssq[slot] = (float)d;
    return;
  }
  const uint16_t* x = (const uint16_t*)e.p + (int64_t)rows.src[slot] * e.sb + (int64_t)(t - 1) * e.st;
  float ss = 0.f;
  for (int c = threadIdx.x * 8; c < d; c += 2048) {
    const uint4 xv = *(const uint4*)(x + c);
    const float4 g0 = *(const float4*)(gain + c), g1 = *(const float4*)(gain + c + 4);
    const uint16_t* xs = (const uint16_t*)&xv;
    const float gs[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
    uint16_t o[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const float v = bf2f(xs[k]);
      ss = fmaf(v, v, ss);
      o[k] = f2bf(v * gs[k]);
    }
    *(uint4*)(out + c) = *(const uint4*)o;
  }
  ss = block_sum(ss, scratch);
  if (threadIdx.x == 0) ssq[slot] = ss;
}

__global__ void k_mem_setlen(const int* len, int B, int* mem_len) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b < B) mem_len[b] = len[b];
}

__global__ void k_mem_commit(const int* rows, int n, const int* t_row, int* mem_len) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  if (t_row[i] > 0) mem_len[rows[i]] = t_row[i];
}

// trajectory log-weight of sequence blockIdx.x: thread i takes positions
// first + i, first + i + 256, ...; the 256 partial sums are added in a fixed
// order
__global__ __launch_bounds__(256) void k_traj_ratio(const int* first, const int* last, const float* logp,
                                                    int64_t logp_sb, const float* logmu, int64_t logmu_sb,
                                                    float* out) {
  __shared__ float scratch[16];
  const int b = blockIdx.x;
  const float* lp = logp + (int64_t)b * logp_sb;
  const float* lm = logmu + (int64_t)b * logmu_sb;
  float acc = 0.f;
  for (int t = first[b] + threadIdx.x; t <= last[b]; t += 256) acc += lp[t] - lm[t];
  acc = block_sum(acc, scratch);
  if (threadIdx.x == 0) out[b] = acc;
}

// ---------------------------------------------------------------------------
// readout: log-sum-exp, argmax, top-k behaviour distribution, sampling
// one workgroup of RB threads per slot; thread i owns logits
// [i*per, (i+1)*per) so that scans over thread order follow id order.
// ---------------------------------------------------------------------------

static constexpr int RB = 1024;
static constexpr int KMAX = 1024;

__device__ __forceinline__ uint32_t order_key(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// exclusive prefix sum over the block of one int per thread (thread order)
__device__ int block_excl_scan(int v, int* sh /* RB + 32 */, int* total) {
  sh[threadIdx.x] = v;
  __syncthreads();
  for (int off = 1; off < RB; off <<= 1) {
    const int x = threadIdx.x >= off ? sh[threadIdx.x - off] : 0;
    __syncthreads();
    sh[threadIdx.x] += x;
    __syncthreads();
  }
  const int incl = sh[threadIdx.x];
  *total = sh[RB - 1];
  __syncthreads();
  return incl - v;
}

__global__ __launch_bounds__(RB) void k_readout(ReadoutArgs a) {
  __shared__ float s_f[RB / 64];
  __shared__ int s_i[RB / 64];
  __shared__ int s_scan[RB];
  __shared__ int s_hist[256];
  __shared__ float c_val[KMAX];
  __shared__ int c_id[KMAX];
  __shared__ int c_ord[KMAX];
  __shared__ float s_bcast[4];
  __shared__ int s_ibcast[4];

  const int slot = blockIdx.x;
  const int t = a.rows.t_row[slot];
  if (t <= 0) return;
  const int V = a.V;
  const float* z = a.logits + (int64_t)slot * V;
  const int per = (V + RB - 1) / RB;
  const int lo = min(V, threadIdx.x * per), hi = min(V, lo + per);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;

  // ---- max and argmax (lowest id among equal maxima) ----
  float bm = -INFINITY;
  int bi = 0x7fffffff;
  for (int i = lo; i < hi; ++i) {
    const float v = z[i];
    if (v > bm) { bm = v; bi = i; }
  }
  for (int off = 32; off > 0; off >>= 1) {
    const float om = __shfl_xor(bm, off);
    const int oi = __shfl_xor(bi, off);
    if (om > bm || (om == bm && oi < bi)) { bm = om; bi = oi; }
  }
  if (lane == 0) { s_f[w] = bm; s_i[w] = bi; }
  __syncthreads();
  if (threadIdx.x == 0) {
    float m = s_f[0];
    int id = s_i[0];
    for (int k = 1; k < RB / 64; ++k)
      if (s_f[k] > m || (s_f[k] == m && s_i[k] < id)) { m = s_f[k]; id = s_i[k]; }
    s_bcast[0] = m;
    s_ibcast[0] = id;
  }
  __syncthreads();
  const float zmax = s_bcast[0];
  const int amax = s_ibcast[0];
  if (threadIdx.x == 0 && a.argmax) a.argmax[slot] = amax;

  // ---- score token ----
  int tok = -1;
  float* lp_out = nullptr;
  if (a.logp) {
    if (a.mode == 0) {
      tok = a.score_tok[slot];
      lp_out = a.logp + slot;
    } else {
      const int b = a.rows.src[slot];
      if (t >= a.split[b]) {
        tok = a.score_tok[(int64_t)b * a.tok_sb + t];  // x_{t+1}
        lp_out = a.logp + (int64_t)b * a.logp_sb + t;
      }
    }
  }
  // ---- log-sum-exp of the raw distribution ----
  if (lp_out || a.ratio) {
    float se = 0.f;
    for (int i = lo; i < hi; ++i) se += __expf(z[i] - zmax);
    float sum = 0.f;
    {
      for (int off = 32; off > 0; off >>= 1) se += __shfl_xor(se, off);
      if (lane == 0) s_f[w] = se;
      __syncthreads();
      for (int k = 0; k < RB / 64; ++k) sum += s_f[k];
      __syncthreads();
    }
    const float lse = zmax + logf(sum);
    if (threadIdx.x == 0 && lp_out && tok >= 0 && tok < V) {
      const float lp = z[tok] - lse;
      *lp_out = lp;
      if (a.ratio && a.logmu_beh) a.ratio[slot] = expf(lp - a.logmu_beh[slot]);
    }
  }

  // ---- behaviour distribution: temperature, top-k, renormalisation ----
  const bool want_sample = a.uniform != nullptr;
  const bool want_mu = a.logmu != nullptr;
  if (!want_sample && !want_mu) return;
  const float inv_tau = 1.0f / a.temperature;
  int K = a.top_k;
  if (K <= 0 || K > V) {
    // no truncation (scoring only): log mu(tok) = (z_tok - zmax)/tau - log sum exp((z - zmax)/tau)
    float se = 0.f;
    for (int i = lo; i < hi; ++i) se += __expf((z[i] - zmax) * inv_tau);
    for (int off = 32; off > 0; off >>= 1) se += __shfl_xor(se, off);
    if (lane == 0) s_f[w] = se;
    __syncthreads();
    if (threadIdx.x == 0) {
      float sum = 0.f;
      for (int k = 0; k < RB / 64; ++k) sum += s_f[k];
      const int tk = a.score_tok[slot];
      a.logmu[slot] = (tk >= 0 && tk < V) ? (z[tk] - zmax) * inv_tau - logf(sum) : -INFINITY;
    }
    return;
  }
  K = min(K, KMAX);
  // radix select of the K-th largest key, 8 bits per pass from the top
  uint32_t prefix = 0, mask = 0;
  int remaining = K;
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int b = threadIdx.x; b < 256; b += RB) s_hist[b] = 0;
    __syncthreads();
    for (int i = lo; i < hi; ++i) {
      const uint32_t k = order_key(z[i]);
      if ((k & mask) == prefix) atomicAdd(&s_hist[(k >> shift) & 0xff], 1);
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      int cum = 0, dg = 0;
      for (int b = 255; b >= 0; --b) {
        if (cum + s_hist[b] >= remaining) { dg = b; break; }
        cum += s_hist[b];
      }
      s_ibcast[1] = dg;
      s_ibcast[2] = remaining - cum;
    }
    __syncthreads();
    prefix |= (uint32_t)s_ibcast[1] << shift;
    mask |= 0xffu << shift;
    remaining = s_ibcast[2];
    __syncthreads();
  }
  const uint32_t thr = prefix;  // key of the K-th largest logit
  // collect: all keys > thr, then the first `remaining` keys == thr in id order
  int ngt = 0, neq = 0;
  for (int i = lo; i < hi; ++i) {
    const uint32_t k = order_key(z[i]);
    ngt += k > thr;
    neq += k == thr;
  }
  int tot_gt, tot_eq;
  int pgt = block_excl_scan(ngt, s_scan, &tot_gt);
  int peq = block_excl_scan(neq, s_scan, &tot_eq);
  for (int i = lo; i < hi; ++i) {
    const uint32_t k = order_key(z[i]);
    if (k > thr) {
      c_val[pgt] = z[i];
      c_id[pgt] = i;
      ++pgt;
    } else if (k == thr) {
      if (peq < remaining) {
        c_val[tot_gt + peq] = z[i];
        c_id[tot_gt + peq] = i;
      }
      ++peq;
    }
  }
  __syncthreads();
  // order candidates by (logit desc, id asc)
  for (int c = threadIdx.x; c < K; c += RB) {
    const float v = c_val[c];
    const int id = c_id[c];
    int rank = 0;
    for (int o = 0; o < K; ++o) {
      const float u = c_val[o];
      rank += (u > v) || (u == v && c_id[o] < id);
    }
    c_ord[rank] = c;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    const float top = c_val[c_ord[0]];
    float total = 0.f;
    for (int r = 0; r < K; ++r) total += __expf((c_val[c_ord[r]] - top) * inv_tau);
    if (a.top_p > 0.f && a.top_p < 1.f) {
      // nucleus: the shortest prefix of the order whose mass reaches top_p
      const float need = a.top_p * total;
      float cum = 0.f;
      int kk = K;
      for (int r = 0; r < K; ++r) {
        cum += __expf((c_val[c_ord[r]] - top) * inv_tau);
        if (cum >= need) {
          kk = r + 1;
          break;
        }
      }
      K = kk;
      total = 0.f;
      for (int r = 0; r < K; ++r) total += __expf((c_val[c_ord[r]] - top) * inv_tau);
    }
    const float ltot = logf(total);
    if (want_sample) {
      const float target = a.uniform[slot] * total;
      float cum = 0.f;
      int pick = K - 1;
      for (int r = 0; r < K; ++r) {
        cum += __expf((c_val[c_ord[r]] - top) * inv_tau);
        if (cum > target) { pick = r; break; }
      }
      const int c = c_ord[pick];
      if (a.sample_tok) a.sample_tok[slot] = c_id[c];
      if (a.sample_logmu) a.sample_logmu[slot] = (c_val[c] - top) * inv_tau - ltot;
    }
    if (want_mu) {
      const int tk = a.score_tok[slot];
      float lm = -INFINITY;
      for (int r = 0; r < K; ++r)
        if (c_id[c_ord[r]] == tk) lm = (c_val[c_ord[r]] - top) * inv_tau - ltot;
      a.logmu[slot] = lm;
    }
  }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------

void launch_prestep(const MiscArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(k_prestep, dim3((a.n + 255) / 256), dim3(256), 0, s, a);
}
void launch_replay_rows(const int* rows, int n, const int* tick_dev, int* t_row, int* pos, const int* mem_len,
                        int* err, hipStream_t s) {
  hipLaunchKernelGGL(k_replay_rows, dim3((n + 255) / 256), dim3(256), 0, s, rows, n, tick_dev, t_row,
                     (const int*)pos, mem_len, err);
}
void launch_poststep(const PostArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(k_poststep, dim3((a.n + 255) / 256), dim3(256), 0, s, a);
}

// counts[rows[i]] = 0 for the rows of a call (rows outside 0..B_cap-1 left
// to the pre-step's own check)
__global__ void k_zero_rows(int* counts, const int* rows, int n, int B_cap) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const int row = rows[i];
  if (row >= 0 && row < B_cap) counts[row] = 0;
}

// Calibration read: n16 16-byte pieces, each read once, with the load
// instruction of the attention kernels' key and value streams (non-temporal
// 16-byte loads) or a plain one; the xor of everything goes to sink only in
// the unlikely case it equals a magic value (so the loads are kept).
typedef unsigned int cal_u32x4 __attribute__((ext_vector_type(4)));
template <bool NT>
__global__ __launch_bounds__(256) void k_stream_read(const cal_u32x4* __restrict__ p, int64_t n16, unsigned* sink) {
  const int64_t nth = (int64_t)gridDim.x * blockDim.x;
  unsigned acc = 0;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += nth) {
    const cal_u32x4 v = NT ? __builtin_nontemporal_load(p + i) : p[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (acc == 0x9e3779b9u) *sink = acc;
}

void launch_stream_read(const void* p, int64_t n16, bool nontemporal, unsigned* sink, hipStream_t s) {
  if (nontemporal)
    hipLaunchKernelGGL(k_stream_read<true>, dim3(4096), dim3(256), 0, s, (const cal_u32x4*)p, n16, sink);
  else
    hipLaunchKernelGGL(k_stream_read<false>, dim3(4096), dim3(256), 0, s, (const cal_u32x4*)p, n16, sink);
}

// Peak calibration of the matrix cores: every wave runs 4 independent
// chains of v_mfma_f32_32x32x16_bf16 (enough to cover the instruction's
// latency) for `iters` steps on register operands; sink is written only if
// the results' xor equals a fixed value (it keeps the chains). 32768 flops
// per instruction.
typedef __bf16 cal_bf16x8 __attribute__((ext_vector_type(8)));
typedef float cal_f32x16 __attribute__((ext_vector_type(16)));
__global__ __launch_bounds__(256) void k_mfma_loop(int iters, unsigned* sink) {
  cal_bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(float)((threadIdx.x + i) & 7);
    b[i] = (__bf16)(float)((threadIdx.x * 3 + i) & 7);
  }
  cal_f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int k = 0; k < iters; ++k) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, a, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, a, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, b, c3, 0, 0, 0);
  }
  unsigned acc = 0;
#pragma unroll
  for (int e = 0; e < 16; ++e)
    acc ^= __float_as_uint(c0[e]) ^ __float_as_uint(c1[e]) ^ __float_as_uint(c2[e]) ^ __float_as_uint(c3[e]);
  if (acc == 0x9e3779b9u) *sink = acc;
}

void launch_mfma_loop(int blocks, int iters, unsigned* sink, hipStream_t s) {
  hipLaunchKernelGGL(k_mfma_loop, dim3(blocks), dim3(256), 0, s, iters, sink);
}

void launch_zero_rows(int* counts, const int* rows, int n, int B_cap, hipStream_t s) {
  hipLaunchKernelGGL(k_zero_rows, dim3((n + 255) / 256), dim3(256), 0, s, counts, rows, n, B_cap);
}
void launch_init(int dtype, const int* rows, int n, const float* s_star, float* st, int* pos, int* pending,
                 void* ring_k, void* ring_v, int L, int B_cap, int W, int d, int poison, hipStream_t s) {
  if (dtype == 0)
    hipLaunchKernelGGL(k_init<float>, dim3(n), dim3(256), 0, s, rows, n, s_star, st, pos, pending,
                       (float*)ring_k, (float*)ring_v, L, B_cap, W - 1, d, poison);
  else
    hipLaunchKernelGGL(k_init<uint16_t>, dim3(n), dim3(256), 0, s, rows, n, s_star, st, pos, pending,
                       (uint16_t*)ring_k, (uint16_t*)ring_v, L, B_cap, W - 1, d, poison);
}
void launch_set_pending(const int* rows, const int* src, int n, const int* tokens, int64_t tok_sb,
                        const int* last_index, int* pending, hipStream_t s) {
  hipLaunchKernelGGL(k_set_pending, dim3((n + 255) / 256), dim3(256), 0, s, rows, src, n, tokens,
                     tok_sb, last_index, pending);
}
void launch_merge_prep(int dtype, const MiscArgs& a, hipStream_t s) {
  if (dtype == 1) {
    Phase p{};
    p.kind = PH_MERGE_PREP;
    p.gx = a.n;
    p.gy = p.gz = 1;
    p.u.mi = a;
    if (record_phase(p)) return;
  }
  if (dtype == 0) hipLaunchKernelGGL(k_merge_prep<float>, dim3(a.n), dim3(256), 0, s, a);
  else hipLaunchKernelGGL(k_merge_prep<uint16_t>, dim3(a.n), dim3(256), 0, s, a);
}
void launch_rmsnorm(int dtype, const MiscArgs& a, hipStream_t s) {
  if (dtype == 0) hipLaunchKernelGGL(k_rmsnorm<float>, dim3(a.n), dim3(256), 0, s, a);
  else hipLaunchKernelGGL(k_rmsnorm<uint16_t>, dim3(a.n), dim3(256), 0, s, a);
}
void launch_final(int dtype, const MiscArgs& a, hipStream_t s) {
  if (dtype == 1) {
    Phase p{};
    p.kind = PH_FINAL;
    p.gx = a.n;
    p.gy = p.gz = 1;
    p.u.mi = a;
    if (record_phase(p)) return;
  }
  if (dtype == 0) hipLaunchKernelGGL(k_final<float>, dim3(a.n), dim3(256), 0, s, a);
  else hipLaunchKernelGGL(k_final<uint16_t>, dim3(a.n), dim3(256), 0, s, a);
}
void launch_copy_f32(const float* src, float* dst, int64_t n, hipStream_t s) {
  {
    Phase p{};
    p.kind = PH_COPY;
    p.gx = (int)((n + 255) / 256);
    p.gy = p.gz = 1;
    p.u.cp = CopyArgs{src, dst, n};
    if (record_phase(p)) return;
  }
  hipLaunchKernelGGL(k_copy_f32, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, src, dst, n);
}
void launch_mem_slots(const int* rows, int n, const int* mem_len, int B_cap, int T_cap, int* t_out, int* err,
                      hipStream_t s) {
  hipLaunchKernelGGL(k_mem_slots, dim3((n + 255) / 256), dim3(256), 0, s, rows, n, mem_len, B_cap, T_cap, t_out,
                     err);
}
void launch_mem_rows(const int* offs, int B, int64_t r0, int n, int* src_out, int* t_out, hipStream_t s) {
  hipLaunchKernelGGL(k_mem_rows, dim3((n + 255) / 256), dim3(256), 0, s, offs, B, r0, n, src_out, t_out);
}
void launch_mem_prep(int dtype, const Rows& rows, EIn e, int d, const float* gain, void* A, float* ssq,
                     hipStream_t s) {
  const bool v8 = dtype == 1 && d % 8 == 0 && (uintptr_t)e.p % 16 == 0 && e.sb % 8 == 0 && e.st % 8 == 0 &&
                  (uintptr_t)A % 16 == 0 && (uintptr_t)gain % 16 == 0;
  if (dtype == 0)
    hipLaunchKernelGGL(k_mem_prep<float>, dim3(rows.n), dim3(256), 0, s, rows, e, d, gain, (float*)A, ssq);
  else if (v8)
    hipLaunchKernelGGL(k_mem_prep_v8, dim3(rows.n), dim3(256), 0, s, rows, e, d, gain, (uint16_t*)A, ssq);
  else
    hipLaunchKernelGGL(k_mem_prep<uint16_t>, dim3(rows.n), dim3(256), 0, s, rows, e, d, gain, (uint16_t*)A, ssq);
}
void launch_traj_ratio(int B, const int* first, const int* last, const float* logp, int64_t logp_sb,
                       const float* logmu, int64_t logmu_sb, float* out, hipStream_t s) {
  hipLaunchKernelGGL(k_traj_ratio, dim3(B), dim3(256), 0, s, first, last, logp, logp_sb, logmu, logmu_sb, out);
}
void launch_mem_setlen(const int* len, int B, int* mem_len, hipStream_t s) {
  hipLaunchKernelGGL(k_mem_setlen, dim3((B + 255) / 256), dim3(256), 0, s, len, B, mem_len);
}
void launch_mem_commit(const int* rows, int n, const int* t_row, int* mem_len, hipStream_t s) {
  hipLaunchKernelGGL(k_mem_commit, dim3((n + 255) / 256), dim3(256), 0, s, rows, n, t_row, mem_len);
}
void launch_readout(const ReadoutArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(k_readout, dim3(a.n), dim3(RB), 0, s, a);
}

}  // namespace rlt
