// Matrix products of the decoder transition with fused epilogues.
//
// Every projection of the step is Y = A W^T with A the [rows][K] activations
// and W a natural-layout [out][in] weight ("Recurrent Looped Transformer",
// §2.5 eqs. (2.9)-(2.16) and §2.3 eq. (2.6)). Weights are streamed once per
// call; the batch is the M dimension, so these products are HBM-bound for
// the batch sizes of a decoder step.
//
// bf16 path (gfx950 MFMA v_mfma_f32_16x16x32_bf16):
//   workgroup = 4 waves; all 4 waves own the same output tile (16*MB rows x
//   one pair of 16-column blocks) and each streams a disjoint quarter of the
//   workgroup's K range, so A and W are each read once per workgroup; the
//   four partial tiles are summed in LDS in wave order. Optional split of K
//   across S workgroups writes partial tiles that a second kernel sums in
//   split order. Both orders are fixed, so results are deterministic.
//   Accumulation is fp32; A (activations) arrive rounded to bf16.
// fp32 path: one thread per output pair, sequential K loop (used by the
//   float32 configuration, where precision rather than speed is the point).
//
// Output columns are handled as pairs of 16-column blocks so that epilogues
// needing two columns of the same row see both in one lane: the rotary
// transform pairs column i with i + dh/2 of the same head, SwiGLU pairs a
// gate column with its up column.
#include "rlt_internal.h"

namespace rlt {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;

template <typename T>
struct Epi {
  EpiArgs a;

  __device__ __forceinline__ float e_at(int m, int c) const {
    const int t = a.rows.t_row[m];
    if (t <= 0) return 0.f;
    const T* p = (const T*)a.e.p + (int64_t)a.rows.src[m] * a.e.sb + (int64_t)(t - 1) * a.e.st;
    return to_f<T>(p[c]);
  }

  // rotary transform of the pair (x_i, x_{i+dh/2}) of one head at position t
  __device__ __forceinline__ void rotate(int m, int c_in_head, float& x, float& y) const {
    const int t = a.rows.t_row[m];
    double sn, cs;
    sincos((double)t * a.inv_freq[c_in_head], &sn, &cs);
    const float c = (float)cs, s = (float)sn;
    const float xr = x * c - y * s;
    const float yr = y * c + x * s;
    x = xr;
    y = yr;
  }

  // next RMSNorm's input: zb = z * gain (the rstd is applied by the consumer)
  __device__ __forceinline__ float produce(int m, int ca, float za, int cb, float zb) const {
    T* o = (T*)a.zb + (int64_t)m * a.d;
    o[ca] = from_f<T>(za * a.gnext[ca]);
    o[cb] = from_f<T>(zb * a.gnext[cb]);
    return za * za + zb * zb;
  }

  // Epilogue of one column pair of row m. rs scales the accumulators of
  // products whose input is z * gain of an RMSNorm (1 otherwise). Returns
  // the squared sum of the produced residual values (0 for non-producers).
  __device__ __forceinline__ float operator()(int m, int ca, float va, int cb, float vb, float rs) const {
    switch (a.kind) {
      case EPI_STORE:
        a.out_f[(int64_t)m * a.ldo + ca] = va * rs;
        a.out_f[(int64_t)m * a.ldo + cb] = vb * rs;
        return 0.f;
      case EPI_QKV: {
        va *= rs;
        vb *= rs;
        const int seg = ca / a.d;
        const int xa = ca - seg * a.d, xb = cb - seg * a.d;
        if (seg < 2 && a.rope) rotate(m, xa % a.dh, va, vb);
        const int64_t o = (int64_t)m * a.d;
        if (seg == 0) {
          a.out_f[o + xa] = va;
          a.out_f[o + xb] = vb;
        } else {
          T* dst = (T*)(seg == 1 ? a.out_k : a.out_v);
          dst[o + xa] = from_f<T>(va);
          dst[o + xb] = from_f<T>(vb);
        }
        return 0.f;
      }
      case EPI_QROT: {
        va *= rs;
        vb *= rs;
        if (a.rope) rotate(m, ca % a.dh, va, vb);
        a.out_f[(int64_t)m * a.d + ca] = va;
        a.out_f[(int64_t)m * a.d + cb] = vb;
        return 0.f;
      }
      case EPI_RESID: {
        float* z = a.out_f + (int64_t)m * a.ldo;
        const float za = z[ca] + va, zb = z[cb] + vb;
        z[ca] = za;
        z[cb] = zb;
        return produce(m, ca, za, cb, zb);
      }
      case EPI_SWIGLU: {
        va *= rs;
        vb *= rs;
        const float act = va * sigmoidf_(va) * vb;
        ((T*)a.out_k)[(int64_t)m * a.ldo + ca] = from_f<T>(act);
        return 0.f;
      }
      case EPI_MGATE: {
        float* g = a.out_f + (int64_t)m * a.ldo;
        g[ca] = sigmoidf_(va + a.bias[ca]);
        g[cb] = sigmoidf_(vb + a.bias[cb]);
        return 0.f;
      }
      case EPI_MOUT: {
        float* z = a.out_f + (int64_t)m * a.ldo;
        const float* g = a.gbuf + (int64_t)m * a.ldo;
        const float za = e_at(m, ca) + a.alpha * g[ca] * va;
        const float zb = e_at(m, cb) + a.alpha * g[cb] * vb;
        z[ca] = za;
        z[cb] = zb;
        return produce(m, ca, za, cb, zb);
      }
      case EPI_CONVEX: {
        float za = 0.f, zb = 0.f;
        if (a.rows.t_row[m] > 0) {
          const float* s = a.s_state + (int64_t)a.rows.rows[m] * a.d;
          const float ga = sigmoidf_(va + a.bias[ca]);
          const float gb = sigmoidf_(vb + a.bias[cb]);
          za = ga * e_at(m, ca) + (1.f - ga) * s[ca];
          zb = gb * e_at(m, cb) + (1.f - gb) * s[cb];
        }
        float* z = a.out_f + (int64_t)m * a.ldo;
        z[ca] = za;
        z[cb] = zb;
        return produce(m, ca, za, cb, zb);
      }
      default:
        return 0.f;
    }
  }
};

template <typename T>
__device__ __forceinline__ const T* weight_row(const GemmArgs& g, int vc) {
  const int seg = vc / g.seg_rows;
  const int r = vc - seg * g.seg_rows;
  return (const T*)g.W[seg] + (int64_t)r * g.K;
}

__device__ __forceinline__ bf16x8_t load8(const uint16_t* p) {
  const uint4 u = *(const uint4*)p;
  return __builtin_bit_cast(bf16x8_t, u);
}

// grid: x = pair, y = split, z = m-tile; block 256 (4 waves)
template <int MB>
__global__ __launch_bounds__(256) void k_gemm_bf16(GemmArgs g, Epi<uint16_t> epi) {
  __shared__ float red[4][MB * 16][32];
  const int pair = blockIdx.x, split = blockIdx.y, mt = blockIdx.z;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  int ba, bb;
  pair_blocks(g, pair, ba, bb);
  const int r16 = lane & 15;
  const int kq = (lane >> 4) * 8;
  const uint16_t* wa = weight_row<uint16_t>(g, ba * 16 + r16) + kq;
  const uint16_t* wb = weight_row<uint16_t>(g, bb * 16 + r16) + kq;
  const int m0 = mt * MB * 16;
  const uint16_t* ap[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
    ap[mb] = (const uint16_t*)g.A + (int64_t)(m0 + mb * 16 + r16) * g.lda + kq;

  // folded RMSNorm: this tile's row sums of squares, loads in flight with the K loop
  const bool norm_here = g.S == 1 && g.ssq_in != nullptr;
  RowRstd<MB * 16> rr(g, norm_here ? m0 : 0);
  f32x4_t acc[MB][2];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    acc[mb][0] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    acc[mb][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  // The workgroup's K range [kw0, kw1) is cut in 32-wide steps dealt to the
  // four waves round-robin (wave w takes steps w, w+4, ...): at any moment
  // the waves read adjacent 64-byte pieces of each weight row, so rows are
  // streamed in long contiguous runs.
  const int kw0 = split * 4 * g.kslice;
  const int kw1 = min(kw0 + 4 * g.kslice, g.K);
  const int all_steps = max(0, (kw1 - kw0) / 32);
  const int k0 = kw0 + 32 * wave;  // step j of this wave is at k0 + 128 j
  // PF K-steps of loads in flight: step i is multiplied while steps
  // i+1 .. i+PF-1 are still arriving (a register ring, statically indexed).
  // The steady-state loop is branch-free so that each step waits only for
  // its own loads: the refill of step i+PF is always issued, its address
  // clamped to the last step (a harmless re-read) near the end.
  constexpr int PF = MB >= 4 ? 4 : 6;
  const int nsteps = (all_steps - wave + 3) / 4;
  bf16x8_t bufa[PF][MB], bufb[PF][2];
  if (nsteps > 0) {
#pragma unroll
    for (int p = 0; p < PF; ++p) {
      const int k = k0 + 128 * min(p, nsteps - 1);
      bufb[p][0] = load8(wa + k);
      bufb[p][1] = load8(wb + k);
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) bufa[p][mb] = load8(ap[mb] + k);
    }
  }
  int i = 0;
  for (; i + PF <= nsteps; i += PF) {
#pragma unroll
    for (int p = 0; p < PF; ++p) {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        acc[mb][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bufa[p][mb], bufb[p][0], acc[mb][0], 0, 0, 0);
        acc[mb][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bufa[p][mb], bufb[p][1], acc[mb][1], 0, 0, 0);
      }
      const int kn = k0 + 128 * min(i + p + PF, nsteps - 1);
      bufb[p][0] = load8(wa + kn);
      bufb[p][1] = load8(wb + kn);
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) bufa[p][mb] = load8(ap[mb] + kn);
    }
  }
  // tail: the remaining nsteps - i (< PF) steps are already in the ring
#pragma unroll
  for (int p = 0; p < PF; ++p) {
    if (i + p < nsteps) {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        acc[mb][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bufa[p][mb], bufb[p][0], acc[mb][0], 0, 0, 0);
        acc[mb][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bufa[p][mb], bufb[p][1], acc[mb][1], 0, 0, 0);
      }
    }
  }
  // C layout: lane holds rows 4*(lane/16)+i, column lane%16
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      red[wave][mb * 16 + (lane >> 4) * 4 + i][r16] = acc[mb][0][i];
      red[wave][mb * 16 + (lane >> 4) * 4 + i][16 + r16] = acc[mb][1][i];
    }
  __shared__ float s_rstd[MB * 16];
  __shared__ float s_part[256];
  if (norm_here) rr.finish(g, m0, s_part, s_rstd);  // uniform branch: contains a barrier
  __syncthreads();
  // every lane runs the same trip count (the 16 lanes of a row reduce together)
  for (int idx = threadIdx.x; idx < MB * 16 * 16; idx += 256) {
    const int m = idx >> 4, r = idx & 15;
    const int slot = m0 + m;
    const float va = ((red[0][m][r] + red[1][m][r]) + red[2][m][r]) + red[3][m][r];
    const float vb = ((red[0][m][16 + r] + red[1][m][16 + r]) + red[2][m][16 + r]) + red[3][m][16 + r];
    if (g.S == 1) {
      float sq = 0.f;
      if (slot < g.M) sq = epi(slot, ba * 16 + r, va, bb * 16 + r, vb, g.ssq_in ? s_rstd[m] : 1.f);
      if (g.ssq_out) {
        sq = sum16(sq);
        if (r == 0 && slot < g.M) g.ssq_out[(int64_t)pair * g.M_pad + slot] = sq;
      }
    } else if (slot < g.M) {
      float* P = g.partial + ((int64_t)split * g.M_pad + slot) * g.Nv;
      P[ba * 16 + r] = va;
      P[bb * 16 + r] = vb;
    }
  }
}

// Wide tile for batches above 32 rows: 4 column pairs (128 columns) x 16*MB
// rows per workgroup. Wave w owns pair 4*blockIdx.x + w over the whole K
// range of the workgroup, so its accumulators are final (no cross-wave
// reduction). The activation tile, which every column of the call needs, is
// loaded from L2 once per workgroup and shared by the four waves through LDS;
// the weights, each read by one wave only, go straight from HBM into
// registers in MFMA operand layout. K advances in stages of 64 with P stages
// of loads in flight (a register ring; the activation part of a stage is
// written to one of two LDS buffers just before it is used).
// LDS layout of a stage: block (mb, s) of 1 KB holds, at lane position L,
// the 8 activations of row mb*16 + L%16 at k = 32 s + 8 (L/16): exactly the
// MFMA A operand of lane L, so both the writes and the reads are contiguous.
// grid: npairs / 4 * S * m-tiles (1-D, decoded below); block 256; K range
// of a workgroup = kslice (a multiple of 64)
template <int MB>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, MB >= 8 ? 1 : 2))) void k_gemm_bf16_wide(
    GemmArgs g, Epi<uint16_t> epi) {
  constexpr int R = MB * 16;
  constexpr int NA = MB / 2;  // 16-byte activation chunks per thread per stage
  constexpr int PW = 4;       // weight stages in flight (even: a stage's LDS buffer is p & 1)
  __shared__ __attribute__((aligned(16))) uint16_t sa[2][MB * 2 * 64 * 8];
  __shared__ float s_rstd[R];
  __shared__ float s_part[256];
  // 1-D grid of T = groups * S * mtiles workgroups, XCD-aware: the hardware
  // deals consecutive workgroup ids to the 8 XCDs in turn, so id b runs on
  // XCD b % 8. Tile t = (b % 8) * (T / 8) + b / 8 gives each XCD a contiguous
  // run of tiles, ordered m-tile fastest, so the row tiles that read the same
  // weight slice run together on one L2 (ids past 8 * (T / 8) map to themselves).
  const int T = gridDim.x, b = blockIdx.x, per = T >> 3;
  const int t = b < 8 * per ? (b & 7) * per + (b >> 3) : b;
  const int nmt = (g.M + R - 1) / R;
  const int mt = t % nmt, split = (t / nmt) % g.S, grp = t / (nmt * g.S);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int pair = grp * 4 + wave;
  int ba, bb;
  pair_blocks(g, pair, ba, bb);
  const int r16 = lane & 15, kq = (lane >> 4) * 8;
  const uint16_t* wa = weight_row<uint16_t>(g, ba * 16 + r16) + kq;
  const uint16_t* wb = weight_row<uint16_t>(g, bb * 16 + r16) + kq;
  const int m0 = mt * R;
  const uint16_t* ap[NA];
#pragma unroll
  for (int c = 0; c < NA; ++c) {
    const int q = c * 256 + tid, blk = q >> 6, L = q & 63;
    ap[c] = (const uint16_t*)g.A + (int64_t)(m0 + (blk >> 1) * 16 + (L & 15)) * g.lda + (blk & 1) * 32 + (L >> 4) * 8;
  }
  const bool norm_here = g.S == 1 && g.ssq_in != nullptr;
  RowRstd<R> rr(g, norm_here ? m0 : 0);
  f32x4_t acc[MB][2];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    acc[mb][0] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    acc[mb][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  const int kw0 = split * g.kslice;
  const int kw1 = min(kw0 + g.kslice, g.K);
  const int nst = max(0, (kw1 - kw0) / 64);
  // ring of register stages: weights PW stages ahead (HBM latency), the
  // activations 2 stages ahead (L2 hits). Loads are issued in stage order
  // and complete in order, so waiting for the activations of stage st also
  // waits for the weights of stage st + 1 only.
  bf16x8_t ra[2][NA];
  bf16x8_t rw[PW][4];
  auto load_a = [&](int pa, int st) {
    const int k = kw0 + 64 * st;
#pragma unroll
    for (int c = 0; c < NA; ++c) ra[pa][c] = load8(ap[c] + k);
  };
  auto load_w = [&](int pw, int st) {
    const int k = kw0 + 64 * st;
    rw[pw][0] = load8(wa + k);
    rw[pw][1] = load8(wb + k);
    rw[pw][2] = load8(wa + k + 32);
    rw[pw][3] = load8(wb + k + 32);
  };
  // The LDS buffer written at stage st is rewritten at st + 2: every wave has
  // passed the barrier of st + 1, which follows its reads of stage st.
  auto run_stage = [&](int p) {
    uint16_t* buf = sa[p & 1];
#pragma unroll
    for (int c = 0; c < NA; ++c) *(bf16x8_t*)(buf + (c * 256 + tid) * 8) = ra[p & 1][c];
    __syncthreads();
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const bf16x8_t a = *(const bf16x8_t*)(buf + ((mb * 2 + s) * 64 + lane) * 8);
        acc[mb][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, rw[p][2 * s], acc[mb][0], 0, 0, 0);
        acc[mb][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, rw[p][2 * s + 1], acc[mb][1], 0, 0, 0);
      }
  };
  // branch-free steady state: refills are always issued, clamped to the last
  // stage near the end (re-reads that hit in cache)
  if (nst > 0) {
    load_a(0, 0);
    load_a(1, min(1, nst - 1));
#pragma unroll
    for (int p = 0; p < PW; ++p) load_w(p, min(p, nst - 1));
  }
  int i = 0;
  for (; i + PW <= nst; i += PW) {
#pragma unroll
    for (int p = 0; p < PW; ++p) {
      run_stage(p);
      load_a(p & 1, min(i + p + 2, nst - 1));
      load_w(p, min(i + p + PW, nst - 1));
    }
  }
  // tail (fewer than PW stages): the weights are all in flight already, the
  // activations still need their 2-ahead refill; uniform conditions (the
  // stage contains a barrier)
#pragma unroll
  for (int p = 0; p < PW; ++p)
    if (i + p < nst) {
      run_stage(p);
      load_a(p & 1, min(i + p + 2, nst - 1));
    }

  if (norm_here) {  // uniform branch
    rr.finish(g, m0, s_part, s_rstd);
    __syncthreads();
  }
  // C layout: lane holds rows 4*(lane/16)+i of each 16-row block, column lane%16
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int mr = mb * 16 + (lane >> 4) * 4 + q;
      const int m = m0 + mr;
      const float va = acc[mb][0][q], vb = acc[mb][1][q];
      if (g.S == 1) {
        float sq = 0.f;
        if (m < g.M) sq = epi(m, ba * 16 + r16, va, bb * 16 + r16, vb, norm_here ? s_rstd[mr] : 1.f);
        if (g.ssq_out) {
          sq = sum16(sq);
          if (r16 == 0 && m < g.M) g.ssq_out[(int64_t)pair * g.M_pad + m] = sq;
        }
      } else if (m < g.M) {
        float* Pp = g.partial + ((int64_t)split * g.M_pad + m) * g.Nv;
        Pp[ba * 16 + r16] = va;
        Pp[bb * 16 + r16] = vb;
      }
    }
}

// sum of the S split partials in split order, then the epilogue
// grid: x = pair, y = ceil(M/16); block 256
template <typename T>
__global__ __launch_bounds__(256) void k_splitk_epi(GemmArgs g, Epi<T> epi) {
  __shared__ float s_rstd[16];
  __shared__ float s_part[256];
  int ba, bb;
  pair_blocks(g, blockIdx.x, ba, bb);
  const int m = blockIdx.y * 16 + (threadIdx.x >> 4), r = threadIdx.x & 15;
  if (g.ssq_in) {
    RowRstd<16> rr(g, blockIdx.y * 16);
    rr.finish(g, blockIdx.y * 16, s_part, s_rstd);
  }
  __syncthreads();
  float sq = 0.f;
  if (m < g.M) {
    float va = 0.f, vb = 0.f;
    for (int s = 0; s < g.S; ++s) {
      const float* P = g.partial + ((int64_t)s * g.M_pad + m) * g.Nv;
      va += P[ba * 16 + r];
      vb += P[bb * 16 + r];
    }
    sq = epi(m, ba * 16 + r, va, bb * 16 + r, vb, g.ssq_in ? s_rstd[threadIdx.x >> 4] : 1.f);
  }
  if (g.ssq_out) {
    sq = sum16(sq);
    if (r == 0 && m < g.M) g.ssq_out[(int64_t)blockIdx.x * g.M_pad + m] = sq;
  }
}

// fp32: one thread per (row, column pair); columns paired per element:
// rotary pairs (i, i+dh/2) of a head, gate/up pairs, or adjacent columns.
__device__ __forceinline__ void pair_cols(const GemmArgs& g, int q, int& ca, int& cb) {
  if (g.pairing == PAIR_PLAIN) {
    ca = 2 * q;
    cb = 2 * q + 1;
  } else if (g.pairing == PAIR_ROPE) {
    const int half = g.dh / 2;
    const int h = q / half, i = q - h * half;
    ca = h * g.dh + i;
    cb = ca + half;
  } else {
    ca = q;
    cb = q + g.seg_rows;
  }
}

// grid: x = ceil(Nv/2 / 64), y = row; block 64
__global__ __launch_bounds__(64) void k_gemm_f32(GemmArgs g, Epi<float> epi) {
  const int q = blockIdx.x * 64 + threadIdx.x;
  const int m = blockIdx.y;
  if (q >= g.Nv / 2 || m >= g.M) return;
  int ca, cb;
  pair_cols(g, q, ca, cb);
  const float* a = (const float*)g.A + (int64_t)m * g.lda;
  const float* wa = weight_row<float>(g, ca);
  const float* wb = weight_row<float>(g, cb);
  float sa = 0.f, sb = 0.f;
  for (int k = 0; k < g.K; k += 4) {
    const float4 x = *(const float4*)(a + k);
    const float4 p = *(const float4*)(wa + k);
    const float4 r = *(const float4*)(wb + k);
    sa = fmaf(x.x, p.x, sa); sa = fmaf(x.y, p.y, sa); sa = fmaf(x.z, p.z, sa); sa = fmaf(x.w, p.w, sa);
    sb = fmaf(x.x, r.x, sb); sb = fmaf(x.y, r.y, sb); sb = fmaf(x.z, r.z, sb); sb = fmaf(x.w, r.w, sb);
  }
  // one column pair per thread: the pair is the unit of the squared sums
  const float sq = epi(m, ca, sa, cb, sb, g.ssq_in ? row_rstd(g, m) : 1.f);
  if (g.ssq_out) g.ssq_out[(int64_t)q * g.M_pad + m] = sq;
}

void launch_gemm(int dtype, const GemmArgs& g0, const EpiArgs& e, hipStream_t s) {
  GemmArgs g = g0;
  if (dtype == 0) {
    dim3 grid((g.Nv / 2 + 63) / 64, g.M);
    hipLaunchKernelGGL(k_gemm_f32, grid, dim3(64), 0, s, g, Epi<float>{e});
    return;
  }
  const int MB = g.mb;
  const int mt = (g.M + 16 * MB - 1) / (16 * MB);
  Epi<uint16_t> epi{e};
  if (g.wide) {
    dim3 grid(g.npairs / 4 * g.S * mt);
    if (MB == 8)
      hipLaunchKernelGGL(k_gemm_bf16_wide<8>, grid, dim3(256), 0, s, g, epi);
    else
      hipLaunchKernelGGL(k_gemm_bf16_wide<4>, grid, dim3(256), 0, s, g, epi);
  } else {
    dim3 grid(g.npairs, g.S, mt);
    switch (MB) {
      case 1: hipLaunchKernelGGL(k_gemm_bf16<1>, grid, dim3(256), 0, s, g, epi); break;
      case 2: hipLaunchKernelGGL(k_gemm_bf16<2>, grid, dim3(256), 0, s, g, epi); break;
      default: hipLaunchKernelGGL(k_gemm_bf16<4>, grid, dim3(256), 0, s, g, epi); break;
    }
  }
  if (g.S > 1) {
    dim3 g2(g.npairs, (g.M + 15) / 16);
    hipLaunchKernelGGL(k_splitk_epi<uint16_t>, g2, dim3(256), 0, s, g, epi);
  }
}

}  // namespace rlt
