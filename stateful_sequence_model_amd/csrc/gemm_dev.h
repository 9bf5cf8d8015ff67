// Device-side building blocks of the matrix products (epilogue functor and
// the per-tile bodies); included by the stand-alone product kernels and by
// the persistent step kernel.
#pragma once
#include "rlt_internal.h"

// No contraction of multiplies and adds into fused multiply-adds below: the
// epilogues are inlined into several kernels (and into different points of
// one kernel), and the compiler's choice to fuse depends on the context, so
// the same expression could round differently from one launch shape to
// another.
#pragma clang fp contract(off)

namespace rlt {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;

template <typename T>
struct Epi {
  EpiArgs a;

  __device__ __forceinline__ float e_at(int m, int c) const {
    const int t = a.rows.t_row[m];
    if (t <= 0) return 0.f;
    const T* p = (const T*)a.e.p + (int64_t)a.rows.src[m] * a.e.sb + (int64_t)(t - 1) * a.e.st;
    return to_f<T>(p[c]);
  }

  // (cos, sin) of the rotary angle of pair index i (< dh/2) at position t:
  // computed (no memory round trip inside an epilogue), or from the table
  // (double-precision sincos, rounded) when loaded ahead of the product. The
  // computed form takes the angle t * theta_i in double precision, reduces it
  // to [-pi, pi] in double (exact to ~1e-12 for t < 2^16) and evaluates the
  // single-precision sincos there: within about an ulp of the table's value,
  // at a fraction of the cost of a double-precision sincos (which made the
  // Q/K/V epilogue 7.6 of its 19.9 us at 128 rows).
  __device__ __forceinline__ float2 rope_cs(int t, int i, bool tab = false) const {
    if (tab && a.rope_tab && t <= a.rope_tmax) return a.rope_tab[(int64_t)t * (a.dh >> 1) + i];
    const double r = (double)t * a.inv_freq[i];
    const double twopi = 6.283185307179586476925286766559;
    const float x = (float)fma(-rint(r * (1.0 / twopi)), twopi, r);
    float sn, cs;
    sincosf(x, &sn, &cs);
    return make_float2(cs, sn);
  }
  __device__ __forceinline__ static void rot(float2 r, float& x, float& y) {
    const float xr = x * r.x - y * r.y;
    const float yr = y * r.x + x * r.y;
    x = xr;
    y = yr;
  }
  // rotary transform of the pair (x_i, x_{i+dh/2}) of one head at position t
  // (the table when it covers t, like the prefetching epilogue: the same
  // angle values on every path)
  __device__ __forceinline__ void rotate(int m, int c_in_head, float& x, float& y) const {
    rot(rope_cs(a.rows.t_row[m], c_in_head, true), x, y);
  }

  // EPI_MEMKV for a row whose position t (> 0) and destination offset
  // (row * msb + (t - 1) * mst elements) the tile loaded ahead
  __device__ __forceinline__ void memkv_at(int t, int64_t off, int ca, float va, int cb, float vb, float rs) const {
    va *= rs;
    vb *= rs;
    const int seg = ca / a.d;
    const int xa = ca - seg * a.d, xb = cb - seg * a.d;
    if (seg == 0 && a.rope) rot(rope_cs(t, xa % a.dh, true), va, vb);
    T* dst = (T*)(seg == 0 ? a.mk : a.mv) + off;
    dst[xa] = from_f<T>(va);
    dst[xb] = from_f<T>(vb);
  }

  // memkv_at for 8 consecutive columns from ca and from cb (one 16-byte
  // store each; same arithmetic per element); needs a.mem_vec
  __device__ __forceinline__ void memkv_at8(int t, int64_t off, int ca, const float* va, int cb, const float* vb,
                                            float rs) const {
    static_assert(sizeof(T) == 2, "16-byte runs of 8 two-byte elements");
    const int seg = ca / a.d;
    const int xa = ca - seg * a.d, xb = cb - seg * a.d;
    float x[8], y[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      x[k] = va[k] * rs;
      y[k] = vb[k] * rs;
    }
    if (seg == 0 && a.rope) {
      const int i0 = xa % a.dh;  // the 8 columns stay in the first half of the head
#pragma unroll
      for (int k = 0; k < 8; ++k) rot(rope_cs(t, i0 + k, true), x[k], y[k]);
    }
    T* dst = (T*)(seg == 0 ? a.mk : a.mv) + off;
    uint16_t px[8], py[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      px[k] = from_f<T>(x[k]);
      py[k] = from_f<T>(y[k]);
    }
    *(uint4*)(dst + xa) = *(const uint4*)px;
    *(uint4*)(dst + xb) = *(const uint4*)py;
  }

  // Values an epilogue reads from memory for (row m, columns ca, cb), loaded
  // ahead of the product by tiles that know their outputs in advance: the
  // residual and the next norm's gains (EPI_RESID), the rotary (cos, sin)
  // (EPI_QKV on q and k, EPI_QROT). apply() with them equals operator().
  struct Pre {
    float2 u, v;
  };
  __device__ __forceinline__ Pre pre(int m, int ca, int cb) const {
    Pre p{};
    if (a.kind == EPI_RESID) {
      const float* z = a.out_f + (int64_t)m * a.ldo;
      p.u = make_float2(z[ca], z[cb]);
      p.v = make_float2(a.gnext[ca], a.gnext[cb]);
    } else if (a.rope && (a.kind == EPI_QROT || (a.kind == EPI_QKV && ca / a.d < 2))) {
      p.u = rope_cs(a.rows.t_row[m], (ca % a.d) % a.dh, true);
    }
    return p;
  }
  __device__ __forceinline__ float apply(int m, int ca, float va, int cb, float vb, float rs, const Pre& p) const {
    if (a.kind == EPI_RESID) {
      float* z = a.out_f + (int64_t)m * a.ldo;
      const float za = p.u.x + va, zb = p.u.y + vb;
      z[ca] = za;
      z[cb] = zb;
      T* o = (T*)a.zb;
      const int64_t ia = a.pk ? pk_off(m, ca, a.d >> 6) : (int64_t)m * a.d + ca;
      const int64_t ib = a.pk ? pk_off(m, cb, a.d >> 6) : (int64_t)m * a.d + cb;
      store_op(o, ia, a.lo, za * p.v.x);
      store_op(o, ib, a.lo, zb * p.v.y);
      return za * za + zb * zb;
    }
    if (a.kind == EPI_QROT) {
      va *= rs;
      vb *= rs;
      if (a.rope) rot(p.u, va, vb);
      a.out_f[(int64_t)m * a.d + ca] = va;
      a.out_f[(int64_t)m * a.d + cb] = vb;
      return 0.f;
    }
    if (a.kind == EPI_QKV) {
      va *= rs;
      vb *= rs;
      const int seg = ca / a.d;
      const int xa = ca - seg * a.d, xb = cb - seg * a.d;
      if (seg < 2 && a.rope) rot(p.u, va, vb);
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
    return (*this)(m, ca, va, cb, vb, rs);
  }

  // next RMSNorm's input: zb = z * gain (the rstd is applied by the consumer)
  __device__ __forceinline__ float produce(int m, int ca, float za, int cb, float zb) const {
    T* o = (T*)a.zb;
    const int64_t ia = a.pk ? pk_off(m, ca, a.d >> 6) : (int64_t)m * a.d + ca;
    const int64_t ib = a.pk ? pk_off(m, cb, a.d >> 6) : (int64_t)m * a.d + cb;
    store_op(o, ia, a.lo, za * a.gnext[ca]);
    store_op(o, ib, a.lo, zb * a.gnext[cb]);
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
        store_op((T*)a.out_k, a.pk ? pk_off(m, ca, (int)(a.ldo >> 6)) : (int64_t)m * a.ldo + ca, a.lo, act);
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
      case EPI_STORE_T: {
        // fragment order ([M][ldo], ldo % 64 == 0) when a.pk: the next product's operand
        const int64_t ia = a.pk ? pk_off(m, ca, (int)(a.ldo >> 6)) : (int64_t)m * a.ldo + ca;
        const int64_t ib = a.pk ? pk_off(m, cb, (int)(a.ldo >> 6)) : (int64_t)m * a.ldo + cb;
        store_op((T*)a.out_k, ia, a.lo, va * rs);
        store_op((T*)a.out_k, ib, a.lo, vb * rs);
        return 0.f;
      }
      case EPI_MEMKV: {
        const int t = a.rows.t_row[m];
        if (t <= 0) return 0.f;
        va *= rs;
        vb *= rs;
        const int seg = ca / a.d;
        const int xa = ca - seg * a.d, xb = cb - seg * a.d;
        // (cos, sin) from the table: the token-parallel prefill rotates
        // millions of keys per call, where the angles dominated the epilogue
        if (seg == 0 && a.rope) rot(rope_cs(t, xa % a.dh, true), va, vb);
        T* dst = (T*)(seg == 0 ? a.mk : a.mv) + (int64_t)a.rows.rows[m] * a.msb + (int64_t)(t - 1) * a.mst;
        dst[xa] = from_f<T>(va);
        dst[xb] = from_f<T>(vb);
        return 0.f;
      }
      default:
        return 0.f;
    }
  }
};

template <typename T>
__device__ __forceinline__ const T* weight_row(const GemmArgs& g, int vc) {
  int seg, r;
  weight_pos(g, vc, seg, r);
  return (const T*)g.W[seg] + (int64_t)r * g.K;
}

__device__ __forceinline__ bf16x8_t load8(const uint16_t* p) {
  const uint4 u = *(const uint4*)p;
  return __builtin_bit_cast(bf16x8_t, u);
}

// LDS floats used by gemm_bf16_body<MB>
constexpr int gemm_lds_floats(int MB) { return 4 * MB * 16 * 32 + MB * 16 + rowrstd_lds<16, 256>() * MB; }

// One (pair, split, m-tile) tile of the product; block 256 (4 waves).
template <int MB>
__device__ __forceinline__ void gemm_bf16_body(const GemmArgs& g, const Epi<uint16_t>& epi, int pair, int split,
                                               int mt, float* lds) {
  float(*red)[MB * 16][32] = reinterpret_cast<float(*)[MB * 16][32]>(lds);
  float* s_rstd = lds + 4 * MB * 16 * 32;
  float* s_part = s_rstd + MB * 16;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  int ba, bb;
  pair_blocks(g, pair, ba, bb);
  const int r16 = narrow_lane_row(lane);
  const int kq = narrow_lane_k(lane);
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
  // The workgroup's K range is cut in 32-wide steps dealt to the four waves
  // round-robin (wave w takes steps w, w+4, ...): at any moment the waves
  // read adjacent 64-byte pieces of each weight row, so rows are streamed in
  // long contiguous runs.
  int k0, nsteps;  // step j of this wave is at k0 + 128 j
  narrow_wave_steps(g, split, wave, k0, nsteps);
  // PF K-steps of loads in flight: step i is multiplied while steps
  // i+1 .. i+PF-1 are still arriving (a register ring, statically indexed).
  // The steady-state loop is branch-free so that each step waits only for
  // its own loads: the refill of step i+PF is always issued, its address
  // clamped to the last step (a harmless re-read) near the end.
  constexpr int PF = MB >= 4 ? 4 : 6;
  bf16x8_t bufa[PF][MB], bufb[PF][2];
  if (nsteps > 0) {
#pragma unroll
    for (int p = 0; p < PF; ++p) {
      const int k = narrow_step_k(k0, p, nsteps);
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
      const int kn = narrow_step_k(k0, i + p + PF, nsteps);
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

constexpr int SPLITK_LDS_FLOATS = 16 + rowrstd_lds<16, 256>();

// Sum of the S split partials of (pair, 16-row block mt) in split order, then
// the epilogue; block 256.
template <typename T>
__device__ __forceinline__ void splitk_epi_body(const GemmArgs& g, const Epi<T>& epi, int pair, int mt, float* lds) {
  float* s_rstd = lds;
  float* s_part = lds + 16;
  int ba, bb;
  pair_blocks(g, pair, ba, bb);
  const int m = mt * 16 + (threadIdx.x >> 4), r = threadIdx.x & 15;
  if (g.ssq_in) {
    RowRstd<16> rr(g, mt * 16);
    rr.finish(g, mt * 16, s_part, s_rstd);
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
    if (r == 0 && m < g.M) g.ssq_out[(int64_t)pair * g.M_pad + m] = sq;
  }
}

}  // namespace rlt
