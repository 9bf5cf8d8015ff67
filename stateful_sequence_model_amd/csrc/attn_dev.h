// Device-side bodies of the attention kernels; included by the stand-alone
// attention kernels and by the persistent step kernel.
#pragma once
#include "rlt_internal.h"

namespace rlt {

// 32 bytes of one head's keys or values held by one lane, unconverted: two
// 16-byte pieces, the second h elements after the first. A lane of a head
// owns elements [jl·PE, jl·PE + PE) and the same range + DH/2, so that the
// lanes of a head read one contiguous span per load instruction (128 bytes
// for 128-wide bf16 heads: every cache line an instruction touches is used
// whole).
struct Raw {
  uint4 a, b;
};

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

// Streamed keys and values are read once per launch: non-temporal loads (a
// read-only probe of the cross-attention access pattern measured 7.3 TB/s
// with them against 6.4 TB/s with the default cache policy).
__device__ __forceinline__ uint4 ld_stream(const void* p) {
  const u32x4_t v = __builtin_nontemporal_load((const u32x4_t*)p);
  return make_uint4(v.x, v.y, v.z, v.w);
}

template <typename T> struct LaneVec;
template <> struct LaneVec<uint16_t> {
  static constexpr int E = 16, PE = 8;
  __device__ static __forceinline__ Raw load(const uint16_t* p, int h) {
    return Raw{ld_stream(p), ld_stream(p + h)};
  }
  __device__ static __forceinline__ float lo(uint32_t w) { return __uint_as_float(w << 16); }
  __device__ static __forceinline__ float hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
  __device__ static __forceinline__ float dot(const float* q, const Raw& r) {
    const uint32_t w[8] = {r.a.x, r.a.y, r.a.z, r.a.w, r.b.x, r.b.y, r.b.z, r.b.w};
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      s = fmaf(q[2 * i], lo(w[i]), s);
      s = fmaf(q[2 * i + 1], hi(w[i]), s);
    }
    return s;
  }
  __device__ static __forceinline__ void axpy(float* o, float p, const Raw& r) {
    const uint32_t w[8] = {r.a.x, r.a.y, r.a.z, r.a.w, r.b.x, r.b.y, r.b.z, r.b.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      o[2 * i] = fmaf(p, lo(w[i]), o[2 * i]);
      o[2 * i + 1] = fmaf(p, hi(w[i]), o[2 * i + 1]);
    }
  }
  // the lane's two pieces to p0 and p1
  __device__ static __forceinline__ void store(uint16_t* p0, uint16_t* p1, const float* f) {
    uint32_t w[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) w[i] = (uint32_t)f2bf(f[2 * i]) | ((uint32_t)f2bf(f[2 * i + 1]) << 16);
    *(uint4*)p0 = make_uint4(w[0], w[1], w[2], w[3]);
    *(uint4*)p1 = make_uint4(w[4], w[5], w[6], w[7]);
  }
};
template <> struct LaneVec<float> {
  static constexpr int E = 8, PE = 4;
  __device__ static __forceinline__ Raw load(const float* p, int h) {
    return Raw{ld_stream(p), ld_stream(p + h)};
  }
  __device__ static __forceinline__ float dot(const float* q, const Raw& r) {
    const uint32_t w[8] = {r.a.x, r.a.y, r.a.z, r.a.w, r.b.x, r.b.y, r.b.z, r.b.w};
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) s = fmaf(q[i], __uint_as_float(w[i]), s);
    return s;
  }
  __device__ static __forceinline__ void axpy(float* o, float p, const Raw& r) {
    const uint32_t w[8] = {r.a.x, r.a.y, r.a.z, r.a.w, r.b.x, r.b.y, r.b.z, r.b.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] = fmaf(p, __uint_as_float(w[i]), o[i]);
  }
  __device__ static __forceinline__ void store(float* p0, float* p1, const float* f) {
    *(float4*)p0 = make_float4(f[0], f[1], f[2], f[3]);
    *(float4*)p1 = make_float4(f[4], f[5], f[6], f[7]);
  }
};

// s + the value of lane (this lane with the DPP permutation CTRL applied)
template <int CTRL>
__device__ __forceinline__ float dpp_add(float s) {
  return s + __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(s), CTRL, 0xf, 0xf, false));
}

// Sum over aligned groups of LPK (1..16) consecutive lanes, the result in
// every lane of the group, through the data-parallel primitives of the
// vector ALU (no LDS round trip): swap neighbours, swap pairs of a quad,
// then mirror within 8 and 16 lanes (each mirror pairs a lane with one of
// the half it has not summed yet, whose values are already uniform).
template <int LPK>
__device__ __forceinline__ float group_sum(float s) {
  static_assert(LPK >= 1 && LPK <= 16 && (LPK & (LPK - 1)) == 0, "group of 1-16 lanes");
  if (LPK >= 2) s = dpp_add<0xb1>(s);   // quad_perm [1,0,3,2]
  if (LPK >= 4) s = dpp_add<0x4e>(s);   // quad_perm [2,3,0,1]
  if (LPK >= 8) s = dpp_add<0x141>(s);  // row_half_mirror
  if (LPK >= 16) s = dpp_add<0x140>(s); // row_mirror
  return s;
}

// online-softmax accumulator of one lane (E output elements)
template <typename T>
struct Acc {
  static constexpr int E = LaneVec<T>::E;
  float m, l, o[E];
  __device__ __forceinline__ void init() {
    m = -INFINITY;
    l = 0.f;
#pragma unroll
    for (int i = 0; i < E; ++i) o[i] = 0.f;
  }
  // fold N keys (scores s[], values v[]) with one max update
  template <int N>
  __device__ __forceinline__ void fold(const float* s, const Raw* v) {
    float mx = m;
#pragma unroll
    for (int u = 0; u < N; ++u) mx = fmaxf(mx, s[u]);
    const float c = exp2f(m - mx);
    l *= c;
#pragma unroll
    for (int i = 0; i < E; ++i) o[i] *= c;
#pragma unroll
    for (int u = 0; u < N; ++u) {
      const float p = exp2f(s[u] - mx);
      l += p;
      LaneVec<T>::axpy(o, p, v[u]);
    }
    m = mx;
  }
};

// Walk keys r = r0, r0 + step, ... < r1 (addressed by kv(r) -> (k, v)
// pointers), U at a time.
// qp: this lane's query elements (pieces at qp and qp + DH/2), unscaled;
// scores are scaled by qscale. The query is loaded after the first batch of
// keys is issued, so no workgroup waits for it before its key loads start.
template <typename T, int LPK, int U, class KV>
__device__ __forceinline__ void walk(Acc<T>& acc, const float* qp, float qscale, int r0, int r1, int step,
                                     const KV& kv) {
  constexpr int h = LPK * LaneVec<T>::PE;  // DH / 2
  constexpr int E = LaneVec<T>::E, PE = LaneVec<T>::PE;
  using LV = LaneVec<T>;
  float q[E];
  // full batches: r0 + i·U·step for i < nb, each with its last key below r1
  const int span = U * step;
  const int last = r1 - 1 - (U - 1) * step;
  const int nb = last >= r0 ? (last - r0) / span + 1 : 0;
  auto issue = [&](Raw* kr, Raw* vr, int r) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const T *kp, *vp;
      kv(r + u * step, kp, vp);
      kr[u] = LV::load(kp, h);
      vr[u] = LV::load(vp, h);
    }
  };
  auto consume = [&](const Raw* kr, const Raw* vr) {
    float s[U];
#pragma unroll
    for (int u = 0; u < U; ++u) s[u] = group_sum<LPK>(LV::dot(q, kr[u])) * qscale;
    acc.template fold<U>(s, vr);
  };
  // two register sets: the next batch's loads are in flight while the
  // current batch is folded (same batches, same fold order as one set)
  Raw ka[U], va[U], kb[U], vb[U];
  if (nb > 0) issue(ka, va, r0);
#pragma unroll
  for (int i = 0; i < PE; ++i) {
    q[i] = qp[i];
    q[PE + i] = qp[h + i];
  }
  for (int i = 0; i < nb; i += 2) {
    if (i + 1 < nb) issue(kb, vb, r0 + (i + 1) * span);
    consume(ka, va);
    if (i + 1 < nb) {
      if (i + 2 < nb) issue(ka, va, r0 + (i + 2) * span);
      consume(kb, vb);
    }
  }
  for (int r = r0 + nb * span; r < r1; r += step) {
    const T *kp, *vp;
    kv(r, kp, vp);
    Raw kr[1] = {LV::load(kp, h)}, vr[1] = {LV::load(vp, h)};
    float s[1] = {group_sum<LPK>(LV::dot(q, kr[0])) * qscale};
    acc.template fold<1>(s, vr);
  }
}

// Merge the key groups' partials of the workgroup (fixed group order), all
// 256 threads at once: thread idx takes (lane li of a key group, element e)
// for idx = threadIdx.x, + 256, ... < G * E, sums that element over the
// groups in group order (the same operations, in the same order, as one
// lane per element would do) and hands emit(li, e, o, M, L) the merged
// unnormalised output element, running max and sum. Contains one barrier.
template <typename T, class Emit>
__device__ __forceinline__ void merge_groups(const Acc<T>& acc, int G, int KPW, float* s_o, float* s_ml,
                                             const Emit& emit) {
  constexpr int E = Acc<T>::E;
#pragma unroll
  for (int i = 0; i < E; ++i) s_o[threadIdx.x * E + i] = acc.o[i];
  s_ml[2 * threadIdx.x] = acc.m;
  s_ml[2 * threadIdx.x + 1] = acc.l;
  __syncthreads();
  for (int idx = threadIdx.x; idx < G * E; idx += 256) {
    const int li = idx / E, e = idx - li * E;
    float M = -INFINITY;
    for (int g = 0; g < KPW; ++g) M = fmaxf(M, s_ml[2 * (g * G + li)]);
    float L = 0.f, o = 0.f;
    for (int g = 0; g < KPW; ++g) {
      const int th = g * G + li;
      const float w = exp2f(s_ml[2 * th] - M);
      L += s_ml[2 * th + 1] * w;
      o = fmaf(s_o[th * E + e], w, o);
    }
    emit(li, e, o, M, L);
  }
}

template <typename T>
// Keys r < nh are ring slots in memory order: position j sits at slot
// (j - 1) mod (W - 1), so the nh retained positions t - nh .. t - 1 occupy
// exactly slots 0 .. nh - 1, before the ring wraps (nh = t - 1 < W - 1) and
// after (nh = W - 1: every slot). Visiting slots in order (not positions)
// reads the window front to back with no modulo; the softmax is
// order-free up to rounding. Key nh is the current (k, v).
struct RingKV {
  const T *rk, *rv, *ck, *cv;
  int nh;
  int64_t d;
  __device__ __forceinline__ void operator()(int r, const T*& kp, const T*& vp) const {
    if (r < nh) {
      kp = rk + r * d;
      vp = rv + r * d;
    } else {
      kp = ck;
      vp = cv;
    }
  }
};

template <typename T>
struct MemKV {
  const T *mk, *mv;
  int64_t st;
  __device__ __forceinline__ void operator()(int r, const T*& kp, const T*& vp) const {
    kp = mk + r * st;
    vp = mv + r * st;
  }
};

constexpr int UNROLL = 4;

// LDS floats used by the attention bodies
template <typename T>
constexpr int attn_lds_floats() { return 256 * LaneVec<T>::E + 512; }

// SWA for (head group hg, slot); block 256
template <typename T, int DH>
__device__ __forceinline__ void swa_body(const AttnArgs& a, int hg, int slot, float* lds) {
  using LV = LaneVec<T>;
  constexpr int E = LV::E;
  constexpr int LPK = DH / E;
  float* s_o = lds;
  float* s_ml = lds + 256 * E;
  const int t = a.rows.t_row[slot];
  if (t <= 0) return;
  const int row = a.rows.rows[slot];
  const int G = a.hpw * LPK;
  const int KPW = 256 / G;
  const int kg = threadIdx.x / G;
  const int hh = (threadIdx.x % G) / LPK;
  const int jl = threadIdx.x % LPK;
  constexpr int PE = LV::PE, h = DH / 2;
  const int col = (hg * a.hpw + hh) * DH + jl * PE;
  const int d = a.d;
  const int W1 = a.W - 1;
  const int nh = min(t - 1, W1);
  RingKV<T> kv;
  kv.rk = (const T*)a.ring_k + (int64_t)row * W1 * d + col;
  kv.rv = (const T*)a.ring_v + (int64_t)row * W1 * d + col;
  kv.ck = (const T*)a.kc + (int64_t)slot * d + col;
  kv.cv = (const T*)a.vc + (int64_t)slot * d + col;
  kv.nh = nh;
  kv.d = d;

  // the cache insert's data (this lane's pieces of the current k and v),
  // loaded before the walk so that the insert at the end is stores only
  const bool ins = W1 > 0 && kg == 0;
  uint4 ik0{}, ik1{}, iv0{}, iv1{};
  if (ins) {
    ik0 = *(const uint4*)kv.ck;
    ik1 = *(const uint4*)(kv.ck + h);
    iv0 = *(const uint4*)kv.cv;
    iv1 = *(const uint4*)(kv.cv + h);
  }
  Acc<T> acc;
  acc.init();
  walk<T, LPK, UNROLL>(acc, a.q + (int64_t)slot * d + col, a.qscale, kg, nh + 1, KPW, kv);
  T* out = (T*)a.out;
  const int c0 = hg * a.hpw * DH;
  merge_groups<T>(acc, G, KPW, s_o, s_ml, [&](int li, int e, float o, float, float L) {
    // element e of lane li: piece e / PE of that lane's two
    const int c = c0 + (li / LPK) * DH + (li % LPK) * PE + (e < PE ? e : h + e - PE);
    store_op(out, a.out_pk ? pk_off(slot, c, d >> 6) : (int64_t)slot * d + c, a.out_lo, o * (1.f / L));
  });
  // cache insert: every read of this workgroup is complete (the barrier in
  // merge_groups follows every thread's walk)
  if (ins) {
    const int sl = (t - 1) % W1;
    T* dk = (T*)a.ring_k + ((int64_t)row * W1 + sl) * d + col;
    T* dv = (T*)a.ring_v + ((int64_t)row * W1 + sl) * d + col;
    *(uint4*)dk = ik0;
    *(uint4*)(dk + h) = ik1;
    *(uint4*)dv = iv0;
    *(uint4*)(dv + h) = iv1;
  }
}

template <typename T, int DH>
__device__ __forceinline__ void xcombine_body(const AttnArgs& a, int head, int slot, int tid, int nt);

// cross-attention partial of (head group hg, chunk ch, slot); block 256.
// With a.cnt set, the chunks of a (row, head group) are also combined in
// this launch: each workgroup publishes its partial and counts itself in
// a.cnt[slot][hg]; the one that arrives last resets the counter and merges
// every chunk's partial (the combine kernel's arithmetic, in chunk order, so
// the result does not depend on which workgroup is last).
template <typename T, int DH>
__device__ __forceinline__ void xattn_body(const AttnArgs& a, int hg, int ch, int slot, float* lds) {
  using LV = LaneVec<T>;
  constexpr int E = LV::E;
  constexpr int LPK = DH / E;
  float* s_o = lds;
  float* s_ml = lds + 256 * E;
  const int t = a.rows.t_row[slot];
  const int j0 = ch * a.chunk;
  if (t <= 0 || j0 >= t) return;
  const int j1 = min(j0 + a.chunk, t);
  const int row = a.rows.rows[slot];
  const int G = a.hpw * LPK;
  const int KPW = 256 / G;
  const int kg = threadIdx.x / G;
  const int hh = (threadIdx.x % G) / LPK;
  const int jl = threadIdx.x % LPK;
  const int head = hg * a.hpw + hh;
  constexpr int PE = LV::PE, h = DH / 2;
  const int col = head * DH + jl * PE;
  const int d = a.d;
  MemKV<T> kv{(const T*)a.mk + (int64_t)row * a.sb + col, (const T*)a.mv + (int64_t)row * a.sb + col, a.st};
  Acc<T> acc;
  acc.init();
  walk<T, LPK, UNROLL>(acc, a.q + (int64_t)slot * d + col, a.qscale, j0 + kg, j1, KPW, kv);
  merge_groups<T>(acc, G, KPW, s_o, s_ml, [&](int li, int e, float o, float M, float L) {
    const int ljl = li % LPK;
    const int eo = ljl * PE + (e < PE ? e : h + e - PE);  // element of the head
    if (a.direct || t <= a.chunk) {
      // the row's only chunk (one chunk per launch, or a row whose position
      // fits the first chunk): what the combine would write for it (weight
      // 2^0 = 1, the same division); the combine skips such rows
      const int c = (hg * a.hpw + li / LPK) * DH + eo;
      store_op((T*)a.out, a.out_pk ? pk_off(slot, c, d >> 6) : (int64_t)slot * d + c, a.out_lo, o * (1.f / L));
      return;
    }
    float* P = a.part + (((int64_t)slot * a.nch + ch) * a.H + hg * a.hpw + li / LPK) * (DH + 2);
    P[eo] = o;
    if (ljl == 0 && e == 0) {
      P[DH] = M;
      P[DH + 1] = L;
    }
  });
  if (a.cnt == nullptr || a.direct || t <= a.chunk) return;  // uniform in the workgroup
  __shared__ int s_last;
  __builtin_amdgcn_s_waitcnt(0);  // this wave's partial stores have reached the cache hierarchy
  __syncthreads();
  if (threadIdx.x == 0) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");  // publish the workgroup's partial
    int* cp = a.cnt + (int64_t)slot * (a.H / a.hpw) + hg;
    const int nc = (t + a.chunk - 1) / a.chunk;
    const int last = __hip_atomic_fetch_add(cp, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == nc - 1;
    if (last) {
      __hip_atomic_store(cp, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);  // ready for the next launch
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");  // every chunk's partial is visible
    }
    s_last = last;
  }
  __syncthreads();
  if (!s_last) return;
  const int ntp = 256 / a.hpw;
  if (ntp >= 64) {
    xcombine_body<T, DH>(a, hg * a.hpw + (int)threadIdx.x / ntp, slot, (int)threadIdx.x % ntp, ntp);
  } else {
    for (int hh = 0; hh < a.hpw; ++hh) xcombine_body<T, DH>(a, hg * a.hpw + hh, slot, threadIdx.x, 256);
  }
}

// chunk combine of (head, slot) by `nt` (>= 64) threads with index `tid`:
// M = max of the chunk maxima, L = sum over chunks in chunk order of
// l_c 2^(m_c - M), o = the same weights applied to the chunk outputs in chunk
// order. Up to CU chunks all partials are loaded at once (one memory round
// trip); more chunks take the same arithmetic in a plain loop. Rows with a
// single chunk (t <= chunk) were written by the cross-attention itself.
template <typename T, int DH>
__device__ __forceinline__ void xcombine_body(const AttnArgs& a, int head, int slot, int tid, int nt) {
  constexpr int CU = 16, EPT = (DH + 63) / 64;  // chunks loaded at once, elements per thread
  const int t = a.rows.t_row[slot];
  if (t <= a.chunk) return;  // no position, or one chunk: written by the cross-attention itself
  const int nc = (t + a.chunk - 1) / a.chunk;
  const float* P = a.part + ((int64_t)slot * a.nch * a.H + head) * (DH + 2);
  const int64_t cs = (int64_t)a.H * (DH + 2);  // chunk stride
  float M = -INFINITY, L = 0.f;
  float o[EPT];
#pragma unroll
  for (int k = 0; k < EPT; ++k) o[k] = 0.f;
  if (nc <= CU) {
    float m[CU], l[CU], p[CU][EPT];
#pragma unroll
    for (int c = 0; c < CU; ++c) {
      if (c < nc) {
        m[c] = P[c * cs + DH];
        l[c] = P[c * cs + DH + 1];
#pragma unroll
        for (int k = 0; k < EPT; ++k) p[c][k] = tid + k * nt < DH ? P[c * cs + tid + k * nt] : 0.f;
      }
    }
#pragma unroll
    for (int c = 0; c < CU; ++c)
      if (c < nc) M = fmaxf(M, m[c]);
#pragma unroll
    for (int c = 0; c < CU; ++c)
      if (c < nc) {
        const float w = exp2f(m[c] - M);
        L += l[c] * w;
#pragma unroll
        for (int k = 0; k < EPT; ++k) o[k] = fmaf(p[c][k], w, o[k]);
      }
  } else {
    for (int c = 0; c < nc; ++c) M = fmaxf(M, P[c * cs + DH]);
    for (int c = 0; c < nc; ++c) {
      const float w = exp2f(P[c * cs + DH] - M);
      L += P[c * cs + DH + 1] * w;
#pragma unroll
      for (int k = 0; k < EPT; ++k)
        if (tid + k * nt < DH) o[k] = fmaf(P[c * cs + tid + k * nt], w, o[k]);
    }
  }
  const float inv = 1.f / L;
  T* out = (T*)a.out;
#pragma unroll
  for (int k = 0; k < EPT; ++k) {
    const int e = tid + k * nt;
    if (e < DH) {
      const int col = head * DH + e;
      store_op(out, a.out_pk ? pk_off(slot, col, a.d >> 6) : (int64_t)slot * a.d + col, a.out_lo, o[k] * inv);
    }
  }
}

}  // namespace rlt
