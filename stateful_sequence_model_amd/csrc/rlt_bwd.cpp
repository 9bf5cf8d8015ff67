// Host side of the replay backward ("Recurrent Looped Transformer" §5.4,
// App. B): full backpropagation through time of a loss linear in the
// replayed log-probabilities. The sequences advance in lockstep as in the
// forward replay (sorted by length, longest first, so the rows active at
// step t are a prefix). A forward pass keeps s_t and every decoder key/value
// (the per-step checkpoint), and every step's activations too when they fit
// the memory budget; the backward pass walks t from the last step to the
// first, recomputes the step's activations from s_{t-1} and the kept
// keys/values unless they were kept, and differentiates it:
//   readout -> blocks L-1..0 (FFN, cross-attention, SWA) -> merge -> s_{t-1}.
// Gradients of a step's current key/value collect the contributions of every
// later step whose window read them (their steps are processed first), so
// the cache path of the state Jacobian (App. B, eq. (B.3)) is carried
// exactly. Parameter, memory and e gradients accumulate step by step in a
// fixed order.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <numeric>
#include <string>
#include <vector>

#include "bwd.h"

namespace rlt {
namespace bwd {
namespace {

// Work buffers of one call, freed when it returns (after its stream has drained).
struct Buf {
  std::vector<void*> owned;
  bool ok = true;
  ~Buf() {
    for (void* p : owned) (void)hipFree(p);
  }
  void* get(size_t bytes) {
    void* p = nullptr;
    if (hipMalloc(&p, std::max<size_t>(bytes, 4)) != hipSuccess) {
      ok = false;
      return nullptr;
    }
    owned.push_back(p);
    return p;
  }
  float* f(size_t n) { return (float*)get(n * sizeof(float)); }
  int* i(size_t n) { return (int*)get(n * sizeof(int)); }
};

float* layer_ptr(float* const* arr, int l) { return arr ? arr[l] : nullptr; }

}  // namespace

int replay_backward(const Model& m, const rlt_backward_io* io, const rlt_grads* gr, hipStream_t s, std::string& err) {
  const rlt_config& c = m.cfg;
  const int L = c.n_layers, d = c.d_model, H = c.n_heads, dh = c.d_head, W = c.window, G = c.n_groups;
  const int F = c.d_ffn, V = c.vocab, dt = m.dt;
  const bool gated = c.merge_kind == RLT_MERGE_GATED, rope_on = c.pos_kind == RLT_POS_ROPE;
  const int B = io->B;
  const size_t es = dt ? 2 : 4;

  // schedule: sequences by length, longest first; rows active at step t = prefix n_t
  std::vector<int> order(B);
  std::iota(order.begin(), order.end(), 0);
  std::stable_sort(order.begin(), order.end(), [&](int a, int b) { return io->len_host[a] > io->len_host[b]; });
  const int Tm = io->len_host[order[0]] - 1;
  if ((size_t)(2 * Tm + 2 * dh) * sizeof(float) > 65536) {
    err = "len - 1 above 8192 - d_head";
    return RLT_EUNSUPPORTED;
  }
  std::vector<int> n_at(Tm + 2, 0), split_sorted(B);
  for (int i = 0; i < B; ++i) {
    split_sorted[i] = io->split_host[order[i]];
    for (int t = 1; t <= io->len_host[order[i]] - 1; ++t) ++n_at[t];
  }

  Buf buf;
  const size_t Bd = (size_t)B * d, BF = (size_t)B * F;
  int* map = buf.i(B);
  int* split = buf.i(B);
  float* S = buf.f((size_t)(Tm + 1) * Bd);                  // s_t of every step, [t][row][d]
  float* KT = buf.f((size_t)L * Tm * Bd);                   // decoder keys   [l][t-1][row][d]
  float* VT = buf.f((size_t)L * Tm * Bd);                   // decoder values
  float* dKT = buf.f((size_t)L * Tm * Bd);                  // their gradients
  float* dVT = buf.f((size_t)L * Tm * Bd);
  // activations of a step (all layers), in one slot per step when they fit
  // the budget (the backward pass then reads the forward pass's values), else
  // in one slot that every step overwrites (recomputed in the backward pass,
  // by the same kernels, so the values are the same bits either way)
  auto pad = [](size_t n) { return (n + 63) / 64 * 64; };  // 256-byte sub-buffers
  const size_t sz[] = {2 * Bd, (size_t)B, Bd, Bd, (size_t)(L + 1) * Bd, (size_t)L * Bd, (size_t)L * Bd,
                       (size_t)L * Bd, (size_t)L * Bd, (size_t)L * Bd, (size_t)L * Bd, (size_t)L * Bd,
                       (size_t)L * Bd, (size_t)L * Bd, (size_t)4 * L * B + B, (size_t)L * BF, (size_t)L * BF,
                       (size_t)L * BF};
  size_t per_step = 0;
  for (size_t n : sz) per_step += pad(n);
  bool keep = m.keep_acts == 2;
  if (m.keep_acts == 0) {
    size_t free_b = 0, total_b = 0;
    keep = hipMemGetInfo(&free_b, &total_b) == hipSuccess && (size_t)Tm * per_step * sizeof(float) <= free_b / 4;
  }
  float* acts = buf.f((keep ? (size_t)Tm : 1) * per_step);
  struct Act {
    float *cat, *rr, *g, *wsr, *zin, *hs, *q, *o, *zb, *hm, *qm, *om, *za, *hd, *rs, *ga, *gu, *act;
  };
  // cat: [e_t; r] or [e_t; s_{t-1}]; zin: layer inputs, zin[L] = s_t; rs: rstd
  // of RMSNorm_S, _M, _D per layer, then _o
  auto act_at = [&](int t) {
    float* p = acts + (keep ? (size_t)(t - 1) * per_step : 0);
    Act a;
    float** dst[] = {&a.cat, &a.rr, &a.g, &a.wsr, &a.zin, &a.hs, &a.q, &a.o, &a.zb, &a.hm, &a.qm, &a.om,
                     &a.za, &a.hd, &a.rs, &a.ga, &a.gu, &a.act};
    for (size_t i = 0; i < sizeof(sz) / sizeof(sz[0]); ++i) {
      *dst[i] = p;
      p += pad(sz[i]);
    }
    return a;
  };
  float* no = buf.f(Bd);
  float* logits = buf.f((size_t)B * V);
  // gradient temporaries
  float* ds = buf.f(Bd);
  float* dz = buf.f(Bd);
  float* t1 = buf.f(Bd);
  float* t2 = buf.f(Bd);
  float* dq = buf.f(Bd);
  float* dF1 = buf.f(BF);
  float* dF2 = buf.f(BF);
  float* dF3 = buf.f(BF);
  float* dlog = buf.f((size_t)B * V);
  float* dcat = buf.f(2 * Bd);
  float* dpre = buf.f(Bd);
  float* dw = buf.f(Bd);
  float* det = buf.f(Bd);
  if (!buf.ok) {
    (void)hipGetLastError();
    err = "work buffers of the replay backward do not fit";
    return RLT_ENOMEM;
  }
  if (hipMemcpyAsync(map, order.data(), B * sizeof(int), hipMemcpyHostToDevice, s) != hipSuccess ||
      hipMemcpyAsync(split, split_sorted.data(), B * sizeof(int), hipMemcpyHostToDevice, s) != hipSuccess ||
      hipMemsetAsync(dKT, 0, (size_t)L * Tm * Bd * sizeof(float), s) != hipSuccess ||
      hipMemsetAsync(dVT, 0, (size_t)L * Tm * Bd * sizeof(float), s) != hipSuccess ||
      hipMemsetAsync(ds, 0, Bd * sizeof(float), s) != hipSuccess) {
    err = "upload of the schedule failed";
    return RLT_EHIP;
  }
  const size_t LT = (size_t)Tm * Bd;  // per-layer extent of the key/value trace
  auto kt_at = [&](float* base, int l, int t) { return base + (size_t)l * LT + (size_t)(t - 1) * Bd; };
  auto mem_kv = [&](int l) {
    const int gi = (l * G) / L;
    KV kv;
    kv.k = (const char*)io->mem.k + (size_t)gi * io->mem.stride_g * es;
    kv.v = (const char*)io->mem.v + (size_t)gi * io->mem.stride_g * es;
    kv.dt = dt;
    kv.s_row = io->mem.stride_b;
    kv.s_pos = io->mem.stride_t;
    kv.map = map;
    return kv;
  };
  auto trace_kv = [&](int l) {
    KV kv;
    kv.k = KT + (size_t)l * LT;
    kv.v = VT + (size_t)l * LT;
    kv.dt = 0;
    kv.s_row = d;
    kv.s_pos = (int64_t)Bd;
    kv.map = nullptr;
    return kv;
  };
  // forward linear Y[n][N] = X[n][K] W^T, W [N][K] in the parameter type
  auto lin = [&](int n, int N, int K, const float* X, int64_t ldx, const void* Wt, float* Y, int64_t ldy, bool acc) {
    mm(n, N, K, X, ldx, 1, Wt, dt, 1, K, Y, ldy, acc, s);
  };
  // dX[n][K] (+)= dY[n][N] W
  auto lin_dx = [&](int n, int N, int K, const float* dY, int64_t ldy, const void* Wt, float* dX, int64_t ldx, bool acc) {
    mm(n, K, N, dY, ldy, 1, Wt, dt, K, 1, dX, ldx, acc, s);
  };
  // dW[N][K] += dY^T X (rows summed in order)
  auto lin_dw = [&](int n, int N, int K, const float* dY, int64_t ldy, const float* X, int64_t ldx, float* dW) {
    if (dW) mm(N, K, n, dY, 1, ldy, X, 0, ldx, 1, dW, K, true, s);
  };

  // one transition of the n active rows at step t, keeping its activations in a
  auto step_forward = [&](int t, int n, const Act& a) {
    float *cat = a.cat, *rr = a.rr, *g = a.g, *wsr = a.wsr, *zin = a.zin, *hs = a.hs, *q = a.q, *o = a.o;
    float *zb = a.zb, *hm = a.hm, *qm = a.qm, *om = a.om, *za = a.za, *hd = a.hd, *ga = a.ga, *gu = a.gu;
    float* act = a.act;
    float *rs_s = a.rs, *rs_m = a.rs + (size_t)L * B, *rs_d = a.rs + (size_t)2 * L * B;
    const float* sp = S + (size_t)(t - 1) * Bd;
    gather_e(cat, 2 * d, io->e, dt, io->e_stride_b, io->e_stride_t, map, t, n, d, s);
    if (gated)
      rms_fwd(sp, d, m.merge_norm, cat + d, 2 * d, rr, n, d, c.rms_eps, s);
    else
      add(cat + d, 2 * d, sp, d, nullptr, 0, n, d, s);
    lin(n, d, 2 * d, cat, 2 * d, m.merge_wg, g, d, false);
    sigmoid_bias(g, d, m.merge_bg, n, d, s);
    if (gated) {
      lin(n, d, d, cat + d, 2 * d, m.merge_ws, wsr, d, false);
      merge_fwd(1, zin, cat, 2 * d, g, wsr, d, c.alpha, n, d, s);
    } else {
      merge_fwd(0, zin, cat, 2 * d, g, sp, d, c.alpha, n, d, s);
    }
    for (int l = 0; l < L; ++l) {
      const size_t o_l = (size_t)l * Bd;
      float* z = zin + o_l;
      // SWA [eqs. (2.12)-(2.14)]
      rms_fwd(z, d, m.norm_s[l], hs + o_l, d, rs_s + (size_t)l * B, n, d, c.rms_eps, s);
      float* kt = kt_at(KT, l, t);
      float* vt = kt_at(VT, l, t);
      lin(n, d, d, hs + o_l, d, m.wq[l], q + o_l, d, false);
      lin(n, d, d, hs + o_l, d, m.wk[l], kt, d, false);
      lin(n, d, d, hs + o_l, d, m.wv[l], vt, d, false);
      if (rope_on) {
        rope(q + o_l, d, n, d, dh, t, m.inv_freq, 1, s);
        rope(kt, d, n, d, dh, t, m.inv_freq, 1, s);
      }
      attn_fwd(q + o_l, d, trace_kv(l), std::max(1, t - W + 1), t, o + o_l, d, n, H, dh, s);
      add(zb + o_l, d, z, d, nullptr, 0, n, d, s);
      lin(n, d, d, o + o_l, d, m.wo[l], zb + o_l, d, true);
      // cross-attention to M_{<=t} [eq. (2.15)]
      rms_fwd(zb + o_l, d, m.norm_m[l], hm + o_l, d, rs_m + (size_t)l * B, n, d, c.rms_eps, s);
      lin(n, d, d, hm + o_l, d, m.wqm[l], qm + o_l, d, false);
      if (rope_on) rope(qm + o_l, d, n, d, dh, t, m.inv_freq, 1, s);
      attn_fwd(qm + o_l, d, mem_kv(l), 1, t, om + o_l, d, n, H, dh, s);
      add(za + o_l, d, zb + o_l, d, nullptr, 0, n, d, s);
      lin(n, d, d, om + o_l, d, m.wom[l], za + o_l, d, true);
      // SwiGLU FFN [eq. (2.16)]
      rms_fwd(za + o_l, d, m.norm_d[l], hd + o_l, d, rs_d + (size_t)l * B, n, d, c.rms_eps, s);
      lin(n, F, d, hd + o_l, d, m.w_gate[l], ga + (size_t)l * BF, F, false);
      lin(n, F, d, hd + o_l, d, m.w_up[l], gu + (size_t)l * BF, F, false);
      swiglu_fwd(ga + (size_t)l * BF, gu + (size_t)l * BF, act + (size_t)l * BF, n, F, s);
      add(zin + o_l + Bd, d, za + o_l, d, nullptr, 0, n, d, s);
      lin(n, d, F, act + (size_t)l * BF, F, m.w_down[l], zin + o_l + Bd, d, true);
    }
  };
  // readout [eq. (2.6)]: log p and its gradient w (onehot - softmax)
  auto readout = [&](int t, int n, float* logp_out, const Act& a) {
    const float* st = a.zin + (size_t)L * Bd;
    rms_fwd(st, d, m.out_norm, no, d, a.rs + (size_t)4 * L * B, n, d, c.rms_eps, s);
    lin(n, V, d, no, d, m.w_out, logits, V, false);
    logsoftmax_bwd(logits, V, io->tokens, io->tok_stride_b, io->w, io->w_stride_b, map, split, t, logp_out,
                   io->logp_stride_b, dlog, n, s);
  };

  // forward pass: s_t and the decoder keys/values of every step
  add(S, d, m.s_star, 0, nullptr, 0, B, d, s);
  for (int t = 1; t <= Tm; ++t) {
    const int n = n_at[t];
    const Act a = act_at(t);
    step_forward(t, n, a);
    add(S + (size_t)t * Bd, d, a.zin + (size_t)L * Bd, d, nullptr, 0, n, d, s);
    if (io->logp) readout(t, n, io->logp, a);
  }

  // backward pass
  for (int t = Tm; t >= 1; --t) {
    const int n = n_at[t];
    const Act a = act_at(t);
    if (!keep) step_forward(t, n, a);
    float *cat = a.cat, *rr = a.rr, *g = a.g, *wsr = a.wsr, *zin = a.zin, *hs = a.hs, *q = a.q, *o = a.o;
    float *zb = a.zb, *hm = a.hm, *qm = a.qm, *om = a.om, *za = a.za, *hd = a.hd, *ga = a.ga, *gu = a.gu;
    float* act = a.act;
    float *rs_s = a.rs, *rs_m = a.rs + (size_t)L * B, *rs_d = a.rs + (size_t)2 * L * B;
    float* rs_o = a.rs + (size_t)4 * L * B;
    add(dz, d, ds, d, nullptr, 0, n, d, s);  // dL/ds_t from step t+1 (zero rows past n_{t+1})
    const float* st = zin + (size_t)L * Bd;
    readout(t, n, nullptr, a);
    lin_dw(n, V, d, dlog, V, no, d, gr->w_out);
    lin_dx(n, V, d, dlog, V, m.w_out, t1, d, false);
    colsum(gr->out_norm, t1, d, st, d, rs_o, n, d, s);
    rms_bwd(st, d, m.out_norm, rs_o, t1, d, dz, d, n, d, true, s);
    for (int l = L - 1; l >= 0; --l) {
      const size_t o_l = (size_t)l * Bd;
      float* gal = ga + (size_t)l * BF;
      float* gul = gu + (size_t)l * BF;
      // FFN: z_out = za + W_down act
      lin_dx(n, d, F, dz, d, m.w_down[l], dF1, F, false);
      lin_dw(n, d, F, dz, d, act + (size_t)l * BF, F, layer_ptr(gr->w_down, l));
      swiglu_bwd(gal, gul, dF1, dF2, dF3, n, F, s);
      lin_dx(n, F, d, dF2, F, m.w_gate[l], t1, d, false);
      lin_dx(n, F, d, dF3, F, m.w_up[l], t1, d, true);
      lin_dw(n, F, d, dF2, F, hd + o_l, d, layer_ptr(gr->w_gate, l));
      lin_dw(n, F, d, dF3, F, hd + o_l, d, layer_ptr(gr->w_up, l));
      colsum(layer_ptr(gr->norm_d, l), t1, d, za + o_l, d, rs_d + (size_t)l * B, n, d, s);
      rms_bwd(za + o_l, d, m.norm_d[l], rs_d + (size_t)l * B, t1, d, dz, d, n, d, true, s);
      // cross-attention: za = zb + W_om om
      lin_dx(n, d, d, dz, d, m.wom[l], t1, d, false);
      lin_dw(n, d, d, dz, d, om + o_l, d, layer_ptr(gr->wom, l));
      DKV dm{};
      if (io->dmem_k) {
        const int gi = (l * G) / L;
        dm.k = io->dmem_k + (size_t)gi * io->dmem_stride_g;
        dm.v = io->dmem_v + (size_t)gi * io->dmem_stride_g;
        dm.s_row = io->dmem_stride_b;
        dm.s_pos = io->dmem_stride_t;
        dm.map = map;
      }
      attn_bwd(qm + o_l, d, mem_kv(l), 1, t, t1, d, dq, d, dm, n, H, dh, s);
      if (rope_on) rope(dq, d, n, d, dh, t, m.inv_freq, -1, s);
      lin_dx(n, d, d, dq, d, m.wqm[l], t2, d, false);
      lin_dw(n, d, d, dq, d, hm + o_l, d, layer_ptr(gr->wqm, l));
      colsum(layer_ptr(gr->norm_m, l), t2, d, zb + o_l, d, rs_m + (size_t)l * B, n, d, s);
      rms_bwd(zb + o_l, d, m.norm_m[l], rs_m + (size_t)l * B, t2, d, dz, d, n, d, true, s);
      // SWA: zb = z + W_o o; the window's keys/values take their gradients in the trace
      lin_dx(n, d, d, dz, d, m.wo[l], t1, d, false);
      lin_dw(n, d, d, dz, d, o + o_l, d, layer_ptr(gr->wo, l));
      DKV dtr{dKT + (size_t)l * LT, dVT + (size_t)l * LT, d, (int64_t)Bd, nullptr};
      attn_bwd(q + o_l, d, trace_kv(l), std::max(1, t - W + 1), t, t1, d, dq, d, dtr, n, H, dh, s);
      // the current key/value has now received the gradient of every step that read it
      float* dk = kt_at(dKT, l, t);
      float* dv = kt_at(dVT, l, t);
      if (rope_on) {
        rope(dq, d, n, d, dh, t, m.inv_freq, -1, s);
        rope(dk, d, n, d, dh, t, m.inv_freq, -1, s);
      }
      lin_dx(n, d, d, dq, d, m.wq[l], t2, d, false);
      lin_dx(n, d, d, dk, d, m.wk[l], t2, d, true);
      lin_dx(n, d, d, dv, d, m.wv[l], t2, d, true);
      lin_dw(n, d, d, dq, d, hs + o_l, d, layer_ptr(gr->wq, l));
      lin_dw(n, d, d, dk, d, hs + o_l, d, layer_ptr(gr->wk, l));
      lin_dw(n, d, d, dv, d, hs + o_l, d, layer_ptr(gr->wv, l));
      colsum(layer_ptr(gr->norm_s, l), t2, d, zin + o_l, d, rs_s + (size_t)l * B, n, d, s);
      rms_bwd(zin + o_l, d, m.norm_s[l], rs_s + (size_t)l * B, t2, d, dz, d, n, d, true, s);
    }
    // merge [eqs. (2.9)-(2.11)] back to e_t and s_{t-1}
    const float* sp = S + (size_t)(t - 1) * Bd;
    merge_bwd(gated ? 1 : 0, dz, cat, 2 * d, g, gated ? wsr : sp, d, c.alpha, dpre, dw, det, d, n, d, s);
    lin_dw(n, d, 2 * d, dpre, d, cat, 2 * d, gr->merge_wg);
    colsum(gr->merge_bg, dpre, d, nullptr, 0, nullptr, n, d, s);
    lin_dx(n, d, 2 * d, dpre, d, m.merge_wg, dcat, 2 * d, false);
    add(det, d, det, d, dcat, 2 * d, n, d, s);
    scatter_add_e(io->de, io->de_stride_b, io->de_stride_t, det, d, map, t, n, d, s);
    if (gated) {
      lin_dw(n, d, d, dw, d, cat + d, 2 * d, gr->merge_ws);
      lin_dx(n, d, d, dw, d, m.merge_ws, dcat + d, 2 * d, true);
      colsum(gr->merge_norm, dcat + d, 2 * d, sp, d, rr, n, d, s);
      rms_bwd(sp, d, m.merge_norm, rr, dcat + d, 2 * d, ds, d, n, d, false, s);
    } else {
      add(ds, d, dw, d, dcat + d, 2 * d, n, d, s);
    }
    if (t == 1) colsum(gr->s_star, ds, d, nullptr, 0, nullptr, n, d, s);
  }
  if (hipGetLastError() != hipSuccess || hipStreamSynchronize(s) != hipSuccess) {
    err = "replay backward kernels failed";
    return RLT_EHIP;
  }
  return RLT_OK;
}

}  // namespace bwd
}  // namespace rlt
