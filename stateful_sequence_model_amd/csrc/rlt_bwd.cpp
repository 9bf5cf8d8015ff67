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

  // Per-step values the backward pass reads: the step's activations and the
  // gradients that feed the weight-gradient products. Each is a field of
  // `nl` layers x slots x B rows x `width`, layer-major, so that one layer's
  // rows of consecutive steps are evenly strided. With one slot per step
  // (kept: the backward pass reads the forward pass's activations, and every
  // weight gradient is one product over all steps' rows at the end) when they
  // fit a quarter of the free device memory; else one slot that every step
  // overwrites (activations recomputed in the backward pass by the same
  // kernels, weight gradients accumulated step by step).
  struct Field {
    int nl;
    size_t width;
    float* base;
  };
  enum {
    CAT, RR, GG, WSR, ZIN, HS, Q, O, ZB, HM, QM, OM, ZA, HD, RS, GA, GU, ACT,  // activations
    NO, DLOG, DPRE, DWM, DZV, DF2, DF3, DQM, DQS,                            // weight-gradient operands
    T1O, T1D, T2M, T2S, DCAT, NFIELD                                         // gain-gradient operands
  };
  Field fl[NFIELD] = {
      {1, 2 * (size_t)d, nullptr}, {1, 1, nullptr}, {1, (size_t)d, nullptr}, {1, (size_t)d, nullptr},
      {L + 1, (size_t)d, nullptr},  // layer inputs; layer L: s_t
      {L, (size_t)d, nullptr}, {L, (size_t)d, nullptr}, {L, (size_t)d, nullptr}, {L, (size_t)d, nullptr},
      {L, (size_t)d, nullptr}, {L, (size_t)d, nullptr}, {L, (size_t)d, nullptr}, {L, (size_t)d, nullptr},
      {L, (size_t)d, nullptr},
      {4 * L + 1, 1, nullptr},  // rstd of RMSNorm_S (layers 0..L-1), _M (L..), _D (2L..), _o (4L)
      {L, (size_t)F, nullptr}, {L, (size_t)F, nullptr}, {L, (size_t)F, nullptr},
      {1, (size_t)d, nullptr}, {1, (size_t)V, nullptr}, {1, (size_t)d, nullptr}, {1, (size_t)d, nullptr},
      {3 * L + 1, (size_t)d, nullptr},  // dL/dz at each sublayer boundary of the step
      {L, (size_t)F, nullptr}, {L, (size_t)F, nullptr}, {L, (size_t)d, nullptr}, {L, (size_t)d, nullptr},
      {1, (size_t)d, nullptr}, {L, (size_t)d, nullptr}, {L, (size_t)d, nullptr}, {L, (size_t)d, nullptr},
      {1, 2 * (size_t)d, nullptr}};
  size_t per_step = 0;
  for (const Field& f : fl) per_step += (size_t)f.nl * B * f.width;
  bool keep = m.keep_acts == 2;
  if (m.keep_acts == 0) {
    size_t free_b = 0, total_b = 0;
    keep = hipMemGetInfo(&free_b, &total_b) == hipSuccess && (size_t)Tm * per_step * sizeof(float) <= free_b / 4;
  }
  const size_t nslot = keep ? (size_t)Tm : 1;
  float* fields = buf.f(nslot * per_step);
  {
    float* p = fields;
    for (Field& f : fl) {
      f.base = p;
      p += (size_t)f.nl * nslot * B * f.width;
    }
  }
  // layer l of field f at step t
  auto at = [&](int f, int l, int t) {
    const Field& x = fl[f];
    return x.base + ((size_t)l * nslot + (keep ? (size_t)(t - 1) : 0)) * B * x.width;
  };
  float* logits = buf.f((size_t)B * V);
  // gradient temporaries
  float* ds = buf.f(Bd);
  float* t1 = buf.f(Bd);
  float* dF1 = buf.f(BF);
  float* det = buf.f(Bd);
  if (!buf.ok) {
    (void)hipGetLastError();
    err = "work buffers of the replay backward do not fit";
    return RLT_ENOMEM;
  }
  // with one slot per step, rows past a step's active prefix are never
  // written: zero (S too), so that they add nothing to the sums over all slots
  if (hipMemcpyAsync(map, order.data(), B * sizeof(int), hipMemcpyHostToDevice, s) != hipSuccess ||
      hipMemcpyAsync(split, split_sorted.data(), B * sizeof(int), hipMemcpyHostToDevice, s) != hipSuccess ||
      hipMemsetAsync(dKT, 0, (size_t)L * Tm * Bd * sizeof(float), s) != hipSuccess ||
      hipMemsetAsync(dVT, 0, (size_t)L * Tm * Bd * sizeof(float), s) != hipSuccess ||
      hipMemsetAsync(fields, 0, nslot * per_step * sizeof(float), s) != hipSuccess ||
      hipMemsetAsync(S, 0, (size_t)(Tm + 1) * Bd * sizeof(float), s) != hipSuccess ||
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
  // Y[n][N] = base + X W^T (the residual add and the projection in one launch)
  auto lin_res = [&](int n, int N, int K, const float* X, int64_t ldx, const void* Wt, const float* base, float* Y,
                     int64_t ldy) { mm_base(n, N, K, X, ldx, 1, Wt, dt, 1, K, base, Y, ldy, s); };
  // dX[n][K] (+)= dY[n][N] W
  auto lin_dx = [&](int n, int N, int K, const float* dY, int64_t ldy, const void* Wt, float* dX, int64_t ldx, bool acc) {
    mm(n, K, N, dY, ldy, 1, Wt, dt, K, 1, dX, ldx, acc, s);
  };
  // dW[N][K] += dY^T X over n rows, in order
  auto lin_dw = [&](int64_t n, int N, int K, const float* dY, int64_t ldy, const float* X, int64_t ldx, float* dW) {
    if (dW) mm(N, K, (int)n, dY, 1, ldy, X, 0, ldx, 1, dW, K, true, s);
  };

  // one transition of the n active rows at step t, keeping its activations
  // in the step's slots
  auto step_forward = [&](int t, int n) {
    float* cat = at(CAT, 0, t);
    float* rr = at(RR, 0, t);
    float* g = at(GG, 0, t);
    float* wsr = at(WSR, 0, t);
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
      merge_fwd(1, at(ZIN, 0, t), cat, 2 * d, g, wsr, d, c.alpha, n, d, s);
    } else {
      merge_fwd(0, at(ZIN, 0, t), cat, 2 * d, g, sp, d, c.alpha, n, d, s);
    }
    for (int l = 0; l < L; ++l) {
      float* z = at(ZIN, l, t);
      float *hs = at(HS, l, t), *q = at(Q, l, t), *o = at(O, l, t), *zb = at(ZB, l, t);
      float *hm = at(HM, l, t), *qm = at(QM, l, t), *om = at(OM, l, t), *za = at(ZA, l, t), *hd = at(HD, l, t);
      float *ga = at(GA, l, t), *gu = at(GU, l, t), *act = at(ACT, l, t);
      // SWA [eqs. (2.12)-(2.14)]
      rms_fwd(z, d, m.norm_s[l], hs, d, at(RS, l, t), n, d, c.rms_eps, s);
      float* kt = kt_at(KT, l, t);
      float* vt = kt_at(VT, l, t);
      {  // q, k, v in one launch
        const void* wt[3] = {m.wq[l], m.wk[l], m.wv[l]};
        float* ys[3] = {q, kt, vt};
        mm_outputs(3, n, d, d, hs, d, 1, wt, dt, 1, d, ys, d, false, s);
      }
      if (rope_on) rope2(q, kt, d, n, d, dh, t, m.inv_freq, 1, s);
      attn_fwd(q, d, trace_kv(l), std::max(1, t - W + 1), t, o, d, n, H, dh, s);
      lin_res(n, d, d, o, d, m.wo[l], z, zb, d);
      // cross-attention to M_{<=t} [eq. (2.15)]
      rms_fwd(zb, d, m.norm_m[l], hm, d, at(RS, L + l, t), n, d, c.rms_eps, s);
      lin(n, d, d, hm, d, m.wqm[l], qm, d, false);
      if (rope_on) rope(qm, d, n, d, dh, t, m.inv_freq, 1, s);
      attn_fwd(qm, d, mem_kv(l), 1, t, om, d, n, H, dh, s);
      lin_res(n, d, d, om, d, m.wom[l], zb, za, d);
      // SwiGLU FFN [eq. (2.16)]
      rms_fwd(za, d, m.norm_d[l], hd, d, at(RS, 2 * L + l, t), n, d, c.rms_eps, s);
      {  // gate and up in one launch
        const void* wt[2] = {m.w_gate[l], m.w_up[l]};
        float* ys[2] = {ga, gu};
        mm_outputs(2, n, F, d, hd, d, 1, wt, dt, 1, d, ys, F, false, s);
      }
      swiglu_fwd(ga, gu, act, n, F, s);
      float* zn = at(ZIN, l + 1, t);
      lin_res(n, d, F, act, F, m.w_down[l], za, zn, d);
    }
  };
  // readout [eq. (2.6)]: log p and its gradient w (onehot - softmax)
  auto readout = [&](int t, int n, float* logp_out) {
    const float* st = at(ZIN, L, t);
    float* no = at(NO, 0, t);
    rms_fwd(st, d, m.out_norm, no, d, at(RS, 4 * L, t), n, d, c.rms_eps, s);
    lin(n, V, d, no, d, m.w_out, logits, V, false);
    logsoftmax_bwd(logits, V, io->tokens, io->tok_stride_b, io->w, io->w_stride_b, map, split, t, logp_out,
                   io->logp_stride_b, at(DLOG, 0, t), n, s);
  };
  // weight gradients: over every step's slot at once (t = 0, kept; rows past
  // a step's prefix are zero there, never written) or over the n_t active
  // rows of step t's slot
  auto weight_grads = [&](int t) {
    const int tt = t > 0 ? t : 1;
    const int64_t R = t > 0 ? (int64_t)n_at[t] : (int64_t)nslot * B;
    lin_dw(R, V, d, at(DLOG, 0, tt), V, at(NO, 0, tt), d, gr->w_out);
    for (int l = 0; l < L; ++l) {
      const int iv = 3 * (L - 1 - l);
      lin_dw(R, d, F, at(DZV, iv, tt), d, at(ACT, l, tt), F, layer_ptr(gr->w_down, l));
      lin_dw(R, F, d, at(DF2, l, tt), F, at(HD, l, tt), d, layer_ptr(gr->w_gate, l));
      lin_dw(R, F, d, at(DF3, l, tt), F, at(HD, l, tt), d, layer_ptr(gr->w_up, l));
      lin_dw(R, d, d, at(DZV, iv + 1, tt), d, at(OM, l, tt), d, layer_ptr(gr->wom, l));
      lin_dw(R, d, d, at(DQM, l, tt), d, at(HM, l, tt), d, layer_ptr(gr->wqm, l));
      lin_dw(R, d, d, at(DZV, iv + 2, tt), d, at(O, l, tt), d, layer_ptr(gr->wo, l));
      lin_dw(R, d, d, at(DQS, l, tt), d, at(HS, l, tt), d, layer_ptr(gr->wq, l));
      lin_dw(R, d, d, kt_at(dKT, l, tt), d, at(HS, l, tt), d, layer_ptr(gr->wk, l));
      lin_dw(R, d, d, kt_at(dVT, l, tt), d, at(HS, l, tt), d, layer_ptr(gr->wv, l));
    }
    lin_dw(R, d, 2 * d, at(DPRE, 0, tt), d, at(CAT, 0, tt), 2 * d, gr->merge_wg);
    if (gated) lin_dw(R, d, d, at(DWM, 0, tt), d, at(CAT, 0, tt) + d, 2 * d, gr->merge_ws);
  };

  // gain and bias gradients (column sums): step by step in the backward
  // pass (one slot), or over every step's slot at once (kept)
  auto colsum_at = [&](float* dst, const float* a, int64_t lda, const float* b, int64_t ldb, const float* rs, int n) {
    if (!keep) colsum(dst, a, lda, b, ldb, rs, n, d, s);
  };
  auto gain_grads = [&]() {
    const int64_t R = (int64_t)nslot * B;
    colsum_rows(gr->out_norm, at(T1O, 0, 1), d, at(ZIN, L, 1), d, at(RS, 4 * L, 1), R, d, s);
    for (int l = 0; l < L; ++l) {
      colsum_rows(layer_ptr(gr->norm_d, l), at(T1D, l, 1), d, at(ZA, l, 1), d, at(RS, 2 * L + l, 1), R, d, s);
      colsum_rows(layer_ptr(gr->norm_m, l), at(T2M, l, 1), d, at(ZB, l, 1), d, at(RS, L + l, 1), R, d, s);
      colsum_rows(layer_ptr(gr->norm_s, l), at(T2S, l, 1), d, at(ZIN, l, 1), d, at(RS, l, 1), R, d, s);
    }
    colsum_rows(gr->merge_bg, at(DPRE, 0, 1), d, nullptr, 0, nullptr, R, d, s);
    // s_{t-1} of step t is S[t - 1]: rows of S[0 .. Tm - 1] in step order
    if (gated) colsum_rows(gr->merge_norm, at(DCAT, 0, 1) + d, 2 * d, S, d, at(RR, 0, 1), R, d, s);
  };

  // forward pass: s_t and the decoder keys/values of every step
  add(S, d, m.s_star, 0, nullptr, 0, B, d, s);
  for (int t = 1; t <= Tm; ++t) {
    const int n = n_at[t];
    step_forward(t, n);
    add(S + (size_t)t * Bd, d, at(ZIN, L, t), d, nullptr, 0, n, d, s);
    if (io->logp) readout(t, n, io->logp);
  }

  // backward pass
  for (int t = Tm; t >= 1; --t) {
    const int n = n_at[t];
    if (!keep) step_forward(t, n);
    const float* st = at(ZIN, L, t);
    readout(t, n, nullptr);
    // dL/ds_t: from step t+1 (zero rows past n_{t+1}) and the readout
    float* dz0 = at(DZV, 0, t);
    add(dz0, d, ds, d, nullptr, 0, n, d, s);
    float* t1o = at(T1O, 0, t);
    lin_dx(n, V, d, at(DLOG, 0, t), V, m.w_out, t1o, d, false);
    colsum_at(gr->out_norm, t1o, d, st, d, at(RS, 4 * L, t), n);
    rms_bwd(st, d, m.out_norm, at(RS, 4 * L, t), t1o, d, dz0, d, n, d, true, s);
    for (int l = L - 1; l >= 0; --l) {
      // dL/dz entering the layer's FFN, cross-attention and SWA backward, and leaving it
      const int iv = 3 * (L - 1 - l);
      float *dzF = at(DZV, iv, t), *dzX = at(DZV, iv + 1, t), *dzS = at(DZV, iv + 2, t), *dzN = at(DZV, iv + 3, t);
      float *za = at(ZA, l, t), *zb = at(ZB, l, t), *z = at(ZIN, l, t);
      float *dF2 = at(DF2, l, t), *dF3 = at(DF3, l, t), *dqm = at(DQM, l, t), *dqs = at(DQS, l, t);
      // FFN: z_out = za + W_down act
      lin_dx(n, d, F, dzF, d, m.w_down[l], dF1, F, false);
      swiglu_bwd(at(GA, l, t), at(GU, l, t), dF1, dF2, dF3, n, F, s);
      float* t1d = at(T1D, l, t);
      {  // t1d = dF2 W_gate + dF3 W_up, one launch
        const float* dys[2] = {dF2, dF3};
        const void* wt[2] = {m.w_gate[l], m.w_up[l]};
        mm_summed(2, n, d, F, dys, F, 1, wt, dt, d, 1, t1d, d, false, s);
      }
      colsum_at(layer_ptr(gr->norm_d, l), t1d, d, za, d, at(RS, 2 * L + l, t), n);
      rms_bwd(za, d, m.norm_d[l], at(RS, 2 * L + l, t), t1d, d, dzX, d, n, d, false, s, dzF, d);
      // cross-attention: za = zb + W_om om
      lin_dx(n, d, d, dzX, d, m.wom[l], t1, d, false);
      DKV dm{};
      if (io->dmem_k) {
        const int gi = (l * G) / L;
        dm.k = io->dmem_k + (size_t)gi * io->dmem_stride_g;
        dm.v = io->dmem_v + (size_t)gi * io->dmem_stride_g;
        dm.s_row = io->dmem_stride_b;
        dm.s_pos = io->dmem_stride_t;
        dm.map = map;
      }
      attn_bwd(at(QM, l, t), d, mem_kv(l), 1, t, t1, d, dqm, d, dm, n, H, dh, s);
      if (rope_on) rope(dqm, d, n, d, dh, t, m.inv_freq, -1, s);
      float* t2m = at(T2M, l, t);
      lin_dx(n, d, d, dqm, d, m.wqm[l], t2m, d, false);
      colsum_at(layer_ptr(gr->norm_m, l), t2m, d, zb, d, at(RS, L + l, t), n);
      rms_bwd(zb, d, m.norm_m[l], at(RS, L + l, t), t2m, d, dzS, d, n, d, false, s, dzX, d);
      // SWA: zb = z + W_o o; the window's keys/values take their gradients in the trace
      lin_dx(n, d, d, dzS, d, m.wo[l], t1, d, false);
      DKV dtr{dKT + (size_t)l * LT, dVT + (size_t)l * LT, d, (int64_t)Bd, nullptr};
      attn_bwd(at(Q, l, t), d, trace_kv(l), std::max(1, t - W + 1), t, t1, d, dqs, d, dtr, n, H, dh, s);
      // the current key/value has now received the gradient of every step that read it
      float* dk = kt_at(dKT, l, t);
      float* dv = kt_at(dVT, l, t);
      if (rope_on) rope2(dqs, dk, d, n, d, dh, t, m.inv_freq, -1, s);
      float* t2s = at(T2S, l, t);
      {  // t2s = dq W_q + dk W_k + dv W_v, one launch
        const float* dys[3] = {dqs, dk, dv};
        const void* wt[3] = {m.wq[l], m.wk[l], m.wv[l]};
        mm_summed(3, n, d, d, dys, d, 1, wt, dt, d, 1, t2s, d, false, s);
      }
      colsum_at(layer_ptr(gr->norm_s, l), t2s, d, z, d, at(RS, l, t), n);
      rms_bwd(z, d, m.norm_s[l], at(RS, l, t), t2s, d, dzN, d, n, d, false, s, dzS, d);
    }
    // merge [eqs. (2.9)-(2.11)] back to e_t and s_{t-1}
    const float* dz = at(DZV, 3 * L, t);
    const float* sp = S + (size_t)(t - 1) * Bd;
    float* cat = at(CAT, 0, t);
    float* dpre = at(DPRE, 0, t);
    float* dw = at(DWM, 0, t);
    merge_bwd(gated ? 1 : 0, dz, cat, 2 * d, at(GG, 0, t), gated ? at(WSR, 0, t) : sp, d, c.alpha, dpre, dw, det, d,
              n, d, s);
    float* dcat = at(DCAT, 0, t);
    colsum_at(gr->merge_bg, dpre, d, nullptr, 0, nullptr, n);
    lin_dx(n, d, 2 * d, dpre, d, m.merge_wg, dcat, 2 * d, false);
    add(det, d, det, d, dcat, 2 * d, n, d, s);
    scatter_add_e(io->de, io->de_stride_b, io->de_stride_t, det, d, map, t, n, d, s);
    if (gated) {
      lin_dx(n, d, d, dw, d, m.merge_ws, dcat + d, 2 * d, true);
      colsum_at(gr->merge_norm, dcat + d, 2 * d, sp, d, at(RR, 0, t), n);
      rms_bwd(sp, d, m.merge_norm, at(RR, 0, t), dcat + d, 2 * d, ds, d, n, d, false, s);
    } else {
      add(ds, d, dw, d, dcat + d, 2 * d, n, d, s);
    }
    if (t == 1) colsum(gr->s_star, ds, d, nullptr, 0, nullptr, n, d, s);
    if (!keep) weight_grads(t);
  }
  if (keep) {
    weight_grads(0);
    gain_grads();
  }
  if (hipGetLastError() != hipSuccess || hipStreamSynchronize(s) != hipSuccess) {
    err = "replay backward kernels failed";
    return RLT_EHIP;
  }
  return RLT_OK;
}

}  // namespace bwd
}  // namespace rlt
