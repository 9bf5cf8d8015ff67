// Host side of the C ABI declared in include/rlt.h: validation, workspace,
// the launch sequence of one transition, the replay schedule and the
// captured-graph cache. No arithmetic of the method happens here; every
// step runs in the HIP kernels.
//
// Batch invariance: rows of one call are independent sequences ("Recurrent
// Looped Transformer" §4.1) and the report's exact-replay arguments (§3.1
// Prop. 3.1, App. A.4) assume deterministic operations. Every launch shape
// that fixes a reduction order (attention heads per workgroup and chunk
// length, the waves that split a product's K loop, K splits) is chosen from
// the configuration and the context's capacities (max_rows, max_ctx) only,
// never from the number of rows in a call, so a row's results do not depend
// on which other rows share its call. Shapes that leave the arithmetic of
// each output unchanged (row and column tiling) still follow the call.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <numeric>
#include <string>
#include <vector>

#include "../../include/rlt.h"
#include "../../include/rlt_debug.h"
#include "bwd.h"
#include "rlt_internal.h"

using namespace rlt;

// Duplicate-row counters of rlt_decoder_step_noalloc: a fixed device array
// (each device holds its own copy until the process ends). In host code this
// name is not a device address: host code uses the per-device address from
// hipGetSymbolAddress (g_scratch_ptr below), never the name itself.
static __device__ __align__(256) int scratch[RLT_NOALLOC_MAX_ROWS];

namespace {

thread_local char g_msg[512] = "";

// device address of `scratch` per device, resolved once per device (with the
// device current) by rlt_create
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
int* g_scratch_ptr[kMaxDevices] = {};

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_msg, sizeof(g_msg), fmt, ap);
  va_end(ap);
  return code;
}

#define HIP_TRY(expr)                                                                  \
  do {                                                                                 \
    hipError_t e_ = (expr);                                                            \
    if (e_ != hipSuccess) return fail(RLT_EHIP, "%s: %s", #expr, hipGetErrorString(e_)); \
  } while (0)

size_t elt_size(int dtype) { return dtype == RLT_BF16 ? 2 : 4; }

// Scratch of one transition pipeline (rows indexed by slot).
struct Workspace {
  void *X, *kc, *vc, *o, *h, *act;
  float *gbuf, *z, *q, *qm, *part, *partial, *logits;
  float* ssq;  // [d/2][M_pad] partial sums of squares of z (folded RMSNorm)
  int* xcnt;   // [M_pad][n_heads] cross-attention chunk arrival counters (zero between launches)
};


}  // namespace

struct rlt_ctx {
  rlt_config cfg;
  int device;      // the HIP device the context was created on
  int dt;          // 0 = f32, 1 = bf16
  size_t es;       // element size
  // parameters (caller-owned device memory)
  const float *s_star, *merge_norm, *merge_bg, *out_norm;
  const void *merge_wg, *merge_ws, *merge_ws_u, *merge_ws_v, *w_out;
  std::vector<const float*> norm_s, norm_m, norm_d;
  std::vector<const void*> wq, wk, wv, wo, wqm, wom, w_gate, w_up, w_down;
  // capacities and the launch shapes that fix reduction orders (chosen at
  // create from the config and the capacities; see the note at the top)
  int max_rows, max_ctx, M_pad;
  int chunk, nch;      // cross-attention positions per partial, partial slots per row
  int xcomb_mode;      // cross-attention chunks merged: 0 by call size, 1 combine kernel, 2 in the launch
  int one_row_pf;      // weight chunks in flight per wave of one-row products
  int bwd_keep;        // replay backward activations: 0 by size, 1 recomputed, 2 kept
  int hpw, hpw_x;      // attention heads per workgroup: SWA, cross-attention
  int narrow_rows;     // row count whose K splits the narrow product tile uses
  int gemm_target;     // K split target of the persistent step's products (0: stand-alone kernels)
  size_t partial_cap;  // floats per workspace
  // bf16: the decoder's weights in fragment order (a
  // library-owned copy, rebuilt by rlt_refresh_weights) and the products
  // that read them; the activations they multiply are then written in
  // fragment order by their producers
  bool pk_ready;
  std::vector<void*> pk_qkv, pk_wo, pk_wqm, pk_wom, pk_gu, pk_down;
  void* pk_out;
  void *pk_mwg, *pk_mws, *pk_mws_u, *pk_mws_v;  // merge products (null: not packed)
  // the operand-order products' activations carry two bf16 terms (x rounded,
  // then the rounding remainder) unless one_term; the second term of each
  // fragment-order buffer lies this many elements after the first
  bool one_term;
  int64_t lo_X, lo_o, lo_h, lo_act;
  // forced operand-order product shape (tuning sweeps): rows 32 * rb, waves,
  // chunks in flight, epilogue prefetch (-1: the library's choice); 0 = none
  int shape_rb, shape_cb, shape_lt, shape_pf, shape_pre;
  // duplicate-row detection of rlt_decoder_step: per state row, the number
  // of slots of the current call naming it (zero between calls)
  int* claim;
  int claim_cap;
  std::vector<std::pair<GemmArgs, void*>> pk_all;
  // persistent step for calls of at most fused_rows rows (bf16; 0 = off)
  int fused_rows;
  int fused_grid;      // workgroups = compute units
  int fused_target;    // workgroups a product aims to fill inside the persistent step
  int64_t fused_spin;  // barrier wait limit in s_memrealtime ticks
  unsigned* fused_sync;
  struct FusedEntry {
    std::vector<Phase> host;
    Phase* dev;
  };
  std::vector<FusedEntry> fused_cache;
  // encoder-memory construction scratch (allocated on first use)
  int mem_rows;        // rows per chunk (multiple of 128)
  void* mem_A;         // [mem_rows][d] product input
  float* mem_ssq;      // [mem_rows]
  int *mem_src, *mem_t;  // [mem_rows]
  int* mem_offs;       // [mem_B + 1] prefill schedule
  int* mem_lens;       // [mem_B]
  int mem_B;
  // shared device buffers
  int *t_row, *ident, *ones, *rows_buf, *src_buf, *split_buf, *last_buf;
  int* tick_dev;        // replay: the current tick, advanced on the device
  int replay_graph_min;  // replay: runs of at least this many ticks of one active set are captured (0: never)
  bool big_tile;         // the memory construction's K/V product on the 256 x 256 tile
  bool lt_dma;           // staged 64 x 128 product tile with its chunks copied straight into LDS
  double* inv_freq;
  float2* rope_tab;  // [rope_tmax + 1][d_head / 2] rotary (cos, sin)
  int rope_tmax;
  Workspace ws[1];
  // pinned host staging for replay schedules
  int* host_stage;
  // error word: host-mapped pinned memory written by kernels
  int* err_host;
  int* err_dev;
  // captured step graph
  hipGraph_t graph;
  hipGraphExec_t graph_exec;
  std::vector<unsigned char> graph_key;
  // optional per-kernel-class timing (HIP events on the launch stream)
  bool prof_on;
  std::vector<hipEvent_t> prof_ev;
  size_t prof_next;
  std::vector<std::pair<int, size_t>> prof_rec;  // (class, index of the start event)
};

namespace {
thread_local std::vector<Phase>* t_rec = nullptr;
}  // namespace

bool rlt::record_phase(const Phase& p) {
  if (!t_rec) return false;
  t_rec->push_back(p);
  return true;
}

namespace {

// Brackets the launches of one kernel class with two events when timing
// is on (never inside a graph capture, never while recording phases).
struct Prof {
  rlt_ctx* c;
  int kind;
  hipStream_t s;
  size_t i0 = 0;
  bool on;
  size_t take() {
    if (c->prof_next >= c->prof_ev.size()) {
      hipEvent_t e;
      if (hipEventCreate(&e) != hipSuccess) return (size_t)-1;
      c->prof_ev.push_back(e);
    }
    return c->prof_next++;
  }
  Prof(rlt_ctx* c_, int k, hipStream_t s_) : c(c_), kind(k), s(s_), on(c_->prof_on && !t_rec) {
    if (on) {
      i0 = take();
      if (i0 == (size_t)-1) on = false;
      else (void)hipEventRecord(c->prof_ev[i0], s);
    }
  }
  ~Prof() {
    if (!on) return;
    const size_t i1 = take();
    if (i1 != i0 + 1) return;
    (void)hipEventRecord(c->prof_ev[i1], s);
    c->prof_rec.push_back({kind, i0});
  }
};

int check_config(const rlt_config* c) {
  if (!c) return fail(RLT_EINVAL, "null config");
  if (c->n_layers < 1 || c->d_model < 1 || c->n_heads < 1 || c->d_head < 1 || c->window < 1 ||
      c->n_groups < 1 || c->d_ffn < 1 || c->vocab < 2)
    return fail(RLT_EINVAL, "config sizes must be positive");
  if (c->n_heads * c->d_head != c->d_model) return fail(RLT_ESHAPE, "d_model != n_heads * d_head");
  if (c->dtype != RLT_F32 && c->dtype != RLT_BF16) return fail(RLT_EINVAL, "dtype");
  if (c->merge_kind != RLT_MERGE_GATED && c->merge_kind != RLT_MERGE_CONVEX)
    return fail(RLT_EINVAL, "merge_kind");
  if (c->pos_kind != RLT_POS_NONE && c->pos_kind != RLT_POS_ROPE) return fail(RLT_EINVAL, "pos_kind");
  const int dh = c->d_head;
  if (dh != 16 && dh != 32 && dh != 64 && dh != 128)
    return fail(RLT_EUNSUPPORTED, "d_head %d not in {16,32,64,128}", dh);
  if (dh == 16 && c->dtype == RLT_BF16) return fail(RLT_EUNSUPPORTED, "d_head 16 needs RLT_F32");
  if (c->d_model % 32 || c->d_ffn % 32 || c->vocab % 32)
    return fail(RLT_EUNSUPPORTED, "d_model, d_ffn and vocab must be multiples of 32");
  if (c->n_groups != 1 && c->n_groups != c->n_layers)
    return fail(RLT_EUNSUPPORTED, "n_groups must be 1 or n_layers");
  if (!(c->rms_eps > 0.f) || !(c->rope_theta > 0.f)) return fail(RLT_EINVAL, "rms_eps, rope_theta");
  if (c->merge_gate != RLT_GATE_VECTOR && c->merge_gate != RLT_GATE_SCALAR) return fail(RLT_EINVAL, "merge_gate");
  if (c->merge_gate == RLT_GATE_SCALAR && c->merge_kind != RLT_MERGE_GATED)
    return fail(RLT_EUNSUPPORTED, "the scalar gate is implemented for the gated merge");
  if (c->merge_rank < 0 || c->merge_rank % 32 || c->merge_rank > c->d_ffn || c->merge_rank > c->d_model)
    return fail(RLT_EUNSUPPORTED, "merge_rank must be 0 or a multiple of 32 up to min(d_model, d_ffn)");
  if (c->merge_rank && c->merge_kind != RLT_MERGE_GATED) return fail(RLT_EINVAL, "merge_rank needs the gated merge");
  if (c->block_order < RLT_ORDER_SXF || c->block_order > RLT_ORDER_FXS) return fail(RLT_EINVAL, "block_order");
  return RLT_OK;
}

int elems_per_lane(int dt) { return dt == 1 ? 16 : 8; }

// heads per attention workgroup: hpw * (dh / E) lanes per key group, which
// must divide 256; default: the widest group of at most 32 lanes. A
// requested value (tuning) is used when valid.
bool hpw_ok(const rlt_config& c, int dt, int h) {
  const int lpk = c.d_head / elems_per_lane(dt);
  return h >= 1 && h <= c.n_heads && c.n_heads % h == 0 && 256 % (h * lpk) == 0;
}
int choose_hpw(const rlt_config& c, int dt, int requested) {
  if (requested > 0 && hpw_ok(c, dt, requested)) return requested;
  const int lpk = c.d_head / elems_per_lane(dt);
  int best = 1;
  for (int h = 1; h <= c.n_heads; ++h)
    if (hpw_ok(c, dt, h) && h * lpk <= 32) best = h;
  return best;
}

template <typename P>
int dev_alloc(P** p, size_t bytes) {
  void* v = nullptr;
  if (bytes == 0) bytes = 16;
  if (hipMalloc(&v, bytes) != hipSuccess) return fail(RLT_ENOMEM, "hipMalloc(%zu) failed", bytes);
  *p = (P*)v;
  return RLT_OK;
}

}  // namespace

// ----------------------------------------------------------------------------
// create / destroy / layout / errors
// ----------------------------------------------------------------------------

extern "C" const char* rlt_last_error(void) { return g_msg; }

extern "C" int rlt_state_layout(const rlt_config* cfg, int32_t B_cap, size_t bytes_out[5]) {
  int rc = check_config(cfg);
  if (rc) return rc;
  if (B_cap < 1 || !bytes_out) return fail(RLT_EINVAL, "B_cap < 1 or null output");
  const size_t es = elt_size(cfg->dtype);
  const size_t ring = (size_t)cfg->n_layers * B_cap * (size_t)(cfg->window - 1) * cfg->d_model * es;
  bytes_out[0] = (size_t)B_cap * cfg->d_model * sizeof(float);
  bytes_out[1] = ring;
  bytes_out[2] = ring;
  bytes_out[3] = (size_t)B_cap * sizeof(int32_t);
  bytes_out[4] = (size_t)B_cap * sizeof(int32_t);
  return RLT_OK;
}

extern "C" void rlt_destroy(rlt_ctx* c) {
  if (!c) return;
  std::vector<void*> ptrs = {c->t_row, c->ident, c->ones, c->rows_buf, c->src_buf, c->split_buf, c->last_buf,
                             c->tick_dev, c->inv_freq, c->rope_tab};
  for (Workspace& w : c->ws) {
    void* p[] = {w.X, w.kc, w.vc, w.o, w.h, w.act, w.gbuf, w.z, w.q, w.qm, w.part, w.partial, w.logits, w.ssq,
                 w.xcnt};
    ptrs.insert(ptrs.end(), std::begin(p), std::end(p));
  }
  for (void* p : ptrs)
    if (p) (void)hipFree(p);
  if (c->fused_sync) (void)hipFree(c->fused_sync);
  for (auto& e : c->pk_all) (void)hipFree(e.second);
  for (void* p : {c->mem_A, (void*)c->mem_ssq, (void*)c->mem_src, (void*)c->mem_t, (void*)c->mem_offs,
                  (void*)c->mem_lens})
    if (p) (void)hipFree(p);
  for (auto& e : c->fused_cache) (void)hipFree(e.dev);
  if (c->graph_exec) (void)hipGraphExecDestroy(c->graph_exec);
  if (c->graph) (void)hipGraphDestroy(c->graph);
  if (c->claim) (void)hipFree(c->claim);
  if (c->err_host) (void)hipHostFree(c->err_host);
  if (c->host_stage) (void)hipHostFree(c->host_stage);
  for (hipEvent_t e : c->prof_ev) (void)hipEventDestroy(e);
  delete c;
}

static int alloc_workspace(rlt_ctx* c, Workspace& w, bool full) {
  const rlt_config& cf = c->cfg;
  const size_t M = c->M_pad, es = c->es, d = cf.d_model, F = cf.d_ffn;
  const size_t nt = c->dt == 1 ? 2 : 1;  // bf16 product operands: room for a second term
  int rc = 0;
  if ((rc = dev_alloc(&w.X, nt * M * 2 * d * es)) || (rc = dev_alloc(&w.kc, M * d * es)) ||
      (rc = dev_alloc(&w.vc, M * d * es)) || (rc = dev_alloc(&w.o, nt * M * d * es)) ||
      (rc = dev_alloc(&w.h, nt * M * d * es)) || (rc = dev_alloc(&w.act, nt * M * F * es)) ||
      (rc = dev_alloc(&w.gbuf, M * d * 4)) || (rc = dev_alloc(&w.z, M * d * 4)) ||
      (rc = dev_alloc(&w.q, M * d * 4)) || (rc = dev_alloc(&w.qm, M * d * 4)) ||
      (rc = dev_alloc(&w.part, M * (size_t)c->nch * cf.n_heads * (cf.d_head + 2) * 4)) ||
      (rc = dev_alloc(&w.partial, c->partial_cap * 4)) ||
      (rc = dev_alloc(&w.logits, (full ? M : 16) * (size_t)cf.vocab * 4)) ||
      (rc = dev_alloc(&w.ssq, M * (size_t)(d / 2) * 4)) ||
      (rc = dev_alloc(&w.xcnt, M * (size_t)cf.n_heads * 4)))
    return rc;
  // rows beyond a call's n are read by the MFMA tiles and discarded: keep
  // them finite
  if (hipMemset(w.X, 0, nt * M * 2 * d * es) != hipSuccess || hipMemset(w.o, 0, nt * M * d * es) != hipSuccess ||
      hipMemset(w.h, 0, nt * M * d * es) != hipSuccess || hipMemset(w.act, 0, nt * M * F * es) != hipSuccess ||
      hipMemset(w.xcnt, 0, M * (size_t)cf.n_heads * 4) != hipSuccess)
    return fail(RLT_EHIP, "workspace initialisation failed");
  return RLT_OK;
}

// Fragment-order copies of the transition's product weights (bf16 contexts):
// one per product as the transition calls it (Q/K/V together, gate/up
// together), the merge's included. Weights not 16-byte aligned leave the
// copies unbuilt and those calls on the other tiles.
static int build_packed(rlt_ctx* c) {
  const rlt_config& cf = c->cfg;
  const int d = cf.d_model, F = cf.d_ffn, L = cf.n_layers, k = cf.merge_rank;
  const bool gated = cf.merge_kind == RLT_MERGE_GATED;
  const bool vec_gate = !gated || cf.merge_gate == RLT_GATE_VECTOR;
  std::vector<const void*> all = {c->w_out};
  for (auto* v : {&c->wq, &c->wk, &c->wv, &c->wo, &c->wqm, &c->wom, &c->w_gate, &c->w_up, &c->w_down})
    all.insert(all.end(), v->begin(), v->end());
  if (vec_gate) all.push_back(c->merge_wg);
  if (gated) {
    if (k > 0) {
      all.push_back(c->merge_ws_u);
      all.push_back(c->merge_ws_v);
    } else {
      all.push_back(c->merge_ws);
    }
  }
  for (const void* p : all)
    if ((uintptr_t)p % 16) return RLT_OK;
  auto pack = [&](std::initializer_list<const void*> W, int seg_rows, int K, int pairing, void** out) -> int {
    GemmArgs g{};
    int i = 0;
    for (const void* p : W) g.W[i++] = p;
    g.nseg = i;
    g.seg_rows = seg_rows;
    g.K = K;
    g.pairing = pairing;
    g.dh = cf.d_head;
    g.Nv = g.nseg * seg_rows;
    g.npairs = g.Nv / 32;
    int rc = dev_alloc(out, (size_t)g.Nv * K * 2);
    if (rc) return rc;
    c->pk_all.push_back({g, *out});
    launch_pack_weights(g, *out, nullptr);
    return RLT_OK;
  };
  for (auto* v : {&c->pk_qkv, &c->pk_wo, &c->pk_wqm, &c->pk_wom, &c->pk_gu, &c->pk_down}) v->assign(L, nullptr);
  int rc = 0;
  for (int l = 0; l < L && !rc; ++l) {
    if ((rc = pack({c->wq[l], c->wk[l], c->wv[l]}, d, d, PAIR_ROPE, &c->pk_qkv[l])) ||
        (rc = pack({c->wo[l]}, d, d, PAIR_PLAIN, &c->pk_wo[l])) ||
        (rc = pack({c->wqm[l]}, d, d, PAIR_ROPE, &c->pk_wqm[l])) ||
        (rc = pack({c->wom[l]}, d, d, PAIR_PLAIN, &c->pk_wom[l])) ||
        (rc = pack({c->w_gate[l], c->w_up[l]}, F, d, PAIR_DUAL, &c->pk_gu[l])) ||
        (rc = pack({c->w_down[l]}, d, F, PAIR_PLAIN, &c->pk_down[l])))
      break;
  }
  if (!rc) rc = pack({c->w_out}, cf.vocab, d, PAIR_PLAIN, &c->pk_out);
  // merge [eqs. (2.9)-(2.11)]: W_g over [e; r] (or [e; s]), W_s (or V then
  // U of a low-rank W_s; U needs a rank that is a multiple of 64)
  if (!rc && vec_gate) rc = pack({c->merge_wg}, d, 2 * d, PAIR_PLAIN, &c->pk_mwg);
  if (!rc && gated && k == 0) rc = pack({c->merge_ws}, d, d, PAIR_PLAIN, &c->pk_mws);
  if (!rc && gated && k > 0) rc = pack({c->merge_ws_v}, k, d, PAIR_PLAIN, &c->pk_mws_v);
  if (!rc && gated && k > 0 && k % 64 == 0) rc = pack({c->merge_ws_u}, d, k, PAIR_PLAIN, &c->pk_mws_u);
  if (rc) return rc;
  HIP_TRY(hipGetLastError());
  HIP_TRY(hipDeviceSynchronize());
  c->pk_ready = true;
  return RLT_OK;
}

extern "C" int rlt_refresh_weights(rlt_ctx* c, uint64_t weights_version, void* stream) {
  if (!c) return fail(RLT_EINVAL, "null context");
  if (weights_version == c->cfg.weights_version)
    return fail(RLT_EINVAL, "changed weights need a new weights_version (the context has %llu)",
                (unsigned long long)weights_version);
  for (auto& e : c->pk_all) launch_pack_weights(e.first, e.second, (hipStream_t)stream);
  HIP_TRY(hipGetLastError());
  c->cfg.weights_version = weights_version;
  return RLT_OK;
}

// Attention heads per workgroup for calls of up to `rows` rows: the widest
// valid group h, narrowed (down to one head) while such a call would have
// fewer than `want` workgroups per key range, so that contexts for small
// calls spread their keys over more compute units. SWA: 256 (batch 1 at
// t ~ 2048: 4.43 -> 4.09 ms per step, batch 16: 6.25 -> 5.91); cross-
// attention, whose chunks multiply its workgroups: 128 (narrower measured
// slower at 16 rows, 6.05 vs 5.92 ms, and faster at one row, 4.02 vs 4.09).
static int narrow_hpw(const rlt_config& cf, int dt, int h, int rows, int want) {
  for (int k = h - 1; k >= 1 && (int64_t)rows * (cf.n_heads / h) < want; --k)
    if (hpw_ok(cf, dt, k)) h = k;
  return h;
}

// Memory positions per cross-attention partial for calls of up to `rows`
// rows: few long workgroups stream faster than many short ones (each pays a
// start-up latency and a merge), so the chunk grows with the rows while the
// grid still fills the chip at mid context (reference depth, t = 2048: 128
// rows 14.7 ms per step with 2048 against 15.4 with 512; 64 rows best at
// 1024, 16 at 512, 1 at 256). One chunk of the whole context up to 4096
// positions when there are enough workgroups: no combine launch.
static int pick_chunk(int wg_per_chunk, int max_ctx) {
  if (wg_per_chunk >= 1024) return max_ctx <= 4096 ? 4096 : 2048;
  return wg_per_chunk >= 512 ? 1024 : wg_per_chunk >= 128 ? 512 : 256;
}

// The device address of the allocation-free step's counters on `dev` (the
// current device), resolved on the first context created there.
static int resolve_scratch(int dev) {
  if (dev < 0 || dev >= kMaxDevices) return fail(RLT_EUNSUPPORTED, "device %d beyond %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (g_scratch_ptr[dev]) return RLT_OK;
  void* p = nullptr;
  const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  if (e != hipSuccess || !p) return fail(RLT_EHIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
  g_scratch_ptr[dev] = (int*)p;
  return RLT_OK;
}

static int create_ctx(const rlt_config* cfg, const rlt_weights* w, int32_t max_rows, int32_t max_ctx,
                      const rlt_dbg_launch* opt, rlt_ctx** out) {
  int rc = check_config(cfg);
  if (rc) return rc;
  if (!w || !out) return fail(RLT_EINVAL, "null weights or output");
  if (max_rows < 1 || max_rows > 65536 || max_ctx < 1) return fail(RLT_EINVAL, "max_rows/max_ctx");
  const int L = cfg->n_layers;
  const bool gated = cfg->merge_kind == RLT_MERGE_GATED;
  const bool low_rank = cfg->merge_rank > 0;
  if (!w->s_star || !w->merge_wg || !w->merge_bg || !w->out_norm || !w->w_out ||
      (gated && (!w->merge_norm || (low_rank ? (!w->merge_ws_u || !w->merge_ws_v) : !w->merge_ws))))
    return fail(RLT_EINVAL, "missing global weight");
  const void* const* per[] = {(const void* const*)w->norm_s, w->wq, w->wk, w->wv, w->wo,
                              (const void* const*)w->norm_m, w->wqm, w->wom,
                              (const void* const*)w->norm_d, w->w_gate, w->w_up, w->w_down};
  for (auto arr : per) {
    if (!arr) return fail(RLT_EINVAL, "missing per-layer weight array");
    for (int l = 0; l < L; ++l)
      if (!arr[l]) return fail(RLT_EINVAL, "missing per-layer weight of layer %d", l);
  }
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(RLT_EHIP, "hipGetDevice failed");
  if ((rc = resolve_scratch(dev))) return rc;
  rlt_ctx* c = new rlt_ctx();  // value-initialised: every pointer starts null
  c->cfg = *cfg;
  c->device = dev;
  c->dt = cfg->dtype == RLT_BF16 ? 1 : 0;
  c->es = elt_size(cfg->dtype);
  c->s_star = w->s_star;
  c->merge_norm = w->merge_norm;
  c->merge_bg = w->merge_bg;
  c->out_norm = w->out_norm;
  c->merge_wg = w->merge_wg;
  c->merge_ws = w->merge_ws;
  c->merge_ws_u = w->merge_ws_u;
  c->merge_ws_v = w->merge_ws_v;
  c->w_out = w->w_out;
  c->norm_s.assign(w->norm_s, w->norm_s + L);
  c->norm_m.assign(w->norm_m, w->norm_m + L);
  c->norm_d.assign(w->norm_d, w->norm_d + L);
  c->wq.assign(w->wq, w->wq + L);
  c->wk.assign(w->wk, w->wk + L);
  c->wv.assign(w->wv, w->wv + L);
  c->wo.assign(w->wo, w->wo + L);
  c->wqm.assign(w->wqm, w->wqm + L);
  c->wom.assign(w->wom, w->wom + L);
  c->w_gate.assign(w->w_gate, w->w_gate + L);
  c->w_up.assign(w->w_up, w->w_up + L);
  c->w_down.assign(w->w_down, w->w_down + L);

  const int d = cfg->d_model, F = cfg->d_ffn, dh = cfg->d_head;
  c->max_rows = max_rows;
  c->max_ctx = max_ctx;
  c->M_pad = (max_rows + 127) / 128 * 128;
  // launch shapes that fix reduction orders: from the config and the
  // capacities only (batch invariance); `opt` overrides them for tests
  const rlt_dbg_launch o = opt ? *opt : rlt_dbg_launch{};
  c->hpw = hpw_ok(*cfg, c->dt, o.swa_hpw) ? o.swa_hpw
                                           : narrow_hpw(*cfg, c->dt, choose_hpw(*cfg, c->dt, 0), max_rows, 256);
  c->hpw_x = hpw_ok(*cfg, c->dt, o.xattn_hpw) ? o.xattn_hpw
                                                : narrow_hpw(*cfg, c->dt, choose_hpw(*cfg, c->dt, 2), max_rows, 128);
  c->chunk = (o.xattn_chunk >= 16 && o.xattn_chunk <= 4096) ? o.xattn_chunk
                                                            : pick_chunk(max_rows * (cfg->n_heads / c->hpw_x), max_ctx);
  c->nch = (max_ctx + c->chunk - 1) / c->chunk;
  c->narrow_rows = std::min(max_rows, 32);
  c->gemm_target = 0;
  // Opt-in only: on MI355X a device-scope grid barrier costs 3.5-8.7 us,
  // so ~15 phases per block make the persistent step slower than the
  // separate kernels at every batch size measured (1-16 rows).
  c->fused_rows = c->dt == 1 ? std::min(32, std::max(0, (int)o.fused_rows)) : 0;
  c->fused_spin = (int64_t)200000000;  // 2 s of the 100 MHz real-time counter
  c->partial_cap = (size_t)8 * c->M_pad * std::max(3 * d, 2 * F);
  const size_t M = c->M_pad;

#define ALLOC(p, bytes)                     \
  do {                                      \
    int r_ = dev_alloc(&(p), (bytes));      \
    if (r_) { rlt_destroy(c); return r_; }  \
  } while (0)
  ALLOC(c->t_row, M * 4);
  ALLOC(c->ident, M * 4);
  ALLOC(c->ones, M * 4);
  ALLOC(c->rows_buf, M * 4);
  ALLOC(c->src_buf, M * 4);
  ALLOC(c->split_buf, M * 4);
  ALLOC(c->last_buf, M * 4);
  ALLOC(c->tick_dev, 4);
  ALLOC(c->inv_freq, (size_t)(dh / 2) * sizeof(double));
  c->rope_tmax = std::min(max_ctx, 65536);  // positions past it compute their angles
  ALLOC(c->rope_tab, (size_t)(c->rope_tmax + 1) * (dh / 2) * sizeof(float2));
#undef ALLOC
  if ((rc = alloc_workspace(c, c->ws[0], true))) {
    rlt_destroy(c);
    return rc;
  }
  std::vector<int> iv(M), ov(M, 1);
  std::iota(iv.begin(), iv.end(), 0);
  std::vector<double> fr(dh / 2);
  for (int i = 0; i < dh / 2; ++i) fr[i] = std::pow((double)cfg->rope_theta, -2.0 * i / dh);
  if (hipMemcpy(c->ident, iv.data(), M * 4, hipMemcpyHostToDevice) != hipSuccess ||
      hipMemcpy(c->ones, ov.data(), M * 4, hipMemcpyHostToDevice) != hipSuccess ||
      hipMemcpy(c->inv_freq, fr.data(), fr.size() * sizeof(double), hipMemcpyHostToDevice) != hipSuccess) {
    rlt_destroy(c);
    return fail(RLT_EHIP, "workspace initialisation failed");
  }
  launch_rope_table(c->inv_freq, dh, c->rope_tmax, c->rope_tab, nullptr);
  if (hipGetLastError() != hipSuccess || hipDeviceSynchronize() != hipSuccess) {
    rlt_destroy(c);
    return fail(RLT_EHIP, "rotary table initialisation failed");
  }
  if (hipHostMalloc((void**)&c->err_host, sizeof(int), hipHostMallocMapped) != hipSuccess ||
      hipHostGetDevicePointer((void**)&c->err_dev, c->err_host, 0) != hipSuccess) {
    rlt_destroy(c);
    return fail(RLT_EHIP, "pinned error word allocation failed");
  }
  *(volatile int*)c->err_host = 0;
  if (c->fused_rows > 0) {
    int dev = 0, ncu = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || ncu < 1 ||
        fused_blocks_per_cu() < 1)
      c->fused_rows = 0;  // no persistent path on this device: separate kernels only
    c->fused_grid = ncu;
    c->fused_target = c->fused_grid;
  }
  if (c->fused_rows > 0 && (dev_alloc(&c->fused_sync, 2 * sizeof(unsigned)) != RLT_OK ||
                            hipMemset(c->fused_sync, 0, 2 * sizeof(unsigned)) != hipSuccess)) {
    rlt_destroy(c);
    return fail(RLT_EHIP, "barrier word allocation failed");
  }
  if (hipHostMalloc((void**)&c->host_stage, (M * 4 + 16) * 4, hipHostMallocDefault) != hipSuccess) {
    rlt_destroy(c);
    return fail(RLT_EHIP, "pinned staging allocation failed");
  }
  if (c->dt == 1 && d % 64 == 0 && F % 64 == 0 && !o.no_packed) {
    if ((rc = build_packed(c))) {
      rlt_destroy(c);
      return rc;
    }
  }
  c->one_term = o.one_term != 0;
  c->replay_graph_min = o.replay_graph_min < 0 ? 0 : (o.replay_graph_min > 0 ? o.replay_graph_min : 4);
  c->big_tile = o.no_big_tile == 0;
  c->lt_dma = o.no_lt_dma == 0;
  c->xcomb_mode = (o.xattn_combine_kernel >= 0 && o.xattn_combine_kernel <= 2) ? o.xattn_combine_kernel : 0;
  c->one_row_pf = (o.one_row_pf >= 2 && o.one_row_pf <= 4) ? o.one_row_pf : 2;
  c->bwd_keep = (o.bwd_activations >= 0 && o.bwd_activations <= 2) ? o.bwd_activations : 0;
  if (c->pk_ready && !c->one_term) {
    c->lo_X = (int64_t)M * 2 * d;
    c->lo_o = c->lo_h = (int64_t)M * d;
    c->lo_act = (int64_t)M * F;
  }
  *out = c;
  return RLT_OK;
}

extern "C" int rlt_create(const rlt_config* cfg, const rlt_weights* w, int32_t max_rows, int32_t max_ctx,
                          rlt_ctx** out) {
  return create_ctx(cfg, w, max_rows, max_ctx, nullptr, out);
}

extern "C" int rlt_dbg_create(const rlt_config* cfg, const rlt_weights* w, int32_t max_rows, int32_t max_ctx,
                              const rlt_dbg_launch* opt, rlt_ctx** out) {
  if (!opt) return fail(RLT_EINVAL, "null launch options");
  return create_ctx(cfg, w, max_rows, max_ctx, opt, out);
}

// a device-detected error from earlier work, if any (cleared when returned)
static int take_device_error(rlt_ctx* c) {
  const int e = *(volatile int*)c->err_host;
  if (e) {
    *(volatile int*)c->err_host = 0;
    if (e == RLT_EHIP && c->fused_sync) {
      // a persistent step gave up at a barrier: rearm the barrier words
      (void)hipDeviceSynchronize();
      (void)hipMemset(c->fused_sync, 0, 2 * sizeof(unsigned));
      (void)hipDeviceSynchronize();
      return fail(e, "device-detected error from an earlier call: a persistent step timed out at a barrier");
    }
    return fail(e, "device-detected error from an earlier call (code %d): rows were skipped", e);
  }
  return RLT_OK;
}

extern "C" int rlt_sync_error(rlt_ctx* c, void* stream) {
  if (!c) return fail(RLT_EINVAL, "null context");
  HIP_TRY(hipStreamSynchronize((hipStream_t)stream));
  return take_device_error(c);
}

// ----------------------------------------------------------------------------
// matrix product wrapper: picks the tile height and K split for the bf16 path
// ----------------------------------------------------------------------------

namespace {

struct Gemm {
  rlt_ctx* c;
  const Workspace* w;
  hipStream_t s;
  int m_pad = 0;       // rows allocated in A (default: the context's M_pad)
  int ssq_units = 0;   // units of ssq_in (default: the decoder producers' units)

  // Wp: the weights in fragment order; A is then in fragment order too
  void run(const void* A, int64_t lda, std::initializer_list<const void*> W, int seg_rows, int K, int pairing,
           int n, EpiArgs e, const float* ssq_in = nullptr, float* ssq_out = nullptr, const void* Wp = nullptr,
           int64_t a_lo = 0) {
    GemmArgs g{};
    g.A = A;
    g.lda = lda;
    g.a_lo = Wp ? a_lo : 0;
    int i = 0;
    for (const void* p : W) g.W[i++] = p;
    g.nseg = i;
    g.seg_rows = seg_rows;
    g.K = K;
    g.pairing = pairing;
    g.dh = c->cfg.d_head;
    g.M = n;
    g.M_pad = m_pad ? m_pad : c->M_pad;
    g.Nv = g.nseg * seg_rows;
    g.npairs = g.Nv / 32;
    g.S = 1;
    g.mb = 1;
    g.kslice = (K + 4 * 32 - 1) / (4 * 32) * 32;
    g.partial = w->partial;
    g.ssq_in = ssq_in;
    g.ssq_out = ssq_out;
    g.ssq_units = ssq_units ? ssq_units : c->cfg.d_model / (c->dt == 1 ? 32 : 2);  // producers' column units
    g.inv_d = 1.0f / (float)c->cfg.d_model;
    g.eps = c->cfg.rms_eps;
    if (Wp) {
      // tile shape (none of these choices changes the arithmetic: fixed
      // stream order, see the kernels), measured per product at 1, 128, 256
      // and 512 rows, reference depth: calls of more than 64 rows whose
      // products have at least 96 staged tiles of 128 rows x 64 columns
      // (64 with K of 4096 or more) take the staged tile (64 x 128 where the
      // columns allow), in one workgroup per tile from 150 tiles, else split
      // over two stream groups (four below 96 tiles); the others the
      // register tile of 32 rows, two chunks in flight per wave (three or
      // four past 32 rows measured no faster: 64 rows 13.64 / 13.70 / 13.74
      // ms per step with 2 / 3 / 4, 128 rows 21.73 / 21.75 / 21.77)
      g.Wp = Wp;
      g.rb = 1;
      g.cb = 1;
      g.pre = -1;
      g.pf = 2;
      g.lt_groups = 0;
      g.lt_rbk = 4;
      g.lt_dma = c->lt_dma ? 1 : 0;
      // one-row calls: activations staged in LDS (the K loop then issues
      // weight loads only; at 4 and 8 rows measured slower)
      g.a_lds = (n == 1 && K / 64 <= PK_LDS_CHUNKS) ? 1 : 0;
      if (g.a_lds) g.pf = c->one_row_pf;
      if (n > 64 && g.npairs % 2 == 0) {
        const int tiles = g.npairs / 2 * ((n + 127) / 128);  // counted in 128 x 64 tiles
        if (tiles >= 96 || (tiles >= 64 && K >= 4096)) g.lt_groups = tiles >= 150 ? 1 : tiles >= 96 ? 2 : 4;
        while (g.lt_groups > 1 && (size_t)g.lt_groups * g.M_pad * g.Nv > c->partial_cap) g.lt_groups /= 2;
        // tiles of 64 rows x 4 column pairs where the columns allow: the same
        // workgroups move a fifth less through LDS per chunk (measured faster
        // for Q/K/V, gate/up and the vocabulary at 128 rows)
        if (g.lt_groups > 0 && g.npairs % 4 == 0) g.lt_rbk = 2;
      }
      // register tile past 128 rows: two column pairs per workgroup while one
      // pair would need more than 256 workgroups (256 rows, 2048-wide: one
      // round of 256 workgroups instead of two of 256, and half the
      // activation re-reads; measured 16 -> 13 us per product)
      if (g.lt_groups == 0 && n > 128 && g.npairs % 2 == 0 && (n + 31) / 32 * g.npairs > 256) {
        g.cb = 2;
        g.pf = 2;
      }
      if (c->shape_rb > 0) {
        if (c->shape_lt > 0) {
          const int lcb = c->shape_cb == 4 ? 4 : 2;  // column pairs per staged tile
          if (g.npairs % lcb == 0 && (size_t)c->shape_lt * g.M_pad * g.Nv <= c->partial_cap) {
            g.lt_groups = c->shape_lt;
            g.lt_rbk = 8 / lcb;
            g.a_lds = 0;
          }
        } else if (g.npairs % c->shape_cb == 0) {
          g.lt_groups = 0;
          g.a_lds = 0;
          g.rb = c->shape_rb;
          g.cb = c->shape_cb;
          g.pf = c->shape_pf;
          g.pre = c->shape_pre;
        }
      }
    } else if (c->dt == 1 && n > 32 && g.npairs % 2 == 0 && K % 64 == 0) {
      // LDS tile of 128 rows x 64 columns (128 when that still leaves two
      // workgroups per compute unit); K split while each split adds a
      // workgroup per compute unit and keeps at least 8 stages of 64
      // (measured best for every product shape at 64-256 rows). The split,
      // which fixes the summation order, is taken for a call of the
      // context's capacity (mt_cap row tiles); the column tile follows the call.
      const int mt = (n + 127) / 128, mt_cap = (std::max(c->max_rows, 33) + 127) / 128;
      const int BN = (g.npairs % 4 == 0 && g.npairs / 2 * mt >= 512) ? 128 : 64;
      const int BN_cap = (g.npairs % 4 == 0 && g.npairs / 2 * mt_cap >= 512) ? 128 : 64;
      const int tiles = g.npairs / (BN_cap / 32) * mt_cap;
      const int kst = K / 64;
      int S = std::max(1, 256 / tiles);
      S = std::min(S, std::max(1, kst / 8));
      while (S > 1 && (size_t)S * g.M_pad * g.Nv > c->partial_cap) --S;
      g.wide = BN;
      g.S = S;
      g.kslice = (kst + S - 1) / S * 64;
      // the memory construction's K/V product (16-byte runs, no split, at
      // least 256 rows): tiles of 256 x 256 with 128 x 64 per wave
      if (BN == 128 && S == 1 && e.kind == EPI_MEMKV && e.mem_vec && g.npairs % 8 == 0 && n >= 256 &&
          c->big_tile)
        g.wide = 256;
    } else if (c->dt == 1) {
      narrow_plan(n, g.npairs, K, c->narrow_rows, c->gemm_target, g.M_pad, g.Nv, c->partial_cap, g.S, g.mb,
                  g.kslice);
    }
    Prof pf(c, RLT_PROF_GEMM, s);
    launch_gemm(c->dt, g, e, s);
  }
};

struct StepPlan {
  Rows R;                 // rows / src / t_row (t_row filled by the pre-step)
  int n;
  int* claim;             // decoder step: per-row slot counts (duplicate rows), else null
  EIn e;
  rlt_memory mem;
  rlt_state* st;
  // outputs (slot-indexed pointers start at this plan's first slot)
  float* s_out;
  float* s_trace;
  int64_t s_trace_sb;
  float* z_trace;         // [L][z_trace_ld][d], this plan's rows at z_trace
  int z_trace_ld;
  bool need_logits;
  float* logits;          // caller's [n][V] or null (workspace)
  ReadoutArgs ro;
  bool do_readout;
};

// the transition for the plan's slots: merge, L_D blocks, final norm, readout
void enqueue_transition(rlt_ctx* c, const Workspace& w, const StepPlan& P, hipStream_t s) {
  const rlt_config& cf = c->cfg;
  const int d = cf.d_model, F = cf.d_ffn, H = cf.n_heads, dh = cf.d_head, L = cf.n_layers;
  const int n = P.n;
  const size_t es = c->es;
  Gemm gm{c, &w, s};

  // bf16 calls run the fragment-order products (except calls taken by the
  // opt-in persistent step, which runs the narrow tile): every producer of
  // their activations (residual / merge epilogues, SwiGLU, attention outputs)
  // then writes in fragment order
  const bool pk = c->pk_ready && !(c->fused_rows > 0 && n <= c->fused_rows);
  auto pw = [&](const std::vector<void*>& v, int l) -> const void* { return pk ? v[l] : nullptr; };

  // second terms of the fragment-order operands (none off the operand-order path)
  const int64_t lo_X = pk ? c->lo_X : 0, lo_o = pk ? c->lo_o : 0, lo_h = pk ? c->lo_h : 0,
                lo_act = pk ? c->lo_act : 0;
  EpiArgs E0{};
  E0.pk = pk ? 1 : 0;
  E0.lo = lo_h;  // the producers' output, the next norm's input w.h
  E0.rows = P.R;
  E0.d = d;
  E0.dh = dh;
  E0.H = H;
  E0.rope = cf.pos_kind == RLT_POS_ROPE;
  E0.inv_freq = c->inv_freq;
  E0.rope_tab = c->rope_tab;
  E0.rope_tmax = c->rope_tmax;
  E0.alpha = cf.alpha;
  E0.e = P.e;
  E0.s_state = P.st->s;

  MiscArgs m{};
  m.rows = P.R;
  m.n = n;
  m.d = d;
  m.eps = cf.rms_eps;
  m.s_state = P.st->s;
  m.e = P.e;
  m.merge_kind = cf.merge_kind;
  m.err = c->err_dev;

  // Sublayer order of every block [RLT §2.5, text after eq. (2.16)]: kinds
  // 0 = SWA, 1 = cross-attention, 2 = FFN, each with its own pre-norm.
  static const int kOrders[6][3] = {{0, 1, 2}, {0, 2, 1}, {1, 0, 2}, {1, 2, 0}, {2, 0, 1}, {2, 1, 0}};
  const int* order = kOrders[cf.block_order];
  auto gain_of = [&](int l, int kind) -> const float* {
    if (l >= L) return c->out_norm;  // after the last block: RMSNorm_o of the readout [eq. (2.6)]
    return kind == 0 ? c->norm_s[l] : kind == 1 ? c->norm_m[l] : c->norm_d[l];
  };

  // ---- merge [eqs. (2.9)-(2.11)] ----
  // Every RMSNorm is folded into the matrix products: the producer of z
  // (merge or residual epilogue) writes z * gain_next into w.h and per-row
  // partial sums of squares into w.ssq; the consumer scales by rstd.
  const bool scalar_gate = cf.merge_gate == RLT_GATE_SCALAR;
  m.gain = c->merge_norm;
  m.out = w.X;
  m.ld_out = 2 * d;
  m.wg = scalar_gate ? c->merge_wg : nullptr;   // scalar gate: computed with the merge input
  m.bg = c->merge_bg;
  m.gbuf = w.gbuf;
  // operand-order merge products: X = [e; r] (or [e; s]) and r alone are
  // written in fragment order ([n][2d] and [n][d]); r alone goes to w.o,
  // which the blocks use only later
  m.pk = pk ? 1 : 0;
  m.out2 = w.o;
  m.lo = lo_X;
  m.lo2 = lo_o;
  m.claim = P.claim;
  { Prof pf(c, RLT_PROF_NORM, s); launch_merge_prep(c->dt, m, s); }
  auto mw = [&](void* p) -> const void* { return pk ? p : nullptr; };
  auto producer = [&](EpiArgs e, const float* gnext) {
    e.gnext = gnext;
    e.zb = w.h;
    return e;
  };
  const float* g_first = gain_of(0, order[0]);
  if (cf.merge_kind == RLT_MERGE_GATED) {
    EpiArgs e = E0;
    if (!scalar_gate) {
      e.kind = EPI_MGATE;
      e.out_f = w.gbuf;
      e.ldo = d;
      e.bias = c->merge_bg;
      gm.run(w.X, 2 * d, {c->merge_wg}, d, 2 * d, PAIR_PLAIN, n, e, nullptr, nullptr, mw(c->pk_mwg), lo_X);
    }
    e.kind = EPI_MOUT;
    e.out_f = w.z;
    e.ldo = d;
    e.gbuf = w.gbuf;
    // RMSNorm_s(s_{t-1}): the fragment-order copy, or the second half of X
    const void* r_in = pk ? w.o : (const char*)w.X + d * es;
    const int64_t ld_r = pk ? d : 2 * d;
    if (cf.merge_rank > 0) {
      // low-rank W_s = U V: y = V r (stored in the dtype), then U y; y is in
      // fragment order when U has an operand-order copy (rank % 64 == 0)
      const int k = cf.merge_rank;
      const bool pk_u = pk && c->pk_mws_u;
      EpiArgs ey = E0;
      ey.kind = EPI_STORE_T;
      ey.out_k = w.act;
      ey.ldo = k;
      ey.pk = pk_u ? 1 : 0;
      ey.lo = pk_u ? lo_act : 0;
      gm.run(r_in, ld_r, {c->merge_ws_v}, k, d, PAIR_PLAIN, n, ey, nullptr, nullptr, mw(c->pk_mws_v), lo_o);
      gm.run(w.act, k, {c->merge_ws_u}, d, k, PAIR_PLAIN, n, producer(e, g_first), nullptr, w.ssq,
             pk_u ? c->pk_mws_u : nullptr, lo_act);
    } else {
      gm.run(r_in, ld_r, {c->merge_ws}, d, d, PAIR_PLAIN, n, producer(e, g_first), nullptr, w.ssq, mw(c->pk_mws),
             lo_o);
    }
  } else {
    EpiArgs e = E0;
    e.kind = EPI_CONVEX;
    e.out_f = w.z;
    e.ldo = d;
    e.bias = c->merge_bg;
    gm.run(w.X, 2 * d, {c->merge_wg}, d, 2 * d, PAIR_PLAIN, n, producer(e, g_first), nullptr, w.ssq,
           mw(c->pk_mwg), lo_X);
  }

  AttnArgs at{};
  at.rows = P.R;
  at.d = d;
  at.H = H;
  at.dh = dh;
  at.qscale = (float)(1.4426950408889634 / std::sqrt((double)dh));
  at.W = cf.window;
  at.chunk = c->chunk;
  at.nch = c->nch;
  at.direct = at.nch == 1 ? 1 : 0;
  at.part = w.part;
  // chunks merged inside the cross-attention launch (no combine launch) for
  // calls of at most 256 workgroups: each workgroup that writes a partial
  // then pays a device-scope release (an L2 write-back), which costs more
  // than the combine launch it saves once many workgroups write partials
  // (reference depth, batch 1: t ~ 40 3.74 -> 3.66 ms per step, t ~ 2048
  // 4.19 -> 4.13; 8 rows: t ~ 40 4.03 -> 3.97, but t ~ 2048 5.30 -> 6.07)
  const bool in_launch = c->xcomb_mode == 2 ||
                         (c->xcomb_mode == 0 && (int64_t)n * (H / c->hpw_x) * c->nch <= 256);
  at.cnt = in_launch ? w.xcnt : nullptr;
  at.out_pk = pk ? 1 : 0;
  at.out_lo = lo_o;
  at.sb = P.mem.stride_b;
  at.st = P.mem.stride_t;

  const size_t ring_layer = (size_t)P.st->B_cap * (cf.window - 1) * d * es;
  // ---- SWA sublayer [eqs. (2.12)-(2.14)]: RMSNorm_S folded into QKV ----
  auto swa = [&](int l, const float* gnext) {
    {
      EpiArgs e = E0;
      e.kind = EPI_QKV;
      e.out_f = w.q;
      e.out_k = w.kc;
      e.out_v = w.vc;
      gm.run(w.h, d, {c->wq[l], c->wk[l], c->wv[l]}, d, d, PAIR_ROPE, n, e, w.ssq, nullptr, pw(c->pk_qkv, l), lo_h);
    }
    at.q = w.q;
    at.kc = w.kc;
    at.vc = w.vc;
    at.ring_k = (char*)P.st->ring_k + l * ring_layer;
    at.ring_v = (char*)P.st->ring_v + l * ring_layer;
    at.out = w.o;
    at.hpw = c->hpw;
    { Prof pf(c, RLT_PROF_SWA, s); launch_swa(c->dt, at, s); }
    EpiArgs e = E0;
    e.kind = EPI_RESID;
    e.out_f = w.z;
    e.ldo = d;
    gm.run(w.o, d, {c->wo[l]}, d, d, PAIR_PLAIN, n, producer(e, gnext), nullptr, w.ssq, pw(c->pk_wo, l), lo_o);
  };
  // ---- cross-attention sublayer [eq. (2.15)]: RMSNorm_M folded into the query ----
  auto cross = [&](int l, const float* gnext) {
    {
      EpiArgs e = E0;
      e.kind = EPI_QROT;
      e.out_f = w.qm;
      gm.run(w.h, d, {c->wqm[l]}, d, d, PAIR_ROPE, n, e, w.ssq, nullptr, pw(c->pk_wqm, l), lo_h);
    }
    const int g = (l * cf.n_groups) / L;
    at.q = w.qm;
    at.mk = (const char*)P.mem.k + (size_t)g * P.mem.stride_g * es;
    at.mv = (const char*)P.mem.v + (size_t)g * P.mem.stride_g * es;
    at.out = w.o;
    at.hpw = c->hpw_x;
    { Prof pf(c, RLT_PROF_XATTN, s); launch_xattn(c->dt, at, s); }
    if (!at.direct) {
      if (at.cnt) {
        launch_xcombine(c->dt, at, s);  // merged in the launch: only records the persistent step's phase
      } else {
        Prof pf(c, RLT_PROF_XCOMBINE, s);
        launch_xcombine(c->dt, at, s);
      }
    }
    EpiArgs e = E0;
    e.kind = EPI_RESID;
    e.out_f = w.z;
    e.ldo = d;
    gm.run(w.o, d, {c->wom[l]}, d, d, PAIR_PLAIN, n, producer(e, gnext), nullptr, w.ssq, pw(c->pk_wom, l), lo_o);
  };
  // ---- FFN sublayer [eq. (2.16)]: RMSNorm_D folded into gate/up ----
  auto ffn = [&](int l, const float* gnext) {
    EpiArgs e = E0;
    e.kind = EPI_SWIGLU;
    e.out_k = w.act;
    e.ldo = F;
    e.lo = lo_act;
    gm.run(w.h, d, {c->w_gate[l], c->w_up[l]}, F, d, PAIR_DUAL, n, e, w.ssq, nullptr, pw(c->pk_gu, l), lo_h);
    e.kind = EPI_RESID;
    e.out_f = w.z;
    e.ldo = d;
    e.lo = lo_h;
    gm.run(w.act, F, {c->w_down[l]}, d, F, PAIR_PLAIN, n, producer(e, gnext), nullptr, w.ssq, pw(c->pk_down, l),
           lo_act);
  };
  for (int l = 0; l < L; ++l) {
    for (int i = 0; i < 3; ++i) {
      // the producer of this sublayer folds the gain of the next norm: the
      // next sublayer's, the next block's first, or RMSNorm_o
      const float* gnext = i + 1 < 3 ? gain_of(l, order[i + 1]) : gain_of(l + 1, order[0]);
      if (order[i] == 0) swa(l, gnext);
      else if (order[i] == 1) cross(l, gnext);
      else ffn(l, gnext);
    }
    if (P.z_trace) launch_copy_f32(w.z, P.z_trace + (size_t)l * P.z_trace_ld * d, (int64_t)n * d, s);
  }
  // ---- s_t write-back [eq. (2.5)] ----
  m.z = w.z;
  m.s_out = P.s_out;
  m.s_trace = P.s_trace;
  m.s_trace_sb = P.s_trace_sb;
  { Prof pf(c, RLT_PROF_NORM, s); launch_final(c->dt, m, s); }
  float* logits = P.logits ? P.logits : w.logits;
  if (P.need_logits) {
    EpiArgs e = E0;
    e.kind = EPI_STORE;
    e.out_f = logits;
    e.ldo = cf.vocab;
    gm.run(w.h, d, {c->w_out}, cf.vocab, d, PAIR_PLAIN, n, e, w.ssq, nullptr,
           pk ? c->pk_out : nullptr, lo_h);  // RMSNorm_o folded in [eq. (2.6)]
  }
  if (P.do_readout) {
    ReadoutArgs ro = P.ro;
    ro.logits = logits;
    Prof pf(c, RLT_PROF_READOUT, s);
    launch_readout(ro, s);
  }
}

// The device copy of a recorded phase list: found in the cache, or
// uploaded (synchronously; never while `s` is being captured). Null when
// unavailable.
const Phase* fused_phases(rlt_ctx* c, const std::vector<Phase>& rec, hipStream_t s) {
  const size_t bytes = rec.size() * sizeof(Phase);
  for (const auto& e : c->fused_cache)
    if (e.host.size() == rec.size() && std::memcmp(e.host.data(), rec.data(), bytes) == 0) return e.dev;
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(s, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone) return nullptr;
  if (c->fused_cache.size() >= 64) {
    if (hipDeviceSynchronize() != hipSuccess) return nullptr;
    for (auto& e : c->fused_cache) (void)hipFree(e.dev);
    c->fused_cache.clear();
  }
  Phase* dev = nullptr;
  if (hipMalloc((void**)&dev, bytes) != hipSuccess) return nullptr;
  if (hipMemcpy(dev, rec.data(), bytes, hipMemcpyHostToDevice) != hipSuccess) {
    (void)hipFree(dev);
    return nullptr;
  }
  c->fused_cache.push_back({rec, dev});
  return dev;
}

// Record the transition of the plan as phases (the readout stays a kernel
// of its own); returns the device phase list or null.
const Phase* fused_prepare(rlt_ctx* c, const StepPlan& P, hipStream_t s, int* nphase) {
  std::vector<Phase> rec;
  StepPlan Q = P;
  Q.do_readout = false;
  t_rec = &rec;
  c->gemm_target = c->fused_target;
  enqueue_transition(c, c->ws[0], Q, s);
  t_rec = nullptr;
  c->gemm_target = 0;
  *nphase = (int)rec.size();
  for (const Phase& p : rec)
    if (p.kind == PH_INVALID) return nullptr;
  return fused_phases(c, rec, s);
}

// Run the plan: one persistent kernel for small calls (opt-in), otherwise
// the separate kernels.
void enqueue_rows(rlt_ctx* c, const StepPlan& P, hipStream_t s, bool allow_fused = true) {
  const int n = P.n;
  if (allow_fused && c->fused_rows > 0 && n <= c->fused_rows) {
    int nph = 0;
    const Phase* ph = fused_prepare(c, P, s, &nph);
    if (ph) {
      {
        Prof pf(c, RLT_PROF_FUSED, s);
        launch_fused(ph, nph, c->fused_sync, c->err_dev, c->fused_grid, c->fused_spin, s);
      }
      if (P.do_readout) {
        ReadoutArgs ro = P.ro;
        ro.logits = P.logits ? P.logits : c->ws[0].logits;
        Prof pf(c, RLT_PROF_READOUT, s);
        launch_readout(ro, s);
      }
      return;
    }
  }
  enqueue_transition(c, c->ws[0], P, s);
}

int check_state(rlt_ctx* c, const rlt_state* st) {
  if (!st || !st->s || !st->pos || !st->pending) return fail(RLT_EINVAL, "null state buffer");
  if (c->cfg.window > 1 && (!st->ring_k || !st->ring_v)) return fail(RLT_EINVAL, "null cache buffer");
  if (st->B_cap < 1) return fail(RLT_EINVAL, "B_cap < 1");
  if (st->version != c->cfg.weights_version)
    return fail(RLT_ESTALE, "state version %llu differs from weights version %llu",
                (unsigned long long)st->version, (unsigned long long)c->cfg.weights_version);
  return RLT_OK;
}

int check_memory(const rlt_memory& m) {
  if (!m.k || !m.v || !m.mem_len) return fail(RLT_EINVAL, "null memory pointer");
  if (m.stride_t < 1 || m.stride_b < 0 || m.stride_g < 0) return fail(RLT_EINVAL, "memory strides");
  return RLT_OK;
}

// the attention kernels read memory entries in 16-byte runs
int check_memory_read(const rlt_ctx* c, const rlt_memory& m) {
  int rc = check_memory(m);
  if (rc) return rc;
  const int64_t run = 16 / c->es;  // elements per 16 bytes
  if ((uintptr_t)m.k % 16 || (uintptr_t)m.v % 16 || m.stride_t % run || m.stride_b % run || m.stride_g % run)
    return fail(RLT_EINVAL, "memory k/v must be 16-byte aligned with strides in multiples of %lld elements",
                (long long)run);
  return RLT_OK;
}

}  // namespace

// ----------------------------------------------------------------------------
// entry points
// ----------------------------------------------------------------------------

extern "C" int rlt_init_state(rlt_ctx* c, rlt_state* st, const int32_t* rows, int32_t n, int32_t flags,
                              void* stream) {
  if (!c) return fail(RLT_EINVAL, "null context");
  int rc = check_state(c, st);
  if (rc) return rc;
  if (!rows || n < 1 || n > st->B_cap) return fail(RLT_EINVAL, "rows/n");
  launch_init(c->dt, rows, n, c->s_star, st->s, st->pos, st->pending, st->ring_k, st->ring_v,
              c->cfg.n_layers, st->B_cap, c->cfg.window, c->cfg.d_model, flags & RLT_INIT_POISON,
              (hipStream_t)stream);
  HIP_TRY(hipGetLastError());
  return RLT_OK;
}

// The duplicate-row counters for states of up to B_cap rows (zero-filled;
// grown outside any capture, waiting for earlier work that may use them).
static int ensure_claim(rlt_ctx* c, int B_cap, hipStream_t s) {
  if (c->claim_cap >= B_cap) return RLT_OK;
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  HIP_TRY(hipStreamIsCapturing(s, &cs));
  if (cs != hipStreamCaptureStatusNone) return fail(RLT_EINVAL, "state rows grew during a graph capture");
  HIP_TRY(hipDeviceSynchronize());
  if (c->claim) (void)hipFree(c->claim);
  c->claim = nullptr;
  c->claim_cap = 0;
  int rc = dev_alloc(&c->claim, (size_t)B_cap * 4);
  if (rc) return rc;
  HIP_TRY(hipMemset(c->claim, 0, (size_t)B_cap * 4));
  c->claim_cap = B_cap;
  return RLT_OK;
}

// dry: only prepare what a capture cannot (the persistent step's phase list
// upload, the duplicate-row counters), before a graph capture.
// fixed_claim: the allocation-free step's counters (cleared here for the
// call's rows; no allocation, no persistent step), else the context's own.
static int step_enqueue(rlt_ctx* c, rlt_state* st, const rlt_step_io* io, hipStream_t s, bool dry = false,
                        int* fixed_claim = nullptr) {
  const int n = io->n;
  int* claim = fixed_claim;
  if (!claim) {
    int rc = ensure_claim(c, st->B_cap, s);
    if (rc) return rc;
    claim = c->claim;
  }
  StepPlan P{};
  P.R = Rows{io->rows, c->ident, c->t_row, n};
  P.n = n;
  P.claim = claim;
  P.e = EIn{io->e, (int64_t)c->cfg.d_model, 0};
  P.mem = io->mem;
  P.st = st;
  P.s_out = io->s_out;
  P.z_trace = io->z_trace;
  P.z_trace_ld = n;
  const bool sampling = io->uniform != nullptr;
  P.need_logits = io->logits || io->argmax || io->logp || sampling;
  P.logits = io->logits;
  P.do_readout = io->argmax || io->logp || sampling;
  ReadoutArgs& ro = P.ro;
  ro.rows = P.R;
  ro.n = n;
  ro.V = c->cfg.vocab;
  ro.argmax = io->argmax;
  ro.mode = 0;
  ro.score_tok = io->score_tok;
  ro.logp = io->logp;
  ro.uniform = io->uniform;
  ro.temperature = io->temperature;
  ro.top_k = io->top_k;
  ro.top_p = io->top_p;
  ro.sample_tok = io->sample_tok;
  ro.sample_logmu = io->sample_logmu;

  MiscArgs m{};
  m.rows = P.R;
  m.n = n;
  m.pos = st->pos;
  m.pending = st->pending;
  m.mem_len = io->mem.mem_len;
  m.consume_tok = io->consume_tok;
  m.t_row_out = c->t_row;
  m.err = c->err_dev;
  m.max_t = c->max_ctx;
  m.B_cap = st->B_cap;
  m.claim = claim;
  if (dry) {
    int nph = 0;
    if (c->fused_rows > 0 && n <= c->fused_rows) (void)fused_prepare(c, P, s, &nph);
    return RLT_OK;
  }
  if (fixed_claim) launch_zero_rows(fixed_claim, io->rows, n, st->B_cap, s);
  launch_prestep(m, s);
  enqueue_rows(c, P, s, fixed_claim == nullptr);
  PostArgs pa{P.R, n, st->pos, st->pending, nullptr, claim, st->B_cap};
  if (io->flags & RLT_STEP_DEFER) pa.next_tok = sampling ? io->sample_tok : io->argmax;
  launch_poststep(pa, s);
  HIP_TRY(hipGetLastError());
  return RLT_OK;
}

static int check_step(rlt_ctx* c, rlt_state* st, const rlt_step_io* io);

extern "C" int rlt_decoder_step_noalloc(rlt_ctx* c, rlt_state* st, const rlt_step_io* io, void* stream) {
  int rc = check_step(c, st, io);
  if (rc) return rc;
  if (st->B_cap > RLT_NOALLOC_MAX_ROWS)
    return fail(RLT_ESHAPE, "B_cap %d exceeds the allocation-free step's maximum of %d rows", st->B_cap,
                RLT_NOALLOC_MAX_ROWS);
  if (io->flags & RLT_STEP_GRAPH)
    return fail(RLT_EINVAL, "RLT_STEP_GRAPH allocates a graph: capture the allocation-free step yourself");
  int* claim = g_scratch_ptr[c->device];
  if (!claim) return fail(RLT_EHIP, "the fixed counter array of device %d is not resolved", c->device);
  if ((rc = take_device_error(c))) return rc;
  const bool prof = c->prof_on;  // the timing hook creates events: off for this call
  c->prof_on = false;
  rc = step_enqueue(c, st, io, (hipStream_t)stream, false, claim);
  c->prof_on = prof;
  return rc;
}

// argument checks shared by the decoder step entry points
static int check_step(rlt_ctx* c, rlt_state* st, const rlt_step_io* io) {
  if (!c || !io) return fail(RLT_EINVAL, "null context or io");
  int rc = check_state(c, st);
  if (rc) return rc;
  if (io->n < 1 || io->n > c->max_rows) return fail(RLT_ESHAPE, "n=%d outside 1..max_rows=%d", io->n, c->max_rows);
  if (io->n > st->B_cap) return fail(RLT_ESHAPE, "n > B_cap");
  if (!io->rows || !io->e) return fail(RLT_EINVAL, "null rows or e");
  if ((rc = check_memory_read(c, io->mem))) return rc;
  if (io->logp && !io->score_tok) return fail(RLT_EINVAL, "logp needs score_tok");
  if (io->uniform) {
    if (!(io->temperature > 0.f)) return fail(RLT_EINVAL, "temperature must be > 0");
    if (io->top_k < 1 || io->top_k > 1024 || io->top_k > c->cfg.vocab)
      return fail(RLT_EUNSUPPORTED, "sampling needs 1 <= top_k <= min(1024, vocab)");
    if (!io->sample_tok && !io->sample_logmu) return fail(RLT_EINVAL, "sampling without outputs");
  }
  if (!(io->top_p == io->top_p)) return fail(RLT_EINVAL, "top_p is NaN");
  if ((io->flags & RLT_STEP_DEFER) && !(io->uniform ? io->sample_tok : io->argmax))
    return fail(RLT_EINVAL, "RLT_STEP_DEFER needs sample_tok (sampling) or argmax");
  return RLT_OK;
}

extern "C" int rlt_decoder_step(rlt_ctx* c, rlt_state* st, const rlt_step_io* io, void* stream) {
  int rc = check_step(c, st, io);
  if (rc) return rc;
  if ((rc = take_device_error(c))) return rc;
  hipStream_t s = (hipStream_t)stream;
  if (!(io->flags & RLT_STEP_GRAPH)) return step_enqueue(c, st, io, s);
  if (!stream) return fail(RLT_EINVAL, "RLT_STEP_GRAPH needs a non-default stream");

  // captured step: replay when the arguments are identical to the capture
  std::vector<unsigned char> key(sizeof(rlt_step_io) + sizeof(rlt_state) + sizeof(void*));
  std::memcpy(key.data(), io, sizeof(rlt_step_io));
  std::memcpy(key.data() + sizeof(rlt_step_io), st, sizeof(rlt_state));
  std::memcpy(key.data() + sizeof(rlt_step_io) + sizeof(rlt_state), &stream, sizeof(void*));
  if (!c->graph_exec || key != c->graph_key) {
    if (c->graph_exec) {
      (void)hipGraphExecDestroy(c->graph_exec);
      c->graph_exec = nullptr;
    }
    if (c->graph) {
      (void)hipGraphDestroy(c->graph);
      c->graph = nullptr;
    }
    if ((rc = step_enqueue(c, st, io, s, true))) return rc;
    HIP_TRY(hipStreamBeginCapture(s, hipStreamCaptureModeThreadLocal));
    const bool prof = c->prof_on;
    c->prof_on = false;
    rc = step_enqueue(c, st, io, s);
    c->prof_on = prof;
    hipGraph_t g = nullptr;
    hipError_t ec = hipStreamEndCapture(s, &g);
    if (rc) {
      if (g) (void)hipGraphDestroy(g);
      return rc;
    }
    if (ec != hipSuccess) return fail(RLT_EHIP, "hipStreamEndCapture: %s", hipGetErrorString(ec));
    c->graph = g;
    HIP_TRY(hipGraphInstantiate(&c->graph_exec, g, nullptr, nullptr, 0));
    c->graph_key = key;
  }
  HIP_TRY(hipGraphLaunch(c->graph_exec, s));
  return RLT_OK;
}

extern "C" int rlt_replay_sequence(rlt_ctx* c, rlt_state* st, const rlt_replay_io* io, void* stream) {
  if (!c || !io) return fail(RLT_EINVAL, "null context or io");
  int rc = check_state(c, st);
  if (rc) return rc;
  const int B = io->B;
  if (B < 1 || B > c->max_rows || B > st->B_cap) return fail(RLT_ESHAPE, "B outside 1..max_rows/B_cap");
  if (!io->len_host || !io->split_host || !io->e || !io->tokens || !io->logp)
    return fail(RLT_EINVAL, "null replay input");
  if ((rc = check_memory_read(c, io->mem))) return rc;
  int maxlen = 0;
  std::vector<int> rows(B);
  for (int b = 0; b < B; ++b) {
    const int len = io->len_host[b], sp = io->split_host[b];
    if (len < 2) return fail(RLT_ESHAPE, "len[%d]=%d < 2", b, len);
    if (len - 1 > c->max_ctx) return fail(RLT_ESHAPE, "len[%d]-1 exceeds max_ctx", b);
    if (sp < 1) return fail(RLT_EINVAL, "split[%d] < 1", b);
    rows[b] = io->rows_host ? io->rows_host[b] : b;
    if (rows[b] < 0 || rows[b] >= st->B_cap) return fail(RLT_EINVAL, "row of sequence %d out of range", b);
    maxlen = std::max(maxlen, len);
  }
  {
    std::vector<int> seen(rows);
    std::sort(seen.begin(), seen.end());
    if (std::adjacent_find(seen.begin(), seen.end()) != seen.end()) return fail(RLT_EINVAL, "duplicate rows");
  }
  if ((rc = take_device_error(c))) return rc;
  hipStream_t s = (hipStream_t)stream;
  // schedule: sequences by length, longest first (stable), so that the
  // active set at tick t (len - 1 >= t) is a prefix of the order
  std::vector<int> order(B);
  std::iota(order.begin(), order.end(), 0);
  std::stable_sort(order.begin(), order.end(),
                   [&](int a, int b) { return io->len_host[a] > io->len_host[b]; });
  int* stg = c->host_stage;
  const size_t M = c->M_pad;
  for (int i = 0; i < B; ++i) {
    stg[i] = rows[order[i]];
    stg[M + i] = order[i];
    stg[2 * M + i] = io->split_host[i];
    stg[3 * M + i] = io->len_host[i] - 1;
  }
  HIP_TRY(hipMemcpyAsync(c->rows_buf, stg, B * 4, hipMemcpyHostToDevice, s));
  HIP_TRY(hipMemcpyAsync(c->src_buf, stg + M, B * 4, hipMemcpyHostToDevice, s));
  HIP_TRY(hipMemcpyAsync(c->split_buf, stg + 2 * M, B * 4, hipMemcpyHostToDevice, s));
  HIP_TRY(hipMemcpyAsync(c->last_buf, stg + 3 * M, B * 4, hipMemcpyHostToDevice, s));
  HIP_TRY(hipStreamSynchronize(s));
  launch_init(c->dt, c->rows_buf, B, c->s_star, st->s, st->pos, st->pending, st->ring_k, st->ring_v,
              c->cfg.n_layers, st->B_cap, c->cfg.window, c->cfg.d_model, 0, s);
  std::vector<int> lens_sorted(B);
  for (int i = 0; i < B; ++i) lens_sorted[i] = io->len_host[order[i]];
  auto active = [&](int t) {
    int nt = 0;
    while (nt < B && lens_sorted[nt] - 1 >= t) ++nt;
    return nt;
  };
  // The launches of a tick depend on the size of the active set only (the
  // tick itself lives on the device): a run of ticks with one active set
  // is captured once and replayed, on a caller's stream that is not itself
  // capturing and with the timing hook off.
  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  if (stream) HIP_TRY(hipStreamIsCapturing(s, &cap));
  const bool graphs = stream && cap == hipStreamCaptureStatusNone && !c->prof_on && c->replay_graph_min > 0 &&
                      c->fused_rows == 0;  // (the persistent path builds its phase tables on first use)
  stg[4 * M] = 1;
  HIP_TRY(hipMemcpyAsync(c->tick_dev, stg + 4 * M, 4, hipMemcpyHostToDevice, s));
  std::vector<hipGraphExec_t> execs;
  std::vector<hipGraph_t> graphs_made;
  auto release = [&]() {
    for (hipGraphExec_t e : execs) (void)hipGraphExecDestroy(e);
    for (hipGraph_t g : graphs_made) (void)hipGraphDestroy(g);
  };
  int t = 1;
  while (t <= maxlen - 1) {
    const int nt = active(t);
    int run = 1;
    while (t + run <= maxlen - 1 && active(t + run) == nt) ++run;
    StepPlan P{};
    P.R = Rows{c->rows_buf, c->src_buf, c->t_row, nt};
    P.n = nt;
    P.e = EIn{io->e, io->e_stride_b, io->e_stride_t};
    P.mem = io->mem;
    P.st = st;
    P.s_trace = io->s_trace;
    P.s_trace_sb = io->s_stride_b;
    P.need_logits = true;
    P.do_readout = true;
    ReadoutArgs& ro = P.ro;
    ro.rows = P.R;
    ro.n = nt;
    ro.V = c->cfg.vocab;
    ro.mode = 1;
    ro.score_tok = io->tokens;
    ro.tok_sb = io->tok_stride_b;
    ro.logp = io->logp;
    ro.logp_sb = io->logp_stride_b;
    ro.split = c->split_buf;
    PostArgs pa{P.R, nt, st->pos, st->pending, nullptr, nullptr, st->B_cap, c->tick_dev};
    auto tick = [&]() {
      launch_replay_rows(c->rows_buf, nt, c->tick_dev, c->t_row, st->pos, io->mem.mem_len, c->err_dev, s);
      enqueue_rows(c, P, s);
      launch_poststep(pa, s);
    };
    if (graphs && run >= c->replay_graph_min) {
      hipGraph_t g = nullptr;
      hipGraphExec_t ge = nullptr;
      if (hipStreamBeginCapture(s, hipStreamCaptureModeThreadLocal) != hipSuccess) {
        release();
        return fail(RLT_EHIP, "replay capture failed to start");
      }
      tick();
      const hipError_t ec = hipStreamEndCapture(s, &g);
      if (g) graphs_made.push_back(g);
      if (ec != hipSuccess || hipGraphInstantiate(&ge, g, nullptr, nullptr, 0) != hipSuccess) {
        (void)hipStreamSynchronize(s);
        release();
        return fail(RLT_EHIP, "replay capture failed");
      }
      execs.push_back(ge);
      for (int r = 0; r < run; ++r)
        if (hipGraphLaunch(ge, s) != hipSuccess) {
          (void)hipStreamSynchronize(s);
          release();
          return fail(RLT_EHIP, "replay graph launch failed");
        }
    } else {
      for (int r = 0; r < run; ++r) tick();
    }
    t += run;
  }
  if (!execs.empty()) {
    // the graphs are released once their launches have run
    const hipError_t es = hipStreamSynchronize(s);
    release();
    if (es != hipSuccess) return fail(RLT_EHIP, "replay: %s", hipGetErrorString(es));
  }
  launch_set_pending(c->rows_buf, c->src_buf, B, io->tokens, io->tok_stride_b, c->last_buf, st->pending, s);
  HIP_TRY(hipGetLastError());
  return RLT_OK;
}

extern "C" int rlt_score_logprobs(rlt_ctx* c, const rlt_score_io* io, void* stream) {
  if (!c || !io) return fail(RLT_EINVAL, "null context or io");
  if (io->n < 1 || io->n > c->max_rows) return fail(RLT_ESHAPE, "n outside 1..max_rows");
  if (!io->s || !io->tokens || !io->logp) return fail(RLT_EINVAL, "null s, tokens or logp");
  if (io->logmu && !(io->temperature > 0.f)) return fail(RLT_EINVAL, "temperature must be > 0");
  if (io->logmu && (io->top_k < 0 || io->top_k > 1024)) return fail(RLT_EUNSUPPORTED, "top_k outside 0..1024");
  if (io->logmu && io->top_p > 0.f && io->top_p < 1.f && io->top_k < 1)
    return fail(RLT_EUNSUPPORTED, "a top-p nucleus is taken within the top-k set: needs top_k >= 1");
  if (io->ratio && !io->logmu_behaviour) return fail(RLT_EINVAL, "ratio needs logmu_behaviour");
  int rc = take_device_error(c);
  if (rc) return rc;
  hipStream_t s = (hipStream_t)stream;
  const Workspace& w = c->ws[0];
  const int n = io->n, d = c->cfg.d_model;
  Rows R{c->ident, c->ident, c->ones, n};
  MiscArgs m{};
  m.rows = R;
  m.n = n;
  m.d = d;
  m.eps = c->cfg.rms_eps;
  m.z = io->s;
  m.gain = c->out_norm;
  m.out = w.h;
  m.ld_out = d;
  launch_rmsnorm(c->dt, m, s);
  EpiArgs e{};
  e.kind = EPI_STORE;
  e.rows = R;
  e.d = d;
  e.out_f = w.logits;
  e.ldo = c->cfg.vocab;
  Gemm gm{c, &w, s};
  gm.run(w.h, d, {c->w_out}, c->cfg.vocab, d, PAIR_PLAIN, n, e);
  ReadoutArgs ro{};
  ro.rows = R;
  ro.n = n;
  ro.V = c->cfg.vocab;
  ro.logits = w.logits;
  ro.mode = 0;
  ro.score_tok = io->tokens;
  ro.logp = io->logp;
  ro.temperature = io->temperature;
  ro.top_k = io->top_k;
  ro.top_p = io->top_p;
  ro.logmu = io->logmu;
  ro.logmu_beh = io->logmu_behaviour;
  ro.ratio = io->ratio;
  launch_readout(ro, s);
  HIP_TRY(hipGetLastError());
  return RLT_OK;
}

// ----------------------------------------------------------------------------
// test / benchmark hooks (include/rlt_debug.h)
// ----------------------------------------------------------------------------

// ----------------------------------------------------------------------------
// exact prefix snapshots [RLT §6]
// ----------------------------------------------------------------------------

extern "C" int rlt_snapshot_bytes(const rlt_config* cfg, size_t* bytes_per_row) {
  int rc = check_config(cfg);
  if (rc) return rc;
  if (!bytes_per_row) return fail(RLT_EINVAL, "null output");
  const size_t es = elt_size(cfg->dtype);
  *bytes_per_row = sizeof(rlt_snapshot_header) + (size_t)cfg->d_model * sizeof(float) +
                   2 * (size_t)cfg->n_layers * (size_t)(cfg->window - 1) * cfg->d_model * es;
  return RLT_OK;
}

namespace {

// the rows' ring bytes: L blocks of (W-1)*d elements, layer stride B_cap*(W-1)*d
struct RingGeom {
  size_t width, pitch;
  int height;
};

RingGeom ring_geom(const rlt_ctx* c, const rlt_state* st) {
  const size_t blk = (size_t)(c->cfg.window - 1) * c->cfg.d_model * c->es;
  return RingGeom{blk, blk * st->B_cap, c->cfg.n_layers};
}

int check_rows_host(const rlt_state* st, const int32_t* rows, int32_t n) {
  if (!rows || n < 1) return fail(RLT_EINVAL, "rows/n");
  std::vector<int> seen(rows, rows + n);
  std::sort(seen.begin(), seen.end());
  if (seen.front() < 0 || seen.back() >= st->B_cap) return fail(RLT_EINVAL, "row outside 0..B_cap-1");
  if (std::adjacent_find(seen.begin(), seen.end()) != seen.end()) return fail(RLT_EINVAL, "duplicate rows");
  return RLT_OK;
}

}  // namespace

extern "C" int rlt_state_snapshot(rlt_ctx* c, const rlt_state* st, const int32_t* rows_host, int32_t n, void* dst,
                                  void* stream) {
  if (!c || !dst) return fail(RLT_EINVAL, "null context or destination");
  int rc = check_state(c, st);
  if (rc) return rc;
  if ((rc = check_rows_host(st, rows_host, n))) return rc;
  size_t per = 0;
  if ((rc = rlt_snapshot_bytes(&c->cfg, &per))) return rc;
  hipStream_t s = (hipStream_t)stream;
  const rlt_config& cf = c->cfg;
  const RingGeom rg = ring_geom(c, st);
  for (int i = 0; i < n; ++i) {
    const int r = rows_host[i];
    char* base = (char*)dst + (size_t)i * per;
    rlt_snapshot_header* h = (rlt_snapshot_header*)base;
    std::memset(h, 0, sizeof(*h));
    h->magic = RLT_SNAPSHOT_MAGIC;
    h->layout = 1;
    h->weights_version = cf.weights_version;
    h->n_layers = cf.n_layers;
    h->d_model = cf.d_model;
    h->window = cf.window;
    h->dtype = cf.dtype;
    char* p = base + sizeof(rlt_snapshot_header);
    HIP_TRY(hipMemcpyAsync(&h->pos, st->pos + r, 4, hipMemcpyDeviceToHost, s));
    HIP_TRY(hipMemcpyAsync(&h->pending, st->pending + r, 4, hipMemcpyDeviceToHost, s));
    HIP_TRY(hipMemcpyAsync(p, st->s + (size_t)r * cf.d_model, (size_t)cf.d_model * 4, hipMemcpyDeviceToHost, s));
    p += (size_t)cf.d_model * 4;
    if (rg.width) {
      for (const void* ring : {(const void*)st->ring_k, (const void*)st->ring_v}) {
        HIP_TRY(hipMemcpy2DAsync(p, rg.width, (const char*)ring + (size_t)r * rg.width, rg.pitch, rg.width,
                                 rg.height, hipMemcpyDeviceToHost, s));
        p += rg.width * rg.height;
      }
    }
  }
  HIP_TRY(hipStreamSynchronize(s));
  return RLT_OK;
}

extern "C" int rlt_state_restore(rlt_ctx* c, rlt_state* st, const int32_t* rows_host, int32_t n, const void* src,
                                 void* stream) {
  if (!c || !src) return fail(RLT_EINVAL, "null context or source");
  int rc = check_state(c, st);
  if (rc) return rc;
  if ((rc = check_rows_host(st, rows_host, n))) return rc;
  size_t per = 0;
  if ((rc = rlt_snapshot_bytes(&c->cfg, &per))) return rc;
  const rlt_config& cf = c->cfg;
  for (int i = 0; i < n; ++i) {
    const rlt_snapshot_header* h = (const rlt_snapshot_header*)((const char*)src + (size_t)i * per);
    if (h->magic != RLT_SNAPSHOT_MAGIC || h->layout != 1) return fail(RLT_EINVAL, "snapshot %d: not a snapshot", i);
    if (h->n_layers != cf.n_layers || h->d_model != cf.d_model || h->window != cf.window || h->dtype != cf.dtype)
      return fail(RLT_ESHAPE, "snapshot %d was taken under another configuration", i);
    if (h->weights_version != cf.weights_version)
      return fail(RLT_ESTALE, "snapshot %d has weights version %llu, the context %llu", i,
                  (unsigned long long)h->weights_version, (unsigned long long)cf.weights_version);
    if (h->pos < 0 || h->pos > c->max_ctx) return fail(RLT_EINVAL, "snapshot %d: position %d", i, h->pos);
  }
  hipStream_t s = (hipStream_t)stream;
  const RingGeom rg = ring_geom(c, st);
  for (int i = 0; i < n; ++i) {
    const int r = rows_host[i];
    const char* base = (const char*)src + (size_t)i * per;
    const rlt_snapshot_header* h = (const rlt_snapshot_header*)base;
    const char* p = base + sizeof(rlt_snapshot_header);
    HIP_TRY(hipMemcpyAsync(st->pos + r, &h->pos, 4, hipMemcpyHostToDevice, s));
    HIP_TRY(hipMemcpyAsync(st->pending + r, &h->pending, 4, hipMemcpyHostToDevice, s));
    HIP_TRY(hipMemcpyAsync(st->s + (size_t)r * cf.d_model, p, (size_t)cf.d_model * 4, hipMemcpyHostToDevice, s));
    p += (size_t)cf.d_model * 4;
    if (rg.width) {
      for (void* ring : {st->ring_k, st->ring_v}) {
        HIP_TRY(hipMemcpy2DAsync((char*)ring + (size_t)r * rg.width, rg.pitch, p, rg.width, rg.width, rg.height,
                                 hipMemcpyHostToDevice, s));
        p += rg.width * rg.height;
      }
    }
  }
  HIP_TRY(hipStreamSynchronize(s));
  return RLT_OK;
}

// ----------------------------------------------------------------------------
// encoder memory [RLT §2.2, eq. (2.2)]
// ----------------------------------------------------------------------------

namespace {

int check_memory_weights(const rlt_ctx* c, const rlt_memory_weights* mw) {
  if (!mw || !mw->norm_e || !mw->wk || !mw->wv) return fail(RLT_EINVAL, "null memory weights");
  for (int g = 0; g < c->cfg.n_groups; ++g)
    if (!mw->norm_e[g] || !mw->wk[g] || !mw->wv[g]) return fail(RLT_EINVAL, "missing memory weight of group %d", g);
  return RLT_OK;
}

// scratch for up to mem_rows entries per chunk (when rows) and B prefill sequences
int ensure_mem_ws(rlt_ctx* c, int B, bool rows = true) {
  if (rows && !c->mem_A) {
    c->mem_rows = std::max(c->M_pad, 8192);
    const size_t R = c->mem_rows;
    int rc = 0;
    if ((rc = dev_alloc(&c->mem_A, R * c->cfg.d_model * c->es)) || (rc = dev_alloc(&c->mem_ssq, R * 4)) ||
        (rc = dev_alloc(&c->mem_src, R * 4)) || (rc = dev_alloc(&c->mem_t, R * 4)))
      return rc;
    if (hipMemset(c->mem_A, 0, R * c->cfg.d_model * c->es) != hipSuccess)
      return fail(RLT_EHIP, "memory scratch initialisation failed");
  }
  if (B > c->mem_B) {
    if (c->mem_offs) (void)hipFree(c->mem_offs);
    if (c->mem_lens) (void)hipFree(c->mem_lens);
    c->mem_offs = c->mem_lens = nullptr;
    c->mem_B = 0;
    int rc = 0;
    if ((rc = dev_alloc(&c->mem_offs, (size_t)(B + 1) * 4)) || (rc = dev_alloc(&c->mem_lens, (size_t)B * 4))) return rc;
    c->mem_B = B;
  }
  return RLT_OK;
}

// entries of the n slots of R (t_row already set) for every group
void enqueue_mem_entries(rlt_ctx* c, const rlt_memory_weights* mw, const rlt_memory* mem, const Rows& R, EIn e,
                         hipStream_t s) {
  const rlt_config& cf = c->cfg;
  const int d = cf.d_model;
  for (int g = 0; g < cf.n_groups; ++g) {
    launch_mem_prep(c->dt, R, e, d, mw->norm_e[g], c->mem_A, c->mem_ssq, s);
    EpiArgs ep{};
    ep.kind = EPI_MEMKV;
    ep.rows = R;
    ep.d = d;
    ep.dh = cf.d_head;
    ep.H = cf.n_heads;
    ep.rope = cf.pos_kind == RLT_POS_ROPE;
    ep.inv_freq = c->inv_freq;
    ep.rope_tab = c->rope_tab;
    ep.rope_tmax = c->rope_tmax;
    ep.mk = (char*)mem->k + (size_t)g * mem->stride_g * c->es;
    ep.mv = (char*)mem->v + (size_t)g * mem->stride_g * c->es;
    ep.msb = mem->stride_b;
    ep.mst = mem->stride_t;
    ep.mem_vec = c->dt == 1 && (uintptr_t)ep.mk % 16 == 0 && (uintptr_t)ep.mv % 16 == 0 && mem->stride_b % 8 == 0 &&
                 mem->stride_t % 8 == 0 && d % 8 == 0;

    Gemm gm{c, &c->ws[0], s};
    gm.m_pad = c->mem_rows;
    gm.ssq_units = 1;
    gm.run(c->mem_A, d, {mw->wk[g], mw->wv[g]}, d, d, PAIR_ROPE, R.n, ep, c->mem_ssq, nullptr);
  }
}

}  // namespace

extern "C" int rlt_memory_append(rlt_ctx* c, const rlt_memory_weights* mw, const rlt_memory* mem, int32_t B_cap,
                                 int32_t T_cap, const int32_t* rows, int32_t n, const void* e, void* stream) {
  if (!c || !mem) return fail(RLT_EINVAL, "null context or memory");
  int rc = check_memory_weights(c, mw);
  if (rc) return rc;
  if ((rc = check_memory(*mem))) return rc;
  if (!rows || !e) return fail(RLT_EINVAL, "null rows or e");
  if (n < 1 || n > c->max_rows) return fail(RLT_ESHAPE, "n=%d outside 1..max_rows=%d", n, c->max_rows);
  if (B_cap < 1 || T_cap < 1) return fail(RLT_EINVAL, "B_cap < 1 or T_cap < 1");
  if ((rc = ensure_mem_ws(c, 0))) return rc;
  hipStream_t s = (hipStream_t)stream;
  int* mem_len = const_cast<int*>(mem->mem_len);
  launch_mem_slots(rows, n, mem_len, B_cap, T_cap, c->mem_t, c->err_dev, s);
  const Rows R{rows, c->ident, c->mem_t, n};  // output row rows[i], input e[i]
  enqueue_mem_entries(c, mw, mem, R, EIn{e, (int64_t)c->cfg.d_model, 0}, s);
  launch_mem_commit(rows, n, c->mem_t, mem_len, s);
  HIP_TRY(hipGetLastError());
  return RLT_OK;
}

extern "C" int rlt_memory_prefill(rlt_ctx* c, const rlt_memory_weights* mw, const rlt_memory* mem, int32_t T_cap,
                                  int32_t B, const int32_t* len_host, const void* e, int64_t e_stride_b,
                                  int64_t e_stride_t, void* stream) {
  if (!c || !mem) return fail(RLT_EINVAL, "null context or memory");
  int rc = check_memory_weights(c, mw);
  if (rc) return rc;
  if ((rc = check_memory(*mem))) return rc;
  if (!len_host || !e) return fail(RLT_EINVAL, "null lengths or e");
  if (B < 1 || T_cap < 1) return fail(RLT_ESHAPE, "B < 1 or T_cap < 1");
  if (e_stride_b < 0 || e_stride_t < 1) return fail(RLT_EINVAL, "e strides");
  std::vector<int> offs(B + 1, 0);
  for (int b = 0; b < B; ++b) {
    if (len_host[b] < 1 || len_host[b] > T_cap) return fail(RLT_ESHAPE, "len[%d]=%d outside 1..T_cap", b, len_host[b]);
    if ((int64_t)offs[b] + len_host[b] > INT32_MAX) return fail(RLT_ESHAPE, "more than 2^31 entries");
    offs[b + 1] = offs[b] + len_host[b];
  }
  if ((rc = ensure_mem_ws(c, B))) return rc;
  hipStream_t s = (hipStream_t)stream;
  HIP_TRY(hipStreamSynchronize(s));  // the schedule buffers may still be read by earlier work
  HIP_TRY(hipMemcpy(c->mem_offs, offs.data(), (size_t)(B + 1) * 4, hipMemcpyHostToDevice));
  HIP_TRY(hipMemcpy(c->mem_lens, len_host, (size_t)B * 4, hipMemcpyHostToDevice));
  const int64_t total = offs[B];
  for (int64_t r0 = 0; r0 < total; r0 += c->mem_rows) {
    const int nrow = (int)std::min<int64_t>(c->mem_rows, total - r0);
    launch_mem_rows(c->mem_offs, B, r0, nrow, c->mem_src, c->mem_t, s);
    const Rows R{c->mem_src, c->mem_src, c->mem_t, nrow};  // sequence b is both memory row and e row
    enqueue_mem_entries(c, mw, mem, R, EIn{e, e_stride_b, e_stride_t}, s);
  }
  launch_mem_setlen(c->mem_lens, B, const_cast<int*>(mem->mem_len), s);
  HIP_TRY(hipGetLastError());
  return RLT_OK;
}

extern "C" int rlt_trajectory_log_ratio(rlt_ctx* c, int32_t B, const int32_t* len_host, const int32_t* split_host,
                                        const float* logp, int64_t logp_stride_b, const float* logmu,
                                        int64_t logmu_stride_b, float* out, void* stream) {
  if (!c || !len_host || !split_host || !logp || !logmu || !out) return fail(RLT_EINVAL, "null argument");
  if (B < 1) return fail(RLT_ESHAPE, "B < 1");
  if (logp_stride_b < 0 || logmu_stride_b < 0) return fail(RLT_EINVAL, "strides");
  int rc = ensure_mem_ws(c, B, false);  // the prefill schedule buffers hold the first / last positions
  if (rc) return rc;
  std::vector<int> range(2 * (size_t)B);
  for (int b = 0; b < B; ++b) {
    if (split_host[b] < 1) return fail(RLT_EINVAL, "split[%d] < 1", b);
    range[b] = split_host[b];
    range[B + b] = len_host[b] - 1;
  }
  hipStream_t s = (hipStream_t)stream;
  HIP_TRY(hipStreamSynchronize(s));
  HIP_TRY(hipMemcpy(c->mem_offs, range.data(), (size_t)B * 4, hipMemcpyHostToDevice));
  HIP_TRY(hipMemcpy(c->mem_lens, range.data() + B, (size_t)B * 4, hipMemcpyHostToDevice));
  launch_traj_ratio(B, c->mem_offs, c->mem_lens, logp, logp_stride_b, logmu, logmu_stride_b, out, s);
  HIP_TRY(hipGetLastError());
  return RLT_OK;
}

extern "C" int rlt_replay_backward(rlt_ctx* c, const rlt_backward_io* io, const rlt_grads* gr, void* stream) {
  if (!c || !io || !gr) return fail(RLT_EINVAL, "null argument");
  if (!io->len_host || !io->split_host || !io->e || !io->tokens || !io->w || !io->mem.k || !io->mem.v)
    return fail(RLT_EINVAL, "null input array");
  if ((io->dmem_k == nullptr) != (io->dmem_v == nullptr)) return fail(RLT_EINVAL, "dmem_k and dmem_v: both or none");
  if (io->B < 1) return fail(RLT_ESHAPE, "B < 1");
  if (io->e_stride_b < 0 || io->e_stride_t < 0 || io->tok_stride_b < 0 || io->w_stride_b < 0 ||
      io->logp_stride_b < 0 || io->de_stride_b < 0 || io->de_stride_t < 0 || io->mem.stride_g < 0 ||
      io->mem.stride_b < 0 || io->mem.stride_t < 0 || io->dmem_stride_g < 0 || io->dmem_stride_b < 0 ||
      io->dmem_stride_t < 0)
    return fail(RLT_EINVAL, "negative stride");
  for (int b = 0; b < io->B; ++b) {
    if (io->len_host[b] < 2) return fail(RLT_ESHAPE, "len[%d] < 2", b);
    if (io->split_host[b] < 1 || io->split_host[b] > io->len_host[b] - 1)
      return fail(RLT_EINVAL, "split[%d] outside 1 .. len - 1", b);
  }
  const rlt_config& cf = c->cfg;
  if (cf.merge_gate != RLT_GATE_VECTOR || cf.merge_rank != 0 || cf.block_order != RLT_ORDER_SXF)
    return fail(RLT_EUNSUPPORTED, "the replay backward covers the vector gate, full-rank W_s and order SXF");
  bwd::Model m;
  m.cfg = cf;
  m.dt = c->dt;
  m.s_star = c->s_star;
  m.merge_norm = c->merge_norm;
  m.merge_bg = c->merge_bg;
  m.out_norm = c->out_norm;
  m.merge_wg = c->merge_wg;
  m.merge_ws = c->merge_ws;
  m.w_out = c->w_out;
  m.norm_s = c->norm_s;
  m.norm_m = c->norm_m;
  m.norm_d = c->norm_d;
  m.wq = c->wq;
  m.wk = c->wk;
  m.wv = c->wv;
  m.wo = c->wo;
  m.wqm = c->wqm;
  m.wom = c->wom;
  m.w_gate = c->w_gate;
  m.w_up = c->w_up;
  m.w_down = c->w_down;
  m.inv_freq = c->inv_freq;
  m.keep_acts = c->bwd_keep;
  std::string err;
  const int rc = bwd::replay_backward(m, io, gr, (hipStream_t)stream, err);
  if (rc) return fail(rc, "%s", err.c_str());
  return RLT_OK;
}

extern "C" int rlt_dbg_gemm(rlt_ctx* c, const void* A, const void* W, int32_t M, int32_t N, int32_t K,
                            float* out, void* stream) {
  if (!c || !A || !W || !out) return fail(RLT_EINVAL, "null argument");
  const int kmax = std::max(2 * c->cfg.d_model, c->cfg.d_ffn);
  if (M < 1 || M > c->max_rows || N < 32 || N % 32 || K < 32 || K % 32 || K > kmax)
    return fail(RLT_ESHAPE, "need 1 <= M <= max_rows, N and K multiples of 32, K <= max(2*d_model, d_ffn)");
  hipStream_t s = (hipStream_t)stream;
  const Workspace& w = c->ws[0];
  // A goes through a padded workspace buffer: the MFMA tiles read whole 16-row blocks
  void* stage = K <= 2 * c->cfg.d_model ? w.X : w.act;
  HIP_TRY(hipMemcpyAsync(stage, A, (size_t)M * K * c->es, hipMemcpyDeviceToDevice, s));
  Rows R{c->ident, c->ident, c->ones, M};
  EpiArgs e{};
  e.kind = EPI_STORE;
  e.rows = R;
  e.out_f = out;
  e.ldo = N;
  Gemm gm{c, &w, s};
  gm.run(stage, K, {W}, N, K, PAIR_PLAIN, M, e);
  HIP_TRY(hipGetLastError());
  return RLT_OK;
}

extern "C" int rlt_dbg_gemm_packed(rlt_ctx* c, const void* A, const void* W, int32_t M, int32_t N, int32_t K,
                                   float* out, void* stream) {
  if (!c || !A || !W || !out) return fail(RLT_EINVAL, "null argument");
  if (c->dt != 1) return fail(RLT_EUNSUPPORTED, "the operand-order path is bf16 only");
  const int kmax = std::max(2 * c->cfg.d_model, c->cfg.d_ffn);
  if (M < 1 || M > c->max_rows || N < 32 || N % 32 || K < 64 || K % 64 || K > kmax)
    return fail(RLT_ESHAPE, "need 1 <= M <= max_rows, N a multiple of 32, K a multiple of 64 <= max(2*d_model, d_ffn)");
  hipStream_t s = (hipStream_t)stream;
  const Workspace& w = c->ws[0];
  const int Mr = (M + 63) / 64 * 64;  // whole row tiles of the 64-row shapes (<= M_pad)
  void *Ap = nullptr, *Wp = nullptr;
  int rc = dev_alloc(&Ap, (size_t)Mr * K * 2);
  if (!rc) rc = dev_alloc(&Wp, (size_t)N * K * 2);
  if (!rc) {
    // rows of A past M (up to the 64-row tile) are zero
    GemmArgs ga{}, gw{};
    ga.W[0] = A;
    ga.nseg = 1;
    ga.seg_rows = Mr;
    ga.K = K;
    ga.pairing = PAIR_PLAIN;
    ga.Nv = Mr;
    ga.npairs = Mr / 32;
    gw = ga;
    gw.W[0] = W;
    gw.seg_rows = gw.Nv = N;
    gw.npairs = N / 32;
    void* stage = w.act;  // [M_pad][d_ffn] >= Mr x K when K <= d_ffn; else X (2 d_model wide)
    if (K > c->cfg.d_ffn) stage = w.X;
    if (hipMemsetAsync(stage, 0, (size_t)Mr * K * 2, s) != hipSuccess ||
        hipMemcpyAsync(stage, A, (size_t)M * K * 2, hipMemcpyDeviceToDevice, s) != hipSuccess) {
      rc = fail(RLT_EHIP, "staging copy failed");
    } else {
      ga.W[0] = stage;
      launch_pack_weights(ga, Ap, s);
      launch_pack_weights(gw, Wp, s);
      Rows R{c->ident, c->ident, c->ones, M};
      EpiArgs e{};
      e.kind = EPI_STORE;
      e.rows = R;
      e.out_f = out;
      e.ldo = N;
      Gemm gm{c, &w, s};
      gm.run(Ap, K, {W}, N, K, PAIR_PLAIN, M, e, nullptr, nullptr, Wp);
      if (hipGetLastError() != hipSuccess || hipStreamSynchronize(s) != hipSuccess)
        rc = fail(RLT_EHIP, "operand-order product failed");
    }
  }
  if (Ap) (void)hipFree(Ap);
  if (Wp) (void)hipFree(Wp);
  return rc;
}

extern "C" int rlt_dbg_narrow_bounds(int32_t n, int32_t npairs, int32_t K, int32_t pairing, int32_t dh,
                                     int32_t nseg, int32_t seg_rows, int32_t M_pad, int32_t narrow_rows,
                                     int32_t target, int64_t partial_cap, rlt_narrow_report* out) {
  if (!out) return fail(RLT_EINVAL, "null report");
  if (n < 1 || n > M_pad || npairs < 1 || K < 32 || nseg < 1 || nseg > 3 || seg_rows < 16 || narrow_rows < 1 ||
      partial_cap < 0 || (pairing == PAIR_ROPE && (dh < 32 || dh % 32)))
    return fail(RLT_EINVAL, "narrow bounds: arguments");
  GemmArgs g{};
  g.K = K;
  g.pairing = pairing;
  g.dh = dh;
  g.nseg = nseg;
  g.seg_rows = seg_rows;
  g.M = n;
  g.M_pad = M_pad;
  g.npairs = npairs;
  g.Nv = nseg * seg_rows;
  narrow_plan(n, npairs, K, narrow_rows, target, M_pad, g.Nv, (size_t)partial_cap, g.S, g.mb, g.kslice);
  rlt_narrow_report r{};
  r.S = g.S;
  r.mb = g.mb;
  r.kslice = g.kslice;
  r.a_row_max = -1;
  r.a_col_end = 0;
  r.w_seg_max = r.w_row_max = -1;
  const int MB = g.mb, mtiles = (n + 16 * MB - 1) / (16 * MB);
  // K coverage of one tile (the same for every tile): each 32-wide step once
  std::vector<int> cover(K / 32 + 1, 0);
  int64_t kend = 0;
  for (int split = 0; split < g.S; ++split)
    for (int wave = 0; wave < 4; ++wave) {
      int k0, ns;
      narrow_wave_steps(g, split, wave, k0, ns);
      for (int j = 0; j < ns; ++j) {
        const int k = narrow_step_k(k0, j, ns);
        if (k / 32 < (int)cover.size()) ++cover[k / 32];
      }
      if (ns > 0)
        for (int lane = 0; lane < 64; ++lane)
          kend = std::max<int64_t>(kend, narrow_step_k(k0, ns - 1, ns) + narrow_lane_k(lane) + 8);
    }
  for (int st = 0; st < K / 32; ++st) {
    if (cover[st] == 0) ++r.steps_missing;
    if (cover[st] > 1) r.steps_repeated += cover[st] - 1;
  }
  for (size_t st = K / 32; st < cover.size(); ++st) r.steps_repeated += cover[st];  // steps past K
  r.a_col_end = kend;
  for (int pair = 0; pair < npairs; ++pair) {
    int ba, bb;
    pair_blocks(g, pair, ba, bb);
    for (int lane = 0; lane < 64; ++lane)
      for (int vc : {ba * 16 + narrow_lane_row(lane), bb * 16 + narrow_lane_row(lane)}) {
        int seg, row;
        weight_pos(g, vc, seg, row);
        r.w_seg_max = std::max(r.w_seg_max, seg);
        r.w_row_max = std::max(r.w_row_max, row);
      }
    for (int mt = 0; mt < mtiles; ++mt) {
      const int m0 = mt * MB * 16;
      for (int lane = 0; lane < 64; ++lane)
        for (int mb = 0; mb < MB; ++mb) r.a_row_max = std::max<int64_t>(r.a_row_max, m0 + mb * 16 + narrow_lane_row(lane));
      // epilogue: item idx of MB * 16 * 16 (row m, column r of the pair's halves); stores only rows < M
      for (int idx = 0; idx < MB * 16 * 16; ++idx) {
        const int slot = m0 + (idx >> 4), c = idx & 15;
        if (slot >= n) continue;
        if (g.S > 1)
          for (int split = 0; split < g.S; ++split)
            r.partial_end = std::max<int64_t>(
                r.partial_end, ((int64_t)split * M_pad + slot) * g.Nv + std::max(ba, bb) * 16 + c + 1);
        else
          r.ssq_end = std::max<int64_t>(r.ssq_end, (int64_t)pair * M_pad + slot + 1);
      }
    }
  }
  *out = r;
  return RLT_OK;
}

extern "C" int rlt_dbg_stream_read(const void* src, int64_t bytes, int32_t nontemporal, uint32_t* sink, void* stream) {
  if (!src || !sink) return fail(RLT_EINVAL, "null argument");
  if (bytes < 16 || bytes % 16 || (uintptr_t)src % 16) return fail(RLT_ESHAPE, "bytes and src must be 16-byte multiples");
  launch_stream_read(src, bytes / 16, nontemporal != 0, sink, (hipStream_t)stream);
  HIP_TRY(hipGetLastError());
  return RLT_OK;
}

extern "C" int rlt_dbg_mfma_loop(int32_t blocks, int32_t iters, uint32_t* sink, void* stream) {
  if (!sink) return fail(RLT_EINVAL, "null argument");
  if (blocks < 1 || blocks > (1 << 20) || iters < 1) return fail(RLT_ESHAPE, "blocks in 1..2^20, iters >= 1");
  launch_mfma_loop(blocks, iters, sink, (hipStream_t)stream);
  HIP_TRY(hipGetLastError());
  return RLT_OK;
}

extern "C" int rlt_dbg_product_shape(rlt_ctx* c, int32_t rb, int32_t cb, int32_t lt, int32_t pf, int32_t pre) {
  if (!c) return fail(RLT_EINVAL, "null context");
  if (rb != 0 && (rb < 1 || rb > 2 || (cb != 1 && cb != 2 && !(cb == 4 && lt > 0)) ||
                  (lt != 0 && lt != 1 && lt != 2 && lt != 4 && lt != 8) || pf < 1 || pf > 4 || pre < -1 || pre > 1))
    return fail(RLT_EINVAL, "product shape");
  c->shape_rb = rb;
  c->shape_cb = cb;
  c->shape_lt = lt;
  c->shape_pf = pf;
  c->shape_pre = pre;
  return RLT_OK;
}

extern "C" int rlt_dbg_profile(rlt_ctx* c, int32_t enable) {
  if (!c) return fail(RLT_EINVAL, "null context");
  c->prof_on = enable != 0;
  if (enable) {
    c->prof_rec.clear();
    c->prof_next = 0;
  }
  return RLT_OK;
}

extern "C" int rlt_dbg_profile_read(rlt_ctx* c, int32_t kind, double* total_ms, int64_t* launches) {
  if (!c || !total_ms || !launches) return fail(RLT_EINVAL, "null argument");
  if (kind < 0 || kind >= RLT_PROF_NCLASS) return fail(RLT_EINVAL, "kernel class");
  double ms = 0.0;
  int64_t cnt = 0;
  for (const auto& r : c->prof_rec) {
    if (r.first != kind) continue;
    HIP_TRY(hipEventSynchronize(c->prof_ev[r.second + 1]));
    float e = 0.f;
    HIP_TRY(hipEventElapsedTime(&e, c->prof_ev[r.second], c->prof_ev[r.second + 1]));
    ms += e;
    ++cnt;
  }
  *total_ms = ms;
  *launches = cnt;
  return RLT_OK;
}
