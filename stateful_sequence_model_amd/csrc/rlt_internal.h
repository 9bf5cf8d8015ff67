// Internal declarations shared by the HIP kernels and the host side of the
// library. Element type T is `float` (RLT_F32) or `uint16_t` holding bf16
// bit patterns (RLT_BF16); the same T is used for weights, SWA cache,
// encoder memory, e and the activations fed to matrix products.
#pragma once
#include <algorithm>

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rlt {

// ----------------------------------------------------------------------------
// device helpers
// ----------------------------------------------------------------------------

__device__ __forceinline__ float bf2f(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// round-to-nearest-even float -> bf16 (finite inputs; NaN stays NaN)
__device__ __forceinline__ uint16_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x7fffffu)) return (uint16_t)((u >> 16) | 0x40);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

template <typename T> __device__ __forceinline__ float to_f(T x);
template <> __device__ __forceinline__ float to_f<float>(float x) { return x; }
template <> __device__ __forceinline__ float to_f<uint16_t>(uint16_t x) { return bf2f(x); }

template <typename T> __device__ __forceinline__ T from_f(float x);
template <> __device__ __forceinline__ float from_f<float>(float x) { return x; }
template <> __device__ __forceinline__ uint16_t from_f<uint16_t>(float x) { return f2bf(x); }

// Store x as a matrix-product operand: p[i] = x in the element type and,
// when lo != 0 (bf16 operands carried as two terms), p[i + lo] = the rounding
// remainder x - p[i] in the element type, so that p[i] + p[i + lo] holds x to
// about 16 significant bits.
template <typename T>
__device__ __forceinline__ void store_op(T* p, int64_t i, int64_t lo, float x) {
  const T h = from_f<T>(x);
  p[i] = h;
  if (lo) p[i + lo] = from_f<T>(x - to_f<T>(h));
}

__device__ __forceinline__ float sigmoidf_(float x) { return 1.0f / (1.0f + __expf(-x)); }

// Block-wide sum of one float per thread, fixed reduction order (wave
// butterfly then waves in index order). blockDim.x must be a multiple of 64.
__device__ __forceinline__ float block_sum(float v, float* scratch /* >= 16 floats */) {
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
  const int w = threadIdx.x >> 6, nw = blockDim.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) scratch[w] = v;
  __syncthreads();
  float s = 0.f;
  for (int i = 0; i < nw; ++i) s += scratch[i];
  return s;
}

// ----------------------------------------------------------------------------
// per-call row bookkeeping
// ----------------------------------------------------------------------------

// Slot i of a launch processes state row rows[i] at 1-based position
// t_row[i] (0 = skip: the row had a device-detected error). src[i] indexes
// the caller's per-sequence inputs/outputs (i itself for a decoder step,
// the sequence id for a replay).
struct Rows {
  const int* rows;
  const int* src;
  const int* t_row;
  int n;
};

// e_t of slot i: e + src[i] * sb + (t - 1) * st elements.
struct EIn {
  const void* p;
  int64_t sb, st;
};

// ----------------------------------------------------------------------------
// matrix products  Y[m][c] = sum_k A[m][k] W(c)[k]
// ----------------------------------------------------------------------------

enum Pairing { PAIR_PLAIN = 0, PAIR_ROPE = 1, PAIR_DUAL = 2 };

// Fragment order of a bf16 operand [R][K] (R a multiple of 32, K of 64) of
// v_mfma_f32_32x32x16_bf16: for 32-row block b, 64-wide K chunk c and step
// s < 4, the 64 lanes' 16-byte fragments are contiguous; lane l holds row
// 32 b + l % 32 and k in [64 c + 32 (l / 32) + 8 s, + 8). The k order inside
// a chunk is a permutation of the plain one, applied alike to both operands
// of a product, so the sums are unchanged. One wave load instruction then
// reads 1 KB of consecutive bytes.
__host__ __device__ inline int64_t pk_off(int m, int k, int nchunk) {
  return ((((int64_t)(m >> 5) * nchunk + (k >> 6)) * 4 + ((k & 31) >> 3)) * 64 + ((k >> 5) & 1) * 32 + (m & 31)) * 8 +
         (k & 7);
}

// 64-wide chunks of K the register tile can stage in LDS for one-row calls
constexpr int PK_LDS_CHUNKS = 96;

struct GemmArgs {
  const void* A;          // [M_pad][lda] activations (T); fragment order when Wp is set
  int64_t lda;
  int64_t a_lo;           // fragment order: elements from A to its second term (0: one term)
  const void* W[3];       // weight segments, each [seg_rows][K] (T), natural layout
  const void* Wp;         // bf16: the same weights in fragment order, virtual column
                          // pairs as 32-row blocks (pair p = block p), or null
  int rb, cb;             // fragment-order tile: 32 rb rows x cb column pairs
  int pf;                 // fragment-order tile: chunks in flight per wave
  int lt_groups;          // fragment order, > 0: staged tile, this many workgroups
                          // per tile over the stream groups (1, 2, 4 or 8); 0: register tile
  int lt_rbk;             // staged tile: 32-row blocks per tile, 4 (128 x 64) or 2 (64 x 128)
  int lt_dma;             // staged tile of 64 x 128: chunks copied straight into LDS (k_gemm_bf16_ltd;
                          // else through registers, k_gemm_bf16_lt)
  int a_lds;              // register tile: 1 (M = 1, K <= 64 PK_LDS_CHUNKS): the
                          // activations staged in LDS for the whole K
  int pre;                // fragment-order tile: -1 = by epilogue kind, 0/1 = epilogue values after / before the K loop
  int nseg, seg_rows;
  int K;
  int npairs;             // output handled as pairs of 16-column blocks
  int pairing;            // Pairing
  int dh;                 // head width for PAIR_ROPE
  int M, M_pad;           // valid rows / allocated rows of A
  int S;                  // splits of K across workgroups (bf16 path)
  int mb;                 // 16-row blocks per tile of the narrow bf16 tile: 1, 2 or 4
  int wide;               // bf16 path: 0 = narrow tile; 64 or 128 = LDS tile of 128 rows x this many columns
  int kslice;             // K elements per (split, wave) slice, multiple of 32;
                          // LDS tile: K elements per split, multiple of 64
  float* partial;         // [S][M_pad][Nv] when S > 1
  int Nv;                 // nseg * seg_rows
  // RMSNorm folded into the products (RMSNorm(z) W^T = rstd * ((z * gain) W^T)):
  // a consumer reads per-row partial sums of squares of z and scales its
  // accumulators by rstd = 1/sqrt(sum/d + eps) before the epilogue; a
  // producer (residual / merge epilogue) writes those partial sums, one per
  // (column unit, row), for the next consumer.
  const float* ssq_in;    // [ssq_units][M_pad] or null
  float* ssq_out;         // [units of this product][M_pad] or null
  int ssq_units;
  float inv_d, eps;
};

// 16-lane sum (lanes 16q .. 16q+15 of a wave), fixed butterfly order
__device__ __forceinline__ float sum16(float v) {
  v += __shfl_xor(v, 1);
  v += __shfl_xor(v, 2);
  v += __shfl_xor(v, 4);
  v += __shfl_xor(v, 8);
  return v;
}

// rstd of row m from the per-unit partial sums of squares (one thread)
__device__ __forceinline__ float row_rstd(const GemmArgs& g, int m) {
  float a = 0.f;
#pragma unroll 8
  for (int u = 0; u < g.ssq_units; ++u) a += g.ssq_in[(int64_t)u * g.M_pad + m];
  return 1.0f / sqrtf(a * g.inv_d + g.eps);
}

// Per-row rstd for R rows starting at m0, computed by the NT threads of a
// workgroup. The partial sums of squares of a row are added in one fixed
// order whatever R and NT are (so that a row's rstd, like every other
// reduction of a product, does not depend on the tile it lands in): unit u
// goes to part u % 4, each part adds its units in increasing u, and the row's
// sum is ((p0 + p1) + p2) + p3.
// Loads: the PA = NT / R threads of a row take the row's first PA * RU
// units round-robin (thread slot sl: units sl, sl + PA, ...) into registers
// when constructed (before the main loop, so the loads are in flight with
// it); finish() stages them in LDS (or stage() does, early, where the main
// loop needs the registers) and the four part sums are then formed by one
// thread each, reading units in increasing order (units past PA * RU, only
// for very wide rows, straight from memory). Rows at or past M load nothing
// (their rstd is never used).
template <int R, int NT = 256>
struct RowRstd {
  static constexpr int PA = NT / R;                 // threads per row
  static constexpr int RU = PA >= 16 ? 4 : (PA >= 4 ? 64 / PA : 16);  // units per thread in registers
  static constexpr int NU = PA * RU;                // units staged
  static_assert(PA >= 2 && (PA & (PA - 1)) == 0, "threads per row");
  float v[RU];
  __device__ __forceinline__ RowRstd(const GemmArgs& g, int m0) {
    const int row = threadIdx.x % R, sl = threadIdx.x / R;
#pragma unroll
    for (int j = 0; j < RU; ++j) v[j] = 0.f;
    if (!g.ssq_in) return;  // uniform
    // no branches around the loads (rows clamped below M: those rows' rstd
    // is never used; units clamped to the last one: units past it are
    // staged but never read, reduce() stops at ssq_units), and no use of the
    // values before they are staged, so the loads stay in flight until then
    const int m = m0 + row < g.M ? m0 + row : g.M - 1;
#pragma unroll
    for (int j = 0; j < RU; ++j) {
      const int u = sl + PA * j;
      v[j] = g.ssq_in[(int64_t)(u < g.ssq_units ? u : g.ssq_units - 1) * g.M_pad + m];
    }
  }
  // the loaded units to s_part (LDS [NU][R] floats)
  __device__ __forceinline__ void stage(float* s_part) const {
    const int row = threadIdx.x % R, sl = threadIdx.x / R;
#pragma unroll
    for (int j = 0; j < RU; ++j) s_part[(sl + PA * j) * R + row] = v[j];
  }
  // s_part: LDS [NU][R] floats (the staged units; its first 4 R floats then
  // hold the part sums); s_rstd: LDS [R]; contains three __syncthreads
  __device__ __forceinline__ void finish(const GemmArgs& g, int m0, float* s_part, float* s_rstd) const {
    stage(s_part);
    reduce(g, m0, s_part, s_rstd);
  }
  // finish() after stage(s_part) ran (in every thread of the workgroup)
  __device__ static __forceinline__ void reduce(const GemmArgs& g, int m0, float* s_part, float* s_rstd) {
    const int row = threadIdx.x % R, sl = threadIdx.x / R;
    __syncthreads();
    // the threads of slots 0 .. 3 form the part sums (slot sl: parts sl, sl + PA, ...)
    constexpr int CPT = PA >= 4 ? 1 : 4 / PA;
    float a[CPT];
    const int nst = g.ssq_units < NU ? g.ssq_units : NU;
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int cp = sl + PA * c;
      a[c] = 0.f;
      if (cp < 4) {
        for (int u = cp; u < nst; u += 4) a[c] += s_part[u * R + row];
        if (m0 + row < g.M)
          for (int u = NU + cp; u < g.ssq_units; u += 4) a[c] += g.ssq_in[(int64_t)u * g.M_pad + m0 + row];
      }
    }
    __syncthreads();
#pragma unroll
    for (int c = 0; c < CPT; ++c)
      if (sl + PA * c < 4) s_part[(sl + PA * c) * R + row] = a[c];
    __syncthreads();
    if (threadIdx.x < R) {
      const float s = ((s_part[threadIdx.x] + s_part[R + threadIdx.x]) + s_part[2 * R + threadIdx.x]) +
                      s_part[3 * R + threadIdx.x];
      s_rstd[threadIdx.x] = 1.0f / sqrtf(s * g.inv_d + g.eps);
    }
  }
};

// LDS floats RowRstd<R, NT>::finish needs for s_part
template <int R, int NT>
constexpr int rowrstd_lds() { return RowRstd<R, NT>::NU * R; }

// 16-row blocks per matrix-product tile for an M-row call (tile <= 64 rows;
// larger M runs several row tiles)
__host__ __device__ inline int gemm_row_blocks(int M) { return M <= 16 ? 1 : M <= 32 ? 2 : 4; }

// virtual column blocks (16 columns each) of pair p
__host__ __device__ inline void pair_blocks(const GemmArgs& g, int p, int& ba, int& bb) {
  if (g.pairing == PAIR_PLAIN) {
    ba = 2 * p;
    bb = 2 * p + 1;
  } else if (g.pairing == PAIR_ROPE) {
    const int per = g.dh / 32;           // pairs per head
    const int h = p / per, j = p - h * per;
    ba = h * (g.dh / 16) + j;
    bb = ba + per;
  } else {
    ba = p;
    bb = p + g.seg_rows / 16;
  }
}

// Index math of the narrow tile (gemm_bf16_body), shared with the host-side
// bounds walk (rlt_dbg_narrow_bounds):
// virtual column vc of a weight = row r of segment seg
__host__ __device__ inline void weight_pos(const GemmArgs& g, int vc, int& seg, int& r) {
  seg = vc / g.seg_rows;
  r = vc - seg * g.seg_rows;
}
// the workgroup's K range [kw0, kw1) = split's 4 kslice, cut in 32-wide steps
// dealt to the four waves round-robin: wave `wave` takes steps at k0 + 128 j,
// j < nsteps
__host__ __device__ inline void narrow_wave_steps(const GemmArgs& g, int split, int wave, int& k0, int& nsteps) {
  const int kw0 = split * 4 * g.kslice;
  const int kw1 = kw0 + 4 * g.kslice < g.K ? kw0 + 4 * g.kslice : g.K;
  const int all = kw1 > kw0 ? (kw1 - kw0) / 32 : 0;
  k0 = kw0 + 32 * wave;
  nsteps = (all - wave + 3) / 4;
}
// K offset of the wave's step j, clamped to its last step (the refills past
// the last step re-read it)
__host__ __device__ inline int narrow_step_k(int k0, int j, int nsteps) { return k0 + 128 * (j < nsteps - 1 ? j : nsteps - 1); }
// lane's row within a 16-row block and its 8-element K offset within a step
__host__ __device__ inline int narrow_lane_row(int lane) { return lane & 15; }
__host__ __device__ inline int narrow_lane_k(int lane) { return (lane >> 4) * 8; }
// The host's choice of K split, row blocks per tile and per-wave K slice of
// the narrow tile for an n-row call (nr = min(max_rows, 32) rows fix the
// split, whatever the call's own row count; target: workgroups the
// persistent step fills, 0 for a stand-alone kernel with 256 compute units).
// The split fixes the summation order. It only splits while each split still
// adds a workgroup per compute unit (splitting further leaves workgroups
// queued behind others and adds partial traffic, which costs more than the
// latency it hides), keeps >= 64 K per wave, partial traffic below the
// weights', and the partials within the workspace.
inline void narrow_plan(int n, int npairs, int K, int nr, int target, int M_pad, int Nv, size_t partial_cap, int& S,
                        int& mb, int& kslice) {
  mb = gemm_row_blocks(n);
  const int MBr = gemm_row_blocks(nr);
  const int tiles = npairs * ((nr + 16 * MBr - 1) / (16 * MBr));
  S = target ? std::max(1, (target + tiles - 1) / tiles) : std::max(1, 256 / tiles);
  S = std::min(S, std::max(1, K / 256));
  S = std::min(S, std::max(1, K / (4 * nr)));
  while (S > 1 && (size_t)S * M_pad * Nv > partial_cap) --S;
  const int per = (K + 4 * S - 1) / (4 * S);
  kslice = (per + 31) / 32 * 32;
}

// Epilogue kinds (functors live in the GEMM translation unit).
enum EpiKind {
  EPI_STORE = 0,   // out[m][c] = v                          (logits)
  EPI_QKV = 1,     // q (f32, rotary), k (T, rotary), v (T)   eqs (2.12)-(2.13)
  EPI_QROT = 2,    // q (f32, rotary)                          eq (2.15) query
  EPI_RESID = 3,   // z[m][c] += v                             residual adds
  EPI_SWIGLU = 4,  // act[m][c] = silu(gate) * up              eq (2.16)
  EPI_MGATE = 5,   // g[m][c] = sigmoid(v + b_g[c])           eq (2.10)
  EPI_MOUT = 6,    // z[m][c] = e + alpha * g * v              eq (2.11)
  EPI_CONVEX = 7,  // g = sigmoid(v + b); z = g e + (1-g) s
  EPI_MEMKV = 8,   // memory entry: k (T, rotary at t) and v (T)   eq (2.2)
  EPI_STORE_T = 9  // out_k[m][c] = v in the element type (low-rank W_s: V r)
};

struct EpiArgs {
  int kind;
  Rows rows;
  int d, dh, H;
  int rope;                 // apply rotary transform
  const double* inv_freq;   // [dh/2] theta^(-2i/dh)
  const float2* rope_tab;   // [rope_tmax + 1][dh/2] (cos, sin) of t * inv_freq[i], or null
  int rope_tmax;
  float* out_f;             // f32 output (q, logits, z, g)
  int64_t ldo;
  void* out_k;              // T outputs (k, act)
  void* out_v;
  const float* bias;        // b_g
  const float* gbuf;        // merge gate
  float alpha;
  EIn e;                    // merge: e_t
  const float* s_state;     // convex merge: s_{t-1} rows
  // producers (EPI_RESID, EPI_MOUT, EPI_CONVEX): gain of the next RMSNorm and
  // the [M][d] (T) buffer receiving z * gain, the next product's input
  const float* gnext;
  void* zb;
  int pk;                   // bf16: zb and the SwiGLU output are written in fragment order
  int64_t lo;               // fragment-order outputs: elements to their second term (0: one term)
  // memory entries (EPI_MEMKV): one group's K / V buffers; the entry of slot
  // m is at rows[m] * msb + (t_row[m] - 1) * mst elements
  void* mk;
  void* mv;
  int64_t msb, mst;
  int mem_vec;  // bf16 and every 8-column run of a destination entry 16-byte aligned
};

// ----------------------------------------------------------------------------
// host-side launchers (defined in the .hip translation units)
// ----------------------------------------------------------------------------

struct AttnArgs {
  Rows rows;
  int d, H, dh;
  int hpw;                  // heads per workgroup
  float qscale;             // log2(e) / sqrt(dh)
  const float* q;           // [n][d]
  // SWA
  const void* kc;           // [n][d] current k (T)
  const void* vc;
  void* ring_k;             // layer base: [B_cap][W-1][d]
  void* ring_v;
  int W;
  // cross-attention
  const void* mk;           // group base (row stride sb, position stride st)
  const void* mv;
  int64_t sb, st;
  int chunk;                // positions per partial
  int nch;                  // chunk slots per row in `part`
  float* part;              // [n][nch][H][dh + 2]
  void* out;                // [n][d] (T) attention output
  int out_pk;               // bf16: out in fragment order (the next product's operand)
  int64_t out_lo;           // fragment-order out: elements to its second term (0: one term)
  int direct;               // cross-attention with one chunk: the normalised output, no combine
  int* cnt;                 // [n][H / hpw] arrival counters, zero between launches: chunks combined
                            // by the cross-attention launch itself (null: by the combine kernel)
};

void launch_gemm(int dtype, const GemmArgs& g, const EpiArgs& e, hipStream_t s);
// tab[t][i] = (cos, sin)(t * inv_freq[i]) for t <= tmax, i < dh/2: the values
// the epilogues' rotary transform computes (double precision, rounded)
void launch_rope_table(const double* inv_freq, int dh, int tmax, float2* tab, hipStream_t s);
// Wp <- g's weights (bf16) in fragment order (K % 64 == 0, Nv % 32 == 0)
void launch_pack_weights(const GemmArgs& g, void* Wp, hipStream_t s);
void launch_swa(int dtype, const AttnArgs& a, hipStream_t s);
void launch_xattn(int dtype, const AttnArgs& a, hipStream_t s);
void launch_xcombine(int dtype, const AttnArgs& a, hipStream_t s);

struct MiscArgs {
  Rows rows;
  int n, d;
  float eps;
  float* s_state;                 // [B_cap][d]
  int* pos;
  int* pending;
  const int* mem_len;
  const int* consume_tok;
  int* t_row_out;
  int* err;                       // device-visible error word (host mapped)
  const float* gain;
  const float* z;                 // [n][d]
  void* out;                      // T [n][ld_out]
  int64_t ld_out;
  EIn e;
  int merge_kind;
  const void* wg;                 // scalar merge gate: w_g [2d] (T), or null (vector gate)
  const float* bg;                // b_g [1] (scalar gate)
  float* gbuf;                    // [n][d] gate values (scalar gate: broadcast)
  float* s_out;                   // optional [n][d]
  float* s_trace;                 // optional replay trace
  int64_t s_trace_sb;
  int max_t;                      // largest position the workspace supports
  int B_cap;                      // rows in the state buffers
  int pk;                         // merge preparation: X (and out2) in fragment order
  void* out2;                     // merge preparation: RMSNorm_s(s_{t-1}) alone (pk, gated)
  int64_t lo, lo2;                // fragment order: elements from out / out2 to their second terms
  int* claim;                     // [B_cap] slots per state row in this call (decoder step), or null
};

void launch_prestep(const MiscArgs& a, hipStream_t s);
void launch_merge_prep(int dtype, const MiscArgs& a, hipStream_t s);
void launch_rmsnorm(int dtype, const MiscArgs& a, hipStream_t s);
void launch_final(int dtype, const MiscArgs& a, hipStream_t s);
void launch_copy_f32(const float* src, float* dst, int64_t n, hipStream_t s);

// encoder memory [RLT §2.2, eq. (2.2)]
void launch_mem_slots(const int* rows, int n, const int* mem_len, int B_cap, int T_cap, int* t_out, int* err,
                      hipStream_t s);
void launch_mem_rows(const int* offs, int B, int64_t r0, int n, int* src_out, int* t_out, hipStream_t s);
// A[slot] = e(slot) * gain (dtype), ssq[slot] = sum of squares of e(slot)
void launch_mem_prep(int dtype, const Rows& rows, EIn e, int d, const float* gain, void* A, float* ssq,
                     hipStream_t s);
void launch_mem_commit(const int* rows, int n, const int* t_row, int* mem_len, hipStream_t s);
void launch_mem_setlen(const int* len, int B, int* mem_len, hipStream_t s);

// out[b] = sum over t = first[b] .. last[b] of logp[b][t] - logmu[b][t] [RLT §5.3]
void launch_traj_ratio(int B, const int* first, const int* last, const float* logp, int64_t logp_sb,
                       const float* logmu, int64_t logmu_sb, float* out, hipStream_t s);

struct ReadoutArgs {
  Rows rows;
  int n, V;
  const float* logits;       // [n][V]
  int32_t* argmax;
  // scoring: token/out located per slot
  int mode;                  // 0: step (arrays by slot), 1: replay (by src,t)
  const int* score_tok;      // step: [n]; replay: tokens base
  int64_t tok_sb;
  float* logp;               // step: [n]; replay: base
  int64_t logp_sb;
  const int* split;          // replay: [B] first scored position
  // sampling / behaviour
  const float* uniform;      // [n] or null
  float temperature;
  int top_k;
  float top_p;               // nucleus after top-k; outside (0, 1): none
  int32_t* sample_tok;
  float* sample_logmu;
  float* logmu;              // behaviour log-prob of score_tok (score call)
  const float* logmu_beh;    // recorded behaviour log-probs (score call)
  float* ratio;
};
void launch_readout(const ReadoutArgs& a, hipStream_t s);

struct PostArgs {
  Rows rows;
  int n;
  int* pos;
  int* pending;
  const int32_t* next_tok;   // token to record as pending (DEFER) or null
  int* claim;                // [B_cap] slot counts to clear (decoder step), or null
  int B_cap;
  int* tick;                 // replay: position counter to advance by one, or null
};
void launch_poststep(const PostArgs& a, hipStream_t s);
// read n16 16-byte pieces once (counter calibration)
void launch_stream_read(const void* p, int64_t n16, bool nontemporal, unsigned* sink, hipStream_t s);
void launch_mfma_loop(int blocks, int iters, unsigned* sink, hipStream_t s);
// counts[rows[i]] = 0 for i < n (a fill kernel: capturable)
void launch_zero_rows(int* counts, const int* rows, int n, int B_cap, hipStream_t s);

// ----------------------------------------------------------------------------
// persistent step: the launches of a transition are recorded as phases and
// run by one kernel that keeps one workgroup per compute unit and crosses a
// grid-wide barrier between phases (small calls, where launch latency rather
// than bandwidth bounds the separate kernels)
// ----------------------------------------------------------------------------

enum PhaseKind {
  PH_GEMM = 0,        // k_gemm_bf16 tile (bf16, 1 or 2 row blocks)
  PH_SPLITK = 1,      // split-K sum + epilogue
  PH_SWA = 2,
  PH_XATTN = 3,
  PH_XCOMBINE = 4,
  PH_MERGE_PREP = 5,
  PH_FINAL = 6,
  PH_COPY = 7,
  PH_INVALID = -1     // marks a recording that contains a launch the persistent kernel cannot run
};

struct CopyArgs {
  const float* src;
  float* dst;
  int64_t n;
};

struct GemmPhase {
  GemmArgs g;
  EpiArgs e;
};

// One recorded launch: a virtual grid of (gx, gy, gz) blocks of 256 threads.
struct Phase {
  int kind;
  int gx, gy, gz;
  union {
    GemmPhase gm;
    AttnArgs at;
    MiscArgs mi;
    CopyArgs cp;
  } u;
};

// Host: while a recorder is installed, the recordable launchers (bf16
// products with up to 2 row blocks, attention, merge preparation, state
// write-back, copies) append a phase and return true instead of launching.
bool record_phase(const Phase& p);

// Grid-barrier words: [0] arrival counter (self-resetting), [1] abort flag.
void launch_fused(const Phase* phases, int nphase, unsigned* sync, int* err, int grid, int64_t spin_ticks,
                  hipStream_t s);
// workgroups of the persistent kernel that fit on one compute unit
int fused_blocks_per_cu();

void launch_init(int dtype, const int* rows, int n, const float* s_star, float* s_state, int* pos,
                 int* pending, void* ring_k, void* ring_v, int L, int B_cap, int W, int d,
                 int poison, hipStream_t s);
void launch_set_pending(const int* rows, const int* src, int n, const int* tokens, int64_t tok_sb,
                        const int* last_index, int* pending, hipStream_t s);
void launch_replay_rows(const int* rows, int n, const int* tick_dev, int* t_row, int* pos, const int* mem_len,
                        int* err, hipStream_t s);

}  // namespace rlt
