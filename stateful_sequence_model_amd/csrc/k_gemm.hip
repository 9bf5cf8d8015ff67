// Matrix products of the decoder transition with fused epilogues.
//
// Every projection of the step is Y = A W^T with A the [rows][K] activations
// and W a natural-layout [out][in] weight ("Recurrent Looped Transformer",
// §2.5 eqs. (2.9)-(2.16) and §2.3 eq. (2.6)). Weights are streamed once per
// call; the batch is the M dimension, so these products are HBM-bound for
// the batch sizes of a decoder step.
//
// bf16 path, calls of at most 32 rows (gfx950 MFMA v_mfma_f32_16x16x32_bf16):
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
#include "gemm_dev.h"

namespace rlt {

// grid: x = pair, y = split, z = m-tile; block 256 (4 waves)
template <int MB>
__global__ __launch_bounds__(256) void k_gemm_bf16(GemmArgs g, Epi<uint16_t> epi) {
  __shared__ float lds[gemm_lds_floats(MB)];
  gemm_bf16_body<MB>(g, epi, blockIdx.x, blockIdx.y, blockIdx.z, lds);
}

// Tile for calls above 32 rows: 128 rows x BN virtual columns per
// workgroup, K in stages of 64. Both operands are staged through LDS: a
// stage is loaded with row-contiguous 16-byte loads (8 lanes read one
// 128-byte row segment), PF stages ahead in registers, then written to one
// of two LDS buffers whose rows are padded by 16 bytes so that the MFMA
// operand reads (32 rows at one k offset) hit distinct banks. Four waves in
// a 2 x 2 arrangement each multiply 64 rows by BN/2 columns with
// v_mfma_f32_32x32x16_bf16, which issues close to its peak rate with four
// accumulators per wave (the 16x16x32 form needs twice as many).
// Virtual columns: the 32-column MFMA block j of a wave holds one column
// pair, its first 16 columns being the pair's block ba and the last 16 its
// block bb, so the epilogue of a pair combines lanes l and l ^ 16, which hold
// the same rows (C layout: lane l holds column l % 32 of the block and rows
// 8 g + 4 (l / 32) + q, g, q < 4).
// grid: npairs / (BN / 32) * S * m-tiles (1-D, decoded as in the other
// tiles); block 256; K range of a workgroup = kslice (a multiple of 64).
template <int BN>
__global__ __launch_bounds__(256) void k_gemm_bf16_tile(GemmArgs g, Epi<uint16_t> epi) {
  constexpr int BM = 128, BK = 64, LDR = BK + 8, PF = 2;
  constexpr int WN = BN / 2, NB = WN / 32;
  constexpr int LA = BM * BK / 8 / 256, LW = BN * BK / 8 / 256;
  constexpr int LDC = BN + 1;  // float row stride of the staged output tile
  constexpr int STAGE_BYTES = 2 * (BM + BN) * LDR * 2, C_BYTES = BM * LDC * 4;
  // the two operand buffers, reused for the output tile after the K loop
  __shared__ __attribute__((aligned(16))) unsigned char smem[STAGE_BYTES > C_BYTES ? STAGE_BYTES : C_BYTES];
  uint16_t(*sA)[BM * LDR] = reinterpret_cast<uint16_t(*)[BM * LDR]>(smem);
  uint16_t(*sW)[BN * LDR] = reinterpret_cast<uint16_t(*)[BN * LDR]>(smem + 2 * BM * LDR * 2);
  __shared__ float s_rstd[BM];
  __shared__ float s_part[rowrstd_lds<BM, 256>()];
  // XCD-aware order: consecutive workgroup ids run on the 8 XCDs in turn, so
  // id b maps to tile (b % 8) * (T / 8) + b / 8 (ids past 8 * (T / 8) map to
  // themselves), m-tile fastest: the row tiles of one weight slice share an L2
  const int T = gridDim.x, b = blockIdx.x, per = T >> 3;
  const int t = b < 8 * per ? (b & 7) * per + (b >> 3) : b;
  const int nmt = (g.M + BM - 1) / BM;
  const int mt = t % nmt, split = (t / nmt) % g.S, grp = t / (nmt * g.S);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int wm = wave >> 1, wn = wave & 1;
  const int m0 = mt * BM, pair0 = grp * (BN / 32);
  const int kw0 = split * g.kslice;
  const int kw1 = min(kw0 + g.kslice, g.K);
  const int nst = max(0, (kw1 - kw0) / BK);
  // loads: thread covers rows lr + 32 i of the stage, 16-byte chunk lc
  const int lr = tid >> 3, lc = (tid & 7) * 8;
  const uint16_t* pa[LA];
#pragma unroll
  for (int i = 0; i < LA; ++i) pa[i] = (const uint16_t*)g.A + (int64_t)(m0 + lr + 32 * i) * g.lda + kw0 + lc;
  const uint16_t* pw[LW];
#pragma unroll
  for (int i = 0; i < LW; ++i) {
    const int v = lr + 32 * i;  // virtual column of the tile
    int ba, bb;
    pair_blocks(g, pair0 + v / 32, ba, bb);
    pw[i] = weight_row<uint16_t>(g, ((v & 16) ? bb : ba) * 16 + (v & 15)) + kw0 + lc;
  }
  const bool norm_here = g.S == 1 && g.ssq_in != nullptr;
  RowRstd<BM> rr(g, norm_here ? m0 : 0);
  // memory entries (the token-parallel prefill): each row's position and
  // destination, loaded now and staged for the epilogue (no dependent loads
  // inside it)
  const bool memkv = g.S == 1 && epi.a.kind == EPI_MEMKV;
  __shared__ int s_t[BM];
  __shared__ int64_t s_off[BM];
  int my_t = 0, my_row = 0;
  if (memkv && tid < BM && m0 + tid < g.M) {
    my_t = epi.a.rows.t_row[m0 + tid];
    my_row = epi.a.rows.rows[m0 + tid];
  }
  bf16x8_t ra[PF][LA], rw[PF][LW];
  auto gload = [&](int p, int st) {
#pragma unroll
    for (int i = 0; i < LA; ++i) ra[p][i] = load8(pa[i] + BK * st);
#pragma unroll
    for (int i = 0; i < LW; ++i) rw[p][i] = load8(pw[i] + BK * st);
  };
  auto lstore = [&](int p, int buf) {
#pragma unroll
    for (int i = 0; i < LA; ++i) *(bf16x8_t*)(sA[buf] + (lr + 32 * i) * LDR + lc) = ra[p][i];
#pragma unroll
    for (int i = 0; i < LW; ++i) *(bf16x8_t*)(sW[buf] + (lr + 32 * i) * LDR + lc) = rw[p][i];
  };
  f32x16_t acc[2][NB];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;
  const int r32 = lane & 31, kh = (lane >> 5) * 8;
  auto compute = [&](int buf) {
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      bf16x8_t a[2], w[NB];
#pragma unroll
      for (int i = 0; i < 2; ++i) a[i] = *(const bf16x8_t*)(sA[buf] + (wm * 64 + i * 32 + r32) * LDR + ks * 16 + kh);
#pragma unroll
      for (int j = 0; j < NB; ++j) w[j] = *(const bf16x8_t*)(sW[buf] + (wn * WN + j * 32 + r32) * LDR + ks * 16 + kh);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], w[j], acc[i][j], 0, 0, 0);
    }
  };
  // Register slot s % PF holds stage s until it is written to LDS buffer
  // s % 2, then takes stage s + PF. Stage st is multiplied from buffer st % 2
  // while stages st + 1 .. st + PF are in flight; the barrier after it
  // publishes stage st + 1 and frees buffer st % 2 for stage st + 2.
  if (nst > 0) {
#pragma unroll
    for (int p = 0; p < PF; ++p) gload(p, min(p, nst - 1));
    lstore(0, 0);
    gload(0, min(PF, nst - 1));
    __syncthreads();
  }
  int st = 0;
  for (; st + PF <= nst; st += PF) {
#pragma unroll
    for (int p = 0; p < PF; ++p) {
      const int cur = st + p;
      compute(cur & 1);
      if (cur + 1 < nst) {  // uniform
        lstore((p + 1) % PF, (cur + 1) & 1);
        gload((p + 1) % PF, min(cur + 1 + PF, nst - 1));
      }
      __syncthreads();
    }
  }
#pragma unroll
  for (int p = 0; p < PF; ++p) {
    const int cur = st + p;
    if (cur < nst) {  // uniform
      compute(cur & 1);
      if (cur + 1 < nst) lstore((p + 1) % PF, (cur + 1) & 1);
      __syncthreads();
    }
  }
  // output tile to LDS (the operand buffers are free after the last barrier),
  // C layout: lane l holds column l % 32 of a 32-column block and rows
  // 8 g + 4 (l / 32) + q (g, q < 4)
  float* Cs = reinterpret_cast<float*>(smem);
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int gq = 0; gq < 16; ++gq)
        Cs[(wm * 64 + i * 32 + 8 * (gq >> 2) + 4 * (lane >> 5) + (gq & 3)) * LDC + wn * WN + j * 32 + r32] =
            acc[i][j][gq];
  __syncthreads();
  // output column of virtual column v of this tile
  auto col_of = [&](int v) {
    int ba, bb;
    pair_blocks(g, pair0 + v / 32, ba, bb);
    return ((v & 16) ? bb : ba) * 16 + (v & 15);
  };
  if (g.S > 1) {
    for (int idx = tid; idx < BM * BN; idx += 256) {
      const int row = idx / BN, v = idx % BN;
      if (m0 + row < g.M) g.partial[((int64_t)split * g.M_pad + m0 + row) * g.Nv + col_of(v)] = Cs[row * LDC + v];
    }
    // summed in split order by k_splitk_epi (an in-kernel reduction by the
    // last workgroup of each tile, with release / acquire at device scope,
    // measured several times slower)
    return;
  }
  if (memkv && tid < BM) {
    s_t[tid] = my_t;
    s_off[tid] = (int64_t)my_row * epi.a.msb + (int64_t)(my_t - 1) * epi.a.mst;
  }
  if (norm_here) rr.finish(g, m0, s_part, s_rstd);  // uniform branch: contains a barrier
  __syncthreads();
  if (memkv && epi.a.mem_vec) {
    // two threads per (row, pair), each 8 consecutive columns of block ba and
    // the same 8 of bb: 16-byte stores (2 bytes per lane and store measured
    // as most of the prefill's epilogue)
    for (int it = tid; it < BM * (BN / 32) * 2; it += 256) {
      const int hh = it & 1, rp = it >> 1;
      const int pl = rp % (BN / 32), row = rp / (BN / 32);
      if (m0 + row >= g.M || s_t[row] <= 0) continue;
      int ba, bb;
      pair_blocks(g, pair0 + pl, ba, bb);
      float va[8], vb[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        va[k] = Cs[row * LDC + pl * 32 + 8 * hh + k];
        vb[k] = Cs[row * LDC + pl * 32 + 16 + 8 * hh + k];
      }
      epi.memkv_at8(s_t[row], s_off[row], ba * 16 + 8 * hh, va, bb * 16 + 8 * hh, vb, norm_here ? s_rstd[row] : 1.f);
    }
    return;
  }
  // 16 consecutive threads take the 16 column positions of one (row, pair):
  // virtual columns c16 (block ba) and 16 + c16 (block bb); every thread runs
  // the same trip count, so the row sums of squares reduce over those 16
  const int c16 = tid & 15;
  for (int it = tid >> 4; it < BM * (BN / 32); it += 16) {
    const int pl = it % (BN / 32), row = it / (BN / 32);
    const int m = m0 + row, pair = pair0 + pl;
    int ba, bb;
    pair_blocks(g, pair, ba, bb);
    const float va = Cs[row * LDC + pl * 32 + c16], vb = Cs[row * LDC + pl * 32 + 16 + c16];
    float sq = 0.f;
    if (memkv) {
      if (m < g.M && s_t[row] > 0)
        epi.memkv_at(s_t[row], s_off[row], ba * 16 + c16, va, bb * 16 + c16, vb, norm_here ? s_rstd[row] : 1.f);
    } else if (m < g.M) {
      sq = epi(m, ba * 16 + c16, va, bb * 16 + c16, vb, norm_here ? s_rstd[row] : 1.f);
    }
    if (g.ssq_out) {
      sq = sum16(sq);
      if (c16 == 0 && m < g.M) g.ssq_out[(int64_t)pair * g.M_pad + m] = sq;
    }
  }
}

// Summation order of the products with both operands in fragment order (the
// same for every kernel and launch shape below, so that a row's result does
// not depend on the call it is in, nor on how the call is tiled):
//   * the K range is n = K / 64 chunks of 64, cut into 8 streams; stream s
//     holds the contiguous chunks [s n / 8, (s + 1) n / 8) (floor; empty
//     streams are zero);
//   * a stream accumulates its chunks in increasing order, each chunk as four
//     16-wide v_mfma_f32_32x32x16_bf16 steps starting from zero (with two
//     activation terms: per step the first term, then the second);
//   * the 8 stream sums combine by a balanced tree of neighbours:
//       ((s0 + s1) + (s2 + s3)) + ((s4 + s5) + (s6 + s7)).
// A group of 2^j consecutive streams is a subtree, so the work can be split
// over waves, over workgroups (partials combined by k_pk_combine), or run in
// sequence by one wave that keeps finished subtrees on a small stack.
__device__ __forceinline__ int stream_begin(int nchunk, int s) { return (s * nchunk) >> 3; }

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

// Fold the running sum r of stream j (of a group of Q) into the stack of
// finished subtrees (st[l] holds a subtree of 2^l streams; log2 Q levels);
// after the last stream r holds the group's sum. r restarts at zero
// otherwise.
template <int Q>
constexpr int fold_levels() { return Q >= 8 ? 3 : (Q >= 4 ? 2 : 1); }
template <int Q>
__device__ __forceinline__ void stream_fold(int j, f32x16_t& r, f32x16_t (&st)[fold_levels<Q>()]) {
  f32x16_t v = r;
  int t = j + 1, l = 0;
#pragma unroll
  for (int h = 0; h < 3; ++h)
    if ((t & 1) == 0 && (1 << h) < Q) {
      v = st[h] + v;
      t >>= 1;
      l = h + 1;
    } else {
      break;
    }
  if (j == Q - 1) {
    r = v;
  } else {
#pragma unroll
    for (int h = 0; h < fold_levels<Q>(); ++h)
      if (h == l) st[h] = v;
#pragma unroll
    for (int e = 0; e < 16; ++e) r[e] = 0.f;
  }
}

// Tile for the token-parallel memory construction (calls of at least 256
// rows whose K/V epilogue stores 16-byte runs, no K split): 256 rows x 256
// virtual columns per workgroup of 8 waves, K in stages of 64. The operands
// are staged through two padded LDS buffers as in k_gemm_bf16_tile (each
// stage's loads issued one stage ahead, its LDS writes before the MFMAs of
// the stage before it); the waves form 2 x 4, each multiplying 128 rows
// by 64 columns (4 x 2 accumulators of v_mfma_f32_32x32x16_bf16), so a wave
// reads 6 KB of LDS per 8 MFMAs of a 16-wide step instead of 4 KB per 4 with
// 64 x 64 wave tiles. The row statistics are loaded after the K loop (their
// registers are taken by the accumulators) and the output is staged in LDS
// 128 rows at a time for the epilogue (virtual columns and C layout as in
// k_gemm_bf16_tile).
// grid: npairs / 8 * m-tiles (1-D, m-tile fastest within an XCD); block 512.
__global__ __launch_bounds__(512) void k_gemm_bf16_big(GemmArgs g, Epi<uint16_t> epi) {
  constexpr int BM = 256, BN = 256, BK = 64, LDR = BK + 8, NT = 512, PF = 1;
  constexpr int LA = BM * BK / 8 / NT, LW = BN * BK / 8 / NT;  // 16-byte pieces per thread and stage
  constexpr int HM = BM / 2, LDC = BN + 1;                     // output staged HM rows at a time
  constexpr int STAGE_BYTES = 2 * (BM + BN) * LDR * 2;
  static_assert(HM * LDC * 4 <= STAGE_BYTES && rowrstd_lds<BM, NT>() * 4 <= STAGE_BYTES,
                "the epilogue reuses the operand buffers");
  __shared__ __attribute__((aligned(16))) unsigned char smem[STAGE_BYTES];
  uint16_t(*sA)[BM * LDR] = reinterpret_cast<uint16_t(*)[BM * LDR]>(smem);
  uint16_t(*sW)[BN * LDR] = reinterpret_cast<uint16_t(*)[BN * LDR]>(smem + 2 * BM * LDR * 2);
  __shared__ float s_rstd[BM];
  __shared__ int s_t[BM];
  __shared__ int64_t s_off[BM];
  const int T = gridDim.x, b = blockIdx.x, per = T >> 3;
  const int t = b < 8 * per ? (b & 7) * per + (b >> 3) : b;
  const int nmt = (g.M + BM - 1) / BM;
  const int mt = t % nmt, grp = t / nmt;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int wm = wave >> 2, wn = wave & 3;
  const int m0 = mt * BM, pair0 = grp * (BN / 32);
  const int nst = g.K / BK;
  // loads: thread covers rows lr + 64 i of the stage (clamped below M, never
  // stored), 16-byte chunk lc
  const int lr = tid >> 3, lc = (tid & 7) * 8;
  const uint16_t* pa[LA];
#pragma unroll
  for (int i = 0; i < LA; ++i) {
    const int m = m0 + lr + 64 * i < g.M ? m0 + lr + 64 * i : g.M - 1;
    pa[i] = (const uint16_t*)g.A + (int64_t)m * g.lda + lc;
  }
  const uint16_t* pw[LW];
#pragma unroll
  for (int i = 0; i < LW; ++i) {
    const int v = lr + 64 * i;  // virtual column of the tile
    int ba, bb;
    pair_blocks(g, pair0 + v / 32, ba, bb);
    pw[i] = weight_row<uint16_t>(g, ((v & 16) ? bb : ba) * 16 + (v & 15)) + lc;
  }
  if (tid < BM) {
    const int m = m0 + tid;
    s_t[tid] = m < g.M ? epi.a.rows.t_row[m] : 0;
    s_off[tid] = m < g.M ? (int64_t)epi.a.rows.rows[m] * epi.a.msb + (int64_t)(s_t[tid] - 1) * epi.a.mst : 0;
  }
  bf16x8_t ra[PF][LA], rw[PF][LW];
  auto gload = [&](int p, int st) {
#pragma unroll
    for (int i = 0; i < LA; ++i) ra[p][i] = load8(pa[i] + BK * st);
#pragma unroll
    for (int i = 0; i < LW; ++i) rw[p][i] = load8(pw[i] + BK * st);
  };
  auto lstore = [&](int p, int buf) {
#pragma unroll
    for (int i = 0; i < LA; ++i) *(bf16x8_t*)(sA[buf] + (lr + 64 * i) * LDR + lc) = ra[p][i];
#pragma unroll
    for (int i = 0; i < LW; ++i) *(bf16x8_t*)(sW[buf] + (lr + 64 * i) * LDR + lc) = rw[p][i];
  };
  f32x16_t acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;
  const int r32 = lane & 31, kh = (lane >> 5) * 8;
  auto compute = [&](int buf) {
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      bf16x8_t a[4], w[2];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = *(const bf16x8_t*)(sA[buf] + (wm * 128 + i * 32 + r32) * LDR + ks * 16 + kh);
#pragma unroll
      for (int j = 0; j < 2; ++j) w[j] = *(const bf16x8_t*)(sW[buf] + (wn * 64 + j * 32 + r32) * LDR + ks * 16 + kh);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], w[j], acc[i][j], 0, 0, 0);
    }
  };
  // the schedule of k_gemm_bf16_tile: register slot s % PF holds stage s
  // until it is written to LDS buffer s % 2; one barrier per stage
  if (nst > 0) {
#pragma unroll
    for (int p = 0; p < PF; ++p) gload(p, min(p, nst - 1));
    lstore(0, 0);
    gload(0, min(PF, nst - 1));
    __syncthreads();
  }
  // The next stage's LDS writes and the refill loads are issued before the
  // current stage's MFMAs (buffer (cur + 1) % 2 was last read before the
  // previous barrier; the refill's register slot was just written out), so
  // that they proceed under the MFMA chain.
  int st = 0;
  for (; st + PF <= nst; st += PF) {
#pragma unroll
    for (int p = 0; p < PF; ++p) {
      const int cur = st + p;
      if (cur + 1 < nst) {  // uniform
        lstore((p + 1) % PF, (cur + 1) & 1);
        gload((p + 1) % PF, min(cur + 1 + PF, nst - 1));
      }
      compute(cur & 1);
      __syncthreads();
    }
  }
#pragma unroll
  for (int p = 0; p < PF; ++p) {
    const int cur = st + p;
    if (cur < nst) {  // uniform
      if (cur + 1 < nst) lstore((p + 1) % PF, (cur + 1) & 1);
      compute(cur & 1);
      __syncthreads();
    }
  }
  // row statistics (into the free operand buffers), then the output in two
  // halves of 128 rows: the waves of half h stage their tile, all threads
  // run the epilogue, 16-byte runs of 8 columns of a pair's two blocks
  const bool norm_here = g.ssq_in != nullptr;
  if (norm_here) {  // uniform branch: contains barriers
    RowRstd<BM, NT> rr(g, m0);
    rr.finish(g, m0, reinterpret_cast<float*>(smem), s_rstd);
  }
  __syncthreads();
  float* Cs = reinterpret_cast<float*>(smem);
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    if (wm == h) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int gq = 0; gq < 16; ++gq)
            Cs[(i * 32 + 8 * (gq >> 2) + 4 * (lane >> 5) + (gq & 3)) * LDC + wn * 64 + j * 32 + r32] = acc[i][j][gq];
    }
    __syncthreads();
    for (int it = tid; it < HM * (BN / 32) * 2; it += NT) {
      const int hh = it & 1, rp = it >> 1;
      const int pl = rp % (BN / 32), rh = rp / (BN / 32), row = h * HM + rh;
      if (m0 + row >= g.M || s_t[row] <= 0) continue;
      int ba, bb;
      pair_blocks(g, pair0 + pl, ba, bb);
      float va[8], vb[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        va[k] = Cs[rh * LDC + pl * 32 + 8 * hh + k];
        vb[k] = Cs[rh * LDC + pl * 32 + 16 + 8 * hh + k];
      }
      epi.memkv_at8(s_t[row], s_off[row], ba * 16 + 8 * hh, va, bb * 16 + 8 * hh, vb, norm_here ? s_rstd[row] : 1.f);
    }
    __syncthreads();
  }
}

// Product for calls of up to 64 rows, both operands in fragment order (see
// pk_off): a workgroup owns 32 RB rows x CB column pairs over the whole K;
// its 8 waves are the 8 streams, each loading its chunks' fragments straight
// into registers (one load instruction reads 1 KB of consecutive bytes; no
// LDS staging and no barrier in the K loop). The K loop is branch-free, so
// that each chunk waits only for its own loads: lanes of rows at or past M
// load the last row below M (the same addresses for all of them, so a call
// of a few rows reads little more than the weights; those outputs are
// discarded), and loads past a wave's last chunk re-read that chunk (never
// used). The epilogue threads add the waves' sums by the stream tree, from
// LDS.
// TWO: the activations carry a second bf16 term at A + a_lo (the rounding
// remainder of the first), so the product sees its float32 input to about 16
// significant bits while the weights stay bf16.
// Tile order: workgroup b runs on XCD b % 8 and takes column tile
// 8 (q / mtiles) + b % 8 and row tile q % mtiles (q = b / 8), so the row
// tiles of one column tile share its weights in one L2.
// PRE: the epilogue's memory reads (residual, gains, rotary table) are issued
// before the K loop.
// MS > 0 (calls of at most MS rows, K at most 64 PK_LDS_CHUNKS; taken for
// one-row calls): the activations' fragments of the call's rows (the only
// lanes whose outputs are kept) are staged once in LDS for the whole K, and
// each chunk reads them from there; the K loop then issues weight loads only.
// (At one row the activation loads, at one address per half-wave but one
// instruction each, otherwise take two of every three load slots of the
// compute unit; the smaller register and LDS footprint also fits two
// workgroups per compute unit.) Same operand values for the kept rows, same
// instructions in the same order.
// grid: 8 * mtiles * ceil(ntiles / 8); block 512.
template <int RB, int CB, int PF, bool PRE, bool TWO, int MS>
__global__ __launch_bounds__(512) void k_gemm_bf16_pk(GemmArgs g, Epi<uint16_t> epi) {
  constexpr int NW = 8, R = 32 * RB, NT = 64 * NW, TERMS = TWO ? 2 : 1;
  constexpr int TILE = RB * CB * 16 * 64;  // floats of one wave's partial tile
  static_assert(MS == 0 || (RB == 1 && MS <= 32), "staged activations: one row block");
  __shared__ float red[NW * TILE];
  __shared__ float s_rstd[R];
  __shared__ float s_part[rowrstd_lds<R, NT>()];
  // staged activations: piece ((term * nchunk + c) * 4 + st) * 2 MS + half * MS + row
  __shared__ bf16x8_t s_a[MS > 0 ? TERMS * PK_LDS_CHUNKS * 8 * MS : 1];
  const int mtiles = (g.M + R - 1) / R, ntiles = g.npairs / CB;
  const int b = blockIdx.x, q = b >> 3;
  const int mt = q % mtiles, nt = 8 * (q / mtiles) + (b & 7);
  if (nt >= ntiles) return;  // whole workgroup, before any barrier
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int m0 = mt * R;
  const int nchunk = g.K >> 6;
  const uint16_t* ap[RB];
  const uint16_t* wp[CB];
  for (int r = 0; r < RB; ++r) {
    // this lane's row of block r, clamped below M (lane l holds row l % 32)
    const int last = g.M - 1 - (m0 + 32 * r);
    const int rl = last < 0 ? 0 : ((lane & 31) < last ? (lane & 31) : last);
    ap[r] = (const uint16_t*)g.A + ((int64_t)(mt * RB + r) * nchunk * 256 + (lane & 32) + rl) * 8;
  }
#pragma unroll
  for (int c = 0; c < CB; ++c) wp[c] = (const uint16_t*)g.Wp + ((int64_t)(nt * CB + c) * nchunk * 256 + lane) * 8;
  const bool norm_here = g.ssq_in != nullptr;
  RowRstd<R, NT> rr(g, norm_here ? m0 : 0);
  // epilogue items: (row, column pair) units of 16 consecutive threads
  constexpr int NU = R * CB, NG = NT / 16, NI = (NU + NG - 1) / NG;
  const int c16 = tid & 15, grp = tid >> 4;
  typename Epi<uint16_t>::Pre pre[PRE ? NI : 1];
#pragma unroll
  for (int j = 0; j < (PRE ? NI : 0); ++j) {
    // (rows clamped below M: loads without branches; rows at or past M are
    // not stored)
    const int it = grp + NG * j < NU ? grp + NG * j : NU - 1;
    const int row = it / CB, pc = it - row * CB;
    int ba, bb;
    pair_blocks(g, nt * CB + pc, ba, bb);
    pre[j] = epi.pre(m0 + row < g.M ? m0 + row : g.M - 1, ba * 16 + c16, bb * 16 + c16);
  }
  // this wave's stream: chunks [c0, c0 + n); c0 < nchunk also when n = 0
  const int c0 = stream_begin(nchunk, wave), n = stream_begin(nchunk, wave + 1) - c0;
  const int clast = n > 0 ? c0 + n - 1 : c0;
  constexpr int AS = MS > 0 ? 1 : PF;  // activation register slots
  bf16x8_t ra[AS][RB][4], rw[PF][CB][4], rl[TWO ? AS : 1][RB][4];
  // staged activations: this lane's row (rows at or past M read row M - 1)
  // and half of the 16-wide step
  const int s_row = (lane & 31) < g.M ? (lane & 31) : g.M - 1, s_half = lane >> 5;
  f32x16_t acc[RB][CB];
#pragma unroll
  for (int r = 0; r < RB; ++r)
#pragma unroll
    for (int c = 0; c < CB; ++c)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[r][c][e] = 0.f;
  // chunk i of the stream into register slot `slot` (past the last chunk:
  // that chunk again, never computed)
  auto load = [&](int slot, int i) {
    const int cidx = c0 + i;
    const int64_t off = (int64_t)(cidx < clast ? cidx : clast) * 256 * 8;
    if (MS == 0) {
#pragma unroll
      for (int r = 0; r < RB; ++r)
#pragma unroll
        for (int st = 0; st < 4; ++st) ra[MS ? 0 : slot][r][st] = load8(ap[r] + off + st * 512);
      if (TWO) {
#pragma unroll
        for (int r = 0; r < RB; ++r)
#pragma unroll
          for (int st = 0; st < 4; ++st) rl[TWO && !MS ? slot : 0][r][st] = load8(ap[r] + g.a_lo + off + st * 512);
      }
    }
#pragma unroll
    for (int c = 0; c < CB; ++c)
#pragma unroll
      for (int st = 0; st < 4; ++st) rw[slot][c][st] = load8(wp[c] + off + st * 512);
  };
  // chunk i of the stream from register slot `slot` (and the staged activations)
  auto compute = [&](int slot, int i) {
    const int as = MS > 0 ? 0 : slot;
    if (MS > 0) {
      const int c = c0 + i;
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        ra[0][0][st] = s_a[(c * 4 + st) * 2 * MS + s_half * MS + s_row];
        if (TWO) rl[0][0][st] = s_a[((nchunk + c) * 4 + st) * 2 * MS + s_half * MS + s_row];
      }
    }
#pragma unroll
    for (int st = 0; st < 4; ++st)
#pragma unroll
      for (int r = 0; r < RB; ++r)
#pragma unroll
        for (int c = 0; c < CB; ++c) {
          acc[r][c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ra[as][r][st], rw[slot][c][st], acc[r][c], 0, 0, 0);
          if (TWO)
            acc[r][c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(rl[TWO ? as : 0][r][st], rw[slot][c][st], acc[r][c],
                                                               0, 0, 0);
        }
  };
#pragma unroll
  for (int p = 0; p < PF; ++p) load(p, p);
  if (MS > 0) {
    // the call's rows of every chunk, both terms (the first weight chunks are
    // already in flight); rows past M: row M - 1 (never used)
    const int npc = TERMS * nchunk * 8 * MS;
    for (int p = tid; p < npc; p += NT) {
      const int row = p % MS, rest = p / MS, half = rest & 1, tcs = rest >> 1, st = tcs & 3, tc = tcs >> 2;
      const int term = tc >= nchunk ? 1 : 0, c = tc - term * nchunk;
      const int rc = row < g.M ? row : g.M - 1;
      s_a[p] = load8((const uint16_t*)g.A + (term ? g.a_lo : 0) + ((int64_t)c * 256 + st * 64 + half * 32 + rc) * 8);
    }
    __syncthreads();
  }
  // steady state, branch-free: every refill is a chunk still to come
  int i = 0;
  for (; i + 2 * PF <= n; i += PF) {
#pragma unroll
    for (int u = 0; u < PF; ++u) {
      compute(u, i + u);
      load(u, i + u + PF);
    }
  }
  // the rest (fewer than 2 PF chunks); i stays a multiple of PF
  for (; i < n; i += PF) {
#pragma unroll
    for (int u = 0; u < PF; ++u)
      if (i + u < n) {
        compute(u, i + u);
        if (i + u + PF < n) load(u, i + u + PF);
      }
  }
  // stream sums to LDS; C layout of a 32x32 block: acc[4 gg + qq] of lane l
  // is row 8 gg + 4 (l / 32) + qq, column l % 32
#pragma unroll
  for (int r = 0; r < RB; ++r)
#pragma unroll
    for (int c = 0; c < CB; ++c)
#pragma unroll
      for (int e = 0; e < 16; ++e) red[wave * TILE + ((r * CB + c) * 16 + e) * 64 + lane] = acc[r][c][e];
  if (norm_here) rr.finish(g, m0, s_part, s_rstd);  // uniform branch: contains a barrier
  __syncthreads();
  // every 16-thread group runs the same trip count (the row sums of squares
  // reduce over its 16 lanes); unrolled where the prefetched values need
  // static indices
#pragma unroll
  for (int j = 0; j < NI; ++j) {
    const int it = grp + NG * j;
    if (it >= NU) break;  // uniform within the 16-thread group
    const int row = it / CB, pc = it - row * CB;
    const int m = m0 + row, pair = nt * CB + pc;
    const int r32 = row & 31;
    const int ia = (((row >> 5) * CB + pc) * 16 + 4 * (r32 >> 3) + (r32 & 3)) * 64 + ((r32 >> 2) & 1) * 32 + c16;
    const int ib = ia + 16;
    // the stream tree: neighbours, then pairs 2 apart, then 4 apart
    float va[NW], vb[NW];
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      va[w] = red[w * TILE + ia];
      vb[w] = red[w * TILE + ib];
    }
#pragma unroll
    for (int h = 1; h < NW; h <<= 1)
#pragma unroll
      for (int w = 0; w < NW; w += 2 * h) {
        va[w] += va[w + h];
        vb[w] += vb[w + h];
      }
    int ba, bb;
    pair_blocks(g, pair, ba, bb);
    float sq = 0.f;
    if (m < g.M) {
      const float rs = norm_here ? s_rstd[row] : 1.f;
      sq = PRE ? epi.apply(m, ba * 16 + c16, va[0], bb * 16 + c16, vb[0], rs, pre[PRE ? j : 0])
               : epi(m, ba * 16 + c16, va[0], bb * 16 + c16, vb[0], rs);
    }
    if (g.ssq_out) {
      sq = sum16(sq);
      if (c16 == 0 && m < g.M) g.ssq_out[(int64_t)pair * g.M_pad + m] = sq;
    }
  }
}

// Product for calls of more than 64 rows, both operands in fragment order:
// a workgroup owns 32 RBK rows (RBK = 4 or 2 row blocks) x 8 / RBK column
// pairs and a group of Q consecutive streams (8 / Q workgroups per tile split
// the K range). Each 64-wide chunk of both operands (RBK = 4: 128 x 64
// activations, one or two terms, and 64 x 64 weights, 40 KB with two terms;
// RBK = 2: 64 x 64 and 128 x 64, 32 KB) is staged once into LDS by all 512
// threads (16-byte pieces; one wave load reads 1 KB of consecutive bytes and
// writes it to consecutive LDS), so the weights are read once per tile's
// rows and the activations once per tile's columns. Wave w computes block
// (w / NCB, w % NCB) from LDS, running through its group's streams in order and folding
// each finished stream into a stack of subtrees (stream_fold), which gives
// the stream tree's order exactly. Three LDS buffers: while a chunk is
// multiplied, each wave reads the next chunk's fragments into registers and
// the workgroup writes the one after into the third buffer (from registers
// loaded two chunks ahead); one barrier per chunk.
// Q = 8 (one group): the epilogue runs here; otherwise each workgroup writes
// its group sum (rows below M) to g.partial[group] and k_pk_combine finishes.
// Rows past the last 32-row block below M load that block (discarded).
// grid: 8 * (mtiles * G) * ceil(ntiles / 8), G = 8 / Q; block 512.
template <int Q, bool TWO, int RBK>
__global__ __launch_bounds__(512) void k_gemm_bf16_lt(GemmArgs g, Epi<uint16_t> epi) {
  constexpr int NT = 512, R = 32 * RBK, NCB = 8 / RBK, G = 8 / Q, TERMS = TWO ? 2 : 1, NF = 4 * (TERMS + 1);
  static_assert(RBK == 4 || RBK == 2, "128 x 64 or 64 x 128 tiles");
  constexpr int A_PIECES = RBK * TERMS * 256, PIECES = A_PIECES + NCB * 256, PPT = PIECES / NT;
  static_assert(PIECES % NT == 0, "16-byte pieces per thread");
  constexpr int TILE = RBK * NCB * 16 * 64;  // floats of the workgroup's tile, C layout
  static_assert(TILE * 4 <= 3 * PIECES * 16, "the epilogue reuses the stage buffers");
  __shared__ u32x4_t stage[3][PIECES];
  __shared__ float s_rstd[R];
  __shared__ float s_part[rowrstd_lds<R, NT>()];
  const int mtiles = (g.M + R - 1) / R, ntiles = g.npairs / NCB;
  const int b = blockIdx.x, q = b >> 3, per = mtiles * G;
  const int sub = q % per, nt = 8 * (q / per) + (b & 7);
  if (nt >= ntiles) return;  // whole workgroup, before any barrier
  const int mt = sub / G, grp = sub - mt * G;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int m0 = mt * R, nchunk = g.K >> 6;
  const int lastblk = (g.M - 1) >> 5;
  // this thread's pieces: global element offsets at chunk 0 (a chunk adds 4 KB)
  const uint16_t* gp[PPT];
#pragma unroll
  for (int k = 0; k < PPT; ++k) {
    const int pc = tid + NT * k;
    if (pc < A_PIECES) {
      const int rbk = pc / (TERMS * 256), rem = pc - rbk * TERMS * 256, term = rem >> 8, sl = rem & 255;
      const int blk = mt * RBK + rbk < lastblk ? mt * RBK + rbk : lastblk;
      gp[k] = (const uint16_t*)g.A + (term ? g.a_lo : 0) + ((int64_t)blk * nchunk * 256 + sl) * 8;
    } else {
      const int pw = pc - A_PIECES, cbk = pw >> 8, sl = pw & 255;
      gp[k] = (const uint16_t*)g.Wp + ((int64_t)(nt * NCB + cbk) * nchunk * 256 + sl) * 8;
    }
  }
  const bool norm_here = (Q == 8) && g.ssq_in != nullptr;
  // the group's chunks [cb, ce)
  const int cb = stream_begin(nchunk, grp * Q), ce = stream_begin(nchunk, grp * Q + Q), n = ce - cb;
  const int clast = n > 0 ? ce - 1 : cb;
  u32x4_t rg[2][PPT];  // staging: global -> registers -> LDS
  u32x4_t fr[2][NF];   // one chunk's fragments of this wave, from LDS
  auto load = [&](int set, int i) __attribute__((always_inline)) {  // chunk cb + i (clamped) into set `set`
    const int c = cb + i < clast ? cb + i : clast;
#pragma unroll
    for (int k = 0; k < PPT; ++k) {
      const u32x4_t* src = (const u32x4_t*)(gp[k] + (int64_t)c * 2048);
      // weights are read once per call: streamed past the caches
      rg[set][k] = k * NT >= A_PIECES ? __builtin_nontemporal_load(src) : *src;
    }
  };
  auto put = [&](int set, int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int k = 0; k < PPT; ++k) stage[buf][tid + NT * k] = rg[set][k];
  };
  const int rw = wave / NCB, cw = wave % NCB;
  auto frag = [&](int f, int buf) __attribute__((always_inline)) {
    const u32x4_t* sa = &stage[buf][rw * TERMS * 256 + lane];
    const u32x4_t* sw = &stage[buf][A_PIECES + cw * 256 + lane];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      fr[f][s * (TERMS + 1)] = sa[s * 64];
      if (TWO) fr[f][s * (TERMS + 1) + 1] = sa[256 + s * 64];
      fr[f][s * (TERMS + 1) + TERMS] = sw[s * 64];
    }
  };
  f32x16_t r, st[fold_levels<Q>()];
#pragma unroll
  for (int e = 0; e < 16; ++e) r[e] = 0.f;
  auto mma = [&](int f) __attribute__((always_inline)) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const bf16x8_t w = __builtin_bit_cast(bf16x8_t, fr[f][s * (TERMS + 1) + TERMS]);
      r = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, fr[f][s * (TERMS + 1)]), w, r, 0, 0, 0);
      if (TWO)
        r = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, fr[f][s * (TERMS + 1) + 1]), w, r, 0, 0,
                                                    0);
    }
  };
  // streams of the group that end at or before chunk c are folded
  int j = 0, nb = stream_begin(nchunk, grp * Q + 1);
  auto fold_until = [&](int c) __attribute__((always_inline)) {
    while (j < Q && nb <= c) {
      stream_fold<Q>(j, r, st);
      ++j;
      nb = stream_begin(nchunk, grp * Q + j + 1);
    }
  };
  // Chunk i: LDS buffer i % 3, fragment set i % 2; register set i % 2 holds
  // chunk i + 2 until it is written to LDS (then chunk i + 4). While chunk i
  // is multiplied, the wave reads chunk i + 1's fragments and the workgroup
  // writes chunk i + 2 into the third buffer.
  // The row statistics are loaded first and staged in LDS before the loop
  // (their registers are needed by the loop; the epilogue then reads LDS only).
  if (norm_here) {  // uniform
    RowRstd<R, NT> rr(g, m0);
    load(0, 0);
    load(1, 1);
    rr.stage(s_part);
  } else {
    load(0, 0);
    load(1, 1);
  }
  put(0, 0);
  put(1, 1);
  load(0, 2);
  load(1, 3);
  __syncthreads();
  frag(0, 0);
  // Per chunk, in this order: the LDS writes of chunk i + 2 and the refill
  // loads, then the next chunk's fragment reads interleaved with chunk i's
  // MFMA chain. The barrier that ends a chunk waits only for this wave's
  // writes (LDS operations complete in order: all but the NF fragment reads
  // just issued), so those reads proceed across it; they target the buffer
  // of chunk i + 1, which no wave writes before the next barrier. A plain
  // barrier would wait for them and serialise the chain behind the reads.
  auto chunk = [&](int u, int i, bool refill) __attribute__((always_inline)) {  // chunk i, u = i % 6
    fold_until(cb + i);
    put(u & 1, (u + 2) % 3);
    if (refill) load(u & 1, i + 4);
    frag((u + 1) & 1, (u + 1) % 3);
    mma(u & 1);
    __builtin_amdgcn_sched_group_barrier(0x200, PPT, 0);  // LDS writes first
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);            // MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, TERMS + 1, 0);    // fragment reads
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);            // MFMA
      __builtin_amdgcn_sched_group_barrier(0x020, 2, 0);            // refill loads
    }
    static_assert(NF <= 15, "lgkmcnt field");
    asm volatile("s_waitcnt lgkmcnt(%0)\n\ts_barrier" ::"n"(NF) : "memory");
  };
  int i = 0;
  for (; i + 10 <= n; i += 6) {  // every refill is a chunk still to come
#pragma unroll
    for (int u = 0; u < 6; ++u) chunk(u, i + u, true);
  }
  for (; i < n; i += 6) {
#pragma unroll
    for (int u = 0; u < 6; ++u)
      if (i + u < n) chunk(u, i + u, i + u + 4 < n);
  }
  __syncthreads();      // every wave's fragment reads done before the stage buffers are reused
  fold_until(ce + 1);  // the group's remaining streams (empty ones included)
  if (Q < 8) {
    // group sum of block (rw, cw), rows below M, to the partial buffer
    int ba, bbk;
    pair_blocks(g, nt * NCB + cw, ba, bbk);
    const int col = (lane & 16) ? bbk * 16 + (lane & 15) : ba * 16 + (lane & 15);
    float* P = g.partial + (int64_t)grp * g.M_pad * g.Nv + col;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int m = m0 + rw * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
      if (m < g.M) P[(int64_t)m * g.Nv] = r[e];
    }
    return;
  }
  // block sums to LDS in C layout (in the stage buffers: their last reads and
  // writes were before the loop's final barrier)
  float* red = (float*)&stage[0][0];
#pragma unroll
  for (int e = 0; e < 16; ++e) red[((rw * NCB + cw) * 16 + e) * 64 + lane] = r[e];
  if (norm_here) {  // uniform branch: contains barriers
    RowRstd<R, NT>::reduce(g, m0, s_part, s_rstd);
  }
  __syncthreads();
  constexpr int NU = R * NCB, NG = NT / 16, NI = NU / NG;
  const int c16 = tid & 15, grp16 = tid >> 4;
  for (int jj = 0; jj < NI; ++jj) {
    const int it = grp16 + NG * jj;
    const int row = it / NCB, pc = it - row * NCB;
    const int m = m0 + row, pair = nt * NCB + pc;
    const int r32 = row & 31;
    const int ia = (((row >> 5) * NCB + pc) * 16 + 4 * (r32 >> 3) + (r32 & 3)) * 64 + ((r32 >> 2) & 1) * 32 + c16;
    int ba, bbk;
    pair_blocks(g, pair, ba, bbk);
    float sq = 0.f;
    if (m < g.M) sq = epi(m, ba * 16 + c16, red[ia], bbk * 16 + c16, red[ia + 16], norm_here ? s_rstd[row] : 1.f);
    if (g.ssq_out) {
      sq = sum16(sq);
      if (c16 == 0 && m < g.M) g.ssq_out[(int64_t)pair * g.M_pad + m] = sq;
    }
  }
}

// The staged tile of 64 rows x 4 column pairs (RBK = 2 of k_gemm_bf16_lt)
// with each chunk copied from memory straight into LDS (global_load_lds,
// 16 bytes per lane: a wave's copy writes 1 KB of consecutive LDS, the layout
// k_gemm_bf16_lt writes from registers) and four LDS buffers: chunk i + 3 is
// requested while chunk i is multiplied and chunk i + 1's fragments are read,
// so a chunk's copy has two chunk times to land, and no register set or LDS
// write instruction stages it. The chunk's closing barrier waits for this
// wave's copy of chunk i + 2 (chunk i + 3's may stay in flight) and, as in
// k_gemm_bf16_lt, leaves the NF fragment reads of chunk i + 1 outstanding:
// they target buffer (i + 1) % 4, which the next copy into it (chunk i + 5,
// requested in chunk i + 2, after two more barriers) cannot overtake.
// Buffer (i + 3) % 4 = (i - 1) % 4 is free when chunk i starts: its last
// reads (chunk i - 1's fragments, issued in chunk i - 2) completed before
// the barrier that closed chunk i - 1. The buffers are four LDS arrays
// indexed at compile time (the chunk loop is unrolled by four), so that the
// compiler can tell a copy in flight from the fragment reads of another
// buffer and does not wait for the copy before them. Same fragments, MFMAs
// and stream folds in the same order as k_gemm_bf16_lt: the same bits.
// grid and block as k_gemm_bf16_lt with RBK = 2.
constexpr int CPOL_NT = 2;  // cache-policy operand of global_load_lds: non-temporal
template <int Q, bool TWO>
__global__ __launch_bounds__(512) void k_gemm_bf16_ltd(GemmArgs g, Epi<uint16_t> epi) {
  constexpr int RBK = 2, NT = 512, R = 32 * RBK, NCB = 8 / RBK, G = 8 / Q, TERMS = TWO ? 2 : 1;
  constexpr int NF = 4 * (TERMS + 1), NB = 4;
  constexpr int A_PIECES = RBK * TERMS * 256, PIECES = A_PIECES + NCB * 256, PPT = PIECES / NT;
  static_assert(PIECES % NT == 0, "16-byte pieces per thread");
  constexpr int TILE = RBK * NCB * 16 * 64;
  constexpr bool RED_IN_STAGE = TILE * 4 <= PIECES * 16;  // the epilogue's block sums fit buffer 0
  __shared__ u32x4_t st0[PIECES], st1[PIECES], st2[PIECES], st3[PIECES];
  __shared__ float red_own[RED_IN_STAGE ? 1 : TILE];
  __shared__ float s_rstd[R];
  __shared__ float s_part[rowrstd_lds<R, NT>()];
  const int mtiles = (g.M + R - 1) / R, ntiles = g.npairs / NCB;
  const int b = blockIdx.x, q = b >> 3, per = mtiles * G;
  const int sub = q % per, nt = 8 * (q / per) + (b & 7);
  if (nt >= ntiles) return;  // whole workgroup, before any barrier
  const int mt = sub / G, grp = sub - mt * G;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  const int m0 = mt * R, nchunk = g.K >> 6;
  const int lastblk = (g.M - 1) >> 5;
  // this thread's pieces (piece tid + NT k of a stage buffer): global element
  // offsets at chunk 0 (a chunk adds 4 KB)
  const uint16_t* gp[PPT];
#pragma unroll
  for (int k = 0; k < PPT; ++k) {
    const int pc = tid + NT * k;
    if (pc < A_PIECES) {
      const int rbk = pc / (TERMS * 256), rem = pc - rbk * TERMS * 256, term = rem >> 8, sl = rem & 255;
      const int blk = mt * RBK + rbk < lastblk ? mt * RBK + rbk : lastblk;
      gp[k] = (const uint16_t*)g.A + (term ? g.a_lo : 0) + ((int64_t)blk * nchunk * 256 + sl) * 8;
    } else {
      const int pw = pc - A_PIECES, cbk = pw >> 8, sl = pw & 255;
      gp[k] = (const uint16_t*)g.Wp + ((int64_t)(nt * NCB + cbk) * nchunk * 256 + sl) * 8;
    }
  }
  const bool norm_here = (Q == 8) && g.ssq_in != nullptr;
  const int cb = stream_begin(nchunk, grp * Q), ce = stream_begin(nchunk, grp * Q + Q), n = ce - cb;
  const int clast = n > 0 ? ce - 1 : cb;
  auto sbuf = [&](int buf) __attribute__((always_inline)) -> u32x4_t* {
    return buf == 0 ? st0 : buf == 1 ? st1 : buf == 2 ? st2 : st3;
  };
  static_assert(NB == 4, "four buffers");
  // chunk cb + i (clamped) into LDS buffer `buf`; the weights (read once
  // per call) streamed past the caches
  auto copy = [&](int buf, int i) __attribute__((always_inline)) {
    const int c = cb + i < clast ? cb + i : clast;
    u32x4_t* dst = sbuf(buf);
#pragma unroll
    for (int k = 0; k < PPT; ++k) {
      if (k * NT >= A_PIECES)
        __builtin_amdgcn_global_load_lds((const void*)(gp[k] + (int64_t)c * 2048),
                                         (__attribute__((address_space(3))) void*)(dst + NT * k + wv * 64), 16, 0,
                                         CPOL_NT);
      else
        __builtin_amdgcn_global_load_lds((const void*)(gp[k] + (int64_t)c * 2048),
                                         (__attribute__((address_space(3))) void*)(dst + NT * k + wv * 64), 16, 0, 0);
    }
  };
  u32x4_t fr[2][NF];  // one chunk's fragments of this wave, from LDS
  const int rw = wave / NCB, cw = wave % NCB;
  auto frag = [&](int f, int buf) __attribute__((always_inline)) {
    const u32x4_t* sa = sbuf(buf) + rw * TERMS * 256 + lane;
    const u32x4_t* sw = sbuf(buf) + A_PIECES + cw * 256 + lane;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      fr[f][s * (TERMS + 1)] = sa[s * 64];
      if (TWO) fr[f][s * (TERMS + 1) + 1] = sa[256 + s * 64];
      fr[f][s * (TERMS + 1) + TERMS] = sw[s * 64];
    }
  };
  f32x16_t r, st[fold_levels<Q>()];
#pragma unroll
  for (int e = 0; e < 16; ++e) r[e] = 0.f;
  auto mma = [&](int f) __attribute__((always_inline)) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const bf16x8_t w = __builtin_bit_cast(bf16x8_t, fr[f][s * (TERMS + 1) + TERMS]);
      r = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, fr[f][s * (TERMS + 1)]), w, r, 0, 0, 0);
      if (TWO)
        r = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, fr[f][s * (TERMS + 1) + 1]), w, r, 0, 0,
                                                    0);
    }
  };
  int j = 0, nb = stream_begin(nchunk, grp * Q + 1);
  auto fold_until = [&](int c) __attribute__((always_inline)) {
    while (j < Q && nb <= c) {
      stream_fold<Q>(j, r, st);
      ++j;
      nb = stream_begin(nchunk, grp * Q + j + 1);
    }
  };
  // the row statistics' loads go first and stay in registers through the
  // loop (it stages nothing in registers); then chunks 0, 1, 2 are requested
  GemmArgs gs = g;
  if (!norm_here) gs.ssq_in = nullptr;
  RowRstd<R, NT> rr(gs, m0);
  copy(0, 0);
  copy(1, 1);
  copy(2, 2);
  // s_waitcnt immediates (gfx9 encoding) that wait for vmcnt only: the
  // compiler sees them, so it knows which copies have landed and inserts no
  // wait of its own before the fragment reads
  constexpr int VM_PPT = 0xF70 | (PPT & 15) | ((PPT >> 4) << 14), VM_0 = 0xF70;
  // chunks 0 and 1 in LDS for every wave (chunk 0 is multiplied and chunk
  // 1's fragments are read in the first chunk; chunk 2 may be in flight)
  __builtin_amdgcn_s_waitcnt(VM_PPT);
  __builtin_amdgcn_s_barrier();
  frag(0, 0);
  // chunk i, u = i % 4 (a compile-time constant); more: chunk i + 3 exists
  auto chunk = [&](int u, int i, bool more) __attribute__((always_inline)) {
    fold_until(cb + i);
    if (more) copy((u + 3) & 3, i + 3);
    frag((u + 1) & 1, (u + 1) & 3);
    mma(u & 1);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);          // MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, TERMS + 1, 0);  // fragment reads
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);          // MFMA
    }
    static_assert(NF <= 15, "lgkmcnt field");
    if (more)
      __builtin_amdgcn_s_waitcnt(VM_PPT);
    else
      __builtin_amdgcn_s_waitcnt(VM_0);
    asm volatile("s_waitcnt lgkmcnt(%0)\n\ts_barrier" ::"n"(NF) : "memory");
  };
  int i = 0;
  for (; i + 7 <= n; i += 4) {  // every chunk of these four requests chunk i + u + 3
#pragma unroll
    for (int u = 0; u < 4; ++u) chunk(u, i + u, true);
  }
  for (; i < n; i += 4) {
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (i + u < n) chunk(u, i + u, i + u + 3 < n);
  }
  // every copy landed (a group of fewer than three chunks leaves prologue
  // copies in flight) and every wave's fragment reads done before the stage
  // buffers are reused or the workgroup ends
  __builtin_amdgcn_s_waitcnt(VM_0);
  __syncthreads();
  fold_until(ce + 1);  // the group's remaining streams (empty ones included)
  if (Q < 8) {
    // group sum of block (rw, cw), rows below M, to the partial buffer
    int ba, bbk;
    pair_blocks(g, nt * NCB + cw, ba, bbk);
    const int col = (lane & 16) ? bbk * 16 + (lane & 15) : ba * 16 + (lane & 15);
    float* P = g.partial + (int64_t)grp * g.M_pad * g.Nv + col;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int m = m0 + rw * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
      if (m < g.M) P[(int64_t)m * g.Nv] = r[e];
    }
    return;
  }
  float* red = RED_IN_STAGE ? (float*)st0 : red_own;
#pragma unroll
  for (int e = 0; e < 16; ++e) red[((rw * NCB + cw) * 16 + e) * 64 + lane] = r[e];
  if (norm_here) {  // uniform branch: contains barriers
    rr.finish(g, m0, s_part, s_rstd);
  }
  __syncthreads();
  constexpr int NU = R * NCB, NG = NT / 16, NI = NU / NG;
  const int c16 = tid & 15, grp16 = tid >> 4;
  for (int jj = 0; jj < NI; ++jj) {
    const int it = grp16 + NG * jj;
    const int row = it / NCB, pc = it - row * NCB;
    const int m = m0 + row, pair = nt * NCB + pc;
    const int r32 = row & 31;
    const int ia = (((row >> 5) * NCB + pc) * 16 + 4 * (r32 >> 3) + (r32 & 3)) * 64 + ((r32 >> 2) & 1) * 32 + c16;
    int ba, bbk;
    pair_blocks(g, pair, ba, bbk);
    float sq = 0.f;
    if (m < g.M) sq = epi(m, ba * 16 + c16, red[ia], bbk * 16 + c16, red[ia + 16], norm_here ? s_rstd[row] : 1.f);
    if (g.ssq_out) {
      sq = sum16(sq);
      if (c16 == 0 && m < g.M) g.ssq_out[(int64_t)pair * g.M_pad + m] = sq;
    }
  }
}

// Combine the G group sums of k_gemm_bf16_lt by the stream tree's top levels
// (neighbours, then pairs 2 apart, then 4 apart) and apply the epilogue.
// grid: (pairs, 16-row tiles); block 256 (16 rows x 16 columns of a pair).
template <int G>
__global__ __launch_bounds__(256) void k_pk_combine(GemmArgs g, Epi<uint16_t> epi) {
  __shared__ float lds[SPLITK_LDS_FLOATS];
  float* s_rstd = lds;
  float* s_part = lds + 16;
  const int pair = blockIdx.x, mt = blockIdx.y;
  int ba, bb;
  pair_blocks(g, pair, ba, bb);
  const int m = mt * 16 + (threadIdx.x >> 4), r = threadIdx.x & 15;
  // the group sums and the epilogue's own inputs are loaded first, so that
  // their round trips overlap the row statistics' (rows at or past M load
  // row M - 1, never used)
  const int mc = m < g.M ? m : g.M - 1;
  float va[G], vb[G];
#pragma unroll
  for (int k = 0; k < G; ++k) {
    const float* P = g.partial + ((int64_t)k * g.M_pad + mc) * g.Nv;
    va[k] = P[ba * 16 + r];
    vb[k] = P[bb * 16 + r];
  }
  const typename Epi<uint16_t>::Pre pv = epi.pre(mc, ba * 16 + r, bb * 16 + r);
  if (g.ssq_in) {
    RowRstd<16> rr(g, mt * 16);
    rr.finish(g, mt * 16, s_part, s_rstd);
  }
  __syncthreads();
  float sq = 0.f;
  if (m < g.M) {
#pragma unroll
    for (int h = 1; h < G; h <<= 1)
#pragma unroll
      for (int k = 0; k < G; k += 2 * h) {
        va[k] += va[k + h];
        vb[k] += vb[k + h];
      }
    sq = epi.apply(m, ba * 16 + r, va[0], bb * 16 + r, vb[0], g.ssq_in ? s_rstd[threadIdx.x >> 4] : 1.f, pv);
  }
  if (g.ssq_out) {
    sq = sum16(sq);
    if (r == 0 && m < g.M) g.ssq_out[(int64_t)pair * g.M_pad + m] = sq;
  }
}

// rotary table: one thread per (t, i)
__global__ __launch_bounds__(256) void k_rope_table(const double* inv_freq, int half, int tmax, float2* tab) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)(tmax + 1) * half) return;
  const int t = (int)(i / half), f = (int)(i % half);
  double sn, cs;
  sincos((double)t * inv_freq[f], &sn, &cs);
  tab[i] = make_float2((float)cs, (float)sn);
}

void launch_rope_table(const double* inv_freq, int dh, int tmax, float2* tab, hipStream_t s) {
  const int64_t n = (int64_t)(tmax + 1) * (dh / 2);
  hipLaunchKernelGGL(k_rope_table, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, inv_freq, dh / 2, tmax, tab);
}

// Weights in fragment order: one thread per 16-byte fragment (pair p = block
// p of the packed rows: its virtual columns 0-15 are block ba, 16-31 block bb).
__global__ __launch_bounds__(256) void k_pack_weights(GemmArgs g, uint16_t* dst) {
  const int nchunk = g.K >> 6;
  const int64_t total = (int64_t)g.npairs * nchunk * 256;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= total) return;
  const int l = (int)(i & 63), st = (int)((i >> 6) & 3);
  const int64_t pc = i >> 8;
  const int c = (int)(pc % nchunk), p = (int)(pc / nchunk);
  int ba, bb;
  pair_blocks(g, p, ba, bb);
  const int v = l & 31;
  const int k = 64 * c + 32 * (l >> 5) + 8 * st;
  const uint16_t* src = weight_row<uint16_t>(g, ((v & 16) ? bb : ba) * 16 + (v & 15)) + k;
  *(uint4*)(dst + i * 8) = *(const uint4*)src;
}

void launch_pack_weights(const GemmArgs& g, void* Wp, hipStream_t s) {
  const int64_t total = (int64_t)g.npairs * (g.K >> 6) * 256;
  hipLaunchKernelGGL(k_pack_weights, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, g, (uint16_t*)Wp);
}

// grid: x = pair, y = ceil(M/16); block 256
template <typename T>
__global__ __launch_bounds__(256) void k_splitk_epi(GemmArgs g, Epi<T> epi) {
  __shared__ float lds[SPLITK_LDS_FLOATS];
  splitk_epi_body<T>(g, epi, blockIdx.x, blockIdx.y, lds);
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
  if (g.Wp) {
    Phase bad{};
    bad.kind = PH_INVALID;  // not runnable by the persistent kernel: the recording is dropped
    if (record_phase(bad)) return;
    Epi<uint16_t> epi{e};
    const bool two = g.a_lo != 0;
    if (g.lt_groups > 0) {
      // staged tile: 32 rbk rows x 8 / rbk column pairs per workgroup, G
      // workgroups per tile over the stream groups
      const int rbk = g.lt_rbk == 2 ? 2 : 4;
      const int G = g.lt_groups, mtiles = (g.M + 32 * rbk - 1) / (32 * rbk), ntiles = g.npairs / (8 / rbk);
      dim3 grid(8 * mtiles * G * ((ntiles + 7) / 8));
#define RLT_LT2(Q_, RBK_)                                                                              \
  do {                                                                                                 \
    if (two) hipLaunchKernelGGL((k_gemm_bf16_lt<Q_, true, RBK_>), grid, dim3(512), 0, s, g, epi);     \
    else hipLaunchKernelGGL((k_gemm_bf16_lt<Q_, false, RBK_>), grid, dim3(512), 0, s, g, epi);        \
  } while (0)
#define RLT_LTD(Q_)                                                                                   \
  do {                                                                                                \
    if (two) hipLaunchKernelGGL((k_gemm_bf16_ltd<Q_, true>), grid, dim3(512), 0, s, g, epi);         \
    else hipLaunchKernelGGL((k_gemm_bf16_ltd<Q_, false>), grid, dim3(512), 0, s, g, epi);            \
  } while (0)
#define RLT_LT(Q_)                       \
  do {                                   \
    if (rbk == 2 && g.lt_dma) RLT_LTD(Q_); \
    else if (rbk == 2) RLT_LT2(Q_, 2);    \
    else RLT_LT2(Q_, 4);                  \
  } while (0)
      switch (G) {
        case 1: RLT_LT(8); break;
        case 2: RLT_LT(4); break;
        case 4: RLT_LT(2); break;
        default: RLT_LT(1); break;
      }
#undef RLT_LT
#undef RLT_LTD
#undef RLT_LT2
      if (G > 1) {
        dim3 g2(g.npairs, (g.M + 15) / 16);
        switch (G) {
          case 2: hipLaunchKernelGGL(k_pk_combine<2>, g2, dim3(256), 0, s, g, epi); break;
          case 4: hipLaunchKernelGGL(k_pk_combine<4>, g2, dim3(256), 0, s, g, epi); break;
          default: hipLaunchKernelGGL(k_pk_combine<8>, g2, dim3(256), 0, s, g, epi); break;
        }
      }
      return;
    }
    const int mtiles = (g.M + 32 * g.rb - 1) / (32 * g.rb), ntiles = g.npairs / g.cb;
    dim3 grid(8 * mtiles * ((ntiles + 7) / 8));
    // the Q/K/V product's epilogue computes its rotary angles (prefetching a
    // table lookup measured slower)
    const bool pre = g.pre >= 0 ? g.pre != 0 : (e.kind == EPI_RESID || e.kind == EPI_QROT);
#define RLT_PK3(RB_, CB_, PF_, PRE_, MS_)                                                                   \
  do {                                                                                                      \
    if (two) hipLaunchKernelGGL((k_gemm_bf16_pk<RB_, CB_, PF_, PRE_, true, MS_>), grid, dim3(512), 0, s, g, epi); \
    else hipLaunchKernelGGL((k_gemm_bf16_pk<RB_, CB_, PF_, PRE_, false, MS_>), grid, dim3(512), 0, s, g, epi);    \
  } while (0)
#define RLT_PK2(RB_, CB_, PF_, PRE_) RLT_PK3(RB_, CB_, PF_, PRE_, 0)
    if (g.a_lds == 1 && g.M == 1 && (g.K >> 6) <= PK_LDS_CHUNKS) {  // one row: activations in LDS
      if (g.pf == 4) {
        if (pre) RLT_PK3(1, 1, 4, true, 1);
        else RLT_PK3(1, 1, 4, false, 1);
      } else if (g.pf == 3) {
        if (pre) RLT_PK3(1, 1, 3, true, 1);
        else RLT_PK3(1, 1, 3, false, 1);
      } else {
        if (pre) RLT_PK3(1, 1, 2, true, 1);
        else RLT_PK3(1, 1, 2, false, 1);
      }
      return;
    }
#define RLT_PK(RB_, CB_, PF_)              \
  do {                                     \
    if (pre) RLT_PK2(RB_, CB_, PF_, true); \
    else RLT_PK2(RB_, CB_, PF_, false);    \
  } while (0)
#define RLT_SHAPE(RB_, CB_, PF_) \
  if (g.rb == RB_ && g.cb == CB_ && g.pf == PF_) RLT_PK(RB_, CB_, PF_); else
    // shapes the host may pick (none changes the arithmetic, see the kernel)
    RLT_SHAPE(1, 1, 2) RLT_SHAPE(1, 1, 3) RLT_SHAPE(1, 1, 4) RLT_SHAPE(2, 1, 1) RLT_SHAPE(2, 1, 2)
    RLT_SHAPE(1, 2, 1) RLT_SHAPE(1, 2, 2) {
      RLT_PK(1, 1, 2);
    }
#undef RLT_SHAPE
#undef RLT_PK
#undef RLT_PK2
#undef RLT_PK3
    return;
  }
  const int MB = g.mb;
  const int mt = (g.M + 16 * MB - 1) / (16 * MB);
  if (g.wide || MB > 2) {
    Phase bad{};
    bad.kind = PH_INVALID;  // not runnable by the persistent kernel: the recording is dropped
    if (record_phase(bad)) return;
  } else {
    Phase p{};
    p.kind = PH_GEMM;
    p.gx = g.npairs;
    p.gy = g.S;
    p.gz = mt;
    p.u.gm.g = g;
    p.u.gm.e = e;
    if (record_phase(p)) {
      if (g.S > 1) {
        p.kind = PH_SPLITK;
        p.gy = (g.M + 15) / 16;
        p.gz = 1;
        record_phase(p);
      }
      return;
    }
  }
  Epi<uint16_t> epi{e};
  if (g.wide == 256) {  // host checked: M >= 256, K % 64 == 0, no split, K/V epilogue with 16-byte runs
    dim3 grid(g.npairs / 8 * ((g.M + 255) / 256));
    hipLaunchKernelGGL(k_gemm_bf16_big, grid, dim3(512), 0, s, g, epi);
    return;
  }
  if (g.wide) {
    const int tiles_m = (g.M + 127) / 128;
    dim3 grid(g.npairs / (g.wide / 32) * g.S * tiles_m);
    if (g.wide == 128)
      hipLaunchKernelGGL(k_gemm_bf16_tile<128>, grid, dim3(256), 0, s, g, epi);
    else
      hipLaunchKernelGGL(k_gemm_bf16_tile<64>, grid, dim3(256), 0, s, g, epi);
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
