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
  __shared__ float s_part[256];
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

// Product with both operands in fragment order (see pk_off): a workgroup owns
// 32 RB rows x CB column pairs over the whole K, so
// there is no K split and no partial traffic; its NW waves take the 64-wide
// K chunks round-robin (wave w: chunks w, w + NW, ...) and load each chunk's
// fragments straight into registers, every load instruction reading 1 KB of
// consecutive bytes, PF chunks ahead. No LDS staging and no barrier inside the
// K loop. Lanes of rows at or past M load no activations (zeros), so a call
// of a few rows reads little more than the weights. The NW wave partials
// are summed in LDS in wave order by the
// epilogue threads (16 consecutive threads per row and column pair, as in the
// other tiles). Tile order: workgroup b runs on XCD b % 8 and takes column
// tile 8 (q / mtiles) + b % 8 and row tile q % mtiles (q = b / 8), so the row
// tiles of one column tile share its weights in one L2.
// PRE: the epilogue reads memory (residual, gains, rotary table) and loads it
// before the K loop (registers that would otherwise halve the occupancy of
// the larger tiles).
// NW = 8 (with 4 chunks in flight per wave) serves the smallest tile when it
// needs at most one workgroup per compute unit: a compute unit holds only so
// many loads in flight, and with few column tiles (64 workgroups for a
// 2048-wide product at one row) the weights stream faster with twice the
// waves per workgroup.
// grid: 8 * mtiles * ceil(ntiles / 8); block 64 NW.
template <int RB, int CB, bool PRE, int NW>
__global__ __launch_bounds__(64 * NW) void k_gemm_bf16_pk(GemmArgs g, Epi<uint16_t> epi) {
  constexpr int R = 32 * RB, PF = NW == 8 && RB * CB == 1 ? 4 : 2, NT = 64 * NW;
  constexpr int TILE = RB * CB * 16 * 64;  // floats of one wave's partial tile
  static_assert((R * CB * 16) % NT == 0, "epilogue items per thread");
  __shared__ float red[NW * TILE];
  __shared__ float s_rstd[R];
  __shared__ float s_part[NT];  // RowRstd uses the first 256; the rest keeps stray writes in bounds
  const int mtiles = (g.M + R - 1) / R, ntiles = g.npairs / CB;
  const int b = blockIdx.x, q = b >> 3;
  const int mt = q % mtiles, nt = 8 * (q / mtiles) + (b & 7);
  if (nt >= ntiles) return;  // whole workgroup, before any barrier
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int m0 = mt * R;
  const int nchunk = g.K >> 6;
  const uint16_t* ap[RB];
  const uint16_t* wp[CB];
#pragma unroll
  for (int r = 0; r < RB; ++r) ap[r] = (const uint16_t*)g.A + ((int64_t)(mt * RB + r) * nchunk * 256 + lane) * 8;
#pragma unroll
  for (int c = 0; c < CB; ++c) wp[c] = (const uint16_t*)g.Wp + ((int64_t)(nt * CB + c) * nchunk * 256 + lane) * 8;
  const bool norm_here = g.ssq_in != nullptr;
  RowRstd<R> rr(g, norm_here ? m0 : 0);
  // this thread's epilogue items (16 consecutive threads per row and pair)
  // and the values their epilogue reads, loaded now, in flight with the K loop
  constexpr int NI = R * CB * 16 / NT;
  const int c16 = tid & 15;
  typename Epi<uint16_t>::Pre pre[PRE ? NI : 1];
#pragma unroll
  for (int j = 0; j < (PRE ? NI : 0); ++j) {
    const int it = (tid >> 4) + (NT / 16) * j;
    const int row = it / CB, pc = it - row * CB;
    int ba, bb;
    pair_blocks(g, nt * CB + pc, ba, bb);
    pre[j] = m0 + row < g.M ? epi.pre(m0 + row, ba * 16 + c16, bb * 16 + c16) : typename Epi<uint16_t>::Pre{};
  }
  const int n = (nchunk - wave + NW - 1) / NW;  // chunks of this wave
  bf16x8_t ra[PF][RB][4], rw[PF][CB][4];
  f32x16_t acc[RB][CB];
#pragma unroll
  for (int r = 0; r < RB; ++r)
#pragma unroll
    for (int c = 0; c < CB; ++c)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[r][c][e] = 0.f;
  bool live[RB];  // this lane's activation row exists
#pragma unroll
  for (int r = 0; r < RB; ++r) live[r] = m0 + 32 * r + (lane & 31) < g.M;
  auto load = [&](int slot, int i) {
    const int64_t off = (int64_t)(wave + NW * i) * 256 * 8;
#pragma unroll
    for (int r = 0; r < RB; ++r)
#pragma unroll
      for (int st = 0; st < 4; ++st) ra[slot][r][st] = live[r] ? load8(ap[r] + off + st * 512) : bf16x8_t{};
#pragma unroll
    for (int c = 0; c < CB; ++c)
#pragma unroll
      for (int st = 0; st < 4; ++st) rw[slot][c][st] = load8(wp[c] + off + st * 512);
  };
  auto compute = [&](int slot) {
#pragma unroll
    for (int st = 0; st < 4; ++st)
#pragma unroll
      for (int r = 0; r < RB; ++r)
#pragma unroll
        for (int c = 0; c < CB; ++c)
          acc[r][c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ra[slot][r][st], rw[slot][c][st], acc[r][c], 0, 0, 0);
  };
#pragma unroll
  for (int p = 0; p < PF; ++p)
    if (p < n) load(p, p);
  int i = 0;
  for (; i + PF <= n; i += PF) {
#pragma unroll
    for (int p = 0; p < PF; ++p) {
      compute(p);
      if (i + p + PF < n) load(p, i + p + PF);
    }
  }
#pragma unroll
  for (int p = 0; p < PF; ++p)
    if (i + p < n) compute(p);
  // wave partials to LDS; C layout of a 32x32 block: acc[4 gg + qq] of lane l
  // is row 8 gg + 4 (l / 32) + qq, column l % 32
#pragma unroll
  for (int r = 0; r < RB; ++r)
#pragma unroll
    for (int c = 0; c < CB; ++c)
#pragma unroll
      for (int e = 0; e < 16; ++e) red[wave * TILE + ((r * CB + c) * 16 + e) * 64 + lane] = acc[r][c][e];
  if (norm_here) rr.finish(g, m0, s_part, s_rstd);  // uniform branch: contains a barrier
  __syncthreads();
  // same trip count on every thread; unrolled only where the prefetched
  // values need static indices (the unrolled Q/K/V epilogue measured slower)
  constexpr int EU = PRE ? NI : 1;
#pragma unroll EU
  for (int j = 0; j < NI; ++j) {
    const int it = (tid >> 4) + (NT / 16) * j;
    const int row = it / CB, pc = it - row * CB;
    const int m = m0 + row, pair = nt * CB + pc;
    const int r32 = row & 31;
    const int ia = (((row >> 5) * CB + pc) * 16 + 4 * (r32 >> 3) + (r32 & 3)) * 64 + ((r32 >> 2) & 1) * 32 + c16;
    const int ib = ia + 16;
    float va = red[ia], vb = red[ib];
#pragma unroll
    for (int w = 1; w < NW; ++w) {
      va += red[w * TILE + ia];
      vb += red[w * TILE + ib];
    }
    int ba, bb;
    pair_blocks(g, pair, ba, bb);
    float sq = 0.f;
    if (m < g.M) {
      const float rs = norm_here ? s_rstd[row] : 1.f;
      sq = PRE ? epi.apply(m, ba * 16 + c16, va, bb * 16 + c16, vb, rs, pre[PRE ? j : 0])
               : epi(m, ba * 16 + c16, va, bb * 16 + c16, vb, rs);
    }
    if (g.ssq_out) {
      sq = sum16(sq);
      if (c16 == 0 && m < g.M) g.ssq_out[(int64_t)pair * g.M_pad + m] = sq;
    }
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
    const int mtiles = (g.M + 32 * g.rb - 1) / (32 * g.rb), ntiles = g.npairs / g.cb;
    dim3 grid(8 * mtiles * ((ntiles + 7) / 8));
    // (the Q/K/V product's 64 x 2 tile measured slower with it, 26.4 vs 19.9
    // us at 128 rows, and slower again with table lookups in its epilogue)
    const bool pre = e.kind == EPI_RESID || e.kind == EPI_QROT;
#define RLT_PK(RB_, CB_, NW_)                                                                          \
  do {                                                                                                 \
    if (pre) hipLaunchKernelGGL((k_gemm_bf16_pk<RB_, CB_, true, NW_>), grid, dim3(64 * NW_), 0, s, g, epi); \
    else hipLaunchKernelGGL((k_gemm_bf16_pk<RB_, CB_, false, NW_>), grid, dim3(64 * NW_), 0, s, g, epi);    \
  } while (0)
    // eight waves where the call needs at most one workgroup per compute
    // unit (8 waves at 344 workgroups of 32 x 1: 15.6 vs 13.0 us)
    const bool w8 = grid.x <= 256;
    if (g.rb == 2 && g.cb == 2) {
      // eight waves load the epilogue's values after the K loop (prefetched
      // they would spill)
      if (w8) hipLaunchKernelGGL((k_gemm_bf16_pk<2, 2, false, 8>), grid, dim3(512), 0, s, g, epi);
      else RLT_PK(2, 2, 4);
    } else if (g.rb == 2) {
      if (w8) RLT_PK(2, 1, 8);
      else RLT_PK(2, 1, 4);
    } else {
      if (w8) RLT_PK(1, 1, 8);
      else RLT_PK(1, 1, 4);
    }
#undef RLT_PK
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
