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
//   across S workgroups writes partial tiles; the last workgroup of a tile
//   to finish (an arrival counter per tile) sums them in split order and
//   runs the epilogue (the persistent step uses a phase of its own for this).
//   Both orders are fixed, so results are deterministic.
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
  __shared__ int s_flag;
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
  const bool norm_here = (g.S == 1 || g.tile_cnt != nullptr) && g.ssq_in != nullptr;
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

  if (g.S > 1) {
    // C layout: lane holds rows 4*(lane/16)+i of each 16-row block, column lane%16
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int m = m0 + mb * 16 + (lane >> 4) * 4 + q;
        if (m < g.M) {
          float* Pp = g.partial + ((int64_t)split * g.M_pad + m) * g.Nv;
          Pp[ba * 16 + r16] = acc[mb][0][q];
          Pp[bb * 16 + r16] = acc[mb][1][q];
        }
      }
    // K split reduced here: the tile's last workgroup sums the partials in
    // split order into its accumulators (its own partial included)
    if (!g.tile_cnt || !last_arrival(g.tile_cnt + grp * nmt + mt, g.S, &s_flag)) return;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int m = m0 + mb * 16 + (lane >> 4) * 4 + q;
        float va = 0.f, vb = 0.f;
        if (m < g.M)
          for (int sp = 0; sp < g.S; ++sp) {
            const float* Pp = g.partial + ((int64_t)sp * g.M_pad + m) * g.Nv;
            va += Pp[ba * 16 + r16];
            vb += Pp[bb * 16 + r16];
          }
        acc[mb][0][q] = va;
        acc[mb][1][q] = vb;
      }
  }
  if (norm_here) {  // uniform branch
    rr.finish(g, m0, s_part, s_rstd);
    __syncthreads();
  }
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int mr = mb * 16 + (lane >> 4) * 4 + q;
      const int m = m0 + mr;
      float sq = 0.f;
      if (m < g.M) sq = epi(m, ba * 16 + r16, acc[mb][0][q], bb * 16 + r16, acc[mb][1][q], norm_here ? s_rstd[mr] : 1.f);
      if (g.ssq_out) {
        sq = sum16(sq);
        if (r16 == 0 && m < g.M) g.ssq_out[(int64_t)pair * g.M_pad + m] = sq;
      }
    }
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
    p.u.gm.g.tile_cnt = nullptr;  // the persistent step sums the partials in a phase of its own
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
  if (g.S > 1 && !g.tile_cnt) {
    dim3 g2(g.npairs, (g.M + 15) / 16);
    hipLaunchKernelGGL(k_splitk_epi<uint16_t>, g2, dim3(256), 0, s, g, epi);
  }
}

}  // namespace rlt
