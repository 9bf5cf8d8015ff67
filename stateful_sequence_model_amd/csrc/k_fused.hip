// Persistent decoder step for small calls ("Recurrent Looped Transformer",
// §2.5 eqs. (2.9)-(2.16), §2.3 eq. (2.6)).
//
// With a few rows per call every kernel of the transition moves little data
// and its duration is set by launch, ramp-up and drain, not by bandwidth.
// Here the host records the launches of one transition as a list of phases
// (the same kernel bodies with the same launch shapes) and a single kernel
// runs them: one workgroup per compute unit, each phase's virtual blocks
// dealt round-robin to the workgroups, and a grid-wide barrier between
// phases. Results equal those of the separate kernels bit for bit (same
// bodies, same shapes, same reduction orders).
//
// Grid barrier: arrival counter whose top bit flips when the last workgroup
// arrives (workgroup 0 adds 2^31 - (G - 1), the others add 1), so it needs
// no reset between barriers or launches. Every wave first waits for its own
// global stores; one thread then publishes them at device scope (release),
// arrives, polls with sleeps and acquires. All workgroups are resident at
// once (grid = compute units, resources for one workgroup each), so the
// barrier cannot wait on an unscheduled workgroup; a wall-clock limit turns
// any anomaly into an abort flag and an error word instead of a hang.
#include "attn_dev.h"
#include "gemm_dev.h"
#include "misc_dev.h"

namespace rlt {

namespace {

constexpr int cmax(int a, int b) { return a > b ? a : b; }
constexpr int FUSED_LDS =
    cmax(cmax(gemm_lds_floats(2), attn_lds_floats<uint16_t>()), cmax(SPLITK_LDS_FLOATS, 16));

constexpr int ERR_HIP = -6;  // RLT_EHIP

// returns false when the step was aborted
__device__ bool grid_barrier(unsigned* sync, int* err, int64_t spin_ticks, int* s_flag) {
  __builtin_amdgcn_s_waitcnt(0);  // this wave's stores have reached the cache hierarchy
  __syncthreads();
  if (threadIdx.x == 0) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    const unsigned add = blockIdx.x == 0 ? 0x80000000u - (gridDim.x - 1) : 1u;
    const unsigned old = __hip_atomic_fetch_add(sync, add, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const int64_t t0 = (int64_t)__builtin_amdgcn_s_memrealtime();
    int ok = 1;
    while (true) {
      const unsigned cur = __hip_atomic_load(sync, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if ((cur ^ old) & 0x80000000u) break;
      if (__hip_atomic_load(sync + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) {
        ok = 0;
        break;
      }
      if ((int64_t)__builtin_amdgcn_s_memrealtime() - t0 > spin_ticks) {
        __hip_atomic_store(sync + 1, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        *(volatile int*)err = ERR_HIP;
        ok = 0;
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    *s_flag = ok;
  }
  __syncthreads();
  return *s_flag != 0;
}

template <int DH>
__device__ __forceinline__ void attn_phase(int kind, const AttnArgs& a, int bx, int by, int bz, float* lds) {
  if (kind == PH_SWA)
    swa_body<uint16_t, DH>(a, bx, by, lds);
  else if (kind == PH_XATTN)
    xattn_body<uint16_t, DH>(a, bx, bz, by, lds);  // (head group, slot, chunk) grid
  else
    xcombine_body<uint16_t, DH>(a, bx, by, threadIdx.x, 256);
}

}  // namespace

// grid: one workgroup per compute unit; block 256
__global__ __launch_bounds__(256) void k_fused(const Phase* __restrict__ ph, int nph, unsigned* sync, int* err,
                                               int64_t spin_ticks) {
  __shared__ float lds[FUSED_LDS];
  __shared__ int s_flag;
  if (__hip_atomic_load(sync + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) return;  // earlier abort
  for (int i = 0; i < nph; ++i) {
    const Phase& P = ph[i];
    const int kind = P.kind;
    const int gx = P.gx, gy = P.gy;
    const int nvb = gx * gy * P.gz;
    for (int vb = blockIdx.x; vb < nvb; vb += gridDim.x) {
      const int bx = vb % gx, r = vb / gx, by = r % gy, bz = r / gy;
      switch (kind) {
        case PH_GEMM: {
          const Epi<uint16_t>& epi = *reinterpret_cast<const Epi<uint16_t>*>(&P.u.gm.e);
          if (P.u.gm.g.mb == 1)
            gemm_bf16_body<1>(P.u.gm.g, epi, bx, by, bz, lds);
          else
            gemm_bf16_body<2>(P.u.gm.g, epi, bx, by, bz, lds);
          break;
        }
        case PH_SPLITK: {
          const Epi<uint16_t>& epi = *reinterpret_cast<const Epi<uint16_t>*>(&P.u.gm.e);
          splitk_epi_body<uint16_t>(P.u.gm.g, epi, bx, by, lds);
          break;
        }
        case PH_SWA:
        case PH_XATTN:
        case PH_XCOMBINE:
          switch (P.u.at.dh) {
            case 16: attn_phase<16>(kind, P.u.at, bx, by, bz, lds); break;
            case 32: attn_phase<32>(kind, P.u.at, bx, by, bz, lds); break;
            case 64: attn_phase<64>(kind, P.u.at, bx, by, bz, lds); break;
            default: attn_phase<128>(kind, P.u.at, bx, by, bz, lds); break;
          }
          break;
        case PH_MERGE_PREP:
          merge_prep_body<uint16_t>(P.u.mi, bx, lds);
          break;
        case PH_FINAL:
          final_body<uint16_t>(P.u.mi, bx);
          break;
        default: {  // PH_COPY
          const int64_t e = (int64_t)bx * 256 + threadIdx.x;
          if (e < P.u.cp.n) P.u.cp.dst[e] = P.u.cp.src[e];
          break;
        }
      }
      __syncthreads();  // the next block of this workgroup reuses the LDS
    }
    if (i + 1 < nph && !grid_barrier(sync, err, spin_ticks, &s_flag)) return;
  }
}

int fused_blocks_per_cu() {
  int nb = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, k_fused, 256, 0) != hipSuccess) return 0;
  return nb;
}

void launch_fused(const Phase* phases, int nphase, unsigned* sync, int* err, int grid, int64_t spin_ticks,
                  hipStream_t s) {
  hipLaunchKernelGGL(k_fused, dim3(grid), dim3(256), 0, s, phases, nphase, sync, err, spin_ticks);
}

}  // namespace rlt
