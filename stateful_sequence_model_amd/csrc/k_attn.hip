// Attention kernels of the decoder block ("Recurrent Looped Transformer",
// §2.5 eqs. (2.14)-(2.15) and the cache rule after eq. (2.16)).
//
// Both attentions are one query per (row, head) against stored keys/values,
// i.e. streaming work of about 1 flop per byte: they are bound by HBM
// bandwidth, so they run on the vector ALU (no MFMA) and are organised for
// coalesced, contiguous reads:
//   * a workgroup handles one row and `hpw` consecutive heads, so every key
//     read is hpw*dh contiguous elements; the head groups of one row are
//     the fastest grid dimension, so the workgroups that together read a
//     full key row are dispatched next to each other;
//   * each lane owns E consecutive elements (32 bytes) of one head; the
//     dh/E lanes of a head reduce the q.k dot with xor-shuffles (all lanes
//     end with the identical sum);
//   * the 256 threads form 256/(hpw*dh/E) key groups; a key group takes
//     U keys at a time (all loads issued first), then one running-max update
//     and rescale for the U keys (online softmax in base 2, the
//     log2(e)/sqrt(dh) scale folded into q); the key groups' (max, sum,
//     output) partials are merged in LDS in group order. Every order is a
//     function of t only, so results do not depend on timing or batch.
//
// SWA (eq. 2.14): keys are the retained positions max(1, t-W+1) .. t-1 from
// the ring (slot (j-1) mod (W-1)) plus the current (k, v); after all reads
// of the workgroup the current (k, v) is written to slot (t-1) mod (W-1),
// the slot of position t-W+1 which leaves the window (nothing else reads
// those columns of this row).
// Cross-attention (eq. 2.15): keys are memory positions 1..t only; the
// range is split into chunks of `chunk` positions (boundaries depend on t
// only), each chunk writes an unnormalised (o, max, sum) partial, and the
// chunks are merged in chunk order, by the last of a row's chunk workgroups
// to finish (arrival counter per row and head group) or by a combine kernel
// (the persistent step's phase list, or on request). A row whose t fits the
// first chunk gets its normalised output from that chunk directly (what the
// combine would write); the combine skips it.
#include "attn_dev.h"

namespace rlt {

// grid: x = head group, y = slot; block 256
template <typename T, int DH>
__global__ __launch_bounds__(256) void k_swa(AttnArgs a) {
  __shared__ float lds[attn_lds_floats<T>()];
  swa_body<T, DH>(a, blockIdx.x, blockIdx.y, lds);
}

// grid: x = head group, y = slot, z = chunk (chunk outermost: with rows at
// similar positions the workgroups of chunks past t, which exit at once, come
// last instead of interleaved with the active ones); block 256
template <typename T, int DH>
__global__ __launch_bounds__(256) void k_xattn(AttnArgs a) {
  __shared__ float lds[attn_lds_floats<T>()];
  xattn_body<T, DH>(a, blockIdx.x, blockIdx.z, blockIdx.y, lds);
}

// grid: x = head, y = slot; block 64
template <typename T, int DH>
__global__ __launch_bounds__(64) void k_xcombine(AttnArgs a) {
  xcombine_body<T, DH>(a, blockIdx.x, blockIdx.y, threadIdx.x, 64);
}

template <typename T, int DH>
static void swa_t(const AttnArgs& a, hipStream_t s) {
  dim3 grid(a.H / a.hpw, a.rows.n);
  hipLaunchKernelGGL((k_swa<T, DH>), grid, dim3(256), 0, s, a);
}
template <typename T, int DH>
static void xattn_t(const AttnArgs& a, hipStream_t s) {
  dim3 grid(a.H / a.hpw, a.rows.n, a.nch);
  hipLaunchKernelGGL((k_xattn<T, DH>), grid, dim3(256), 0, s, a);
}
template <typename T, int DH>
static void xcomb_t(const AttnArgs& a, hipStream_t s) {
  dim3 grid(a.H, a.rows.n);
  hipLaunchKernelGGL((k_xcombine<T, DH>), grid, dim3(64), 0, s, a);
}

#define RLT_DISPATCH_DH(FN, T, a, s)            \
  switch ((a).dh) {                             \
    case 16: FN<T, 16>(a, s); break;            \
    case 32: FN<T, 32>(a, s); break;            \
    case 64: FN<T, 64>(a, s); break;            \
    default: FN<T, 128>(a, s); break;           \
  }

void launch_swa(int dtype, const AttnArgs& a, hipStream_t s) {
  if (dtype == 1) {
    Phase p{};
    p.kind = PH_SWA;
    p.gx = a.H / a.hpw;
    p.gy = a.rows.n;
    p.gz = 1;
    p.u.at = a;
    if (record_phase(p)) return;
  }
  if (dtype == 0) { RLT_DISPATCH_DH(swa_t, float, a, s); }
  else { RLT_DISPATCH_DH(swa_t, uint16_t, a, s); }
}
void launch_xattn(int dtype, const AttnArgs& a, hipStream_t s) {
  if (dtype == 1) {
    Phase p{};
    p.kind = PH_XATTN;
    p.gx = a.H / a.hpw;
    p.gy = a.rows.n;
    p.gz = a.nch;
    p.u.at = a;
    p.u.at.cnt = nullptr;  // the persistent step runs the combine as a phase of its own
    if (record_phase(p)) return;
  }
  if (dtype == 0) { RLT_DISPATCH_DH(xattn_t, float, a, s); }
  else { RLT_DISPATCH_DH(xattn_t, uint16_t, a, s); }
}
void launch_xcombine(int dtype, const AttnArgs& a, hipStream_t s) {
  if (dtype == 1) {
    Phase p{};
    p.kind = PH_XCOMBINE;
    p.gx = a.H;
    p.gy = a.rows.n;
    p.gz = 1;
    p.u.at = a;
    if (record_phase(p)) return;
  }
  if (a.cnt) return;  // merged by the cross-attention launch
  if (dtype == 0) { RLT_DISPATCH_DH(xcomb_t, float, a, s); }
  else { RLT_DISPATCH_DH(xcomb_t, uint16_t, a, s); }
}

}  // namespace rlt
