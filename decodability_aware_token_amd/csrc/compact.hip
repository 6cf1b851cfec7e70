// Compaction and gather (state compaction, ragged execution): AI Engineering Academy article on
// FOCUS, section "Arquitetura do FOCUS" (compact the state, drop evicted tokens); project page
// "FOCUS: DLLMs Know How to Tame Their Compute Bound", card "Runtime Action" (ragged execution).
//
// The base offset of request r (kept tokens of the requests before it) comes one of two ways:
//  * up to kScanFromB requests: each workgroup counts its predecessors' nonzero keep bytes
//    itself (O(B) per workgroup, from L2; its loads are issued first and overlap the rest);
//  * above: compact_scan_kernel, one workgroup, scans the kept counts into offsets first (O(B)
//    in total), and each workgroup reads its base from there.
// compact_kernel, one workgroup per request r:
//  a. wave 0: lane j tests keep[r, j]; a ballot gives k_r and each kept lane's rank (mbcnt), so
//     the kept positions come out in ascending order;
//  b. all threads issue the loads of the first batch of the k_r rows to gather (16 bytes each);
//     they do not depend on where the rows go;
//  c. the base offset, as above;
//  d. kept_pos[base + rank] = j, offsets[r + 1] (counting workgroups) and the gathered rows are
//     stored.
#include "compact_impl.h"

namespace focus {
namespace {

// Largest batch whose workgroups count their predecessors themselves.  Measured (two row sets
// of 8 KiB, 4 kept per request): the scan launch costs 3.3 us more at 128 requests and 5.3 us
// more at 1024, the two are equal at 2048, and the counts (0.5 GB read from L2 in all at 4096)
// cost 4.7 us more at 3072 and 6.3 us more at 4096.
constexpr int kScanFromB = 2048;

template <int BLK>
__global__ __launch_bounds__(256) void compact_scan_kernel(const uint8_t* __restrict__ keep,
                                                           int B, int32_t* __restrict__ offsets) {
  __shared__ int s_part[256];
  scan_kept(
      B, [&](int r) { return row_count<BLK>(keep + (size_t)r * BLK); },
      [&](int r, int base, int k) {
        offsets[r + 1] = base + k;
        if (r == 0) offsets[0] = 0;
      },
      s_part);
}

constexpr int kCountBatch = 16;  // predecessor keep words per thread in the first batch

// COUNT: the workgroup counts its predecessors' kept tokens; else it reads offsets[r].
template <bool COUNT>
__global__ __launch_bounds__(256) void compact_kernel(CompactArgs a) {
  __shared__ int s_wsum[4];
  __shared__ int s_pos[64];
  __shared__ int s_k;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int r = blockIdx.x;
  const int blk = a.blk;
  const int words = blk / 4;  // keep row as 32-bit words (rows are 16/32/64 bytes)

  // Loads first and branch-free (clamped addresses, results masked afterwards), so that the
  // compiler can wait for each group of loads alone: this request's keep byte (every wave: the
  // ballot below needs no branch), then the base's inputs.
  const uint8_t kb = a.keep[(size_t)r * blk + min(lane, blk - 1)];
  const uint32_t* kw = reinterpret_cast<const uint32_t*>(a.keep);
  const int nw = r * words;  // predecessor keep words
  uint32_t cw[COUNT ? kCountBatch : 1];
  int base_read = 0;
  if constexpr (COUNT) {
#pragma unroll
    for (int u = 0; u < kCountBatch; ++u) cw[u] = kw[min(tid + 256 * u, max(nw - 1, 0))];
  } else {
    base_read = a.offsets[max(r, 0)];
  }
  __builtin_amdgcn_sched_barrier(0);  // issue all of them before the ballot waits
  if constexpr (COUNT) {
#pragma unroll
    for (int u = 0; u < kCountBatch; ++u)
      if (tid + 256 * u >= nw) cw[u] = 0u;
  }

  // a. this request's kept positions (every wave computes the ballot; wave 0 publishes it)
  const bool kj = lane < blk && kb != 0;
  const uint64_t bits = __ballot(kj);
  const int rank = __builtin_amdgcn_mbcnt_hi((uint32_t)(bits >> 32),
                                             __builtin_amdgcn_mbcnt_lo((uint32_t)bits, 0u));
  if (wv == 0) {
    if (kj) s_pos[rank] = lane;
    if (lane == 0) s_k = __popcll(bits);
  }
  __syncthreads();

  compact_finish(a, r, kj, rank, s_k, s_pos, s_wsum, a.keep + (size_t)r * blk, 0, 1, COUNT,
                 [&]() {
                   if constexpr (COUNT) {
                     int cnt = 0;
#pragma unroll
                     for (int u = 0; u < kCountBatch; ++u) cnt += nonzero_bytes(cw[u]);
                     for (int w = tid + 256 * kCountBatch; w < nw; w += 256)
                       cnt += nonzero_bytes(kw[w]);
                     return cnt;
                   } else {
                     return (tid == 0 && r > 0) ? base_read : 0;
                   }
                 });
}

// Second launch of the two-launch front end: reduction of the score partials, selection with
// the caller's budgets and compaction.  The score launch has written offsets (from the masks
// and budgets alone), so each workgroup reads its base; nsplit workgroups per request (grid
// [B, nsplit]), each gathering its share of the request's rows.
template <int BLK>
__global__ __launch_bounds__(256) void select_compact_kernel(SelectCompactArgs a) {
  __shared__ int s_wsum[4];
  __shared__ int s_pos[64];
  __shared__ int s_k;
  const int tid = threadIdx.x, lane = tid & 63;
  const int r = blockIdx.x, split = blockIdx.y;
  // every input first, so that their round trips overlap: the selection's mask byte and
  // budget, the base offset, then the partials
  const SelectInputs in = select_inputs(a.sel, r, lane);
  const int base = (tid == 0 && r > 0) ? a.cmp.offsets[r] : 0;

  // delta of position lane: the Hkv partials summed in kv-head order.  Eight partials are
  // loaded before any is added (a loop adding each as it arrives waits for every load in turn)
  const float* pr = a.part + (size_t)r * a.Hkv * BLK + min(lane, BLK - 1);
  float dj = 0.f;
  for (int g0 = 0; g0 < a.Hkv; g0 += 8) {
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = pr[(size_t)min(g0 + u, a.Hkv - 1) * BLK];
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (g0 + u < a.Hkv) dj += v[u];
  }
  if (lane >= BLK) dj = 0.f;
  select_compact_request<BLK>(a, r, dj, in, split, gridDim.y, false, s_pos, s_wsum, &s_k,
                              [&]() { return base; });
}

}  // namespace

hipError_t launch_compact(const CompactArgs& a, hipStream_t s) {
  if (a.B <= kScanFromB) {
    hipLaunchKernelGGL(compact_kernel<true>, dim3(a.B), dim3(256), 0, s, a);
    return hipGetLastError();
  }
  if (a.blk == 16)
    hipLaunchKernelGGL(compact_scan_kernel<16>, dim3(1), dim3(256), 0, s, a.keep, a.B, a.offsets);
  else if (a.blk == 32)
    hipLaunchKernelGGL(compact_scan_kernel<32>, dim3(1), dim3(256), 0, s, a.keep, a.B, a.offsets);
  else
    hipLaunchKernelGGL(compact_scan_kernel<64>, dim3(1), dim3(256), 0, s, a.keep, a.B, a.offsets);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(compact_kernel<false>, dim3(a.B), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_select_compact(const SelectCompactArgs& a, hipStream_t s) {
  if (a.sel.blk == 16)
    hipLaunchKernelGGL(select_compact_kernel<16>, dim3(a.sel.B, a.nsplit), dim3(256), 0, s, a);
  else if (a.sel.blk == 32)
    hipLaunchKernelGGL(select_compact_kernel<32>, dim3(a.sel.B, a.nsplit), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(select_compact_kernel<64>, dim3(a.sel.B, a.nsplit), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace focus
