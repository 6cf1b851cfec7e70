// Compaction and gather (state compaction, ragged execution): AI Engineering Academy article on
// FOCUS, section "Arquitetura do FOCUS" (compact the state, drop evicted tokens); project page
// "FOCUS: DLLMs Know How to Tame Their Compute Bound", card "Runtime Action" (ragged execution).
//
// One workgroup per request r, 256 threads, ordered so that the memory round trips overlap:
//  1. Every thread issues its loads of the predecessors' keep rows (4 bytes at a time, a first
//     batch of up to 16 words per thread in flight at once).
//  2. Wave 0: lane j tests keep[r, j]; a ballot gives k_r and each kept lane's rank (mbcnt), so
//     the kept positions come out in ascending order.
//  3. All threads issue the loads of the first batch of the k_r rows to gather (16 bytes each);
//     they do not depend on where the rows go.
//  4. base = offsets[r] = kept tokens of requests 0..r-1: the nonzero bytes of the predecessors'
//     keep rows, summed per wave by a fixed xor butterfly and over the 4 waves in order.
//     Integer arithmetic: exact and deterministic.  (Quadratic in B in total, which is cheap
//     for the supported B <= 4096 since the keep rows are read from L2.)
//  5. kept_pos[base + rank] = j, offsets[r + 1] = base + k_r, and the gathered rows are stored.
#include "device_common.h"
#include "launch.h"

namespace focus {
namespace {

__device__ __forceinline__ int nonzero_bytes(uint32_t w) {
  w |= w >> 4;
  w |= w >> 2;
  w |= w >> 1;
  return __popc(w & 0x01010101u);
}

__device__ __forceinline__ int wave_sum_int(int v) {
#pragma unroll
  for (int m = 32; m > 0; m >>= 1) v += __shfl_xor(v, m, 64);
  return v;
}

constexpr int kCountBatch = 16;  // predecessor keep words per thread in the first batch
constexpr int kGatherBatch = 8;  // 16-byte chunks per thread per gather batch

__global__ __launch_bounds__(256) void compact_kernel(CompactArgs a) {
  __shared__ int s_wsum[4];
  __shared__ int s_pos[64];
  __shared__ int s_k;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int r = blockIdx.x;
  const int blk = a.blk;
  const int words = blk / 4;  // keep row as 32-bit words (rows are 16/32/64 bytes)

  // Loads are branch-free (clamped addresses, results masked afterwards), so that the compiler
  // can wait for each group of loads alone instead of for everything in flight.
  // this request's keep byte (every wave: the ballot below needs no branch), loaded first so
  // that the ballot waits for it alone
  const uint8_t kb = a.keep[(size_t)r * blk + min(lane, blk - 1)];

  // 1. first batch of predecessor keep words
  const uint32_t* kw = reinterpret_cast<const uint32_t*>(a.keep);
  const int nw = r * words;
  uint32_t cw[kCountBatch];
#pragma unroll
  for (int u = 0; u < kCountBatch; ++u) {
    const int w = tid + 256 * u;
    cw[u] = kw[min(w, max(nw - 1, 0))];
  }
  __builtin_amdgcn_sched_barrier(0);  // issue all of them before the ballot waits
#pragma unroll
  for (int u = 0; u < kCountBatch; ++u)
    if (tid + 256 * u >= nw) cw[u] = 0u;

  // 2. this request's kept positions (every wave computes the ballot; wave 0 publishes it)
  const bool kj = lane < blk && kb != 0;
  const uint64_t bits = __ballot(kj);
  const int rank = __builtin_amdgcn_mbcnt_hi((uint32_t)(bits >> 32),
                                             __builtin_amdgcn_mbcnt_lo((uint32_t)bits, 0u));
  if (wv == 0) {
    if (kj) s_pos[rank] = lane;
    if (lane == 0) s_k = __popcll(bits);
  }
  __syncthreads();
  const int k_all = s_k;

  // 3. first gather batch of each row set: loads only.  Unconditional (a request with nothing
  // to gather reads 16 bytes of its own keep row), so that no join makes the compiler wait for
  // these loads before the count below.
  const unsigned char* dummy = a.keep + (size_t)r * blk;
  const bool gather = a.nsets > 0 && k_all > 0;
  int chunks[kMaxSets], total[kMaxSets];
#pragma unroll
  for (int si = 0; si < kMaxSets; ++si) {
    chunks[si] = (gather && si < a.nsets) ? (int)(a.row_bytes[si] / 16) : 0;  // <= 2^20
    total[si] = k_all * chunks[si];
  }
  auto src_of = [&](int si, int c) {
    const int t = c / chunks[si], cc = c - t * chunks[si];
    return static_cast<const unsigned char*>(a.rows[si]) +
           ((int64_t)r * blk + s_pos[t]) * a.row_bytes[si] + (int64_t)cc * 16;
  };
  uint4 v[kMaxSets][kGatherBatch];
#pragma unroll
  for (int si = 0; si < kMaxSets; ++si)
#pragma unroll
    for (int u = 0; u < kGatherBatch; ++u)
      v[si][u] = load16(total[si] > 0 ? src_of(si, min(tid + u * 256, total[si] - 1)) : dummy);

  // 4. base = kept tokens of the predecessors
  int cnt = 0;
#pragma unroll
  for (int u = 0; u < kCountBatch; ++u) cnt += nonzero_bytes(cw[u]);
  for (int w = tid + 256 * kCountBatch; w < nw; w += 256) cnt += nonzero_bytes(kw[w]);
  cnt = wave_sum_int(cnt);
  if (lane == 0) s_wsum[wv] = cnt;
  __syncthreads();
  const int base = s_wsum[0] + s_wsum[1] + s_wsum[2] + s_wsum[3];

  // 5. outputs
  if (wv == 0) {
    if (kj && a.kept_pos != nullptr && base + rank < a.cap) a.kept_pos[base + rank] = lane;
    if (lane == 0) {
      a.offsets[r + 1] = base + k_all;
      if (r == 0) a.offsets[0] = 0;
    }
  }
  if (!gather) return;
  const int k = min(k_all, a.cap - base);  // rows at or past cap are not written
  if (k <= 0) return;
#pragma unroll
  for (int si = 0; si < kMaxSets; ++si) {
    if (si >= a.nsets) break;
    const int limit = k * chunks[si];
    unsigned char* dst = static_cast<unsigned char*>(a.gathered[si]);
    auto dst_of = [&](int c) {
      const int t = c / chunks[si], cc = c - t * chunks[si];
      return dst + ((int64_t)base + t) * a.row_bytes[si] + (int64_t)cc * 16;
    };
#pragma unroll
    for (int u = 0; u < kGatherBatch; ++u) {
      const int c = tid + u * 256;
      if (c < limit) *reinterpret_cast<uint4*>(dst_of(c)) = v[si][u];
    }
    for (int c0 = tid + 256 * kGatherBatch; c0 < limit; c0 += 256 * kGatherBatch) {
      uint4 w[kGatherBatch];
#pragma unroll
      for (int u = 0; u < kGatherBatch; ++u)
        w[u] = load16(src_of(si, min(c0 + u * 256, limit - 1)));
#pragma unroll
      for (int u = 0; u < kGatherBatch; ++u) {
        const int c = c0 + u * 256;
        if (c < limit) *reinterpret_cast<uint4*>(dst_of(c)) = w[u];
      }
    }
  }
}

}  // namespace

hipError_t launch_compact(const CompactArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(compact_kernel, dim3(a.B), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace focus
