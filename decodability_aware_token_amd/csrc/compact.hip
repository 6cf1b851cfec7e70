// Compaction and gather (state compaction, ragged execution): AI Engineering Academy article on
// FOCUS, section "Arquitetura do FOCUS" (compact the state, drop evicted tokens); project page
// "FOCUS: DLLMs Know How to Tame Their Compute Bound", card "Runtime Action" (ragged execution).
//
// One workgroup per request r, 256 threads.
//  1. base = offsets[r] = number of kept tokens of requests 0..r-1: every thread counts the
//     nonzero bytes of a strided subset of the predecessors' keep rows (4 bytes at a time), then a
//     fixed-order LDS tree sums the 256 partial counts.  Integer arithmetic: exact and
//     deterministic.  (Quadratic in B in total, which is cheap for the supported B <= 4096 since
//     the keep rows are read from L2.)
//  2. Wave 0: lane j tests keep[r, j]; a ballot gives k_r and the lane's rank among the kept
//     lanes (mbcnt), so kept_pos[base + rank] = j lists positions in ascending order.
//  3. All threads copy the k_r rows with 16-byte loads, several chunks in flight per thread.
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

__global__ __launch_bounds__(256) void compact_kernel(CompactArgs a) {
  __shared__ int s_cnt[256];
  __shared__ int s_pos[64];
  __shared__ int s_base, s_k;
  const int tid = threadIdx.x;
  const int r = blockIdx.x;
  const int blk = a.blk;
  const int words = blk / 4;  // keep row as 32-bit words (rows are 16/32/64 bytes)

  // 1. kept tokens of the predecessors
  int cnt = 0;
  const uint32_t* kw = reinterpret_cast<const uint32_t*>(a.keep);
  const int nw = r * words;
  for (int w = tid; w < nw; w += 256) cnt += nonzero_bytes(kw[w]);
  s_cnt[tid] = cnt;
  __syncthreads();
  for (int stride = 128; stride > 0; stride >>= 1) {
    if (tid < stride) s_cnt[tid] += s_cnt[tid + stride];
    __syncthreads();
  }

  // 2. this request's kept positions
  if (tid < 64) {
    const bool kj = tid < blk && a.keep[(size_t)r * blk + tid] != 0;
    const uint64_t bits = __ballot(kj);
    const int rank = __builtin_amdgcn_mbcnt_hi((uint32_t)(bits >> 32),
                                               __builtin_amdgcn_mbcnt_lo((uint32_t)bits, 0u));
    const int base = s_cnt[0];
    const int k = __popcll(bits);
    if (kj) {
      s_pos[rank] = tid;
      if (a.kept_pos != nullptr && base + rank < a.cap) a.kept_pos[base + rank] = tid;
    }
    if (tid == 0) {
      s_base = base;
      s_k = k;
      a.offsets[r + 1] = base + k;
      if (r == 0) a.offsets[0] = 0;
    }
  }
  __syncthreads();

  // 3. gather
  if (a.gathered == nullptr) return;
  const int base = s_base;
  const int k = min(s_k, a.cap - base);
  if (k <= 0) return;
  const int64_t chunks = a.row_bytes / 16;
  const int64_t total = (int64_t)k * chunks;
  const unsigned char* src = reinterpret_cast<const unsigned char*>(a.rows);
  unsigned char* dst = reinterpret_cast<unsigned char*>(a.gathered);
  constexpr int U = 4;
  for (int64_t c0 = tid; c0 < total; c0 += 256 * U) {
    uint4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t c = c0 + (int64_t)u * 256;
      if (c < total) {
        const int t = (int)(c / chunks);
        const int64_t cc = c - (int64_t)t * chunks;
        v[u] = load16(src + ((int64_t)r * blk + s_pos[t]) * a.row_bytes + cc * 16);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t c = c0 + (int64_t)u * 256;
      if (c < total) {
        const int t = (int)(c / chunks);
        const int64_t cc = c - (int64_t)t * chunks;
        *reinterpret_cast<uint4*>(dst + ((int64_t)base + t) * a.row_bytes + cc * 16) = v[u];
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
