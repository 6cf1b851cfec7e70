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
#include "select_impl.h"

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

// Steps 3-5, shared by both kernels: request r keeps k_all positions, this lane's (kj) at rank
// `rank`; s_pos[t] is the position of rank t.  count() is this thread's share of the kept
// tokens of the predecessors (its loads may still be in flight: it is called after the first
// gather batch has been issued).  dummy: any 16 readable bytes.  The request's rows are gathered
// by nsplit workgroups, part `split` of each row set's chunks here; part 0 writes the positions
// and offsets.
template <typename CountFn>
__device__ __forceinline__ void compact_finish(const CompactArgs& a, int r, bool kj, int rank,
                                               int k_all, const int* s_pos, int* s_wsum,
                                               const unsigned char* dummy, int split, int nsplit,
                                               CountFn count) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int blk = a.blk;

  // 3. first gather batch of each row set: loads only.  Unconditional (a request with nothing
  // to gather reads the dummy bytes), so that no join makes the compiler wait for these loads
  // before the count below.
  const bool gather = a.nsets > 0 && k_all > 0;
  int chunks[kMaxSets], c_lo[kMaxSets], total[kMaxSets];  // this part: chunks [c_lo, total)
#pragma unroll
  for (int si = 0; si < kMaxSets; ++si) {
    chunks[si] = (gather && si < a.nsets) ? (int)(a.row_bytes[si] / 16) : 0;  // <= 2^20
    const int all = k_all * chunks[si], per = (all + nsplit - 1) / nsplit;
    c_lo[si] = min(split * per, all);
    total[si] = min(c_lo[si] + per, all);
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
      v[si][u] = load16(total[si] > c_lo[si]
                            ? src_of(si, min(c_lo[si] + tid + u * 256, total[si] - 1)) : dummy);

  // 4. base = kept tokens of the predecessors: per-thread counts summed per wave by a fixed xor
  // butterfly and over the 4 waves in order (integers: exact and deterministic)
  int cnt = wave_sum_int(count());
  if (lane == 0) s_wsum[wv] = cnt;
  __syncthreads();
  const int base = s_wsum[0] + s_wsum[1] + s_wsum[2] + s_wsum[3];

  // 5. outputs
  if (wv == 0 && split == 0) {
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
    const int limit = min(k * chunks[si], total[si]);
    unsigned char* dst = static_cast<unsigned char*>(a.gathered[si]);
    auto dst_of = [&](int c) {
      const int t = c / chunks[si], cc = c - t * chunks[si];
      return dst + ((int64_t)base + t) * a.row_bytes[si] + (int64_t)cc * 16;
    };
#pragma unroll
    for (int u = 0; u < kGatherBatch; ++u) {
      const int c = c_lo[si] + tid + u * 256;
      if (c < limit) *reinterpret_cast<uint4*>(dst_of(c)) = v[si][u];
    }
    for (int c0 = c_lo[si] + tid + 256 * kGatherBatch; c0 < limit; c0 += 256 * kGatherBatch) {
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

  compact_finish(a, r, kj, rank, s_k, s_pos, s_wsum, a.keep + (size_t)r * blk, 0, 1, [&]() {
    int cnt = 0;
#pragma unroll
    for (int u = 0; u < kCountBatch; ++u) cnt += nonzero_bytes(cw[u]);
    for (int w = tid + 256 * kCountBatch; w < nw; w += 256) cnt += nonzero_bytes(kw[w]);
    return cnt;
  });
}

// Score reduction + selection + compaction for budgets that do not depend on delta (the
// caller's per-request integers): request r keeps min(max(budget[r], 0), m_r) tokens, m_r its
// masked count, so every workgroup knows its base offset from the masks and budgets of its
// predecessors alone and no pass over the selections is needed.  nsplit workgroups per request
// (grid [B, nsplit]), each gathering its share of the request's rows:
//  1. every thread loads the mask row and budget of its first predecessor;
//  2. every wave sums the request's score partials over the kv heads (lane j: position j, heads
//     in order, the same arithmetic as the score reduction) and runs the selection; wave 0
//     stores delta, keep, the kept count and the kept positions' order;
//  3-5. as in the compaction kernel, with the predecessors' kept counts from step 1.
template <int BLK>
__global__ __launch_bounds__(256) void select_compact_kernel(SelectCompactArgs a) {
  __shared__ int s_wsum[4];
  __shared__ int s_pos[64];
  __shared__ int s_k;
  constexpr int WORDS = BLK / 4;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int r = blockIdx.x, split = blockIdx.y;
  const SelectArgs& sl = a.sel;

  // 1. the first predecessor of this thread (clamped: loads are unconditional)
  const int rp0 = min(tid, max(r - 1, 0));
  const uint32_t* mw0 = reinterpret_cast<const uint32_t*>(sl.masked + (size_t)rp0 * BLK);
  uint32_t w0[WORDS];
#pragma unroll
  for (int i = 0; i < WORDS; ++i) w0[i] = mw0[i];
  const int b0 = sl.budget[rp0];

  // 2. delta of position lane (fixed head order), then the selection
  const float* pr = a.part + (size_t)r * a.Hkv * BLK + min(lane, BLK - 1);
  // eight partials loaded before any is added (a loop adding each as it arrives waits for every
  // load in turn), then summed in head order
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
  const Selection sel = select_compute(sl, r, dj, lane);
  const bool kj = sel.kept;
  const uint64_t bits = __ballot(kj);
  const int rank = __builtin_amdgcn_mbcnt_hi((uint32_t)(bits >> 32),
                                             __builtin_amdgcn_mbcnt_lo((uint32_t)bits, 0u));
  if (wv == 0) {
    if (lane < BLK && split == 0) {
      a.delta[(size_t)r * BLK + lane] = dj;
      sl.keep[(size_t)r * BLK + lane] = kj ? 1 : 0;
    }
    if (kj) s_pos[rank] = lane;
    if (lane == 0) {
      s_k = sel.k;
      if (split == 0) sl.kept_count[r] = sel.k;
    }
  }
  __syncthreads();

  auto kept_of = [&](const uint32_t* w, int b) {
    int m = 0;
#pragma unroll
    for (int i = 0; i < WORDS; ++i) m += nonzero_bytes(w[i]);
    return min(max(b, 0), m);
  };
  compact_finish(a.cmp, r, kj, rank, s_k, s_pos, s_wsum, sl.masked + (size_t)r * BLK, split,
                 gridDim.y, [&]() {
    int cnt = tid < r ? kept_of(w0, b0) : 0;
    for (int rp = tid + 256; rp < r; rp += 256) {
      uint32_t w[WORDS];
      const uint32_t* mw = reinterpret_cast<const uint32_t*>(sl.masked + (size_t)rp * BLK);
#pragma unroll
      for (int i = 0; i < WORDS; ++i) w[i] = mw[i];
      cnt += kept_of(w, sl.budget[rp]);
    }
    return cnt;
  });
}

}  // namespace

hipError_t launch_compact(const CompactArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(compact_kernel, dim3(a.B), dim3(256), 0, s, a);
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
