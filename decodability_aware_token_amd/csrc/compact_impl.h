// Compaction pieces shared by the compaction kernels and the one-launch front end (state
// compaction, ragged execution): AI Engineering Academy article on FOCUS, section "Arquitetura
// do FOCUS" (compact the state, drop evicted tokens); project page "FOCUS: DLLMs Know How to
// Tame Their Compute Bound", card "Runtime Action" (ragged execution).
//
// A request's place in the compacted order is the number of tokens kept by the requests before
// it.  It is found in O(B) by one workgroup: each thread takes ceil(B/256) consecutive requests,
// their kept counts (from the inputs alone) are summed per thread and scanned across the 256
// threads in a fixed order -- integers, so exact and deterministic.
#pragma once

#include "select_impl.h"

namespace focus {

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

// nonzero bytes of a BLK-byte row (4-byte aligned)
template <int BLK>
__device__ __forceinline__ int row_count(const uint8_t* row) {
  const uint32_t* w = reinterpret_cast<const uint32_t*>(row);
  int m = 0;
#pragma unroll
  for (int i = 0; i < BLK / 4; ++i) m += nonzero_bytes(w[i]);
  return m;
}

// kept tokens of request r under a per-request budget: min(max(budget[r], 0), m_r)
template <int BLK>
__device__ __forceinline__ int budget_kept(const SelectArgs& sl, int r) {
  return min(max(sl.budget[r], 0), row_count<BLK>(sl.masked + (size_t)r * BLK));
}

// Exclusive prefix sum of one value per thread over the 256 threads of the workgroup, in thread
// order.  s_part: 256 ints of LDS, free again on return.  Every thread must call it.
__device__ __forceinline__ int block_exclusive_scan(int local, int* s_part) {
  const int tid = threadIdx.x, lane = tid & 63;
  s_part[tid] = local;
  __syncthreads();
  if (tid < 64) {  // wave 0: four values per lane, then a lane scan
    int v[4], s = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[i] = s_part[4 * tid + i];
      s += v[i];
    }
    int incl = s;
#pragma unroll
    for (int dd = 1; dd < 64; dd <<= 1) {
      const int y = __shfl_up(incl, dd, 64);
      if (lane >= dd) incl += y;
    }
    int run = incl - s;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      s_part[4 * tid + i] = run;
      run += v[i];
    }
  }
  __syncthreads();
  const int out = s_part[tid];
  __syncthreads();
  return out;
}

// Kept counts of requests 0..B-1 and their exclusive prefix sums, by the whole workgroup:
// emit(r, base_r, k_r) once per request.  kept_of(r) reads request r's inputs; the loads of a
// thread's requests are issued together (addresses clamped into the batch).
template <typename KeptFn, typename EmitFn>
__device__ __forceinline__ void scan_kept(int B, KeptFn kept_of, EmitFn emit, int* s_part) {
  constexpr int PER = kMaxB / 256;
  const int tid = threadIdx.x;
  const int per = (B + 255) / 256;
  int kv[PER];
  int local = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    kv[i] = 0;
    if (i < per) {  // uniform
      const int r = tid * per + i;
      kv[i] = kept_of(min(r, B - 1));
      if (r >= B) kv[i] = 0;
      local += kv[i];
    }
  }
  int run = block_exclusive_scan(local, s_part);
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    if (i < per) {
      const int r = tid * per + i;
      if (r < B) emit(r, run, kv[i]);
      run += kv[i];
    }
  }
}

constexpr int kGatherBatch = 8;  // 16-byte chunks per thread per gather batch

// Compaction of request r, which keeps k_all positions, this lane's (kj) at rank `rank`;
// s_pos[t] is the position of rank t.  base() gives this thread's share of r's base offset (the
// shares are summed over the workgroup; it is called after the first gather batch has been
// issued, so that whatever it waits for overlaps those loads).  dummy: any 16 readable bytes.
// The request's rows are gathered by nsplit workgroups, part `split` of each row set's chunks
// here; part 0 writes the positions and, if write_offsets, offsets[r + 1] (and offsets[0]).
template <typename BaseFn>
__device__ __forceinline__ void compact_finish(const CompactArgs& a, int r, bool kj, int rank,
                                               int k_all, const int* s_pos, int* s_wsum,
                                               const unsigned char* dummy, int split, int nsplit,
                                               bool write_offsets, BaseFn base) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int blk = a.blk;

  // first gather batch of each row set: loads only.  Unconditional (a request with nothing
  // to gather reads the dummy bytes), so that no join makes the compiler wait for these loads
  // before the base below.
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

  // base offset: the threads' shares summed per wave by a fixed xor butterfly and over the 4
  // waves in order (integers: exact and deterministic)
  const int cnt = wave_sum_int(base());
  if (lane == 0) s_wsum[wv] = cnt;
  __syncthreads();
  const int b0 = s_wsum[0] + s_wsum[1] + s_wsum[2] + s_wsum[3];

  if (wv == 0 && split == 0) {
    if (kj && a.kept_pos != nullptr && b0 + rank < a.cap) a.kept_pos[b0 + rank] = lane;
    if (write_offsets && lane == 0) {
      a.offsets[r + 1] = b0 + k_all;
      if (r == 0) a.offsets[0] = 0;
    }
  }
  if (!gather) return;
  const int k = min(k_all, a.cap - b0);  // rows at or past cap are not written
  if (k <= 0) return;
#pragma unroll
  for (int si = 0; si < kMaxSets; ++si) {
    if (si >= a.nsets) break;
    const int limit = min(k * chunks[si], total[si]);
    unsigned char* dst = static_cast<unsigned char*>(a.gathered[si]);
    auto dst_of = [&](int c) {
      const int t = c / chunks[si], cc = c - t * chunks[si];
      return dst + ((int64_t)b0 + t) * a.row_bytes[si] + (int64_t)cc * 16;
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

// Selection with the caller's budget and compaction of request r from its delta (dj: position
// lane, 0 for lanes >= BLK) and its selection inputs already loaded, by a whole workgroup: every wave computes the selection (so no barrier is needed
// before the gather), wave 0 of part 0 stores delta, keep and kept_count.
// LDS: s_pos [64], s_wsum [4], s_k [1].
template <int BLK, typename BaseFn>
__device__ __forceinline__ void select_compact_request(const SelectCompactArgs& a, int r,
                                                       float dj, SelectInputs in, int split,
                                                       int nsplit, bool write_offsets,
                                                       int* s_pos, int* s_wsum, int* s_k,
                                                       BaseFn base) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const SelectArgs& sl = a.sel;
  const Selection sel = select_decide(sl, in.m_byte, in.budget, dj, lane);
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
      *s_k = sel.k;
      if (split == 0) sl.kept_count[r] = sel.k;
    }
  }
  __syncthreads();
  compact_finish(a.cmp, r, kj, rank, *s_k, s_pos, s_wsum, sl.masked + (size_t)r * BLK, split,
                 nsplit, write_offsets, base);
}

}  // namespace focus
