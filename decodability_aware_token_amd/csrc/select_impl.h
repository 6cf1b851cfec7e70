// Budgeted selection of one request by one wavefront (shared by the selection kernel and the
// fused score + select kernel).  Project page "FOCUS: DLLMs Know How to Tame Their Compute
// Bound", cards "Design" (adaptive budget over likely-decodable candidates) and "Runtime
// Action" (dynamic budgeting, token eviction).
//
// Lane j holds block position j (blk <= 64) and its delta.  The budget is either the caller's
// per-request integer or clamp(#{delta > mean + beta*std}, lo, hi) over the masked candidates,
// with mean and population std reduced in f32 by a fixed xor butterfly.  The top-k is a
// rank-by-count: rank_j = #{masked i : delta_i > delta_j, or delta_i == delta_j and i < j}, kept
// iff rank_j < k_r.  This makes ties go to the lower position and needs no sorting network.
#pragma once

#include "device_common.h"
#include "launch.h"

namespace focus {

__device__ __forceinline__ float wave_sum_all(float v) {
  v = wave_sum_xor(v, 32);
  v = wave_sum_xor(v, 16);
  v = wave_sum_xor(v, 8);
  v = wave_sum_xor(v, 4);
  v = wave_sum_xor(v, 2);
  v = wave_sum_xor(v, 1);
  return v;
}

struct Selection {
  bool kept;  // this lane's position is kept
  int k;      // the request's kept count
};

// Every lane of the wave must call this (lanes >= blk pass any dj).  Reads the request's mask
// (and budget) and returns the decision; stores nothing.
__device__ __forceinline__ Selection select_compute(const SelectArgs& a, int r, float dj,
                                                    int lane) {
  const int blk = a.blk;
  const bool in_blk = lane < blk;
  const bool mj = in_blk && a.masked[(size_t)r * blk + lane] != 0;
  const uint64_t mbits = __ballot(mj);
  const int m = __popcll(mbits);

  int b;
  if (a.adaptive) {
    const float inv_m = m > 0 ? 1.f / (float)m : 0.f;
    const float mu = wave_sum_all(mj ? dj : 0.f) * inv_m;
    const float dev = mj ? (dj - mu) : 0.f;
    const float sigma = sqrtf(wave_sum_all(dev * dev) * inv_m);
    const float thr = mu + a.beta * sigma;
    const int c = m > 0 ? __popcll(__ballot(mj && dj > thr)) : 0;
    b = min(max(c, a.lo), a.hi);
  } else {
    b = a.budget[r];
  }
  const int k = min(max(b, 0), m);

  int rank = 0;
  for (int i = 0; i < blk; ++i) {
    const float di = __shfl(dj, i, 64);
    const bool mi = (mbits >> i) & 1ull;
    rank += (mi && (di > dj || (di == dj && i < lane))) ? 1 : 0;
  }
  return Selection{mj && rank < k, k};
}

// Every lane of the wave must call this (lanes >= blk pass any dj).
__device__ __forceinline__ void select_request(const SelectArgs& a, int r, float dj, int lane) {
  const Selection sel = select_compute(a, r, dj, lane);
  if (lane < a.blk) a.keep[(size_t)r * a.blk + lane] = sel.kept ? 1 : 0;
  if (lane == 0) a.kept_count[r] = sel.k;
}

}  // namespace focus
