// Importance scoring: delta[r, j] = I_1[r, j] - I_0[r, j], where I_l[r, j] is the softmax mass
// block token j receives from all block queries and query heads of layer l (softmax over the
// block's keys).  Project page "FOCUS: DLLMs Know How to Tame Their Compute Bound", Overview
// cards "Design" and "Decodability Signal"; the paper's abstract (attention-derived importance).
//
// One workgroup per (request r, kv head g), 4 waves.  For each layer the K tile of kv head g
// and the Q tiles of GS of its query heads are staged in LDS with coalesced 16-byte loads, all
// issued before the LDS writes, with the next pass in flight.  A wave takes one (query head,
// 16-query tile) unit at a time and computes S^T = K Q^T (keys x queries) on MFMA, so a lane
// holds one query's scores for 4 keys of each 16-key tile: the row softmax over keys needs a
// local reduction plus two cross-lane steps, and the column sums accumulate in registers across
// units and both layers (layer 0 subtracts, layer 1 adds).  The 16 query lanes are summed once
// at the end, the 4 waves in LDS in a fixed order.  A second small kernel sums each request's
// Hkv partials in kv-head order (deterministic, no float atomics) and can run the request's
// selection right away.
//
// Front end with per-request budgets: workgroup 0 first scans the kept counts, known from the
// masks and budgets alone, into the compacted offsets (O(B)), which the reduction + selection +
// compaction kernel then reads.
#include "device_common.h"
#include "launch.h"
#include "compact_impl.h"

namespace focus {
namespace {

// One pass = one layer's K tile of kv head g plus the Q tiles of GS of its query heads.
template <typename T, int BLK, int D, int GS>
struct Pass {
  static constexpr int VEC = 16 / sizeof(T);         // elements per 16-byte chunk
  static constexpr int CH = D / VEC;                 // chunks per row
  static constexpr int CHUNKS = BLK * CH * (1 + GS); // K rows, then Q rows of GS heads
  static constexpr int PER_THREAD = (CHUNKS + 255) / 256;
  uint4 v[PER_THREAD];
};

template <typename T, int BLK, int D, int GS>
__device__ __forceinline__ void load_pass(Pass<T, BLK, D, GS>& ps, const T* Q, const T* K, int r,
                                          int g, int Hq, int Hkv, int G, int h0, int tid) {
  using PS = Pass<T, BLK, D, GS>;
#pragma unroll
  for (int u = 0; u < PS::PER_THREAD; ++u) {
    const int c = tid + 256 * u;
    if (PS::CHUNKS % 256 != 0 && c >= PS::CHUNKS) break;
    const T* src;
    if (c < BLK * PS::CH) {
      const int row = c / PS::CH, cc = c % PS::CH;
      src = K + ((size_t)(r * BLK + row) * Hkv + g) * D + cc * PS::VEC;
    } else {
      const int q = c - BLK * PS::CH;
      const int row = q / (GS * PS::CH), rem = q % (GS * PS::CH);
      const int hh = rem / PS::CH, cc = rem % PS::CH;
      src = Q + ((size_t)(r * BLK + row) * Hq + g * G + h0 + hh) * D + cc * PS::VEC;
    }
    ps.v[u] = load16(src);
  }
}

template <typename T, int BLK, int D, int GS>
__device__ __forceinline__ void store_pass(const Pass<T, BLK, D, GS>& ps, T* Ks, T* Qs, int tid) {
  using PS = Pass<T, BLK, D, GS>;
  constexpr int ROW = D + PS::VEC;
#pragma unroll
  for (int u = 0; u < PS::PER_THREAD; ++u) {
    const int c = tid + 256 * u;
    if (PS::CHUNKS % 256 != 0 && c >= PS::CHUNKS) break;
    T* dst;
    if (c < BLK * PS::CH) {
      const int row = c / PS::CH, cc = c % PS::CH;
      dst = Ks + row * ROW + cc * PS::VEC;
    } else {
      const int q = c - BLK * PS::CH;
      const int row = q / (GS * PS::CH), rem = q % (GS * PS::CH);
      const int hh = rem / PS::CH, cc = rem % PS::CH;
      dst = Qs + (row * GS + hh) * ROW + cc * PS::VEC;
    }
    *reinterpret_cast<uint4*>(dst) = ps.v[u];
  }
}

// Column sums of the row softmax of S^T = K Q^T for one (query head, 16-query tile) unit,
// accumulated into colacc with sign -1 (layer 0) or +1 (layer 1).  Block-only domain: the row is
// normalised over the BLK block keys.  Full domain (FULL): the row's log-sum-exp over prefix and
// block keys is given (row_lse_log2, in log2 units, for this lane's query), and the block keys'
// weights are exp2(z - row_lse_log2).
template <typename T, int BLK, int D, int GS, bool FULL>
__device__ __forceinline__ void score_unit(const T* Ks, const T* Qs, int hh, int nt, int n16,
                                           int j4, float scale_log2, float sign,
                                           float row_lse_log2, float (&colacc)[BLK / 16][4]) {
  constexpr int ES = sizeof(T);
  constexpr int ROW = D + 16 / ES;
  constexpr int NMT = BLK / 16;
  f32x4_t acc[NMT];
#pragma unroll
  for (int mt = 0; mt < NMT; ++mt) acc[mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const T* qrow = Qs + ((16 * nt + n16) * GS + hh) * ROW;
  if constexpr (ES == 2) {
    constexpr int NK = D / 32;
    u32x4_t qf[NK];
#pragma unroll
    for (int kk = 0; kk < NK; ++kk)
      qf[kk] = *reinterpret_cast<const u32x4_t*>(qrow + (4 * kk + j4) * 8);
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt) {
      const T* krow = Ks + (16 * mt + n16) * ROW;
#pragma unroll
      for (int kk = 0; kk < NK; ++kk) {
        const u32x4_t a = *reinterpret_cast<const u32x4_t*>(krow + (4 * kk + j4) * 8);
        acc[mt] = mfma_bf16(a, qf[kk], acc[mt]);
      }
    }
  } else {
    constexpr int NK = D / 4;
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt) {
      const T* krow = Ks + (16 * mt + n16) * ROW;
#pragma unroll 8
      for (int kk = 0; kk < NK; ++kk)
        acc[mt] = mfma_f32(krow[4 * kk + j4], qrow[4 * kk + j4], acc[mt]);
    }
  }
  // acc[mt][i] = S[key 16mt + 4*j4 + i][query 16nt + n16]
  if constexpr (FULL) {
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        colacc[mt][i] += sign * fast_exp2(acc[mt][i] * scale_log2 - row_lse_log2);
    return;
  }
  // softmax over all BLK keys
  float mx = -INFINITY;
#pragma unroll
  for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i) mx = fmaxf(mx, acc[mt][i]);
  mx = wave_max_xor(mx, 16);
  mx = wave_max_xor(mx, 32);
  float p[NMT][4];
  float sum = 0.f;
#pragma unroll
  for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      p[mt][i] = fast_exp2((acc[mt][i] - mx) * scale_log2);
      sum += p[mt][i];
    }
  sum = wave_sum_xor(sum, 16);
  sum = wave_sum_xor(sum, 32);
  const float w = sign / sum;
#pragma unroll
  for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i) colacc[mt][i] += p[mt][i] * w;
}

// Passes run (layer, head group) in order; the next pass's global loads are in flight (in
// registers) while the current one is computed from LDS.
template <typename T, int BLK, int D, int GS, bool FULL>
__global__ __launch_bounds__(256) void score_partial_kernel(const T* __restrict__ q0,
                                                            const T* __restrict__ k0,
                                                            const T* __restrict__ q1,
                                                            const T* __restrict__ k1, int Hq,
                                                            int Hkv, float scale_log2,
                                                            const float* __restrict__ lse0,
                                                            const float* __restrict__ lse1,
                                                            float* __restrict__ part,
                                                            int scan_offsets, SelectArgs sel,
                                                            int32_t* __restrict__ offsets) {
  extern __shared__ __align__(16) unsigned char smem[];
  constexpr int ROW = D + 16 / sizeof(T);
  constexpr int NMT = BLK / 16;
  T* Ks = reinterpret_cast<T*>(smem);               // [BLK][ROW]
  T* Qs = Ks + BLK * ROW;                            // [BLK][GS][ROW]
  float* red = reinterpret_cast<float*>(Qs + BLK * GS * ROW);  // [4][BLK]

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int n16 = lane & 15, j4 = lane >> 4;
  const int G = Hq / Hkv;
  const int r = blockIdx.x / Hkv, g = blockIdx.x % Hkv;
  const int groups = G / GS;        // head groups per layer
  const int npass = 2 * groups;

  float colacc[NMT][4];
#pragma unroll
  for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i) colacc[mt][i] = 0.f;

  if constexpr (!FULL) {
    if (scan_offsets && blockIdx.x == 0) {  // the scanning workgroup (LDS still free)
      scan_kept(gridDim.x / Hkv, [&](int rr) { return budget_kept<BLK>(sel, rr); },
                [&](int rr, int base, int k) {
                  offsets[rr + 1] = base + k;
                  if (rr == 0) offsets[0] = 0;
                },
                reinterpret_cast<int*>(smem));
    }
  }

  Pass<T, BLK, D, GS> ps;
  load_pass<T, BLK, D, GS>(ps, q0, k0, r, g, Hq, Hkv, G, 0, tid);
  for (int pi = 0; pi < npass; ++pi) {
    if (pi > 0) __syncthreads();  // every wave is done with the previous pass's tiles
    store_pass<T, BLK, D, GS>(ps, Ks, Qs, tid);
    __syncthreads();
    const int layer = pi / groups, h0 = (pi % groups) * GS;
    const float sign = layer ? 1.f : -1.f;
    // this wave's units of the pass: u = wave + 4k.  Full domain: their rows' log-sum-exps are
    // loaded before the next pass's tiles, since loads complete in issue order and a wait for
    // one issued after the prefetch would wait for the whole prefetch
    constexpr int NU = GS * NMT, UPW = (NU + 3) / 4;
    float row_lse_log2[UPW];
#pragma unroll
    for (int k = 0; k < UPW; ++k) {
      row_lse_log2[k] = 0.f;
      if constexpr (FULL) {
        const int u = min(wave + 4 * k, NU - 1), hh = u / NMT, nt = u % NMT;
        const float* lse = layer ? lse1 : lse0;  // [B, BLK, Hq], natural log
        row_lse_log2[k] = lse[((size_t)r * BLK + 16 * nt + n16) * Hq + g * G + h0 + hh];
      }
    }
    if (pi + 1 < npass) {
      const int nl = (pi + 1) / groups, nh = ((pi + 1) % groups) * GS;
      load_pass<T, BLK, D, GS>(ps, nl ? q1 : q0, nl ? k1 : k0, r, g, Hq, Hkv, G, nh, tid);
    }
#pragma unroll
    for (int k = 0; k < UPW; ++k) {
      const int u = wave + 4 * k;
      if (u >= NU) break;
      const int hh = u / NMT, nt = u % NMT;
      score_unit<T, BLK, D, GS, FULL>(Ks, Qs, hh, nt, n16, j4, scale_log2, sign,
                                      row_lse_log2[k] * kLog2e, colacc);
    }
  }

  // Sum over the 16 query lanes of each lane group, then over the 4 waves.
#pragma unroll
  for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float v = colacc[mt][i];
      v = wave_sum_xor(v, 1);
      v = wave_sum_xor(v, 2);
      v = wave_sum_xor(v, 4);
      v = wave_sum_xor(v, 8);
      if (n16 == 0) red[wave * BLK + 16 * mt + 4 * j4 + i] = v;
    }
  __syncthreads();
  if (tid < BLK)
    part[(size_t)blockIdx.x * BLK + tid] =
        ((red[tid] + red[BLK + tid]) + red[2 * BLK + tid]) + red[3 * BLK + tid];
}

// One wave per request: lane j sums the Hkv partials of position j in kv-head order (fixed
// order: deterministic), writes delta, and optionally runs the request's selection on it.
__global__ __launch_bounds__(256) void score_reduce_kernel(const float* __restrict__ part, int B,
                                                           int blk, int Hkv,
                                                           float* __restrict__ delta,
                                                           int fuse_select, SelectArgs sel) {
  const int lane = threadIdx.x & 63;
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= B) return;  // uniform per wave
  // the selection's inputs first, so that their round trip overlaps the partials'
  const SelectInputs in = fuse_select ? select_inputs(sel, r, lane) : SelectInputs{0, 0};
  float sum = 0.f;
  if (lane < blk) {
    const float* pr = part + (size_t)r * Hkv * blk + lane;
    // eight partials loaded before any is added (a loop adding each as it arrives waits for
    // every load in turn), then summed in head order
    for (int g0 = 0; g0 < Hkv; g0 += 8) {
      float v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = pr[(size_t)min(g0 + u, Hkv - 1) * blk];
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (g0 + u < Hkv) sum += v[u];
    }
    delta[(size_t)r * blk + lane] = sum;
  }
  if (fuse_select) select_request(sel, r, in, sum, lane);
}

template <typename T, int BLK, int D, int GS>
hipError_t launch_t(const ScoreArgs& a, hipStream_t s) {
  constexpr int ROW = D + 16 / sizeof(T);
  const size_t shmem = (size_t)BLK * (1 + GS) * ROW * sizeof(T) + 4 * BLK * sizeof(float);
  if (a.lse0 != nullptr)
    hipLaunchKernelGGL((score_partial_kernel<T, BLK, D, GS, true>), dim3(a.B * a.Hkv), dim3(256),
                       shmem, s, (const T*)a.q0, (const T*)a.k0, (const T*)a.q1, (const T*)a.k1,
                       a.Hq, a.Hkv, a.scale_log2, a.lse0, a.lse1, a.part, 0, a.sel, nullptr);
  else
    hipLaunchKernelGGL((score_partial_kernel<T, BLK, D, GS, false>), dim3(a.B * a.Hkv),
                       dim3(256), shmem, s, (const T*)a.q0, (const T*)a.k0, (const T*)a.q1,
                       (const T*)a.k1, a.Hq, a.Hkv, a.scale_log2, nullptr, nullptr, a.part,
                       a.scan_offsets, a.sel, a.offsets);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.partial_only) return e;
  hipLaunchKernelGGL(score_reduce_kernel, dim3((a.B + 3) / 4), dim3(256), 0, s, a.part, a.B,
                     a.blk, a.Hkv, a.delta, a.fuse_select, a.sel);
  return hipGetLastError();
}

// Heads staged per pass: as many of the G heads (at most 4) as keep one pass within ~54 KB of
// LDS, so that three workgroups share a CU.
template <typename T, int BLK, int D>
hipError_t launch_g(const ScoreArgs& a, hipStream_t s) {
  const int G = a.Hq / a.Hkv;
  constexpr size_t row = (size_t)(D + 16 / sizeof(T)) * sizeof(T);
  constexpr size_t budget = 54 * 1024;
  constexpr bool fit4 = (size_t)BLK * 5 * row <= budget;
  constexpr bool fit2 = (size_t)BLK * 3 * row <= budget;
  if (G >= 4 && fit4) return launch_t<T, BLK, D, 4>(a, s);
  if (G >= 2 && fit2) return launch_t<T, BLK, D, 2>(a, s);
  return launch_t<T, BLK, D, 1>(a, s);
}

template <typename T>
hipError_t launch_dt(const ScoreArgs& a, hipStream_t s) {
  if (a.d == 64) {
    if (a.blk == 16) return launch_g<T, 16, 64>(a, s);
    if (a.blk == 32) return launch_g<T, 32, 64>(a, s);
    return launch_g<T, 64, 64>(a, s);
  }
  if (a.blk == 16) return launch_g<T, 16, 128>(a, s);
  if (a.blk == 32) return launch_g<T, 32, 128>(a, s);
  return launch_g<T, 64, 128>(a, s);
}

}  // namespace

size_t score_workspace_bytes(int B, int blk, int Hkv) {
  return (size_t)B * Hkv * blk * sizeof(float);
}

hipError_t launch_score(const ScoreArgs& a, hipStream_t s) {
  if (a.is_bf16) return launch_dt<uint16_t>(a, s);
  return launch_dt<float>(a, s);
}

}  // namespace focus
