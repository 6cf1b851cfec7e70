// Importance scoring: delta[r, j] = I_1[r, j] - I_0[r, j], where I_l[r, j] is the softmax mass
// block token j receives from all block queries and query heads of layer l (softmax over the
// block's keys).  Project page "FOCUS: DLLMs Know How to Tame Their Compute Bound", Overview
// cards "Design" and "Decodability Signal"; the paper's abstract (attention-derived importance).
//
// Kernel 1 (score_partial): one workgroup per (request r, kv head g), 4 waves.  For each layer
// the K tile of kv head g and the Q tiles of up to HS of its query heads are staged in LDS with
// coalesced 16-byte loads.  A wave takes one (query head, 16-query tile) unit at a time and
// computes S^T = K Q^T (keys x queries) on MFMA, so a lane holds one query's scores for 4 keys
// of each 16-key tile: the row softmax over keys needs a local reduction plus two cross-lane
// steps, and the column sums accumulate in registers across units and both layers (layer 0
// subtracts, layer 1 adds).  The 16 query lanes are summed once at the end, the 4 waves in LDS
// in a fixed order.  Kernel 2 (score_reduce) sums the Hkv partials in kv-head order.
#include "device_common.h"
#include "launch.h"

namespace focus {
namespace {

template <typename T, int BLK, int D>
__global__ __launch_bounds__(256) void score_partial_kernel(const T* __restrict__ q0,
                                                            const T* __restrict__ k0,
                                                            const T* __restrict__ q1,
                                                            const T* __restrict__ k1, int Hq,
                                                            int Hkv, int HS, float scale_log2,
                                                            float* __restrict__ part) {
  extern __shared__ __align__(16) unsigned char smem[];
  constexpr int ES = sizeof(T);
  constexpr int VEC = 16 / ES;        // elements per 16-byte chunk
  constexpr int ROW = D + VEC;        // padded LDS row (elements)
  constexpr int CH = D / VEC;         // 16-byte chunks per row
  constexpr int NMT = BLK / 16;       // 16-key (and 16-query) tiles
  T* Ks = reinterpret_cast<T*>(smem);           // [BLK][ROW]
  T* Qs = Ks + BLK * ROW;                       // [BLK][HS][ROW]
  float* red = reinterpret_cast<float*>(Qs + BLK * HS * ROW);  // [4][BLK]

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int n16 = lane & 15, j4 = lane >> 4;
  const int G = Hq / Hkv;
  const int r = blockIdx.x / Hkv, g = blockIdx.x % Hkv;

  float colacc[NMT][4];
#pragma unroll
  for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i) colacc[mt][i] = 0.f;

  for (int layer = 0; layer < 2; ++layer) {
    const T* Q = layer ? q1 : q0;
    const T* K = layer ? k1 : k0;
    const float sign = layer ? 1.f : -1.f;
    for (int h0 = 0; h0 < G; h0 += HS) {
      const int hs = min(HS, G - h0);
      __syncthreads();  // the previous stage's readers are done
      for (int c = tid; c < BLK * CH; c += 256) {
        const int row = c / CH, cc = c % CH;
        const T* src = K + ((size_t)(r * BLK + row) * Hkv + g) * D + cc * VEC;
        *reinterpret_cast<uint4*>(Ks + row * ROW + cc * VEC) = load16(src);
      }
      for (int c = tid; c < BLK * hs * CH; c += 256) {
        const int row = c / (hs * CH), rem = c % (hs * CH);
        const int hh = rem / CH, cc = rem % CH;
        const T* src = Q + ((size_t)(r * BLK + row) * Hq + g * G + h0 + hh) * D + cc * VEC;
        *reinterpret_cast<uint4*>(Qs + (row * HS + hh) * ROW + cc * VEC) = load16(src);
      }
      __syncthreads();

      for (int u = wave; u < hs * NMT; u += 4) {
        const int hh = u / NMT, nt = u % NMT;
        f32x4_t acc[NMT];
#pragma unroll
        for (int mt = 0; mt < NMT; ++mt) acc[mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        const T* qrow = Qs + ((16 * nt + n16) * HS + hh) * ROW;
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
        // acc[mt][i] = S[key 16mt + 4*j4 + i][query 16nt + n16]; softmax over all BLK keys.
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

__global__ __launch_bounds__(256) void score_reduce_kernel(const float* __restrict__ part, int B,
                                                           int blk, int Hkv,
                                                           float* __restrict__ delta) {
  const int idx = blockIdx.x * 256 + threadIdx.x;
  if (idx >= B * blk) return;
  const int r = idx / blk, j = idx % blk;
  const float* p = part + (size_t)r * Hkv * blk + j;
  float s = 0.f;
  for (int g = 0; g < Hkv; ++g) s += p[(size_t)g * blk];
  delta[idx] = s;
}

template <typename T, int BLK, int D>
hipError_t launch_t(const ScoreArgs& a, hipStream_t s) {
  constexpr int ES = sizeof(T);
  constexpr int ROW = D + 16 / ES;
  const int G = a.Hq / a.Hkv;
  // heads staged per pass: as many as fit in 96 KB of LDS, at most 4
  int HS = G < 4 ? G : 4;
  auto lds = [&](int hs) { return (size_t)(BLK + BLK * hs) * ROW * ES + 4 * BLK * sizeof(float); };
  while (HS > 1 && lds(HS) > 96 * 1024) HS >>= 1;
  const size_t shmem = lds(HS);
  hipLaunchKernelGGL((score_partial_kernel<T, BLK, D>), dim3(a.B * a.Hkv), dim3(256), shmem, s,
                     (const T*)a.q0, (const T*)a.k0, (const T*)a.q1, (const T*)a.k1, a.Hq, a.Hkv,
                     HS, a.scale_log2, a.part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(score_reduce_kernel, dim3((a.B * a.blk + 255) / 256), dim3(256), 0, s,
                     a.part, a.B, a.blk, a.Hkv, a.delta);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_dt(const ScoreArgs& a, hipStream_t s) {
  if (a.d == 64) {
    if (a.blk == 16) return launch_t<T, 16, 64>(a, s);
    if (a.blk == 32) return launch_t<T, 32, 64>(a, s);
    return launch_t<T, 64, 64>(a, s);
  }
  if (a.blk == 16) return launch_t<T, 16, 128>(a, s);
  if (a.blk == 32) return launch_t<T, 32, 128>(a, s);
  return launch_t<T, 64, 128>(a, s);
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
