// Ragged paged attention of the kept queries over each request's paged prefix KV plus its
// intra-block KV.  AI Engineering Academy article on FOCUS, "Arquitetura do FOCUS" (ragged paged
// attention, KV-cache management); project page "FOCUS: DLLMs Know How to Tame Their Compute
// Bound", cards "Runtime Action" (ragged execution, intra-block KV caching) and "Motivation"
// (block diffusion: the prefix is exactly KV-cached, the block attends bidirectionally).
//
// Work item = (request r, kv head g, query group, key split).  The G query heads of kv head g
// are packed with the request's kept tokens into rows rho = t*G + hh (16 rows per MFMA tile,
// QT tiles per item), so one pass over the KV serves every query head that reads it.
//
// Each of the 4 waves streams its own 32-key tiles (tiles w, w+4, ... of the item) straight
// from HBM into MFMA operand registers, double buffered:
//   * K layout [page, Hkv, d/8, S, 8]: a lane's 16-byte load is 8 dims of one key, and the 16
//     lanes of a quarter-wave read 4 runs of 4 consecutive keys (64 B each).  The tile is the
//     A operand of S^T = K Q^T; key slot m of subtile s is key 8*(m/4) + 4*s + m%4, chosen so
//     that the result lane group j holds exactly keys 8j..8j+7 of the tile.
//   * V layout [page, Hkv, S/8, d, 8]: a lane's 16-byte load is one dim of 8 consecutive keys,
//     which is exactly the A operand of O^T = V^T P^T for lane group j; a quarter-wave reads 256
//     contiguous bytes.  P^T (bf16) comes straight from the S^T registers.
// Softmax is online in the exp2 domain (f32).  The 4 waves merge (max, sum, O) in LDS in a fixed
// order; items of long prefixes are split along the keys and merged by attn_combine_kernel, also
// in a fixed order, so results are bitwise reproducible.
#include "device_common.h"
#include "launch.h"

namespace focus {
namespace {

#ifndef FOCUS_ATTN_MAX_TILES_PER_SPLIT
#define FOCUS_ATTN_MAX_TILES_PER_SPLIT 32
#endif
constexpr int kWaves = 4;
constexpr int kMaxTilesPerSplit = FOCUS_ATTN_MAX_TILES_PER_SPLIT;  // 32-key tiles per work item

struct Params {
  const uint16_t* q;
  const int32_t* offsets;
  const uint16_t* k_cache;
  const uint16_t* v_cache;
  const int32_t* page_table;
  const int32_t* prefix_len;
  const uint16_t* k_blk;
  const uint16_t* v_blk;
  uint16_t* out;
  float* lse;
  float* ws_o;   // [slots][16*QT][D]
  float* ws_ml;  // [slots][2][16*QT]   (max in log2 units, sum)
  int cap, num_pages, max_pages, B, blk, Hq, Hkv, G, log2G, S, log2S, log2blk, max_kept;
  int tiles_split, nsplit_max, nqg;
  float scale_log2;
};

template <int D>
struct Tile {
  u32x4_t k[2][D / 32];
  u32x4_t v[D / 16];
};

// Loads tile `it` of the item's key sequence (prefix tiles first, then block tiles) into T.
// Branch-free, so the compiler can keep the next tile's loads in flight (it counts them): each
// lane's 8-key group is clamped to the group holding the segment's last valid key, which always
// lies in an allocated page, and the keys past the valid length are masked in compute_tile.  An
// out-of-range page id is replaced by page 0 and reported through `bad`.
template <int D>
__device__ __forceinline__ void load_tile(Tile<D>& T, const Params& p, int it, int ntp, int P,
                                          int r, int g, const int* s_pages, int pg0, int lane,
                                          bool& bad) {
  constexpr int NK = D / 32, ND = D / 16;
  const int m16 = lane & 15, j4 = lane >> 4;
  const bool paged = it < ntp;  // wave-uniform
  const int key0 = paged ? it * 32 : (it - ntp) * 32;
  const int nvalid = paged ? P : p.blk;
  const int log2S = paged ? p.log2S : p.log2blk;
  const int S = 1 << log2S;
  const size_t page_elems = (size_t)D << log2S;  // one (page, kv head) block
  const int last_group = (nvalid - 1) & ~7;

  // K: keys kg + (m16 & 3) + 4*s of the lane's 8-key group kg (s = 0, 1: the two subtiles)
  const int kg = min(key0 + 8 * (m16 >> 2), last_group);
  // V: the 8 keys vg .. vg+7 of lane group j4
  const int vg = min(key0 + 8 * j4, last_group);
  const uint16_t* kbase;
  const uint16_t* vbase;
  if (paged) {
    int pk = s_pages[(kg >> log2S) - pg0];
    int pv = s_pages[(vg >> log2S) - pg0];
    const bool okk = pk >= 0 && pk < p.num_pages, okv = pv >= 0 && pv < p.num_pages;
    bad = bad || !okk || !okv;
    pk = okk ? pk : 0;
    pv = okv ? pv : 0;
    kbase = p.k_cache + ((size_t)pk * p.Hkv + g) * page_elems;
    vbase = p.v_cache + ((size_t)pv * p.Hkv + g) * page_elems;
  } else {
    kbase = p.k_blk + ((size_t)r * p.Hkv + g) * page_elems;
    vbase = p.v_blk + ((size_t)r * p.Hkv + g) * page_elems;
  }
  const int kslot = (kg & (S - 1)) + (m16 & 3);
  const uint16_t* kp = kbase + ((size_t)((j4 << log2S) + kslot) << 3);
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int kk = 0; kk < NK; ++kk)
      T.k[s][kk] = load16v(kp + ((size_t)(((4 * kk) << log2S) + 4 * s) << 3));
  const uint16_t* vp = vbase + ((size_t)((vg & (S - 1)) >> 3) * D + m16) * 8;
#pragma unroll
  for (int dt = 0; dt < ND; ++dt) T.v[dt] = load16v(vp + 16 * dt * 8);
}

template <int D, int QT>
__device__ __forceinline__ void compute_tile(Tile<D>& T, int key0, int nvalid,
                                             const u32x4_t (&qf)[QT][D / 32],
                                             f32x4_t (&o)[QT][D / 16], float (&mrun)[QT],
                                             float (&lrun)[QT], float scale_log2, int lane) {
  constexpr int NK = D / 32, ND = D / 16;
  const int j4 = lane >> 4;
  const int kbase = key0 + 8 * j4;  // this lane group's 8 keys: kbase + 0..7
  // Values of keys past the end are zeroed: their weights are zero, but the loaded values may
  // be anything and 0 * NaN would not vanish.  Branch-free (all-ones masks on full tiles).
  const int nv = nvalid - kbase;
  u32x4_t vmask;
#pragma unroll
  for (int w = 0; w < 4; ++w)
    vmask[w] = (2 * w + 1 < nv) ? 0xffffffffu : ((2 * w < nv) ? 0x0000ffffu : 0u);
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    f32x4_t s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) {
      s0 = mfma_bf16(T.k[0][kk], qf[qt][kk], s0);
      s1 = mfma_bf16(T.k[1][kk], qf[qt][kk], s1);
    }
    float x[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[i] = s0[i] * scale_log2;
      x[4 + i] = s1[i] * scale_log2;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = (e < nv) ? x[e] : -INFINITY;
    float mx = x[0];
#pragma unroll
    for (int e = 1; e < 8; ++e) mx = fmaxf(mx, x[e]);
    mx = wave_max_xor(mx, 16);
    mx = wave_max_xor(mx, 32);
    const float mnew = fmaxf(mrun[qt], mx);
    float alpha = 1.f, msub = 0.f;
    if (mnew != -INFINITY) {
      alpha = fast_exp2(mrun[qt] - mnew);
      msub = mnew;
    }
    float pe[8];
    float ls = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      pe[e] = fast_exp2(x[e] - msub);
      ls += pe[e];
    }
    lrun[qt] = lrun[qt] * alpha + ls;
    mrun[qt] = mnew;
    u32x4_t pf;
    pf[0] = pack_bf16x2(pe[0], pe[1]);
    pf[1] = pack_bf16x2(pe[2], pe[3]);
    pf[2] = pack_bf16x2(pe[4], pe[5]);
    pf[3] = pack_bf16x2(pe[6], pe[7]);
#pragma unroll
    for (int dt = 0; dt < ND; ++dt) {
      o[qt][dt] *= alpha;
      o[qt][dt] = mfma_bf16(T.v[dt] & vmask, pf, o[qt][dt]);
    }
  }
}

template <int D, int QT>
__global__ __launch_bounds__(256, (QT >= 4 ? 1 : 2)) void attn_kernel(Params p) {
  constexpr int NK = D / 32, ND = D / 16, R = 16 * QT;
  constexpr int OROW = D + 4;  // padded LDS row (floats)
  constexpr int MAXPG = kMaxTilesPerSplit * 32 / 16 + 2;
  __shared__ __align__(16) float s_o[kWaves][16][OROW];
  __shared__ float s_m[kWaves][16];
  __shared__ float s_l[kWaves][16];
  __shared__ int s_pages[MAXPG];
  __shared__ int s_bad;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int m16 = lane & 15, j4 = lane >> 4;
  const int BH = p.B * p.Hkv;
  const int rg = blockIdx.x % BH, split = blockIdx.x / BH;
  const int r = rg / p.Hkv, g = rg % p.Hkv;
  const int qg = blockIdx.y;

  const int off0 = p.offsets[r], off1 = p.offsets[r + 1];
  const int kr = min(off1 - off0, p.max_kept);
  if (off0 < 0 || kr <= 0 || off0 >= p.cap) return;
  const int nrows = kr << p.log2G;
  const int row0 = qg * R;
  if (row0 >= nrows) return;
  int P = p.prefix_len[r];
  const bool bad_len = P < 0 || P > (p.max_pages << p.log2S);
  if (bad_len) P = 0;
  const int ntp = (P + 31) >> 5;
  const int nt = ntp + ((p.blk + 31) >> 5);
  const int nsplit = (nt + p.tiles_split - 1) / p.tiles_split;
  if (split >= nsplit) return;
  const int t0 = split * p.tiles_split;
  const int t1 = min(nt, t0 + p.tiles_split);

  // this split's page ids
  int pg0 = 0;
  if (tid == 0) s_bad = bad_len ? 1 : 0;
  if (t0 < ntp) {
    pg0 = (t0 * 32) >> p.log2S;
    const int pg1 = min((P - 1) >> p.log2S, ((min(t1, ntp) * 32 - 1) >> p.log2S)) + 1;
    for (int i = tid; i < pg1 - pg0; i += 256)
      s_pages[i] = p.page_table[(size_t)r * p.max_pages + pg0 + i];
  }
  __syncthreads();

  // queries of this item (B operand): lane (n = m16, j4) row rho = row0 + 16*qt + n
  u32x4_t qf[QT][NK];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const int rho = row0 + 16 * qt + m16;
    const int tok = off0 + (rho >> p.log2G);
    const bool valid = rho < nrows && tok < p.cap;
    const uint16_t* qrow =
        p.q + ((size_t)tok * p.Hq + g * p.G + (rho & (p.G - 1))) * D;
#pragma unroll
    for (int kk = 0; kk < NK; ++kk)
      qf[qt][kk] = valid ? load16v(qrow + (4 * kk + j4) * 8) : u32x4_t{0u, 0u, 0u, 0u};
  }

  f32x4_t o[QT][ND];
  float mrun[QT], lrun[QT];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    mrun[qt] = -INFINITY;
    lrun[qt] = 0.f;
#pragma unroll
    for (int dt = 0; dt < ND; ++dt) o[qt][dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }

  // Each wave streams tiles wave, wave+4, ... of [t0, t1), loading tile k+1 while it computes
  // tile k.  The prefetch is unconditional (after the wave's last tile it re-reads that tile, a
  // cache hit), so the wait before each compute only drains the older tile's loads.
  bool bad = false;
  Tile<D> ta, tb;
  const int nk = t0 + wave < t1 ? (t1 - t0 - wave + kWaves - 1) / kWaves : 0;
  auto tile_of = [&](int k) { return t0 + wave + kWaves * min(k, nk - 1); };
  static_assert(kMaxTilesPerSplit % (2 * kWaves) == 0, "tile loop unrolls by two buffers");
  auto seg_key0 = [&](int i) { return i < ntp ? i * 32 : (i - ntp) * 32; };
  auto seg_len = [&](int i) { return i < ntp ? P : p.blk; };
  if (nk > 0) {
    // fully unrolled (a wave takes at most kMaxTilesPerSplit / kWaves tiles of a split), so the
    // code is straight-line and the buffers alternate statically
    load_tile<D>(ta, p, tile_of(0), ntp, P, r, g, s_pages, pg0, lane, bad);
#pragma unroll
    for (int k = 0; k < kMaxTilesPerSplit / kWaves; k += 2) {
      load_tile<D>(tb, p, tile_of(k + 1), ntp, P, r, g, s_pages, pg0, lane, bad);
      __builtin_amdgcn_sched_barrier(0);  // keep the prefetch ahead of the compute
      int it = tile_of(k);
      compute_tile<D, QT>(ta, seg_key0(it), seg_len(it), qf, o, mrun, lrun, p.scale_log2, lane);
      if (k + 1 >= nk) break;
      load_tile<D>(ta, p, tile_of(k + 2), ntp, P, r, g, s_pages, pg0, lane, bad);
      __builtin_amdgcn_sched_barrier(0);
      it = tile_of(k + 1);
      compute_tile<D, QT>(tb, seg_key0(it), seg_len(it), qf, o, mrun, lrun, p.scale_log2, lane);
      if (k + 2 >= nk) break;
    }
  }

  // Merge the 4 waves (fixed order), one 16-row query tile at a time, and write the result or
  // this split's partial.
  const int slot = (rg * p.nsplit_max + split) * p.nqg + qg;
  constexpr int C4 = D / 4;
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    // per-wave totals: the 4 lane groups hold disjoint keys' partial sums
    float lt = wave_sum_xor(lrun[qt], 16);
    lt = wave_sum_xor(lt, 32);
    if (qt > 0) __syncthreads();  // the previous tile's readers are done
    if (j4 == 0) {
      s_m[wave][m16] = mrun[qt];
      s_l[wave][m16] = lt;
    }
#pragma unroll
    for (int dt = 0; dt < ND; ++dt)
      *reinterpret_cast<f32x4_t*>(&s_o[wave][m16][16 * dt + 4 * j4]) = o[qt][dt];
    if (bad) s_bad = 1;
    __syncthreads();
    const bool isbad = s_bad != 0;
    for (int item = tid; item < 16 * C4; item += 256) {
      const int rl = item / C4, c4 = item % C4;
      const int row = 16 * qt + rl;
      float M = s_m[0][rl];
#pragma unroll
      for (int w = 1; w < kWaves; ++w) M = fmaxf(M, s_m[w][rl]);
      float L = 0.f;
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float sc = s_m[w][rl] == -INFINITY ? 0.f : fast_exp2(s_m[w][rl] - M);
        L += s_l[w][rl] * sc;
        acc += *reinterpret_cast<const f32x4_t*>(&s_o[w][rl][4 * c4]) * sc;
      }
      const int rho = row0 + row;
      if (nsplit == 1) {
        const int tok = off0 + (rho >> p.log2G);
        if (rho >= nrows || tok >= p.cap) continue;
        const int h = g * p.G + (rho & (p.G - 1));
        const float inv = isbad ? __builtin_nanf("") : 1.f / L;
        uint2 w2;
        w2.x = pack_bf16x2(acc[0] * inv, acc[1] * inv);
        w2.y = pack_bf16x2(acc[2] * inv, acc[3] * inv);
        *reinterpret_cast<uint2*>(p.out + ((size_t)tok * p.Hq + h) * D + 4 * c4) = w2;
        if (c4 == 0 && p.lse != nullptr)
          p.lse[(size_t)tok * p.Hq + h] = isbad ? __builtin_nanf("") : (M + __log2f(L)) * kLn2;
      } else {
        if (isbad) {
          acc = f32x4_t{__builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""),
                        __builtin_nanf("")};
          L = __builtin_nanf("");
        }
        *reinterpret_cast<f32x4_t*>(p.ws_o + ((size_t)slot * R + row) * D + 4 * c4) = acc;
        if (c4 == 0) {
          p.ws_ml[((size_t)slot * 2) * R + row] = M;
          p.ws_ml[((size_t)slot * 2 + 1) * R + row] = L;
        }
      }
    }
  }
}

// Merges the key splits of every (request, kv head, query group) with more than one split.
template <int D, int QT>
__global__ __launch_bounds__(256) void attn_combine_kernel(Params p) {
  constexpr int R = 16 * QT, C4 = D / 4;
  const int tid = threadIdx.x;
  const int rg = blockIdx.x, qg = blockIdx.y;
  const int r = rg / p.Hkv, g = rg % p.Hkv;
  const int off0 = p.offsets[r], off1 = p.offsets[r + 1];
  const int kr = min(off1 - off0, p.max_kept);
  if (off0 < 0 || kr <= 0 || off0 >= p.cap) return;
  const int nrows = kr << p.log2G;
  const int row0 = qg * R;
  if (row0 >= nrows) return;
  int P = p.prefix_len[r];
  if (P < 0 || P > (p.max_pages << p.log2S)) P = 0;
  const int nt = ((P + 31) >> 5) + ((p.blk + 31) >> 5);
  const int nsplit = (nt + p.tiles_split - 1) / p.tiles_split;
  if (nsplit <= 1) return;
  for (int item = tid; item < R * C4; item += 256) {
    const int row = item / C4, c4 = item % C4;
    const int rho = row0 + row;
    const int tok = off0 + (rho >> p.log2G);
    if (rho >= nrows || tok >= p.cap) continue;
    float M = -INFINITY;
    for (int s = 0; s < nsplit; ++s) {
      const int slot = (rg * p.nsplit_max + s) * p.nqg + qg;
      M = fmaxf(M, p.ws_ml[((size_t)slot * 2) * R + row]);
    }
    float L = 0.f;
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    for (int s = 0; s < nsplit; ++s) {
      const int slot = (rg * p.nsplit_max + s) * p.nqg + qg;
      const float ms = p.ws_ml[((size_t)slot * 2) * R + row];
      const float sc = ms == -INFINITY ? 0.f : fast_exp2(ms - M);
      L += p.ws_ml[((size_t)slot * 2 + 1) * R + row] * sc;
      acc += *reinterpret_cast<const f32x4_t*>(p.ws_o + ((size_t)slot * R + row) * D + 4 * c4) *
             sc;
    }
    const int h = g * p.G + (rho & (p.G - 1));
    const float inv = 1.f / L;
    uint2 w2;
    w2.x = pack_bf16x2(acc[0] * inv, acc[1] * inv);
    w2.y = pack_bf16x2(acc[2] * inv, acc[3] * inv);
    *reinterpret_cast<uint2*>(p.out + ((size_t)tok * p.Hq + h) * D + 4 * c4) = w2;
    if (c4 == 0 && p.lse != nullptr) p.lse[(size_t)tok * p.Hq + h] = (M + __log2f(L)) * kLn2;
  }
}

int ilog2(int x) {
  int l = 0;
  while ((1 << l) < x) ++l;
  return l;
}

template <int D, int QT>
hipError_t launch_dq(const Params& prm, const AttnPlan& plan, hipStream_t s) {
  dim3 grid(prm.B * prm.Hkv * plan.nsplit_max, plan.nqg);
  hipLaunchKernelGGL((attn_kernel<D, QT>), grid, dim3(256), 0, s, prm);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || plan.nsplit_max <= 1) return e;
  hipLaunchKernelGGL((attn_combine_kernel<D, QT>), dim3(prm.B * prm.Hkv, plan.nqg), dim3(256), 0,
                     s, prm);
  return hipGetLastError();
}

}  // namespace

AttnPlan plan_attn(int B, int blk, int Hq, int Hkv, int d, int S, int max_pages, int max_kept) {
  AttnPlan pl{};
  const int G = Hq / Hkv;
  const int rows = max_kept * G;
  pl.qt = rows <= 16 ? 1 : (rows <= 32 ? 2 : 4);
  pl.nqg = (rows + 16 * pl.qt - 1) / (16 * pl.qt);
  const long long ntiles_max = ((long long)max_pages * S + 31) / 32 + (blk + 31) / 32;
  // Split the keys so that even a batch of maximal prefixes offers ~2048 work items.
  int ts = kMaxTilesPerSplit;
  while (ts > 8 && (long long)B * Hkv * pl.nqg * ((ntiles_max + ts - 1) / ts) < 2048) ts >>= 1;
  pl.tiles_split = ts;
  pl.nsplit_max = (int)((ntiles_max + ts - 1) / ts);
  if (pl.nsplit_max > 1) {
    const size_t slots = (size_t)B * Hkv * pl.nsplit_max * pl.nqg;
    const size_t R = 16 * (size_t)pl.qt;
    pl.ws_bytes = slots * R * (size_t)d * sizeof(float) + slots * 2 * R * sizeof(float);
  } else {
    pl.ws_bytes = 0;
  }
  return pl;
}

hipError_t launch_attn(const AttnArgs& a, const AttnPlan& plan, hipStream_t s) {
  Params prm{};
  prm.q = a.q;
  prm.offsets = a.offsets;
  prm.k_cache = a.k_cache;
  prm.v_cache = a.v_cache;
  prm.page_table = a.page_table;
  prm.prefix_len = a.prefix_len;
  prm.k_blk = a.k_blk;
  prm.v_blk = a.v_blk;
  prm.out = a.out;
  prm.lse = a.lse;
  prm.cap = a.cap;
  prm.num_pages = a.num_pages;
  prm.max_pages = a.max_pages;
  prm.B = a.B;
  prm.blk = a.blk;
  prm.Hq = a.Hq;
  prm.Hkv = a.Hkv;
  prm.G = a.Hq / a.Hkv;
  prm.log2G = ilog2(prm.G);
  prm.S = a.S;
  prm.log2S = ilog2(a.S);
  prm.log2blk = ilog2(a.blk);
  prm.max_kept = a.max_kept;
  prm.tiles_split = plan.tiles_split;
  prm.nsplit_max = plan.nsplit_max;
  prm.nqg = plan.nqg;
  prm.scale_log2 = a.scale_log2;
  if (plan.nsplit_max > 1) {
    const size_t slots = (size_t)a.B * a.Hkv * plan.nsplit_max * plan.nqg;
    const size_t R = 16 * (size_t)plan.qt;
    prm.ws_o = reinterpret_cast<float*>(a.workspace);
    prm.ws_ml = prm.ws_o + slots * R * a.d;
  }
  if (a.d == 64) {
    if (plan.qt == 1) return launch_dq<64, 1>(prm, plan, s);
    if (plan.qt == 2) return launch_dq<64, 2>(prm, plan, s);
    return launch_dq<64, 4>(prm, plan, s);
  }
  if (plan.qt == 1) return launch_dq<128, 1>(prm, plan, s);
  if (plan.qt == 2) return launch_dq<128, 2>(prm, plan, s);
  return launch_dq<128, 4>(prm, plan, s);
}

}  // namespace focus
