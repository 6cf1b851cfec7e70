// Ragged paged attention of the kept queries over each request's paged prefix KV plus its
// intra-block KV.  AI Engineering Academy article on FOCUS, "Arquitetura do FOCUS" (ragged paged
// attention, KV-cache management); project page "FOCUS: DLLMs Know How to Tame Their Compute
// Bound", cards "Runtime Action" (ragged execution, intra-block KV caching) and "Motivation"
// (block diffusion: the prefix is exactly KV-cached, the block attends bidirectionally).
//
// Work decomposition.  An item is (request r, kv head g, query group qg): the G query heads of
// kv head g are packed with the request's kept tokens into rows rho = t*G + hh, 16*QT rows per
// query group, so one pass over a head's KV serves all its query heads.  An item's keys are
// streamed as 32-key tiles (columns), the prefix tiles first, then the block tiles.  The columns
// of all requests form one global list.
//
// Column groups.  The grid is persistent, one 4-wave workgroup per CU (two for shared tiles and
// for the 32- and 64-row tiles without the output, as far as the LDS holds them all at once:
// the staged metadata grows with the batch), its waves in groups of Hkv*nqg, one wave per
// (kv head, query group).  Group i takes the i-th of equal contiguous slices
// of the column list, so the waves of a group stream the same pages of the same requests at the
// same time, each its own kv head's part of the page: every page is read by all its heads
// together, which keeps the DRAM accesses local wherever the slices fall.  A wave streams its
// columns with the next tile's loads in flight while it computes the current one, crossing
// request boundaries (page ids come from scalar loads that mostly hit the scalar cache; a new
// item's queries are loaded as it starts).  A wave that holds a whole item writes its output
// directly.  An item cut by slice boundaries has one piece per group it overlaps; the pieces
// meet through an arrival counter: a piece that is not the last to finish stores its partial
// (running max, sum, unnormalised O) and arrives; the last one merges every piece in key order
// (its own from registers) and writes the output.  The piece at the end of a slice usually
// finishes last, and sees that before storing anything.  Partials and counters use device-scope
// atomic accesses, which stay coherent across the XCDs' separate L2 caches without an L2
// write-back.  Every group does the same amount of streaming, so no wave waits for another.
//
// Register operands straight from HBM (no LDS):
//   * K pages [page, Hkv, d/8, S, 8]: a lane's 16-byte load is 8 dims of one key; the tile is the
//     A operand of S^T = K Q^T, key slot m of subtile s being key 16s + m (whole 256-byte runs
//     per load instruction).
//   * V pages [page, Hkv, S/8, d, 8]: a lane's two 8-byte loads are one dim of the two 4-key
//     runs its S^T lane group holds, which is exactly the A operand of O^T = V^T P^T for that
//     lane group; P^T (bf16) comes straight from the S^T registers.
// Shared tiles.  Items of 33..64 rows, and of more with the output, take all four waves of a
// workgroup, one 16- or 32-row query group each, on the same kv head (one workgroup per 128
// rows): the workgroup loads each tile once (every thread loads a 1/256 share straight into a
// ring of four LDS tile buffers, three tiles ahead, one barrier per tile), and each wave reads
// the MFMA fragments above from LDS -- the keys, then, after its scores, the values into the
// same registers.
// Queries.  Either compacted rows [cap, Hq, d] (row n is the n-th kept token), or, in the POS
// instantiations, the block's query tensor [B, blk, Hq, d] read in place at the kept positions
// (row n of request r is q[r, q_pos[n]]): the same operands, without a gather beforehand.
// Softmax is online in the exp2 domain (f32).  Merges run in a fixed order, so results are
// bitwise reproducible.
#include <algorithm>

#include "device_common.h"
#include "launch.h"

namespace focus {
namespace {

constexpr int kWaves = 4;  // waves per workgroup
// Tile buffers per wave (NB - 1 tiles in flight during a compute) and workgroups per CU for one
// query tile per item.  Measured on MI355X: one wave per SIMD with one tile in flight streams
// faster than two waves per SIMD or deeper prefetch; fewer concurrent streams keep the DRAM
// accesses more local, and the CU's outstanding misses are the limit, not the wave count.
constexpr int kPrefetchQt1 = 2;
constexpr int kWgsPerCuQt1 = 1;
// Shared tiles: tiles on their way into LDS per workgroup (ahead of the one computed), and
// workgroups per CU.  (Shared waves read a tile's key fragments from LDS, compute every query
// tile's scores, then read the value fragments into the same registers: the two are never live
// together.)
constexpr int kShPrefetch = 3;     // 16-row waves
constexpr int kShPrefetchQt2 = 3;  // 32-row waves
constexpr int kShWgsPerCu = 2;     // 32-row waves
constexpr int kShWgsPerCuQt1 = 2;  // 16-row waves
// LDS per CU (gfx950); the planner caps the workgroups per CU so that they are all resident
constexpr size_t kLdsPerCu = 160 * 1024;
// the most workgroups per CU of any mode (the log-sum-exp-only one-wave kernels take two)
constexpr int kMaxWgsPerCu = std::max({2, kWgsPerCuQt1, kShWgsPerCu, kShWgsPerCuQt1});
// cache-policy bits of a vector memory access with device scope (SC1): stores write through to
// the device-coherent level, loads read from it (what device-scope atomics use on gfx950)
constexpr int kCpolDevice = 16;
// third word of a raw (unswizzled, 32-bit format) buffer resource
constexpr int kRawBufferFormat = 0x00020000;
// how far (log2 units) a row's logits may exceed its reference max before the running output
// is rescaled: softmax weights stay below 2^8
constexpr float kRescaleSlack = 8.f;
// pieces of a cut item merged with all their loads in flight together (more go one by one)
constexpr int kMaxMerge = 8;
// the grid shrinks for small problems so that each wave streams at least this many tiles
constexpr int kMinTilesPerWave = 12;

struct Params {
  const uint16_t* q;       // [cap, Hq, d] compacted rows, or [B, blk, Hq, d] with q_pos
  const int32_t* q_pos;    // null, or [cap]: row n of request r is q[r, q_pos[n]]
  const int32_t* offsets;
  const uint16_t* k_cache;
  const uint16_t* v_cache;
  const int32_t* page_table;
  const int32_t* prefix_len;
  const uint16_t* k_blk;
  const uint16_t* v_blk;
  uint16_t* out;
  float* lse;
  float* ws_o;     // [2W][QT][D/16][64 lanes][4] partial O (unnormalised), in register order
  int ws_o_bytes;  // its size (the buffer-access range)
  float* ws_ml;    // [2W][2][16*QT] partial running max (log2 units) and sum
  int* counters;   // [W] arrivals per cut item, indexed by the item's first group and wave slot;
                   // zero between calls (the last arrival resets it)
  int cap, num_pages, max_pages, B, blk, Hq, Hkv, G, log2G, S, log2S, log2blk, max_kept, nqg;
  int W;           // waves in the grid
  int gs;          // waves per column group (Hkv * nqg)
  int ngroups;     // column groups (W / gs; waves beyond ngroups * gs stay idle)
  float scale_log2;
};

__device__ __forceinline__ int uni(int x) { return __builtin_amdgcn_readfirstlane(x); }

template <int X>
constexpr int kLog2() {
  static_assert(X > 0 && (X & (X - 1)) == 0, "power of two");
  int l = 0;
  while ((1 << l) < X) ++l;
  return l;
}

template <int D>
struct Tile {
  u32x4_t k[2][D / 32];
  u32x4_t v[D / 16];
  bool bad;  // a page id of the tile was out of range (page 0 was read instead)
};

// Per-request metadata staged in LDS by every workgroup.
struct Meta {
  int* cum;   // [B+1] exclusive prefix sums of the requests' column counts
  int* P;     // [B] prefix length, -1 if out of range (the request's rows become NaN)
  int* off;   // [B] first compacted row
  int* rows;  // [B] kept rows * G (0: request has no work)
};

// Position in the global column list (all fields wave-uniform).  Tile counts are derived from
// the prefix length on demand to keep the scalar state small.  A wave's kv head and query group
// never change.
struct Cursor {
  int r, g, qg, tt;  // request, kv head, query group, tile within the item
  int P;             // prefix length of r, -1 if out of range (the item's rows become NaN)
  int off0, nrows;   // first compacted row of r, its kept rows * G
  int start;         // global index of the request's first column
  __device__ __forceinline__ int plen() const { return P < 0 ? 0 : P; }
  __device__ __forceinline__ int ntp() const { return (plen() + 31) >> 5; }
};

__device__ __forceinline__ int item_tiles(const Cursor& c, const Params& p) {
  return c.ntp() + ((p.blk + 31) >> 5);
}

__device__ __forceinline__ void set_request(Cursor& c, int r, const Meta& m) {
  c.r = r;
  c.P = uni(m.P[r]);
  c.off0 = uni(m.off[r]);
  c.nrows = uni(m.rows[r]);
}

__device__ __forceinline__ void advance(Cursor& c, const Meta& m, const Params& p) {
  const int nt = item_tiles(c, p);
  if (++c.tt < nt) return;
  c.start += nt;
  c.tt = 0;
  int r = c.r + 1;
  while (r < p.B - 1 && uni(m.cum[r + 1]) == uni(m.cum[r])) ++r;
  set_request(c, r, m);
}

// Page ids of the (at most two) pages a prefix tile touches, as scalar loads (consecutive tiles
// share the page table's cache lines).
struct Pages {
  int a, b;
};
// Branch-free (indices clamped into the request's row; a block tile reads its row's first entry
// and ignores it), so that the loads can be issued at the start of a step, ahead of the work
// that does not need them.  A table without columns (max_pages == 0) is never read.
__device__ __forceinline__ Pages fetch_pages(const Cursor& c, const Params& p,
                                             const int32_t* __restrict__ page_table) {
  Pages pg{0, 0};
  if (p.max_pages > 0) {
    const int last = max((c.plen() - 1) >> p.log2S, 0);
    const int p0 = min((c.tt * 32) >> p.log2S, last);
    const int32_t* row = page_table + (size_t)c.r * p.max_pages;
    pg.a = row[p0];
    pg.b = row[min(p0 + 1, last)];
  }
  return pg;
}

// Loads the cursor's tile.  Key slot m of K subtile s is key 16s + m, so each K load
// instruction reads 16 consecutive keys of one 8-dim group: whole 256-byte runs.  The S^T
// result lane group j then holds keys 4j..4j+3 (subtile 0) and 16+4j..16+4j+3 (subtile 1), and
// the V operand of that lane group is loaded as the same two 4-key runs (8 bytes each; a load
// instruction again covers whole 256-byte runs).  Branch-free: keys are clamped to the last
// valid key (runs to the last valid run), which lie in allocated pages; keys past the valid
// length are masked in compute_tile.  An out-of-range page id is replaced by page 0 and
// reported in T.bad.
template <int D, bool WO>
__device__ __forceinline__ void load_tile(Tile<D>& T, const Cursor& c, Pages pg, const Params& p,
                                          int lane) {
  constexpr int NK = D / 32, ND = D / 16;
  const int m16 = lane & 15, j4 = lane >> 4;
  const int ntp = c.ntp();
  const bool paged = c.tt < ntp;
  const int key0 = paged ? c.tt * 32 : (c.tt - ntp) * 32;
  const int nvalid = paged ? c.plen() : p.blk;
  const int log2S = paged ? p.log2S : p.log2blk;
  const int S = 1 << log2S;
  const int last = nvalid - 1, last_run = last & ~3;
  // Base addresses of the (at most two) (page, kv head) blocks the tile touches, computed once
  // per tile with wave-uniform (scalar) arithmetic; a lane then picks one of two bases.  A tile
  // of 32 keys starts at a multiple of 32, so with S >= 32 (and in the block) it lies in one
  // block: only S = 16 uses the second.
  const int blk_shift = kLog2<D>() + log2S;  // log2 of one (page, kv head) block's elements
  const uint16_t *k0p, *k1p, *v0p, *v1p;
  bool bad = false;
  if (paged) {
    int a = pg.a, b = pg.b;
    const bool oka = a >= 0 && a < p.num_pages, okb = b >= 0 && b < p.num_pages;
    bad = !oka || !okb;
    a = oka ? a : 0;
    b = okb ? b : 0;
    // (page, kv head) block index times the block size, a power of two: a 32-bit index and
    // one 64-bit shift (page ids are below num_pages, so the index fits)
    const size_t oa = (size_t)(uint32_t)(a * p.Hkv + c.g) << blk_shift;
    const size_t ob = (size_t)(uint32_t)(b * p.Hkv + c.g) << blk_shift;
    k0p = p.k_cache + oa;
    k1p = p.k_cache + ob;
    v0p = p.v_cache + oa;
    v1p = p.v_cache + ob;
  } else {
    const size_t o = (size_t)(uint32_t)(c.r * p.Hkv + c.g) << blk_shift;
    k0p = k1p = p.k_blk + o;
    v0p = v1p = p.v_blk + o;
  }
  const int p0 = key0 >> log2S;
  const bool two = paged && S < 32;
  T.bad = bad;
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const int kkey = min(key0 + 16 * s + m16, last);
    const uint16_t* kb = (two && (kkey >> log2S) != p0) ? k1p : k0p;
    const uint16_t* kp = kb + ((uint32_t)((j4 << log2S) + (kkey & (S - 1))) << 3);
#pragma unroll
    for (int kk = 0; kk < NK; ++kk)
      T.k[s][kk] = load16_stream(kp + ((uint32_t)((4 * kk) << log2S) << 3));
  }
  if constexpr (!WO) return;  // log-sum-exp only: no values
  const uint16_t* vp[2];
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const int vrun = min(key0 + 16 * s + 4 * j4, last_run);
    const uint16_t* vb = (two && (vrun >> log2S) != p0) ? v1p : v0p;
    vp[s] = vb + ((uint32_t)((vrun & (S - 1)) >> 3) * D + m16) * 8 + (vrun & 4);
  }
#pragma unroll
  for (int dt = 0; dt < ND; ++dt) {
    const u32x2_t lo = load8_stream(vp[0] + 16 * dt * 8);
    const u32x2_t hi = load8_stream(vp[1] + 16 * dt * 8);
    T.v[dt] = u32x4_t{lo[0], lo[1], hi[0], hi[1]};
  }
}

// Shared tiles.  When an item's rows need several query groups, the four waves of a workgroup
// are four query groups of the same kv head: they stream the same tiles, so the workgroup loads
// each tile once.  Every thread loads a 1/256 share of a tile (D/64 chunks of 16 bytes of K and
// as many of V) straight into an LDS tile buffer (no registers), NB tiles ahead of use; one
// barrier per tile, and each wave reads its MFMA fragments from LDS.
// Tile buffer layout (16-byte chunks): K chunk (dim group c, key k) at c*32 + k, then V chunk
// (key group q, dim e) at 4*D + q*D + e -- the global layouts restricted to the tile's 32 keys.
// Thread t's chunk u is chunk 256u + t, so each wave's loads fill 64 consecutive chunks.

// cache-policy bits of a load of data read exactly once (non-temporal)
constexpr int kCpolNontemporal = 2;

// 16 bytes per lane from global memory straight into LDS (global_load_lds_dwordx4): lane l
// writes bytes [16l, 16l + 16) after the wave-uniform LDS address dst.  Completion is counted
// by the wave's vector memory counter like any load.
__device__ __forceinline__ void load16_to_lds(const void* src, u32x4_t* dst) {
  __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)src,
                                   (__attribute__((address_space(3))) void*)dst, 16, 0,
                                   kCpolNontemporal);
}

// s_waitcnt immediate with vmcnt = n (0..63) and the other counters at their maxima
constexpr int wait_vmcnt_imm(int n) { return 0x0F70 | (n & 15) | ((n >> 4) << 14); }

// Issues this thread's share of the cursor's tile into tile buffer buf, branch-free and clamped
// like load_tile: K chunks of keys past the valid length hold the last valid key, V chunks of
// key groups past it hold the last valid group (compute_tile masks both).  Returns whether a
// page id of the tile was out of range (page 0 is read instead).  Loads per thread: D/64 for
// K, as many for V with the output.
template <int D, bool WO>
__device__ __forceinline__ bool issue_share(const Cursor& c, Pages pg, const Params& p, int tid,
                                            u32x4_t* buf) {
  constexpr int NC = D / 64;
  const int ntp = c.ntp();
  const bool paged = c.tt < ntp;
  const int key0 = paged ? c.tt * 32 : (c.tt - ntp) * 32;
  const int nvalid = paged ? c.plen() : p.blk;
  const int log2S = paged ? p.log2S : p.log2blk;
  const int S = 1 << log2S;
  const int last = nvalid - 1;
  const int blk_shift = kLog2<D>() + log2S;  // log2 of one (page, kv head) block's elements
  const uint16_t *k0p, *k1p, *v0p, *v1p;
  bool bad = false;
  if (paged) {
    int a = pg.a, b = pg.b;
    const bool oka = a >= 0 && a < p.num_pages, okb = b >= 0 && b < p.num_pages;
    bad = !oka || !okb;
    a = oka ? a : 0;
    b = okb ? b : 0;
    // (page, kv head) block index times the block size, a power of two: a 32-bit index and
    // one 64-bit shift (page ids are below num_pages, so the index fits)
    const size_t oa = (size_t)(uint32_t)(a * p.Hkv + c.g) << blk_shift;
    const size_t ob = (size_t)(uint32_t)(b * p.Hkv + c.g) << blk_shift;
    k0p = p.k_cache + oa;
    k1p = p.k_cache + ob;
    v0p = p.v_cache + oa;
    v1p = p.v_cache + ob;
  } else {
    const size_t o = (size_t)(uint32_t)(c.r * p.Hkv + c.g) << blk_shift;
    k0p = k1p = p.k_blk + o;
    v0p = v1p = p.v_blk + o;
  }
  const int p0 = key0 >> log2S;
  const bool two = paged && S < 32;
  u32x4_t* dst = buf + uni(tid & ~63);  // this wave's 64 chunks
#pragma unroll
  for (int u = 0; u < NC; ++u) {
    const int i = tid + 256 * u;
    const int key = min(key0 + (i & 31), last);
    const uint16_t* kb = (two && (key >> log2S) != p0) ? k1p : k0p;
    load16_to_lds(kb + ((uint32_t)(((i >> 5) << log2S) + (key & (S - 1))) << 3), dst + 256 * u);
  }
  if constexpr (WO) {
#pragma unroll
    for (int u = 0; u < NC; ++u) {
      const int j = tid + 256 * u;
      const int grp = min(key0 + 8 * (j / D), last & ~7);
      const uint16_t* vb = (two && (grp >> log2S) != p0) ? v1p : v0p;
      load16_to_lds(vb + ((uint32_t)(((grp & (S - 1)) >> 3) * D + (j & (D - 1))) << 3),
                    dst + 4 * D + 256 * u);
    }
  }
  return bad;
}

// The wave's MFMA fragments of a tile from its LDS buffer, the registers load_tile fills: the
// key fragments (read_tile_k), the value fragments (read_tile_v).
template <int D>
__device__ __forceinline__ void read_tile_k(Tile<D>& T, const u32x4_t* buf, int lane) {
  constexpr int NK = D / 32;
  const int m16 = lane & 15, j4 = lane >> 4;
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) T.k[s][kk] = buf[(4 * kk + j4) * 32 + 16 * s + m16];
}
template <int D>
__device__ __forceinline__ void read_tile_v(Tile<D>& T, const u32x4_t* buf, int lane) {
  constexpr int ND = D / 16;
  const int m16 = lane & 15, j4 = lane >> 4;
  const u32x2_t* v8 = reinterpret_cast<const u32x2_t*>(buf + 4 * D);
#pragma unroll
  for (int dt = 0; dt < ND; ++dt) {
    const u32x2_t lo = v8[((j4 >> 1) * D + 16 * dt + m16) * 2 + (j4 & 1)];
    const u32x2_t hi = v8[((2 + (j4 >> 1)) * D + 16 * dt + m16) * 2 + (j4 & 1)];
    T.v[dt] = u32x4_t{lo[0], lo[1], hi[0], hi[1]};
  }
}
// Workgroup barrier for the LDS tile ring: this wave's LDS writes are complete, and the
// compiler moves no memory access across it (no wait on the vector memory loads in flight).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(kWaitLgkmcnt0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// The B operand (Q^T) of the current item.  With up to two query tiles it lives in registers;
// with four (64 rows) it lives in the wave's slice of LDS, which keeps the QT = 4 kernel within
// its registers (o alone takes 128, the two tile buffers another 128).
template <int D, int QT>
struct QOperand {
  static constexpr int NK = D / 32;
  static constexpr bool kLds = QT >= 4;
  u32x4_t r[kLds ? 1 : QT][kLds ? 1 : NK];
  u32x4_t* lds;  // [QT][NK][64 lanes] when kLds
  __device__ __forceinline__ u32x4_t get(int qt, int kk, int lane) const {
    if constexpr (kLds)
      return lds[(qt * NK + kk) * 64 + lane];
    else
      return r[qt][kk];
  }
};

// The kept positions of the cursor's query rows (one per query tile and lane; row rho is
// token rho / G of the item), when the queries are read in place (POS); issued ahead of the
// row loads so that their round trip can overlap others (the page ids of the first tile).
template <int QT>
struct QPos {
  int j[QT];
};
template <int QT, bool POS>
__device__ __forceinline__ QPos<QT> fetch_qpos(const Cursor& c, const Params& p, int lane) {
  constexpr int R = 16 * QT;
  QPos<QT> q;
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    q.j[qt] = 0;
    if constexpr (POS) {
      const int rho = min(c.qg * R + 16 * qt + (lane & 15), c.nrows - 1);
      q.j[qt] = p.q_pos[min(c.off0 + (rho >> p.log2G), p.cap - 1)];
    }
  }
  return q;
}

// Loads the Q operand of the cursor's item.  Rows past the item's rows (or past cap) are
// clamped to a valid row: their results are never written, and finite inputs keep them finite.
// POS: the rows are read where they are, at the kept positions qp of the request's block
// (q is [B, blk, Hq, d]); a position outside the block reads position 0 and is reported (true:
// the item's rows become NaN).  Otherwise q holds the compacted rows and qp is not used.
template <int D, int QT, bool POS>
__device__ __forceinline__ bool load_q_at(QOperand<D, QT>& qf, const Cursor& c, const Params& p,
                                          int lane, const QPos<QT>& qp) {
  constexpr int NK = D / 32, R = 16 * QT;
  const int m16 = lane & 15, j4 = lane >> 4;
  bool bad = false;
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const int rho = min(c.qg * R + 16 * qt + m16, c.nrows - 1);
    int src = min(c.off0 + (rho >> p.log2G), p.cap - 1);
    if constexpr (POS) {
      const bool out = (unsigned)qp.j[qt] >= (unsigned)p.blk;
      bad = bad || out;
      src = c.r * p.blk + (out ? 0 : qp.j[qt]);
    }
    const uint16_t* qrow =
        p.q + ((size_t)src * p.Hq + c.g * p.G + (rho & (p.G - 1))) * D + 8 * j4;
    if constexpr (QOperand<D, QT>::kLds) {
      u32x4_t t[NK];
#pragma unroll
      for (int kk = 0; kk < NK; ++kk) t[kk] = load16v(qrow + 32 * kk);
#pragma unroll
      for (int kk = 0; kk < NK; ++kk) qf.lds[(qt * NK + kk) * 64 + lane] = t[kk];
    } else {
#pragma unroll
      for (int kk = 0; kk < NK; ++kk) qf.r[qt][kk] = load16v(qrow + 32 * kk);
    }
  }
  return bad;
}

template <int D, int QT, bool POS>
__device__ __forceinline__ bool load_q(QOperand<D, QT>& qf, const Cursor& c, const Params& p,
                                       int lane) {
  return load_q_at<D, QT, POS>(qf, c, p, lane, fetch_qpos<QT, POS>(c, p, lane));
}

// Scores of one query tile from its Q^T fragments: S^T (32 keys x 16 rows) as two 16-key
// subtiles.
template <int D>
__device__ __forceinline__ void tile_scores_q(const Tile<D>& T, const u32x4_t (&q)[D / 32],
                                              f32x4_t& s0, f32x4_t& s1) {
  constexpr int NK = D / 32;
  s0 = f32x4_t{0.f, 0.f, 0.f, 0.f};
  s1 = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kk = 0; kk < NK; ++kk) {
    s0 = mfma_bf16(T.k[0][kk], q[kk], s0);
    s1 = mfma_bf16(T.k[1][kk], q[kk], s1);
  }
}

// Scores of query tile qt.
template <int D, int QT>
__device__ __forceinline__ void tile_scores(const Tile<D>& T, const QOperand<D, QT>& qf, int qt,
                                            int lane, f32x4_t& s0, f32x4_t& s1) {
  constexpr int NK = D / 32;
  u32x4_t q[NK];
#pragma unroll
  for (int kk = 0; kk < NK; ++kk) q[kk] = qf.get(qt, kk, lane);
  tile_scores_q<D>(T, q, s0, s1);
}

// One 32-key tile for every query tile of the wave.  Online softmax in the exp2 domain against
// a reference max per row that moves only when a key's logit exceeds it by more than
// kRescaleSlack: that test is lane-local (no cross-lane step), and only when some lane finds
// such a key does the wave take the rows' maxima across lanes and rescale o and l (always on
// the first tile of a piece, whose reference is -inf).  Otherwise the weights exp2(x - m) stay
// below 2^kRescaleSlack, which the fp32 sums and bf16 weights hold without loss, and o is
// touched by the matrix unit only.  With up to two query tiles the scores of tile qt+1 are issued
// before the softmax of tile qt, so the matrix unit works while the vector unit does.  WO = false:
// log-sum-exp only
// (no values, no output accumulation).
// nq (wave-uniform): query tiles of this item's query group that hold rows.  With four query
// tiles per wave the others are padding and are skipped (their m, l and O stay at the initial
// -inf, 0, 0, are never written out and weigh zero in a merge), and a group without rows
// computes nothing: 16-token blocks, whose items mostly fill one of the four tiles, 171 -> 153
// us.  With two the check measured slower (the pair's scores are issued together).
// AHEAD (up to two query tiles): the next query tile's scores are issued before this one's
// softmax; off where registers are short (shared tiles with two query tiles per wave).
// SPLIT (shared tiles): T holds only the key fragments; the scores of every query tile are
// computed first, then the value fragments are read from the LDS buffer vbuf into the same
// registers, so keys and values are never live together.
template <int D, int QT, bool WO, bool AHEAD = true, bool SPLIT = false>
__device__ __forceinline__ void compute_tile(Tile<D>& T, int key0, int nvalid, int nq,
                                             const QOperand<D, QT>& qf,
                                             f32x4_t (&o)[QT][D / 16], float (&mrun)[QT],
                                             float (&lrun)[QT], float scale_log2, int lane,
                                             const u32x4_t* vbuf = nullptr) {
  constexpr int ND = D / 16;
  if (QT > 2 && nq <= 0) return;
  const int j4 = lane >> 4;
  // this lane group's 8 keys: slots 0..3 are keys key0 + 4j + (0..3), slots 4..7 are keys
  // key0 + 16 + 4j + (0..3); nv[r] = valid keys of run r
  const int nv[2] = {nvalid - (key0 + 4 * j4), nvalid - (key0 + 16 + 4 * j4)};
  const bool full = key0 + 32 <= nvalid;  // wave-uniform: only the last tile of a range is short
  auto mask_values = [&]() {
    // Values of keys past the end are zeroed: their weights are zero, but the loaded values
    // may be anything and 0 * NaN would not vanish.
    u32x4_t vmask;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const int n = nv[w >> 1], b = 2 * (w & 1);
      vmask[w] = (b + 1 < n) ? 0xffffffffu : ((b < n) ? 0x0000ffffu : 0u);
    }
#pragma unroll
    for (int dt = 0; dt < ND; ++dt) T.v[dt] &= vmask;
  };
  f32x4_t scs[SPLIT ? QT : 1][2];
  if constexpr (SPLIT) {
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) tile_scores<D, QT>(T, qf, qt, lane, scs[qt][0], scs[qt][1]);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (WO) {
      read_tile_v<D>(T, vbuf, lane);
      if (!full) mask_values();
    }
  } else if (WO && !full) {
    mask_values();
  }
  const float inv_scale = 1.f / scale_log2;
  f32x4_t sc[2][2];
  // four query tiles without the output (registers to spare): the next query tile's Q^T
  // fragments are read from LDS one iteration ahead, so the score products do not wait for
  // LDS (with the output the extra registers cost more than the waits)
  constexpr int NK = D / 32;
  constexpr bool kQAhead = QT >= 4 && !WO;
  u32x4_t qfr[2][NK];  // fragments of the query tiles of parity 0 and 1
  if constexpr (SPLIT) {
  } else if constexpr (kQAhead) {
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) qfr[0][kk] = qf.get(0, kk, lane);
    tile_scores_q<D>(T, qfr[0], sc[0][0], sc[0][1]);
  } else {
    tile_scores<D, QT>(T, qf, 0, lane, sc[0][0], sc[0][1]);
  }
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    // with four query tiles, one iteration at a time: otherwise the scheduler hoists every
    // tile's operand reads and keeps them live, which no longer fits the registers
    if (QT > 2) __builtin_amdgcn_sched_barrier(0);
    if (QT > 2 && qt > 0 && qt >= nq) break;
    const int cur = qt & 1;
    // up to two query tiles: the next tile's scores are issued ahead; with four the extra
    // registers would spill, so each tile's scores are computed at its turn
    if (!SPLIT && AHEAD && QT < 4 && qt + 1 < QT)
      tile_scores<D, QT>(T, qf, qt + 1, lane, sc[cur ^ 1][0], sc[cur ^ 1][1]);
    if constexpr (SPLIT) {
      sc[cur][0] = scs[qt][0];
      sc[cur][1] = scs[qt][1];
    } else if constexpr (kQAhead) {
      if (qt > 0) tile_scores_q<D>(T, qfr[cur], sc[cur][0], sc[cur][1]);
      if (qt + 1 < QT && qt + 1 < nq) {
#pragma unroll
        for (int kk = 0; kk < NK; ++kk) qfr[cur ^ 1][kk] = qf.get(qt + 1, kk, lane);
      }
    } else if ((QT >= 4 || !AHEAD) && qt > 0) {
      tile_scores<D, QT>(T, qf, qt, lane, sc[cur][0], sc[cur][1]);
    }
    float s[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      s[i] = sc[cur][0][i];
      s[4 + i] = sc[cur][1][i];
    }
    // Lane-local test against the reference on the raw scores (scale_log2 > 0).  Slots past the
    // end of a short tile hold the score of the last valid key (their keys are clamped to it),
    // so they need no masking here: they neither raise the row max nor change the test.
    float smax = fmaxf(fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3])),
                       fmaxf(fmaxf(s[4], s[5]), fmaxf(s[6], s[7])));
    if (__ballot(smax > (mrun[qt] + kRescaleSlack) * inv_scale) != 0) {
      float mx = smax * scale_log2;
      mx = wave_max_xor(mx, 16);
      mx = wave_max_xor(mx, 32);
      const float mnew = fmaxf(mrun[qt], mx);
      const float alpha =
          mnew == -INFINITY || mrun[qt] == -INFINITY ? 0.f : fast_exp2(mrun[qt] - mnew);
      lrun[qt] *= alpha;
      if constexpr (WO) {
#pragma unroll
        for (int dt = 0; dt < ND; ++dt) o[qt][dt] *= alpha;
      }
      mrun[qt] = mnew;
    }
    const float msub = mrun[qt] == -INFINITY ? 0.f : mrun[qt];
    float pe[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) pe[e] = fast_exp2(__builtin_fmaf(s[e], scale_log2, -msub));
    if (!full) {  // slots past the end weigh nothing
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if ((e & 3) >= nv[e >> 2]) pe[e] = 0.f;
    }
    float ls = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) ls += pe[e];
    lrun[qt] += ls;
    if constexpr (!WO) continue;
    u32x4_t pf;
    pf[0] = pack_bf16x2(pe[0], pe[1]);
    pf[1] = pack_bf16x2(pe[2], pe[3]);
    pf[2] = pack_bf16x2(pe[4], pe[5]);
    pf[3] = pack_bf16x2(pe[6], pe[7]);
#pragma unroll
    for (int dt = 0; dt < ND; ++dt) o[qt][dt] = mfma_bf16(T.v[dt], pf, o[qt][dt]);
  }
}

// Workgroup b runs on XCD b mod 8 (round-robin dispatch).  A column group of gs waves spans
// gs/4 workgroups; they are placed on one XCD (consecutive groups alternate XCDs), which
// measured ~1-3% faster than groups split across two XCDs.  Identity where the grid does not
// divide evenly.
__device__ __forceinline__ int logical_wg(int b, int nwg, int gs) {
  constexpr int kXcds = 8;
  const int m = gs / kWaves;  // workgroups per group
  if (m < 2 || gs % kWaves != 0 || nwg % kXcds != 0 || (nwg / kXcds) % m != 0) return b;
  const int xcd = b % kXcds, k = b / kXcds;
  return ((k / m) * kXcds + xcd) * m + k % m;
}

// Column group whose slice holds column t: the largest i with floor(i*T/n) <= t.
__device__ __forceinline__ int group_of(int t, int total, int n) {
  return (int)(((long long)(t + 1) * n - 1) / total);
}
__device__ __forceinline__ int slice_begin(int i, int total, int n) {
  return (int)(((long long)i * total) / n);
}

// page_table is a separate restrict argument so that its (uniform) reads become scalar loads.
// SH: shared tiles (the workgroup's four waves are four query groups of one kv head; NB is then
// the number of tiles whose shares are in flight in registers).
template <int D, int QT, int NB, bool WO, bool SH, bool POS>
__global__ __launch_bounds__(256, SH ? (QT == 1 ? kShWgsPerCuQt1 : kShWgsPerCu)
                                     : ((NB == 2 && QT == 1) ? 2 : 1)) void attn_kernel(
    Params p, const int32_t* __restrict__ page_table) {
  constexpr int NK = D / 32, ND = D / 16, R = 16 * QT;
  extern __shared__ __align__(16) int smem_i[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = uni(tid >> 6);
  const int m16 = lane & 15, j4 = lane >> 4;
  const int B = p.B;

  // ---- stage the requests' metadata and tile counts in LDS (every workgroup does this)
  Meta meta;
  meta.cum = smem_i;
  meta.P = smem_i + (B + 1);
  meta.off = meta.P + B;
  meta.rows = meta.off + B;
  int* s_part = meta.rows + B;  // [256]
  // per-wave Q operand (QT = 4 only), 16-byte aligned after the metadata
  unsigned char* s_q = reinterpret_cast<unsigned char*>(smem_i) +
                       ((((size_t)4 * B + 1 + 256) * sizeof(int) + 15) & ~(size_t)15);
  const int per = (B + 255) / 256;
  int local = 0;
  for (int i = 0; i < per; ++i) {
    const int r = tid * per + i;
    if (r >= B) break;
    const int off0 = p.offsets[r], off1 = p.offsets[r + 1];
    int P = p.prefix_len[r];
    const int kr = min(off1 - off0, p.max_kept);
    const bool has = off0 >= 0 && kr > 0 && off0 < p.cap;
    const int nrows = has ? kr << p.log2G : 0;
    const bool badP = P < 0 || P > (p.max_pages << p.log2S);
    meta.P[r] = badP ? -1 : P;
    meta.off[r] = off0;
    meta.rows[r] = nrows;
    if (badP) P = 0;
    const int nt = ((P + 31) >> 5) + ((p.blk + 31) >> 5);
    const int tiles = has ? nt : 0;
    meta.cum[r + 1] = tiles;
    local += tiles;
  }
  s_part[tid] = local;
  __syncthreads();
  if (tid < 64) {  // exclusive scan of the 256 partial sums by wave 0
    int v[4], s = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[i] = s_part[4 * tid + i];
      s += v[i];
    }
    int incl = s;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int y = __shfl_up(incl, d, 64);
      if (lane >= d) incl += y;
    }
    int run = incl - s;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      s_part[4 * tid + i] = run;
      run += v[i];
    }
  }
  __syncthreads();
  {
    int run = s_part[tid];
    for (int i = 0; i < per; ++i) {
      const int r = tid * per + i;
      if (r >= B) break;
      run += meta.cum[r + 1];
      meta.cum[r + 1] = run;
    }
    if (tid == 0) meta.cum[0] = 0;
  }
  __syncthreads();

  // ---- this wave's group, and the group's slice [a, b) of the global column list
  const int total = uni(meta.cum[B]);
  const int w = logical_wg(blockIdx.x, gridDim.x, p.gs) * kWaves + wave;
  const int gi = w / p.gs, hi = w - gi * p.gs;
  const int a = slice_begin(gi, total, p.ngroups);
  const int b = slice_begin(gi + 1, total, p.ngroups);
  if (gi >= p.ngroups || a >= b) return;

  // largest r with cum[r] <= col (requests without columns are skipped by the search)
  // (cum is non-decreasing, so each ballot below is a prefix of the lanes: two LDS reads per
  // lane instead of a chain of log2(B) dependent ones)
  auto locate = [&](int col) {
    const int s = (B + 63) >> 6;  // requests per lane in the first round
    if (s <= 64) {
      const int i1 = lane * s;
      const uint64_t m1 = __ballot(i1 < B && meta.cum[min(i1, B - 1)] <= col);
      const int base = (__popcll(m1) - 1) * s;  // lane 0 always holds: cum[0] = 0 <= col
      const int i2 = base + lane;
      const uint64_t m2 = __ballot(lane < s && i2 < B && meta.cum[min(i2, B - 1)] <= col);
      return uni(base + __popcll(m2) - 1);
    }
    int lo = 0, hi_r = B;
    while (hi_r - lo > 1) {
      const int mid = (lo + hi_r) >> 1;
      if (uni(meta.cum[mid]) <= col)
        lo = mid;
      else
        hi_r = mid;
    }
    return lo;
  };
  // The slice is processed rotated: first [x, b), where x is the start of the request holding
  // the slice's last column (or a), then [a, x).  So both pieces that may be cut at the slice
  // boundaries come first and their merges happen while the other waves still stream, instead
  // of at the end of the kernel.
  Cursor Ca;
  {
    const int r = locate(a);
    set_request(Ca, r, meta);
    Ca.g = hi / p.nqg;
    Ca.qg = hi - Ca.g * p.nqg;
    Ca.start = uni(meta.cum[r]);
    Ca.tt = a - Ca.start;
  }
  Cursor C = Ca;
  int x = a;
  {
    const int r = locate(b - 1);
    const int sb = uni(meta.cum[r]);
    if (sb > a) {
      x = sb;
      set_request(C, r, meta);
      C.start = sb;
      C.tt = 0;
    }
  }
  const int n = b - a, n1 = b - x;  // tiles in the slice, in the first segment

  f32x4_t o[QT][ND];
  float mrun[QT], lrun[QT];
  auto reset = [&]() {
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      mrun[qt] = -INFINITY;
      lrun[qt] = 0.f;
#pragma unroll
      for (int dt = 0; dt < ND; ++dt) o[qt][dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
  };
  reset();

  // Writes the finished piece of item c: the output itself if the slice holds the whole item,
  // else the piece takes part in the item's arrival protocol.
  auto finalize = [&](const Cursor& c, bool piece_bad) {
    float lt[QT];
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      lt[qt] = wave_sum_xor(lrun[qt], 16);
      lt[qt] = wave_sum_xor(lt[qt], 32);
    }
    const int end = c.start + item_tiles(c, p);
    // a bad page id seen by any lane taints every row (the products mix all lanes)
    const bool nan_out = __ballot(piece_bad) != 0 || c.P < 0;
    auto write_out = [&](int qt, const f32x4_t (&acc)[ND], float m, float l) {
      const int rho = c.qg * R + 16 * qt + m16;
      const int tok = c.off0 + (rho >> p.log2G);
      if (rho < c.nrows && tok < p.cap) {
        const int h = c.g * p.G + (rho & (p.G - 1));
        if constexpr (WO) {
          const float inv = nan_out ? __builtin_nanf("") : 1.f / l;
          uint16_t* orow = p.out + ((size_t)tok * p.Hq + h) * D + 4 * j4;
#pragma unroll
          for (int dt = 0; dt < ND; ++dt) {
            uint2 w2;
            w2.x = pack_bf16x2(acc[dt][0] * inv, acc[dt][1] * inv);
            w2.y = pack_bf16x2(acc[dt][2] * inv, acc[dt][3] * inv);
            *reinterpret_cast<uint2*>(orow + 16 * dt) = w2;
          }
        }
        if (j4 == 0 && p.lse != nullptr)
          p.lse[(size_t)tok * p.Hq + h] = nan_out ? __builtin_nanf("") : (m + __log2f(l)) * kLn2;
      }
    };
    if (a <= c.start && end <= b) {
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) write_out(qt, o[qt], mrun[qt], lt[qt]);
      return;
    }
    if (c.qg * R >= c.nrows) return;  // the request has no rows in this query group
    // pieces of the item in key order: the group holding the item's first column, then the
    // groups whose slices start inside it; the counter belongs to the first group's wave slot
    const int gf = group_of(c.start, total, p.ngroups);
    int* counter = p.counters + gf * p.gs + hi;
    int npieces = 0;
    for (int tp = c.start; tp < end; tp = slice_begin(group_of(tp, total, p.ngroups) + 1, total,
                                                       p.ngroups))
      ++npieces;
    const int own_slot = a > c.start ? 2 * w : 2 * w + 1;
    // partial O through buffer accesses with device scope (write-through, coherent reads): each
    // instruction moves 1 KiB of one (slot, query tile, 16-dim block) in lane order
    const __amdgpu_buffer_rsrc_t rs_o =
        __builtin_amdgcn_make_buffer_rsrc(p.ws_o, 0, p.ws_o_bytes, kRawBufferFormat);
    auto o_off = [&](int slot, int qt, int dt) {
      return (((slot * QT + qt) * ND + dt) * 64 + lane) * 16;
    };
    int seen = 0;
    if (lane == 0) seen = __hip_atomic_load(counter, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    bool last = uni(seen) == npieces - 1;
    if (!last) {
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) {
        const int row = 16 * qt + m16;
        if constexpr (WO) {
#pragma unroll
          for (int dt = 0; dt < ND; ++dt)
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, o[qt][dt]), rs_o,
                                                   o_off(own_slot, qt, dt), 0, kCpolDevice);
        }
        if (j4 == 0) {
          __hip_atomic_store(p.ws_ml + ((size_t)own_slot * 2) * R + row, mrun[qt],
                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          __hip_atomic_store(p.ws_ml + ((size_t)own_slot * 2 + 1) * R + row,
                             nan_out ? __builtin_nanf("") : lt[qt], __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
        }
      }
      // the partial must be complete at device scope before the arrival is counted: the
      // compiler may not move the increment above the wait, and the wait returns only once
      // every store of this wave has been acknowledged by the device-coherent level
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      int old = 0;
      if (lane == 0)
        old = __hip_atomic_fetch_add(counter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      last = uni(old) == npieces - 1;
    }
    // The merge's loads may not be hoisted above the counter value that selects this wave:
    // issued after it has returned, device-scope loads see every partial whose arrival it
    // counts (each was complete at that level before its increment).
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    if (!last) return;
    // last arrival: merge every piece in key order (own piece from registers), then reset the
    // counter for the next call.  The same operations whether a piece comes from registers or
    // from memory, so the result does not depend on which piece arrived last.  Up to
    // kMaxMerge pieces, their slots are found once, every piece's max and sum loads are issued
    // together, and piece k+1's partial O is loaded while piece k is accumulated (no chain of
    // dependent round trips); items cut into more pieces take them one by one.
    // (32-row tiles only: the 16-row kernel is held to 256 registers and its items are long,
    // and the 64-row kernels are short of registers; those merge piece by piece)
    constexpr int MM = kMaxMerge;
    if (QT == 2 && !SH && npieces <= MM) {
      int slot[MM];
      {
        int tp = c.start;
#pragma unroll
        for (int k = 0; k < MM; ++k) {
          slot[k] = own_slot;
          if (k < npieces) {
            const int gv = group_of(tp, total, p.ngroups);
            slot[k] = tp == c.start ? 2 * (gv * p.gs + hi) + 1 : 2 * (gv * p.gs + hi);
            tp = slice_begin(gv + 1, total, p.ngroups);
          }
        }
      }
      auto fetch_o = [&](int sl, int qt, f32x4_t (&dst)[ND]) {
        if (sl == own_slot) return;
#pragma unroll
        for (int dt = 0; dt < ND; ++dt)
          dst[dt] = __builtin_bit_cast(
              f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rs_o, o_off(sl, qt, dt), 0,
                                                             kCpolDevice));
      };
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) {
        const int row = 16 * qt + m16;
        float ms[MM], ls[MM];
#pragma unroll
        for (int k = 0; k < MM; ++k) {
          ms[k] = -INFINITY;
          ls[k] = 0.f;
          if (k < npieces) {
            if (slot[k] == own_slot) {
              ms[k] = mrun[qt];
              ls[k] = nan_out ? __builtin_nanf("") : lt[qt];
            } else {
              ms[k] = __hip_atomic_load(p.ws_ml + ((size_t)slot[k] * 2) * R + row,
                                        __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
              ls[k] = __hip_atomic_load(p.ws_ml + ((size_t)slot[k] * 2 + 1) * R + row,
                                        __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
          }
        }
        f32x4_t ob[2][ND];
        if constexpr (WO) fetch_o(slot[0], qt, ob[0]);
        float M = -INFINITY;
#pragma unroll
        for (int k = 0; k < MM; ++k)
          if (k < npieces) M = fmaxf(M, ms[k]);
        float L = 0.f;
        f32x4_t acc[ND];
#pragma unroll
        for (int dt = 0; dt < ND; ++dt) acc[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int k = 0; k < MM; ++k) {
          if (k < npieces) {
            if constexpr (WO) {
              if (k + 1 < npieces) fetch_o(slot[k + 1], qt, ob[(k + 1) & 1]);
            }
            const float sc = ms[k] == -INFINITY ? 0.f : fast_exp2(ms[k] - M);
            L = __builtin_fmaf(ls[k], sc, L);
            if constexpr (WO) {
              const bool own = slot[k] == own_slot;
#pragma unroll
              for (int dt = 0; dt < ND; ++dt) {
                const f32x4_t v = own ? o[qt][dt] : ob[k & 1][dt];
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[dt][i] = __builtin_fmaf(v[i], sc, acc[dt][i]);
              }
            }
          }
        }
        write_out(qt, acc, M, L);
      }
      if (lane == 0) __hip_atomic_store(counter, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      return;
    }
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      const int row = 16 * qt + m16;
      float M = -INFINITY;
      for (int tp = c.start; tp < end;) {
        const int gv = group_of(tp, total, p.ngroups);
        const int sl = tp == c.start ? 2 * (gv * p.gs + hi) + 1 : 2 * (gv * p.gs + hi);
        tp = slice_begin(gv + 1, total, p.ngroups);
        const float ms = sl == own_slot ? mrun[qt]
                                        : __hip_atomic_load(p.ws_ml + ((size_t)sl * 2) * R + row,
                                                            __ATOMIC_RELAXED,
                                                            __HIP_MEMORY_SCOPE_AGENT);
        M = fmaxf(M, ms);
      }
      float L = 0.f;
      f32x4_t acc[ND];
#pragma unroll
      for (int dt = 0; dt < ND; ++dt) acc[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      for (int tp = c.start; tp < end;) {
        const int gv = group_of(tp, total, p.ngroups);
        const int sl = tp == c.start ? 2 * (gv * p.gs + hi) + 1 : 2 * (gv * p.gs + hi);
        tp = slice_begin(gv + 1, total, p.ngroups);
        // the same operations whether a piece comes from registers or from memory, so the
        // result does not depend on which piece arrived last
        const bool own = sl == own_slot;
        float ms, ls;
        if (own) {
          ms = mrun[qt];
          ls = nan_out ? __builtin_nanf("") : lt[qt];
        } else {
          ms = __hip_atomic_load(p.ws_ml + ((size_t)sl * 2) * R + row, __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_AGENT);
          ls = __hip_atomic_load(p.ws_ml + ((size_t)sl * 2 + 1) * R + row, __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_AGENT);
        }
        const float sc = ms == -INFINITY ? 0.f : fast_exp2(ms - M);
        L = __builtin_fmaf(ls, sc, L);
        if constexpr (WO) {
#pragma unroll
        for (int dt = 0; dt < ND; ++dt) {
          const f32x4_t v =
              own ? o[qt][dt]
                  : __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                                                    rs_o, o_off(sl, qt, dt), 0, kCpolDevice));
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[dt][i] = __builtin_fmaf(v[i], sc, acc[dt][i]);
        }
        }
      }
      write_out(qt, acc, M, L);
    }
    if (lane == 0) __hip_atomic_store(counter, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  };
  // ---- stream: compute tile tv (cursor C) from buffer tv % NB while the next NB-1 tiles
  // (up to cursor L) are in flight; tv counts tiles in processing order.  Past the slice end L
  // stays on the last tile, so the prefetch is unconditional (it re-reads that tile: cache
  // hits).  When C starts a piece its queries are loaded before the next prefetch, so the
  // compute's wait does not drain the tiles in flight.
  QOperand<D, QT> qf;
  if constexpr (QOperand<D, QT>::kLds)
    qf.lds = reinterpret_cast<u32x4_t*>(s_q) + (size_t)wave * QT * NK * 64;
  // POS: the first piece's query positions and its first tile's page ids are requested
  // together, then its query rows (a second round trip that overlaps the first tile's)
  const QPos<QT> qp0 = fetch_qpos<QT, POS>(C, p, lane);
  Pages pg0{0, 0};
  if constexpr (POS) pg0 = fetch_pages(C, p, page_table);
  bool qbad = load_q_at<D, QT, POS>(qf, C, p, lane, qp0);  // the item's rows read a bad position
  Cursor L = C;
  int tvl = 0, tvc = 0;  // processing indices of L and C
  auto next = [&](Cursor& c, int& idx) {
    if (idx + 1 == n1)
      c = Ca;
    else
      advance(c, meta, p);
    ++idx;
  };
  bool bad = false;
  if constexpr (SH) {
    // ---- shared tiles: tiles tv+1 .. tv+NB-1 are on their way into LDS while tile tv is
    // computed from buffer tv % (NB+1).  At step tv every thread waits for its own share of
    // tile tv (its loads complete in issue order: only the NB-1 later tiles' may be pending),
    // the barrier then makes every share of tile tv visible, and the share of tile tv+NB is
    // issued into the buffer of tile tv-1, which every wave finished before this barrier.  All
    // four waves take the same steps.
    constexpr int NBUF = NB + 1;
    constexpr int CH = 8 * D;                     // 16-byte chunks per tile buffer (K, then V)
    constexpr int NL = (WO ? 2 : 1) * (D / 64);   // loads per thread and tile
    u32x4_t* ring = reinterpret_cast<u32x4_t*>(s_q);
    int badbits = 0;  // bit i: the tile in buffer i read an invalid page id
#pragma unroll
    for (int k = 0; k < NB; ++k) {
      if (k > 0 && tvl + 1 < n) next(L, tvl);
      const bool b = issue_share<D, WO>(L, (POS && k == 0) ? pg0 : fetch_pages(L, p, page_table),
                                        p, tid, ring + (size_t)k * CH);
      badbits |= (b ? 1 : 0) << k;
    }
    if (tvl + 1 < n) next(L, tvl);
    int tv = 0;
    auto sh_step = [&](int rb) {  // rb = tv % NBUF
      const bool live = tv < n;
      const Pages pg = fetch_pages(L, p, page_table);  // in flight during the wait
      if (live && tv > 0 && (C.tt == 0 || tv == n1)) {
        // a new piece's queries: the newest loads, so waiting for them waits for every tile
        // in flight too (the alternative, a wait at each use, would drain every step)
        qbad = load_q<D, QT, POS>(qf, C, p, lane);
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
      }
      __builtin_amdgcn_s_waitcnt(wait_vmcnt_imm((NB - 1) * NL));
      lds_barrier();
      const int wb = (rb + NB) % NBUF;  // the buffer of tile tv-1
      const bool b = issue_share<D, WO>(L, pg, p, tid, ring + (size_t)wb * CH);
      badbits = (badbits & ~(1 << wb)) | ((b ? 1 : 0) << wb);
      if (live) {
        const int nq = (C.nrows - C.qg * R + 15) >> 4;
        if (nq > 0) {
          Tile<D> X;
          const int ntp = C.ntp();
          const bool pgd = C.tt < ntp;
          read_tile_k<D>(X, ring + (size_t)rb * CH, lane);
          compute_tile<D, QT, WO, false, true>(X, pgd ? C.tt * 32 : (C.tt - ntp) * 32,
                                               pgd ? C.plen() : p.blk, nq, qf, o, mrun, lrun,
                                               p.scale_log2, lane, ring + (size_t)rb * CH);
        }
        bad = bad || ((badbits >> rb) & 1);
        if (C.tt == item_tiles(C, p) - 1 || tv == n1 - 1 || tv == n - 1) {
          finalize(C, bad || qbad);
          reset();
          bad = false;
        }
      }
      if (tvc + 1 < n) next(C, tvc);
      if (tvl + 1 < n) next(L, tvl);
      ++tv;
    };
    while (true) {
#pragma unroll
      for (int j = 0; j < NBUF; ++j) sh_step(j);
      if (tv >= n) break;
    }
    // no load into LDS may be pending when the workgroup ends
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    return;
  }
  Tile<D> tl[NB];
#pragma unroll
  for (int k = 0; k < NB - 1; ++k) {
    if (k > 0 && tvl + 1 < n) next(L, tvl);
    load_tile<D, WO>(tl[k], L, (POS && k == 0) ? pg0 : fetch_pages(L, p, page_table), p, lane);
  }
  if (tvl + 1 < n) next(L, tvl);
  int tv = 0;

  // A step past the slice end only issues its (cache-hitting) prefetch, so that the loop has a
  // single exit, after every NB steps: an exit between two buffer roles would let the compiler
  // merge the roles' pending loads at the loop head and drain the prefetch there.
  auto step = [&](Tile<D>& X, Tile<D>& Y) {
    const bool live = tv < n;
    const Pages pg = fetch_pages(L, p, page_table);
    if (live && tv > 0 && (C.tt == 0 || tv == n1)) qbad = load_q<D, QT, POS>(qf, C, p, lane);
    load_tile<D, WO>(Y, L, pg, p, lane);
    __builtin_amdgcn_sched_barrier(0);  // keep the prefetch ahead of the compute
    if (live) {
      const int ntp = C.ntp();
      const bool pg = C.tt < ntp;
      const int nq = (C.nrows - C.qg * R + 15) >> 4;
      compute_tile<D, QT, WO>(X, pg ? C.tt * 32 : (C.tt - ntp) * 32, pg ? C.plen() : p.blk, nq,
                              qf, o, mrun, lrun, p.scale_log2, lane);
      bad = bad || X.bad;
      if (C.tt == item_tiles(C, p) - 1 || tv == n1 - 1 || tv == n - 1) {
        finalize(C, bad || qbad);
        reset();
        bad = false;
      }
    }
    if (tvc + 1 < n) next(C, tvc);
    if (tvl + 1 < n) next(L, tvl);
    ++tv;
  };
  while (true) {
#pragma unroll
    for (int j = 0; j < NB; ++j) step(tl[j], tl[(j + NB - 1) % NB]);
    if (tv >= n) break;
  }
}

int ilog2(int x) {
  int l = 0;
  while ((1 << l) < x) ++l;
  return l;
}

int device_cus() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0)
      n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

// Tiles in flight per wave (one-wave kernels: tile buffers) or per workgroup (shared tiles).
constexpr int prefetch_of(int QT, bool SH) {
  return SH ? (QT == 1 ? kShPrefetch : kShPrefetchQt2) : (QT == 1 ? kPrefetchQt1 : 2);
}

// LDS of one workgroup: the requests' metadata, then the query operands of 64-row waves or the
// tile ring of shared tiles.
size_t attn_lds_bytes(int B, int D, int QT, bool SH) {
  size_t b = (size_t)(4 * B + 1 + 256) * sizeof(int);
  if (QT >= 4) b = ((b + 15) & ~(size_t)15) + (size_t)kWaves * QT * (D / 32) * 64 * 16;
  if (SH) b = ((b + 15) & ~(size_t)15) + (size_t)(prefetch_of(QT, SH) + 1) * 8 * D * 16;
  return b;
}

template <int D, int QT, bool WO, bool SH = false>
hipError_t launch_dq(const Params& prm, const AttnPlan& plan, hipStream_t s) {
  constexpr int NB = prefetch_of(QT, SH);
  if constexpr (WO) {
    if (prm.q_pos != nullptr) {  // queries read in place (with the output only)
      hipLaunchKernelGGL((attn_kernel<D, QT, NB, WO, SH, true>), dim3(plan.wgs), dim3(256),
                         attn_lds_bytes(prm.B, D, QT, SH), s, prm, prm.page_table);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((attn_kernel<D, QT, NB, WO, SH, false>), dim3(plan.wgs), dim3(256),
                     attn_lds_bytes(prm.B, D, QT, SH), s, prm, prm.page_table);
  return hipGetLastError();
}

}  // namespace

AttnPlan plan_attn(int B, int blk, int Hq, int Hkv, int d, int S, int max_pages, int max_kept,
                   bool lse_only) {
  AttnPlan pl{};
  const int G = Hq / Hkv;
  const int rows = max_kept * G;
  const int cus = device_cus();
  // shared tiles: 33..64 rows (16 per wave), and with the output any count above 64 (32 per
  // wave, one workgroup per 128 rows: two or more workgroups of an item stream the same tiles,
  // the later reads mostly from the XCD's L2)
  const bool shared = rows > 32 && (rows <= 64 || !lse_only);
  if (!shared) {
    // one wave per item: 16, 32 or 64 rows (several query groups per (request, kv head) past
    // 64 rows, without the output).  One 4-wave workgroup per CU (one wave per SIMD, each with
    // NB tiles of 32 keys in flight); without the output the larger query tiles are light
    // enough for two workgroups per CU, which hides their instruction latencies behind each
    // other.
    pl.shared = false;
    pl.qt = rows <= 16 ? 1 : (rows <= 32 ? 2 : 4);
    pl.nqg = (rows + 16 * pl.qt - 1) / (16 * pl.qt);
    pl.wgs = (pl.qt > 1 && lse_only) ? 2 : kWgsPerCuQt1;
  } else {
    // the four waves of a workgroup on one (request, kv head)'s tiles; past 128 rows several
    // workgroups per item
    pl.shared = true;
    pl.qt = rows <= 64 ? 1 : 2;
    pl.nqg = kWaves * ((rows + kWaves * 16 * pl.qt - 1) / (kWaves * 16 * pl.qt));
    pl.wgs = pl.qt == 1 ? kShWgsPerCuQt1 : kShWgsPerCu;
  }
  // workgroups per CU, as many as the LDS holds at once (large batches: larger metadata)
  {
    const int fit = (int)(kLdsPerCu / attn_lds_bytes(B, d, pl.qt, pl.shared));
    pl.wgs = cus * std::max(1, std::min(pl.wgs, fit));
  }
  const long long ntiles_max = ((long long)max_pages * S + 31) / 32 + (blk + 31) / 32;
  pl.tiles_bound = (long long)B * ntiles_max;
  pl.gs = Hkv * pl.nqg;
  // Small problems: fewer workgroups, so that a wave has at least kMinTilesPerWave tiles even
  // at the longest possible prefixes.  Per wave the setup, the item starts and the cut-item
  // protocol cost a fixed time; with a handful of tiles each they dominate (measured: the
  // 32-request configuration, about 5 tiles per wave on the full grid, 38.5 -> 36.2 us).
  {
    const long long wave_tiles = pl.tiles_bound * pl.gs;
    long long want = (wave_tiles / kMinTilesPerWave + kWaves - 1) / kWaves;
    const int unit = 8 * (pl.gs >= kWaves ? pl.gs / kWaves : 1);  // whole groups on every XCD
    want = want < unit ? unit : (want + unit - 1) / unit * unit;
    if (want < pl.wgs) pl.wgs = (int)want;
  }
  pl.ngroups = pl.wgs * kWaves / pl.gs;
  const size_t W = (size_t)pl.wgs * kWaves;
  const size_t R = 16 * (size_t)pl.qt;
  // arrival counters sized for the largest grid of either mode, so that the counters of one
  // workspace never overlap another mode's partials
  pl.cnt_bytes = ((size_t)kMaxWgsPerCu * cus * kWaves * sizeof(int) + 255) & ~(size_t)255;
  pl.ws_o_bytes = lse_only ? 0 : 2 * W * R * (size_t)d * sizeof(float);
  pl.ws_ml_bytes = 2 * W * 2 * R * sizeof(float);
  pl.ws_bytes = pl.cnt_bytes + pl.ws_o_bytes + pl.ws_ml_bytes;
  return pl;
}

hipError_t launch_attn(const AttnArgs& a, const AttnPlan& plan, hipStream_t s) {
  Params prm{};
  prm.q = a.q;
  prm.q_pos = a.q_pos;
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
  prm.nqg = plan.nqg;
  prm.W = plan.wgs * kWaves;
  prm.gs = plan.gs;
  prm.ngroups = plan.ngroups;
  prm.scale_log2 = a.scale_log2;
  unsigned char* ws = static_cast<unsigned char*>(a.workspace);
  prm.counters = reinterpret_cast<int*>(ws);
  prm.ws_o = reinterpret_cast<float*>(ws + plan.cnt_bytes);
  prm.ws_o_bytes = (int)plan.ws_o_bytes;
  prm.ws_ml = reinterpret_cast<float*>(ws + plan.cnt_bytes + plan.ws_o_bytes);
  if (a.out == nullptr) {  // log-sum-exp only
    if (plan.shared)
      return a.d == 64 ? launch_dq<64, 1, false, true>(prm, plan, s)
                       : launch_dq<128, 1, false, true>(prm, plan, s);
    if (a.d == 64) {
      if (plan.qt == 1) return launch_dq<64, 1, false>(prm, plan, s);
      if (plan.qt == 2) return launch_dq<64, 2, false>(prm, plan, s);
      return launch_dq<64, 4, false>(prm, plan, s);
    }
    if (plan.qt == 1) return launch_dq<128, 1, false>(prm, plan, s);
    if (plan.qt == 2) return launch_dq<128, 2, false>(prm, plan, s);
    return launch_dq<128, 4, false>(prm, plan, s);
  }
  if (plan.shared) {
    if (plan.qt == 2) return a.d == 64 ? launch_dq<64, 2, true, true>(prm, plan, s)
                                       : launch_dq<128, 2, true, true>(prm, plan, s);
    return a.d == 64 ? launch_dq<64, 1, true, true>(prm, plan, s)
                     : launch_dq<128, 1, true, true>(prm, plan, s);
  }
  if (a.d == 64) {
    if (plan.qt == 1) return launch_dq<64, 1, true>(prm, plan, s);
    if (plan.qt == 2) return launch_dq<64, 2, true>(prm, plan, s);
    return launch_dq<64, 4, true>(prm, plan, s);
  }
  if (plan.qt == 1) return launch_dq<128, 1, true>(prm, plan, s);
  if (plan.qt == 2) return launch_dq<128, 2, true>(prm, plan, s);
  return launch_dq<128, 4, true>(prm, plan, s);
}

}  // namespace focus
