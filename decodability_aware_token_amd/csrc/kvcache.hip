// Intra-block KV write-back and block commit.  Project page "FOCUS: DLLMs Know How to Tame Their
// Compute Bound", cards "Runtime Action" (intra-block KV caching) and "Motivation" (finished
// blocks are exactly KV-cached); AI Engineering Academy article on FOCUS, section "Arquitetura do
// FOCUS" (KV-cache management).  Both are byte moves between the MFMA-native layouts (as is the
// conversion of plain token-row K/V into them, at the end of this file):
//   K [.., Hkv, d/8, n, 8]: key (token t, dim c) at [c/8][t][c%8] -- 16-byte chunks per token
//   V [.., Hkv, n/8, d, 8]: value (t, c) at [t/8][c][t%8]       -- 16-byte chunks per 8 tokens
#include <algorithm>

#include "device_common.h"
#include "launch.h"

namespace focus {
namespace {

constexpr int kBatch = 8;  // 16-byte chunks per thread with their loads in flight together
constexpr int kWritebackSplit = 2;  // workgroups per request in the write-back

// kWritebackSplit workgroups per request, each moving its share of the request's kept rows' fresh
// K/V into the block KV at their positions.  First the request's positions are mapped to the
// rows that write them in LDS (a position named by several rows takes the last of them, as a
// sequential write would, so every destination is written once), then:
//  * keys: one 16-byte chunk per (position, head, 8-dim group), a whole run of 8 dims;
//  * values: one 2-byte element per (position, head, dim): the V layout interleaves 8 positions
//    per 16-byte chunk.  (Rebuilding each touched chunk whole -- the cached chunk merged with
//    the written values, one 16-byte store -- measured slower: its extra loads cost more than
//    the stores it saves.)
// Loads of a batch are all issued before its stores (source and destination may alias as far
// as the compiler knows, so a load after a store would wait for it).
__global__ __launch_bounds__(256) void kv_writeback_kernel(WritebackArgs a) {
  __shared__ int s_row[64];  // position -> row writing it, -1 if none
  __shared__ int s_pos[64];  // positions with a row, ascending
  __shared__ int s_np;
  const int r = blockIdx.x, split = blockIdx.y, tid = threadIdx.x, lane = tid & 63;
  const int n0 = a.offsets[r];
  const int n1 = min(a.offsets[r + 1], a.cap);
  const int nrows = min(n1 - n0, a.blk);  // a request keeps at most blk rows
  if (n0 < 0 || nrows <= 0) return;
  if (tid < 64) s_row[tid] = -1;
  __syncthreads();
  if (tid < nrows) {
    const int j = a.kept_pos[n0 + tid];
    // invalid device data (a position outside the block): the row is skipped
    if (j >= 0 && j < a.blk) atomicMax(&s_row[j], n0 + tid);
  }
  __syncthreads();
  if (tid < 64) {
    const bool has = lane < a.blk && s_row[lane] >= 0;
    const uint64_t m = __ballot(has);
    const int rank = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                               __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
    if (has) s_pos[rank] = lane;
    if (lane == 0) s_np = __popcll(m);
  }
  __syncthreads();
  const int np = s_np;
  const int D8 = a.d / 8;
  // keys
  const int kchunks = np * a.Hkv * D8;
  const int kper = (kchunks + gridDim.y - 1) / gridDim.y;
  const int k_lo = split * kper, k_hi = min(k_lo + kper, kchunks);
  for (int c0 = k_lo + tid; c0 < k_hi; c0 += 256 * kBatch) {
    uint4 v[kBatch];
    int64_t dst[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int c = min(c0 + 256 * u, k_hi - 1);
      const int q = c / (a.Hkv * D8), rem = c % (a.Hkv * D8);
      const int g = rem / D8, c8 = rem % D8;
      const int j = s_pos[q], n = s_row[j];
      v[u] = load16(a.k_rows + ((size_t)n * a.Hkv + g) * a.d + 8 * c8);
      dst[u] = c0 + 256 * u < k_hi ? ((((int64_t)r * a.Hkv + g) * D8 + c8) * a.blk + j) : -1;
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u)
      if (dst[u] >= 0) *reinterpret_cast<uint4*>(a.k_blk + dst[u] * 8) = v[u];
  }
  // values: one 2-byte element per (written position, head, dim)
  const int velems = np * a.Hkv * a.d;
  const int vper = (velems + gridDim.y - 1) / gridDim.y;
  const int v_lo = split * vper, v_hi = min(v_lo + vper, velems);
  for (int e0 = v_lo + tid; e0 < v_hi; e0 += 256 * kBatch) {
    uint16_t v[kBatch];
    int64_t dst[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int e = min(e0 + 256 * u, v_hi - 1);
      const int q = e / (a.Hkv * a.d), rem = e % (a.Hkv * a.d);
      const int g = rem / a.d, c = rem % a.d;
      const int j = s_pos[q], n = s_row[j];
      v[u] = a.v_rows[((size_t)n * a.Hkv + g) * a.d + c];
      dst[u] = e0 + 256 * u < v_hi
                   ? ((((int64_t)r * a.Hkv + g) * (a.blk / 8) + j / 8) * a.d + c) * 8 + j % 8
                   : -1;
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u)
      if (dst[u] >= 0) a.v_blk[dst[u]] = v[u];
  }
}

__device__ __forceinline__ int ceil_div(int x, int y) { return (x + y - 1) / y; }

// The commit's workgroups: grid [B, nsplit], part `split` of request r moves its share of the
// request's K and V chunks (at most kBatch per thread of each, by the choice of nsplit).  Every
// workgroup first derives the whole commit's outcome from the inputs alone (so all of them take
// the same decision without a grid-wide barrier): each committed request's page need, the
// total, this request's first free-stack slot and new pages, and the status; part 0 of a request
// writes its table entries, prefix length and (request 0) the status and free count.  Inputs and
// outputs of the prefix lengths and free count are distinct arrays, so no workgroup can see
// another's update.  The block sources do not depend on that outcome: their loads are issued
// first and fly while it is derived.  Bounded to three waves per SIMD (168 registers, a few
// spilled), so that the 3·B workgroups of the headline batch all fit at once: 21.5 us there
// instead of 26 us with two waves per SIMD.
__global__ __launch_bounds__(256, 3) void block_commit_kernel(CommitArgs a) {
  __shared__ int s_red[3][4];
  __shared__ int s_pages[8];
  const int r = blockIdx.x, split = blockIdx.y, tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int cap_tokens = a.max_pages * a.S;
  const int D8 = a.d / 8, nsrc = a.blk / 8;
  const int P = a.prefix_len_in[r];
  // this part's chunk ranges: keys (head, 8-dim group, token); values [slot/8][dim] chunks of
  // 8 consecutive prefix positions p0 = (P & ~7) + 8q .. p0 + 7, i.e. block tokens
  // t0 = p0 - P .. t0 + 7, taken from at most two source chunks
  const int kchunks = a.blk * a.Hkv * D8;
  const int kper = ceil_div(kchunks, gridDim.y);
  const int k_lo = split * kper, k_hi = min(k_lo + kper, kchunks);
  const int nq = ((P & 7) + a.blk + 7) / 8;
  const int vchunks = nq * a.Hkv * a.d;
  const int vper = ceil_div(vchunks, gridDim.y);
  const int v_lo = split * vper, v_hi = min(v_lo + vper, vchunks);
  const int t0_base = (P & ~7) - P;  // t0 of chunk q is t0_base + 8q, in [-7, blk)

  // ---- source loads (clamped into the block: unconditional, masked when used)
  uint4 kv[kBatch], va[kBatch], vb[kBatch];
#pragma unroll
  for (int u = 0; u < kBatch; ++u) {
    const int c = max(min(k_lo + tid + 256 * u, k_hi - 1), 0);
    const int t = c % a.blk, gc = c / a.blk;  // tokens fastest: whole runs on both sides
    kv[u] = load16(a.k_blk + (((size_t)r * a.Hkv * D8 + gc) * a.blk + t) * 8);
  }
#pragma unroll
  for (int u = 0; u < kBatch; ++u) {
    const int c = max(min(v_lo + tid + 256 * u, v_hi - 1), 0);
    const int q = c / (a.Hkv * a.d), rem = c % (a.Hkv * a.d);
    const int g = rem / a.d, dim = rem % a.d;
    const int t0 = t0_base + 8 * q;
    const int sa = t0 >= 0 ? t0 >> 3 : -1;  // source chunk of t0 (floor division)
    const uint16_t* src = a.v_blk + (((size_t)r * a.Hkv + g) * nsrc * a.d + dim) * 8;
    va[u] = load16(src + (size_t)min(max(sa, 0), nsrc - 1) * a.d * 8);
    vb[u] = load16(src + (size_t)min(sa + 1, nsrc - 1) * a.d * 8);
  }

  // the one older page that can receive tokens (the partly filled last one), clamped
  const int old_page = a.page_table[(size_t)r * a.max_pages +
                                    min(max(P, 0) / a.S, max(a.max_pages - 1, 0))];
  const int fc = a.free_count_in[0];
  // pass 1: needs of all requests (and invalid data), this request's prefix of needs
  int total = 0, before = 0, bad = 0, badid = 0;
  for (int i = tid; i < a.B; i += 256) {
    if (!a.commit[i]) continue;
    const int Pi = a.prefix_len_in[i];
    if (Pi < 0 || Pi + a.blk > cap_tokens) {
      bad = 1;
      continue;
    }
    if (Pi % a.S != 0) {  // the partly filled last page receives tokens: its id must be valid
      const int id = a.page_table[(size_t)i * a.max_pages + Pi / a.S];
      badid |= (id < 0 || id >= a.num_pages);
    }
    const int need = ceil_div(Pi + a.blk, a.S) - ceil_div(Pi, a.S);
    total += need;
    if (i < r) before += need;
  }
  for (int m = 32; m > 0; m >>= 1) {
    total += __shfl_xor(total, m, 64);
    before += __shfl_xor(before, m, 64);
    bad |= __shfl_xor(bad, m, 64);
    badid |= __shfl_xor(badid, m, 64);
  }
  if (lane == 0) {
    s_red[0][wv] = total;
    s_red[1][wv] = before;
    s_red[2][wv] = bad | (badid << 1);
  }
  __syncthreads();
  total = s_red[0][0] + s_red[0][1] + s_red[0][2] + s_red[0][3];
  before = s_red[1][0] + s_red[1][1] + s_red[1][2] + s_red[1][3];
  const int flags = s_red[2][0] | s_red[2][1] | s_red[2][2] | s_red[2][3];
  int status = 0;
  if (flags & 1)
    status = 2;
  else if ((flags & 2) || fc < 0 || fc > a.free_cap)
    status = 3;
  else if (total > fc)
    status = 1;
  __syncthreads();
  // pass 2: the free-stack entries the commit takes must be valid page ids; this request's own
  // entries (its new pages, in position order, from the top of the stack) are kept
  if (status == 0) {
    int badfree = 0;
    for (int i = tid; i < total; i += 256) {
      const int id = a.free_pages[fc - 1 - i];
      badfree |= (id < 0 || id >= a.num_pages);
      if (i >= before && i - before < 8) s_pages[i - before] = id;
    }
    for (int m = 32; m > 0; m >>= 1) badfree |= __shfl_xor(badfree, m, 64);
    if (lane == 0) s_red[2][wv] = badfree;
    __syncthreads();
    if (s_red[2][0] | s_red[2][1] | s_red[2][2] | s_red[2][3]) status = 3;
  }
  const bool mine = status == 0 && a.commit[r] != 0;
  if (tid == 0 && split == 0) {
    a.prefix_len_out[r] = mine ? P + a.blk : P;
    if (r == 0) {
      a.status[0] = status;
      a.free_count_out[0] = status == 0 ? fc - total : fc;
    }
  }
  if (!mine) return;
  // allocate: the new pages (read in pass 2, published by its barrier) enter the table
  const int first_new = ceil_div(P, a.S);
  const int need = ceil_div(P + a.blk, a.S) - first_new;
  int32_t* row = a.page_table + (size_t)r * a.max_pages;
  if (tid < need && split == 0) row[first_new + tid] = s_pages[tid];
  auto page_of = [&](int p) {  // p: prefix position of an appended token
    const int pi = p / a.S;
    return pi < first_new ? old_page : s_pages[pi - first_new];  // pi < first_new: pi == P/S
  };

  // ---- keys: stores of the prefetched chunks
#pragma unroll
  for (int u = 0; u < kBatch; ++u) {
    const int c = k_lo + tid + 256 * u;
    if (c >= k_hi) break;
    const int t = c % a.blk, gc = c / a.blk;  // gc = head * D8 + 8-dim group
    const int p = P + t, page = page_of(p), slot = p % a.S;
    *reinterpret_cast<uint4*>(a.k_cache + (((size_t)page * a.Hkv * D8 + gc) * a.S + slot) * 8) =
        kv[u];
  }
  // ---- values: the destination's own contents for the chunks that are only partly appended
  // (first and last when P is not a multiple of 8), then the shifted and merged chunks
  // the 8 source elements starting at token t0 are elements sh.. of A:B (sh = t0 mod 8, the
  // same for every chunk of the request): a right shift of the 256-bit A:B by 16*sh bits
  const int sh = t0_base & 7;
  uint4 ve[kBatch];
  size_t dst[kBatch];
#pragma unroll
  for (int u = 0; u < kBatch; ++u) {
    const int c = max(min(v_lo + tid + 256 * u, v_hi - 1), 0);
    const int q = c / (a.Hkv * a.d), rem = c % (a.Hkv * a.d);
    const int g = rem / a.d, dim = rem % a.d;
    const int p0 = (P & ~7) + 8 * q, t0 = t0_base + 8 * q;
    const int page = page_of(max(p0, P)), slot = p0 % a.S;
    dst[u] = ((((size_t)page * a.Hkv + g) * (a.S / 8) + slot / 8) * a.d + dim) * 8;
    const bool partial = t0 < 0 || t0 + 8 > a.blk;
    ve[u] = partial ? load16(a.v_cache + dst[u]) : make_uint4(0, 0, 0, 0);
  }
#pragma unroll
  for (int u = 0; u < kBatch; ++u) {
    const int c = v_lo + tid + 256 * u;
    if (c >= v_hi) break;
    const int q = c / (a.Hkv * a.d);
    const int t0 = t0_base + 8 * q;
    const int sa = t0 >= 0 ? t0 >> 3 : -1;
    const uint4 Au = sa >= 0 ? va[u] : make_uint4(0, 0, 0, 0);
    const uint4 Bu = sa + 1 < nsrc ? vb[u] : make_uint4(0, 0, 0, 0);
    const uint64_t a0 = Au.x | ((uint64_t)Au.y << 32), a1 = Au.z | ((uint64_t)Au.w << 32);
    const uint64_t b0 = Bu.x | ((uint64_t)Bu.y << 32), b1 = Bu.z | ((uint64_t)Bu.w << 32);
    const bool upper = sh >= 4;  // the shift crosses the first 64-bit word
    const uint64_t x0 = upper ? a1 : a0, x1 = upper ? b0 : a1, x2 = upper ? b1 : b0;
    const int bits = 16 * (sh & 3);
    const uint64_t r0 = bits ? (x0 >> bits) | (x1 << (64 - bits)) : x0;
    const uint64_t r1 = bits ? (x1 >> bits) | (x2 << (64 - bits)) : x1;
    const uint32_t v[4] = {(uint32_t)r0, (uint32_t)(r0 >> 32), (uint32_t)r1,
                           (uint32_t)(r1 >> 32)};
    const uint32_t Ew[4] = {ve[u].x, ve[u].y, ve[u].z, ve[u].w};
    uint32_t ow[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = t0 + 2 * i;  // tokens of the word's two elements: t, t + 1
      const uint32_t m = ((t >= 0 && t < a.blk) ? 0x0000ffffu : 0u) |
                         ((t + 1 >= 0 && t + 1 < a.blk) ? 0xffff0000u : 0u);
      ow[i] = (v[i] & m) | (Ew[i] & ~m);
    }
    *reinterpret_cast<uint4*>(a.v_cache + dst[u]) = make_uint4(ow[0], ow[1], ow[2], ow[3]);
  }
}

// Conversion of plain K/V (token rows of d elements) into the layouts above, for callers whose
// cache is stored row by row.  A workgroup takes kPackChunks 16-byte chunks of each matrix:
// one or more consecutive (block, kv head) pairs, whose outputs are one contiguous range.  The
// source rows are loaded (neighbouring threads read neighbouring chunks of a row) into LDS as
// they are (rows padded by one chunk, so that reading down a column is free of bank
// conflicts), then every thread builds output chunks in output order -- a key chunk is one
// 16-byte piece of a row, a value chunk gathers one dim of 8 consecutive rows -- so that the
// stores of a wave cover whole consecutive runs.
constexpr int kPackChunks = 1024;

__global__ __launch_bounds__(256) void kv_pack_kernel(PackArgs a) {
  constexpr int kMaxRows = kPackChunks / 8;  // d = 64: 8 chunks per row
  __shared__ uint4 s_k[kPackChunks + kMaxRows], s_v[kPackChunks + kMaxRows];
  const int tid = threadIdx.x;
  const int D8 = a.d / 8, pitch = D8 + 1;     // row pitch in chunks
  const int S = a.S, per_pair = S * D8;        // chunks of one (block, kv head) pair
  const int pp = kPackChunks / per_pair;       // pairs per workgroup (1 .. 8)
  const long long pairs = (long long)a.n_blocks * a.Hkv;
  const long long pair0 = (long long)blockIdx.x * pp;
  const bool has_k = a.k_src != nullptr, has_v = a.v_src != nullptr;
  constexpr int U = kPackChunks / 256;
  uint4 kv[U], vv[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int i = tid + 256 * u, row = i / D8, c8 = i % D8;
    const int p = row / S, s = row % S;
    const long long pair = min(pair0 + p, pairs - 1);  // the last workgroup's unused rows
    const long long n = pair / a.Hkv, g = pair % a.Hkv;
    const size_t off = a.token_major ? (((size_t)n * S + s) * a.Hkv + g) * a.d + 8 * c8
                                     : (((size_t)n * a.Hkv + g) * S + s) * a.d + 8 * c8;
    if (has_k) kv[u] = load16(a.k_src + off);
    if (has_v) vv[u] = load16(a.v_src + off);
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int i = tid + 256 * u, row = i / D8, c8 = i % D8;
    if (has_k) s_k[row * pitch + c8] = kv[u];
    if (has_v) s_v[row * pitch + c8] = vv[u];
  }
  __syncthreads();
  const size_t out0 = (size_t)pair0 * S * a.d;  // first element of this workgroup's outputs
  const long long live = min((long long)pp, pairs - pair0) * per_pair;  // chunks to write
  if (has_k) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = tid + 256 * u;  // output chunk: pair p, dim group c8, token s
      if (j >= live) break;
      const int p = j / per_pair, rem = j % per_pair, c8 = rem / S, s = rem % S;
      reinterpret_cast<uint4*>(a.k_out + out0)[j] = s_k[(p * S + s) * pitch + c8];
    }
  }
  if (has_v) {
    const uint16_t* sv = reinterpret_cast<const uint16_t*>(s_v);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = tid + 256 * u;  // output chunk: pair p, token group q, dim c
      if (j >= live) break;
      const int p = j / per_pair, rem = j % per_pair, q = rem / a.d, c = rem % a.d;
      const uint16_t* col = sv + (size_t)(p * S + 8 * q) * pitch * 8 + c;
      uint32_t w[4];
#pragma unroll
      for (int k = 0; k < 4; ++k)
        w[k] = (uint32_t)col[(2 * k) * pitch * 8] | ((uint32_t)col[(2 * k + 1) * pitch * 8] << 16);
      reinterpret_cast<uint4*>(a.v_out + out0)[j] = make_uint4(w[0], w[1], w[2], w[3]);
    }
  }
}

}  // namespace

hipError_t launch_kv_pack(const PackArgs& a, hipStream_t s) {
  const int pp = kPackChunks / (a.S * (a.d / 8));
  const long long pairs = (long long)a.n_blocks * a.Hkv;
  const int grid = (int)((pairs + pp - 1) / pp);
  hipLaunchKernelGGL(kv_pack_kernel, dim3(grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_writeback(const WritebackArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(kv_writeback_kernel, dim3(a.B, kWritebackSplit), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_commit(const CommitArgs& a, hipStream_t s) {
  // parts per request: at most kBatch chunks per thread of keys and of values
  const int per_wg = 256 * kBatch;
  const int kchunks = a.blk * a.Hkv * (a.d / 8);
  const int vchunks = (a.blk / 8 + 1) * a.Hkv * a.d;  // P not a multiple of 8: one more group
  const int nsplit = std::max((kchunks + per_wg - 1) / per_wg, (vchunks + per_wg - 1) / per_wg);
  hipLaunchKernelGGL(block_commit_kernel, dim3(a.B, nsplit), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace focus
