// Intra-block KV write-back and block commit.  Project page "FOCUS: DLLMs Know How to Tame Their
// Compute Bound", cards "Runtime Action" (intra-block KV caching) and "Motivation" (finished
// blocks are exactly KV-cached); AI Engineering Academy article on FOCUS, section "Arquitetura do
// FOCUS" (KV-cache management).  Both are byte moves between the MFMA-native layouts:
//   K [.., Hkv, d/8, n, 8]: key (token t, dim c) at [c/8][t][c%8] -- 16-byte chunks per token
//   V [.., Hkv, n/8, d, 8]: value (t, c) at [t/8][c][t%8]       -- 16-byte chunks per 8 tokens
#include "device_common.h"
#include "launch.h"

namespace focus {
namespace {

// One workgroup per request: its kept rows' fresh K/V replace the block KV at their positions.
__global__ __launch_bounds__(256) void kv_writeback_kernel(WritebackArgs a) {
  const int r = blockIdx.x, tid = threadIdx.x;
  const int n0 = a.offsets[r];
  const int n1 = min(a.offsets[r + 1], a.cap);
  const int nrows = min(n1 - n0, a.blk);  // a request keeps at most blk rows
  if (n0 < 0 || nrows <= 0) return;
  const int D8 = a.d / 8;
  // keys: one 16-byte chunk per (row, head, 8-dim group)
  const int kchunks = nrows * a.Hkv * D8;
  for (int c = tid; c < kchunks; c += 256) {
    const int n = n0 + c / (a.Hkv * D8), rem = c % (a.Hkv * D8);
    const int g = rem / D8, c8 = rem % D8;
    const int j = a.kept_pos[n];
    if (j < 0 || j >= a.blk) continue;  // invalid device data: the row is skipped
    const uint4 v = load16(a.k_rows + ((size_t)n * a.Hkv + g) * a.d + 8 * c8);
    *reinterpret_cast<uint4*>(a.k_blk + ((((size_t)r * a.Hkv + g) * D8 + c8) * a.blk + j) * 8) = v;
  }
  // values: one 2-byte element per (row, head, dim)
  const int velems = nrows * a.Hkv * a.d;
  for (int e = tid; e < velems; e += 256) {
    const int n = n0 + e / (a.Hkv * a.d), rem = e % (a.Hkv * a.d);
    const int g = rem / a.d, c = rem % a.d;
    const int j = a.kept_pos[n];
    if (j < 0 || j >= a.blk) continue;
    a.v_blk[((((size_t)r * a.Hkv + g) * (a.blk / 8) + j / 8) * a.d + c) * 8 + j % 8] =
        a.v_rows[((size_t)n * a.Hkv + g) * a.d + c];
  }
}

__device__ __forceinline__ int ceil_div(int x, int y) { return (x + y - 1) / y; }

// One workgroup per request.  Every workgroup first derives the whole commit's outcome from the
// inputs alone (so all of them take the same decision without a grid-wide barrier): each
// committed request's page need, the total, this request's first free-stack slot, and the
// status.  Inputs and outputs of the prefix lengths and free count are distinct arrays, so no
// workgroup can see another's update.
__global__ __launch_bounds__(256) void block_commit_kernel(CommitArgs a) {
  __shared__ int s_red[3][4];
  __shared__ int s_pages[8];
  const int r = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int cap_tokens = a.max_pages * a.S;
  const int fc = a.free_count_in[0];
  // pass 1: needs of all requests (and invalid data), this request's prefix of needs
  int total = 0, before = 0, bad = 0, badid = 0;
  for (int i = tid; i < a.B; i += 256) {
    if (!a.commit[i]) continue;
    const int P = a.prefix_len_in[i];
    if (P < 0 || P + a.blk > cap_tokens) {
      bad = 1;
      continue;
    }
    if (P % a.S != 0) {  // the partly filled last page receives tokens: its id must be valid
      const int id = a.page_table[(size_t)i * a.max_pages + P / a.S];
      badid |= (id < 0 || id >= a.num_pages);
    }
    const int need = ceil_div(P + a.blk, a.S) - ceil_div(P, a.S);
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
  // pass 2: the free-stack entries the commit takes must be valid page ids
  if (status == 0) {
    int badfree = 0;
    for (int i = tid; i < total; i += 256) {
      const int id = a.free_pages[fc - 1 - i];
      badfree |= (id < 0 || id >= a.num_pages);
    }
    for (int m = 32; m > 0; m >>= 1) badfree |= __shfl_xor(badfree, m, 64);
    if (lane == 0) s_red[2][wv] = badfree;
    __syncthreads();
    if (s_red[2][0] | s_red[2][1] | s_red[2][2] | s_red[2][3]) status = 3;
  }
  const int P = a.prefix_len_in[r];
  const bool mine = status == 0 && a.commit[r] != 0;
  if (tid == 0) {
    a.prefix_len_out[r] = mine ? P + a.blk : P;
    if (r == 0) {
      a.status[0] = status;
      a.free_count_out[0] = status == 0 ? fc - total : fc;
    }
  }
  if (!mine) return;
  // allocate: this request's new pages, in position order, from the top of the stack
  const int first_new = ceil_div(P, a.S);
  const int need = ceil_div(P + a.blk, a.S) - first_new;
  int32_t* row = a.page_table + (size_t)r * a.max_pages;
  if (tid < need) {
    const int id = a.free_pages[fc - 1 - (before + tid)];
    row[first_new + tid] = id;
    s_pages[tid] = id;
  }
  __syncthreads();
  auto page_of = [&](int p) {  // p: prefix position of an appended token
    const int pi = p / a.S;
    return pi < first_new ? row[pi] : s_pages[pi - first_new];
  };
  const int D8 = a.d / 8;
  // keys: 16-byte chunks (token, head, 8-dim group)
  const int kchunks = a.blk * a.Hkv * D8;
  for (int c = tid; c < kchunks; c += 256) {
    const int t = c / (a.Hkv * D8), rem = c % (a.Hkv * D8);
    const int g = rem / D8, c8 = rem % D8;
    const int p = P + t, page = page_of(p), slot = p % a.S;
    const uint4 v = load16(a.k_blk + ((((size_t)r * a.Hkv + g) * D8 + c8) * a.blk + t) * 8);
    *reinterpret_cast<uint4*>(a.k_cache + ((((size_t)page * a.Hkv + g) * D8 + c8) * a.S + slot) * 8) =
        v;
  }
  // values: 16-byte chunks [slot/8][dim] of 8 consecutive prefix positions.  Destination chunk
  // q covers positions p0 = (P & ~7) + 8q .. p0+7, i.e. block tokens t0 = p0 - P .. t0+7, taken
  // from at most two source chunks; slots outside [P, P + blk) keep their contents.
  const int nq = (P % 8 + a.blk + 7) / 8;
  const int vchunks = nq * a.Hkv * a.d;
  const int nsrc = a.blk / 8;
  for (int c = tid; c < vchunks; c += 256) {
    const int q = c / (a.Hkv * a.d), rem = c % (a.Hkv * a.d);
    const int g = rem / a.d, dim = rem % a.d;
    const int p0 = (P & ~7) + 8 * q, t0 = p0 - P;
    const int page = page_of(max(p0, P)), slot = p0 % a.S;
    uint16_t* dst =
        a.v_cache + ((((size_t)page * a.Hkv + g) * (a.S / 8) + slot / 8) * a.d + dim) * 8;
    const uint16_t* src = a.v_blk + (((size_t)r * a.Hkv + g) * nsrc * a.d + dim) * 8;
    const int sa = t0 >= 0 ? t0 >> 3 : -1;  // source chunk of t0 (floor division)
    uint4 A = make_uint4(0, 0, 0, 0), Bv = make_uint4(0, 0, 0, 0), E = make_uint4(0, 0, 0, 0);
    if (sa >= 0) A = load16(src + (size_t)sa * a.d * 8);
    if (sa + 1 < nsrc) Bv = load16(src + (size_t)(sa + 1) * a.d * 8);
    const bool partial = t0 < 0 || t0 + 8 > a.blk;
    if (partial) E = load16(dst);
    // the 8 source elements starting at token t0 are elements sh.. of A:B (sh = t0 mod 8, the
    // same for every chunk of the request): a right shift of the 256-bit A:B by 16*sh bits
    const int sh = t0 & 7;
    const uint64_t a0 = A.x | ((uint64_t)A.y << 32), a1 = A.z | ((uint64_t)A.w << 32);
    const uint64_t b0 = Bv.x | ((uint64_t)Bv.y << 32), b1 = Bv.z | ((uint64_t)Bv.w << 32);
    const bool upper = sh >= 4;          // the shift crosses the first 64-bit word
    const uint64_t x0 = upper ? a1 : a0, x1 = upper ? b0 : a1, x2 = upper ? b1 : b0;
    const int bits = 16 * (sh & 3);
    const uint64_t r0 = bits ? (x0 >> bits) | (x1 << (64 - bits)) : x0;
    const uint64_t r1 = bits ? (x1 >> bits) | (x2 << (64 - bits)) : x1;
    const uint32_t v[4] = {(uint32_t)r0, (uint32_t)(r0 >> 32), (uint32_t)r1, (uint32_t)(r1 >> 32)};
    const uint32_t Ew[4] = {E.x, E.y, E.z, E.w};
    uint32_t ow[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = t0 + 2 * i;  // tokens of the word's two elements: t, t + 1
      const uint32_t m = ((t >= 0 && t < a.blk) ? 0x0000ffffu : 0u) |
                         ((t + 1 >= 0 && t + 1 < a.blk) ? 0xffff0000u : 0u);
      ow[i] = (v[i] & m) | (Ew[i] & ~m);
    }
    const uint4 o = make_uint4(ow[0], ow[1], ow[2], ow[3]);
    *reinterpret_cast<uint4*>(dst) = o;
  }
}

}  // namespace

hipError_t launch_writeback(const WritebackArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(kv_writeback_kernel, dim3(a.B), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_commit(const CommitArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(block_commit_kernel, dim3(a.B), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace focus
