// C ABI of the focused block-diffusion step (declared in include/focus.h): validates every
// argument on the host, sizes the launch and hands over to the kernels' launchers.  Nothing
// here allocates memory or synchronises the host.
#include "focus.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <mutex>

#include "launch.h"

namespace {

constexpr int kVersion = 100;  // 0.1.0
constexpr int kMaxB = focus::kMaxB;
constexpr int64_t kMaxRowBytes = int64_t(1) << 24;  // 16 MiB per gathered row

bool pow2_in(int x, int lo, int hi) { return x >= lo && x <= hi && (x & (x - 1)) == 0; }
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }
bool group_ok(int Hq, int Hkv) {
  if (Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0) return false;
  const int G = Hq / Hkv;
  return G == 1 || G == 2 || G == 4 || G == 8;
}
int status_of(hipError_t e) { return e == hipSuccess ? FOCUS_OK : FOCUS_ERR_HIP; }

}  // namespace

// Scratch of focus_score_select_compact_noalloc: the score partials [B, Hkv, blk] f32 live in
// this array, one copy per GPU, held until the process ends.  Host code never uses the name
// itself (on the host it is a stand-in, not a device address): the device address comes from
// hipGetSymbolAddress, looked up once per device.
static constexpr size_t kScratchBytes = size_t(4) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's address of `scratch`, or FOCUS_ERR_HIP.
int scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return FOCUS_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
      return FOCUS_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return FOCUS_OK;
}
}  // namespace

extern "C" {

const char* focus_status_string(int code) {
  switch (code) {
    case FOCUS_OK: return "ok";
    case FOCUS_ERR_INVALID_ARG: return "invalid argument";
    case FOCUS_ERR_UNSUPPORTED: return "unsupported size";
    case FOCUS_ERR_WORKSPACE: return "workspace missing or too small";
    case FOCUS_ERR_HIP: return "HIP launch error";
    default: return "unknown status";
  }
}

int focus_version(void) { return kVersion; }

size_t focus_score_l01_workspace_size(int B, int blk, int Hq, int Hkv, int d) {
  (void)Hq;
  (void)d;
  if (B <= 0 || blk <= 0 || Hkv <= 0) return 0;
  return focus::score_workspace_bytes(B, blk, Hkv);
}

namespace {
// Validates the scoring arguments and fills a; FOCUS_OK or the error code.
int score_prepare(const void* q0, const void* k0, const void* q1, const void* k1,
                  const float* lse0, const float* lse1, int dtype, int B, int blk, int Hq,
                  int Hkv, int d, float sm_scale, float* delta, void* workspace,
                  size_t workspace_bytes, focus::ScoreArgs& a) {
  if (!q0 || !k0 || !q1 || !k1 || !delta) return FOCUS_ERR_INVALID_ARG;
  if (B <= 0 || blk <= 0 || Hq <= 0 || Hkv <= 0 || d <= 0) return FOCUS_ERR_INVALID_ARG;
  if (!(sm_scale > 0.f) || !std::isfinite(sm_scale)) return FOCUS_ERR_INVALID_ARG;
  if (dtype != FOCUS_F32 && dtype != FOCUS_BF16) return FOCUS_ERR_UNSUPPORTED;
  if (Hq % Hkv != 0) return FOCUS_ERR_INVALID_ARG;
  if (!group_ok(Hq, Hkv) || Hkv > 64) return FOCUS_ERR_UNSUPPORTED;
  if (!pow2_in(blk, 16, 64) || (d != 64 && d != 128) || B > kMaxB) return FOCUS_ERR_UNSUPPORTED;
  if (!aligned16(q0) || !aligned16(k0) || !aligned16(q1) || !aligned16(k1))
    return FOCUS_ERR_INVALID_ARG;
  if (lse0 && (!aligned4(lse0) || !aligned4(lse1))) return FOCUS_ERR_INVALID_ARG;
  const size_t need = focus::score_workspace_bytes(B, blk, Hkv);
  if (need > 0 && (!workspace || workspace_bytes < need)) return FOCUS_ERR_WORKSPACE;
  a = focus::ScoreArgs{};
  a.q0 = q0;
  a.k0 = k0;
  a.q1 = q1;
  a.k1 = k1;
  a.is_bf16 = dtype == FOCUS_BF16;
  a.B = B;
  a.blk = blk;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.d = d;
  a.scale_log2 = sm_scale * 1.4426950408889634f;
  a.lse0 = lse0;
  a.lse1 = lse1;
  a.delta = delta;
  a.part = static_cast<float*>(workspace);
  return FOCUS_OK;
}

int score_common(const void* q0, const void* k0, const void* q1, const void* k1,
                 const float* lse0, const float* lse1, int dtype, int B, int blk, int Hq,
                 int Hkv, int d, float sm_scale, float* delta, void* workspace,
                 size_t workspace_bytes, hipStream_t stream,
                 const focus::SelectArgs* sel = nullptr) {
  focus::ScoreArgs a;
  const int rc = score_prepare(q0, k0, q1, k1, lse0, lse1, dtype, B, blk, Hq, Hkv, d, sm_scale,
                               delta, workspace, workspace_bytes, a);
  if (rc != FOCUS_OK) return rc;
  if (sel) {
    a.fuse_select = 1;
    a.sel = *sel;
  }
  return status_of(focus::launch_score(a, stream));
}
}  // namespace

int focus_score_l01(const void* q0, const void* k0, const void* q1, const void* k1, int dtype,
                    int B, int blk, int Hq, int Hkv, int d, float sm_scale, float* delta,
                    void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return score_common(q0, k0, q1, k1, nullptr, nullptr, dtype, B, blk, Hq, Hkv, d, sm_scale,
                      delta, workspace, workspace_bytes, stream);
}

int focus_score_l01_lse(const void* q0, const void* k0, const void* q1, const void* k1,
                        const float* lse0, const float* lse1, int dtype, int B, int blk, int Hq,
                        int Hkv, int d, float sm_scale, float* delta, void* workspace,
                        size_t workspace_bytes, hipStream_t stream) {
  if (!lse0 || !lse1) return FOCUS_ERR_INVALID_ARG;
  return score_common(q0, k0, q1, k1, lse0, lse1, dtype, B, blk, Hq, Hkv, d, sm_scale, delta,
                      workspace, workspace_bytes, stream);
}

int focus_score_select(const void* q0, const void* k0, const void* q1, const void* k1,
                       int dtype, int B, int blk, int Hq, int Hkv, int d, float sm_scale,
                       const uint8_t* masked, const int32_t* budget, int adaptive, float beta,
                       int lo, int hi, float* delta, uint8_t* keep, int32_t* kept_count,
                       void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!masked || !keep || !kept_count) return FOCUS_ERR_INVALID_ARG;
  if (!adaptive && !budget) return FOCUS_ERR_INVALID_ARG;
  if (adaptive && (!std::isfinite(beta) || lo > hi)) return FOCUS_ERR_INVALID_ARG;
  focus::SelectArgs sa{};
  sa.delta = delta;
  sa.masked = masked;
  sa.budget = budget;
  sa.adaptive = adaptive ? 1 : 0;
  sa.beta = beta;
  sa.lo = lo;
  sa.hi = hi;
  sa.B = B;
  sa.blk = blk;
  sa.keep = keep;
  sa.kept_count = kept_count;
  return score_common(q0, k0, q1, k1, nullptr, nullptr, dtype, B, blk, Hq, Hkv, d, sm_scale,
                      delta, workspace, workspace_bytes, stream, &sa);
}

int focus_select_budget(const float* delta, const uint8_t* masked, const int32_t* budget,
                        int adaptive, float beta, int lo, int hi, int B, int blk, uint8_t* keep,
                        int32_t* kept_count, hipStream_t stream) {
  if (!delta || !masked || !keep || !kept_count) return FOCUS_ERR_INVALID_ARG;
  if (!adaptive && !budget) return FOCUS_ERR_INVALID_ARG;
  if (B <= 0 || blk <= 0) return FOCUS_ERR_INVALID_ARG;
  if (adaptive && (!std::isfinite(beta) || lo > hi)) return FOCUS_ERR_INVALID_ARG;
  if (!pow2_in(blk, 16, 64) || B > kMaxB) return FOCUS_ERR_UNSUPPORTED;
  focus::SelectArgs a{};
  a.delta = delta;
  a.masked = masked;
  a.budget = budget;
  a.adaptive = adaptive ? 1 : 0;
  a.beta = beta;
  a.lo = lo;
  a.hi = hi;
  a.B = B;
  a.blk = blk;
  a.keep = keep;
  a.kept_count = kept_count;
  return status_of(focus::launch_select(a, stream));
}

namespace {
// Validates the compaction arguments other than keep and fills a (keep left null).
int compact_prepare(int B, int blk, int nsets, const void* const* rows, const int64_t* row_bytes,
                    void* const* gathered, int cap, int32_t* offsets, int32_t* kept_pos,
                    focus::CompactArgs& a) {
  if (!offsets) return FOCUS_ERR_INVALID_ARG;
  if (B <= 0 || blk <= 0 || cap < 0 || nsets < 0) return FOCUS_ERR_INVALID_ARG;
  if (nsets > 0 && (!rows || !row_bytes || !gathered)) return FOCUS_ERR_INVALID_ARG;
  if (!pow2_in(blk, 16, 64) || B > kMaxB || nsets > focus::kMaxSets) return FOCUS_ERR_UNSUPPORTED;
  a = focus::CompactArgs{};
  for (int si = 0; si < nsets; ++si) {
    if (!rows[si] || !gathered[si] || row_bytes[si] <= 0) return FOCUS_ERR_INVALID_ARG;
    if (row_bytes[si] % 16 != 0 || row_bytes[si] > kMaxRowBytes || !aligned16(rows[si]) ||
        !aligned16(gathered[si]))
      return FOCUS_ERR_UNSUPPORTED;
    a.rows[si] = rows[si];
    a.row_bytes[si] = row_bytes[si];
    a.gathered[si] = gathered[si];
  }
  a.B = B;
  a.blk = blk;
  a.nsets = nsets;
  a.cap = cap;
  a.offsets = offsets;
  a.kept_pos = kept_pos;
  return FOCUS_OK;
}

int compact_common(const uint8_t* keep, int B, int blk, int nsets, const void* const* rows,
                   const int64_t* row_bytes, void* const* gathered, int cap, int32_t* offsets,
                   int32_t* kept_pos, hipStream_t stream) {
  if (!keep) return FOCUS_ERR_INVALID_ARG;
  focus::CompactArgs a;
  const int rc =
      compact_prepare(B, blk, nsets, rows, row_bytes, gathered, cap, offsets, kept_pos, a);
  if (rc != FOCUS_OK) return rc;
  if (!aligned4(keep)) return FOCUS_ERR_INVALID_ARG;
  a.keep = keep;
  return status_of(focus::launch_compact(a, stream));
}
}  // namespace

int focus_compact(const uint8_t* keep, int B, int blk, const void* rows, int64_t row_bytes,
                  int cap, int32_t* offsets, int32_t* kept_pos, void* gathered,
                  hipStream_t stream) {
  if ((rows == nullptr) != (gathered == nullptr)) return FOCUS_ERR_INVALID_ARG;
  if (rows && row_bytes <= 0) return FOCUS_ERR_INVALID_ARG;
  return compact_common(keep, B, blk, rows ? 1 : 0, &rows, &row_bytes, &gathered, cap, offsets,
                        kept_pos, stream);
}

int focus_compact_multi(const uint8_t* keep, int B, int blk, int nsets, const void* const* rows,
                        const int64_t* row_bytes, void* const* gathered, int cap,
                        int32_t* offsets, int32_t* kept_pos, hipStream_t stream) {
  return compact_common(keep, B, blk, nsets, rows, row_bytes, gathered, cap, offsets, kept_pos,
                        stream);
}

namespace {
// The two launches of focus_score_select_compact, validated and ready to go.
struct FrontEnd {
  focus::ScoreArgs sa;
  focus::SelectCompactArgs a;
};

int front_end_prepare(const void* q0, const void* k0, const void* q1, const void* k1, int dtype,
                      int B, int blk, int Hq, int Hkv, int d, float sm_scale,
                      const uint8_t* masked, const int32_t* budget, float* delta, uint8_t* keep,
                      int32_t* kept_count, int nsets, const void* const* rows,
                      const int64_t* row_bytes, void* const* gathered, int cap,
                      int32_t* offsets, int32_t* kept_pos, int max_kept, void* workspace,
                      size_t workspace_bytes, FrontEnd& fe) {
  if (!masked || !budget || !keep || !kept_count) return FOCUS_ERR_INVALID_ARG;
  if (max_kept < 1 || max_kept > blk) return FOCUS_ERR_INVALID_ARG;
  focus::ScoreArgs& sa = fe.sa;
  int rc = score_prepare(q0, k0, q1, k1, nullptr, nullptr, dtype, B, blk, Hq, Hkv, d, sm_scale,
                         delta, workspace, workspace_bytes, sa);
  if (rc != FOCUS_OK) return rc;
  focus::CompactArgs ca;
  rc = compact_prepare(B, blk, nsets, rows, row_bytes, gathered, cap, offsets, kept_pos, ca);
  if (rc != FOCUS_OK) return rc;
  if (!aligned4(masked)) return FOCUS_ERR_INVALID_ARG;
  sa.partial_only = 1;
  focus::SelectCompactArgs& a = fe.a;
  a = focus::SelectCompactArgs{};
  a.part = sa.part;
  a.Hkv = Hkv;
  a.delta = delta;
  a.sel.masked = masked;
  a.sel.budget = budget;
  a.sel.adaptive = 0;
  a.sel.B = B;
  a.sel.blk = blk;
  a.sel.keep = keep;
  a.sel.kept_count = kept_count;
  a.cmp = ca;
  // workgroups per request: one 32 KiB gather batch each for max_kept rows of every set
  int64_t bytes = 0;
  for (int si = 0; si < nsets; ++si) bytes += row_bytes[si];
  const int64_t per_wg = 256 * 8 * 16;
  a.nsplit = (int)std::min<int64_t>(
      16, std::max<int64_t>(1, (max_kept * bytes + per_wg - 1) / per_wg));
  // the score launch writes the offsets (from the masks and budgets), the second reads them
  sa.scan_offsets = 1;
  sa.sel = a.sel;
  sa.offsets = offsets;
  return FOCUS_OK;
}

int front_end_launch(const FrontEnd& fe, hipStream_t stream) {
  if (focus::launch_score(fe.sa, stream) != hipSuccess) return FOCUS_ERR_HIP;
  return status_of(focus::launch_select_compact(fe.a, stream));
}

}  // namespace

int focus_score_select_compact(const void* q0, const void* k0, const void* q1, const void* k1,
                               int dtype, int B, int blk, int Hq, int Hkv, int d, float sm_scale,
                               const uint8_t* masked, const int32_t* budget, float* delta,
                               uint8_t* keep, int32_t* kept_count, int nsets,
                               const void* const* rows, const int64_t* row_bytes,
                               void* const* gathered, int cap, int32_t* offsets,
                               int32_t* kept_pos, int max_kept, void* workspace,
                               size_t workspace_bytes, hipStream_t stream) {
  FrontEnd fe;
  const int rc = front_end_prepare(q0, k0, q1, k1, dtype, B, blk, Hq, Hkv, d, sm_scale, masked,
                                   budget, delta, keep, kept_count, nsets, rows, row_bytes,
                                   gathered, cap, offsets, kept_pos, max_kept, workspace,
                                   workspace_bytes, fe);
  if (rc != FOCUS_OK) return rc;
  return front_end_launch(fe, stream);
}

size_t focus_noalloc_scratch_bytes(void) { return kScratchBytes; }

int focus_score_select_compact_noalloc(const void* q0, const void* k0, const void* q1,
                                       const void* k1, int dtype, int B, int blk, int Hq,
                                       int Hkv, int d, float sm_scale, const uint8_t* masked,
                                       const int32_t* budget, float* delta, uint8_t* keep,
                                       int32_t* kept_count, int nsets, const void* const* rows,
                                       const int64_t* row_bytes, void* const* gathered, int cap,
                                       int32_t* offsets, int32_t* kept_pos, int max_kept,
                                       hipStream_t stream) {
  // every argument is checked before the device is touched; the partials must fit the array
  if (B > 0 && blk > 0 && Hkv > 0 && focus::score_workspace_bytes(B, blk, Hkv) > kScratchBytes)
    return FOCUS_ERR_UNSUPPORTED;
  FrontEnd fe;
  // validated against a stand-in workspace of the scratch's size (never dereferenced)
  int rc = front_end_prepare(q0, k0, q1, k1, dtype, B, blk, Hq, Hkv, d, sm_scale, masked,
                             budget, delta, keep, kept_count, nsets, rows, row_bytes, gathered,
                             cap, offsets, kept_pos, max_kept, reinterpret_cast<void*>(256),
                             kScratchBytes, fe);
  if (rc != FOCUS_OK) return rc;
  void* ptr = nullptr;
  rc = scratch_address(&ptr);
  if (rc != FOCUS_OK) return rc;
  fe.sa.part = static_cast<float*>(ptr);
  fe.a.part = static_cast<const float*>(ptr);
  return front_end_launch(fe, stream);
}

size_t focus_ragged_paged_attn_workspace_size(int B, int blk, int Hq, int Hkv, int d, int S,
                                              int max_pages, int max_kept) {
  if (B <= 0 || blk <= 0 || !group_ok(Hq, Hkv) || d <= 0 || S <= 0 || max_pages < 0 ||
      max_kept <= 0)
    return 0;
  // enough for the call with the output and for the log-sum-exp-only call
  return std::max(focus::plan_attn(B, blk, Hq, Hkv, d, S, max_pages, max_kept).ws_bytes,
                  focus::plan_attn(B, blk, Hq, Hkv, d, S, max_pages, max_kept, true).ws_bytes);
}

namespace {

// The attention's checks and launch; q_pos == nullptr: q holds the compacted rows [cap, Hq, d],
// else the block's queries [B, blk, Hq, d], read at q_pos (call 4b).
int attn_call(const void* q, const int32_t* q_pos, const int32_t* offsets, int cap,
              const void* k_cache, const void* v_cache, int num_pages,
              const int32_t* page_table, int max_pages, const int32_t* prefix_len,
              const void* k_blk, const void* v_blk, int B, int blk, int Hq, int Hkv, int d, int S,
              int max_kept, float sm_scale, void* out, float* lse, void* workspace,
              size_t workspace_bytes, bool positional, hipStream_t stream) {
  // out == NULL: log-sum-exp only (lse required; the values are then not read and may be NULL)
  const bool lse_only = out == nullptr;
  if (!offsets || !prefix_len || !k_blk || (!lse_only && !v_blk)) return FOCUS_ERR_INVALID_ARG;
  if (cap > 0 && (!q || (lse_only && !lse))) return FOCUS_ERR_INVALID_ARG;
  if (positional && cap > 0 && !q_pos) return FOCUS_ERR_INVALID_ARG;
  if (positional && lse_only && cap > 0) return FOCUS_ERR_UNSUPPORTED;  // with the output only
  if (B <= 0 || blk <= 0 || Hq <= 0 || Hkv <= 0 || d <= 0 || S <= 0 || cap < 0 ||
      num_pages < 0 || max_pages < 0 || max_kept <= 0)
    return FOCUS_ERR_INVALID_ARG;
  if (max_pages > 0 && (!k_cache || (!lse_only && !v_cache) || !page_table || num_pages <= 0))
    return FOCUS_ERR_INVALID_ARG;
  if (!(sm_scale > 0.f) || !std::isfinite(sm_scale)) return FOCUS_ERR_INVALID_ARG;
  if (Hq % Hkv != 0 || max_kept > blk) return FOCUS_ERR_INVALID_ARG;
  if (!group_ok(Hq, Hkv) || Hkv > 64) return FOCUS_ERR_UNSUPPORTED;
  if ((d != 64 && d != 128) || !pow2_in(S, 16, 64) || !pow2_in(blk, 16, 64) || B > kMaxB)
    return FOCUS_ERR_UNSUPPORTED;
  if ((long long)max_pages * S > (1LL << 24)) return FOCUS_ERR_UNSUPPORTED;
  // (page, kv head) block indices are 32-bit in the kernel
  if ((long long)num_pages * Hkv >= (1LL << 32)) return FOCUS_ERR_UNSUPPORTED;
  if (!aligned16(q) || !aligned16(k_blk) || !aligned16(v_blk) || !aligned16(out) ||
      (k_cache && !aligned16(k_cache)) || (v_cache && !aligned16(v_cache)))
    return FOCUS_ERR_INVALID_ARG;
  const focus::AttnPlan plan =
      focus::plan_attn(B, blk, Hq, Hkv, d, S, max_pages, max_kept, lse_only);
  if (plan.tiles_bound >= (1LL << 31) || plan.ngroups < 1) return FOCUS_ERR_UNSUPPORTED;
  if (!workspace || workspace_bytes < plan.ws_bytes) return FOCUS_ERR_WORKSPACE;
  if (cap == 0) return FOCUS_OK;
  focus::AttnArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.q_pos = positional ? q_pos : nullptr;
  a.offsets = offsets;
  a.cap = cap;
  a.k_cache = static_cast<const uint16_t*>(k_cache);
  a.v_cache = static_cast<const uint16_t*>(v_cache);
  a.num_pages = num_pages;
  a.page_table = page_table;
  a.max_pages = max_pages;
  a.prefix_len = prefix_len;
  a.k_blk = static_cast<const uint16_t*>(k_blk);
  a.v_blk = static_cast<const uint16_t*>(v_blk);
  a.B = B;
  a.blk = blk;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.d = d;
  a.S = S;
  a.max_kept = max_kept;
  a.scale_log2 = sm_scale * 1.4426950408889634f;
  a.out = static_cast<uint16_t*>(out);
  a.lse = lse;
  a.workspace = workspace;
  return status_of(focus::launch_attn(a, plan, stream));
}

}  // namespace

int focus_ragged_paged_attn(const void* q, const int32_t* offsets, int cap, const void* k_cache,
                            const void* v_cache, int num_pages, const int32_t* page_table,
                            int max_pages, const int32_t* prefix_len, const void* k_blk,
                            const void* v_blk, int B, int blk, int Hq, int Hkv, int d, int S,
                            int max_kept, float sm_scale, void* out, float* lse, void* workspace,
                            size_t workspace_bytes, hipStream_t stream) {
  return attn_call(q, nullptr, offsets, cap, k_cache, v_cache, num_pages, page_table, max_pages,
                   prefix_len, k_blk, v_blk, B, blk, Hq, Hkv, d, S, max_kept, sm_scale, out, lse,
                   workspace, workspace_bytes, false, stream);
}

int focus_ragged_paged_attn_pos(const void* q_block, const int32_t* kept_pos,
                                const int32_t* offsets, int cap, const void* k_cache,
                                const void* v_cache, int num_pages, const int32_t* page_table,
                                int max_pages, const int32_t* prefix_len, const void* k_blk,
                                const void* v_blk, int B, int blk, int Hq, int Hkv, int d, int S,
                                int max_kept, float sm_scale, void* out, float* lse,
                                void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return attn_call(q_block, kept_pos, offsets, cap, k_cache, v_cache, num_pages, page_table,
                   max_pages, prefix_len, k_blk, v_blk, B, blk, Hq, Hkv, d, S, max_kept, sm_scale,
                   out, lse, workspace, workspace_bytes, true, stream);
}


int focus_kv_writeback(const void* k_rows, const void* v_rows, const int32_t* offsets,
                       const int32_t* kept_pos, int cap, int B, int blk, int Hkv, int d,
                       void* k_blk, void* v_blk, hipStream_t stream) {
  if (!k_rows || !v_rows || !offsets || !kept_pos || !k_blk || !v_blk) return FOCUS_ERR_INVALID_ARG;
  if (cap < 0 || B <= 0 || blk <= 0 || Hkv <= 0 || d <= 0) return FOCUS_ERR_INVALID_ARG;
  if (!pow2_in(blk, 16, 64) || (d != 64 && d != 128) || Hkv > 64 || B > kMaxB)
    return FOCUS_ERR_UNSUPPORTED;
  if (!aligned16(k_rows) || !aligned16(v_rows) || !aligned16(k_blk) || !aligned16(v_blk))
    return FOCUS_ERR_INVALID_ARG;
  if (cap == 0) return FOCUS_OK;
  focus::WritebackArgs a{};
  a.k_rows = static_cast<const uint16_t*>(k_rows);
  a.v_rows = static_cast<const uint16_t*>(v_rows);
  a.offsets = offsets;
  a.kept_pos = kept_pos;
  a.cap = cap;
  a.B = B;
  a.blk = blk;
  a.Hkv = Hkv;
  a.d = d;
  a.k_blk = static_cast<uint16_t*>(k_blk);
  a.v_blk = static_cast<uint16_t*>(v_blk);
  return status_of(focus::launch_writeback(a, stream));
}

int focus_block_commit(const uint8_t* commit, const void* k_blk, const void* v_blk, int B,
                       int blk, int Hkv, int d, int S, void* k_cache, void* v_cache,
                       int num_pages, int32_t* page_table, int max_pages,
                       const int32_t* prefix_len_in, int32_t* prefix_len_out,
                       const int32_t* free_pages, int free_cap, const int32_t* free_count_in,
                       int32_t* free_count_out, int32_t* status, hipStream_t stream) {
  if (!commit || !k_blk || !v_blk || !k_cache || !v_cache || !page_table || !prefix_len_in ||
      !prefix_len_out || !free_count_in || !free_count_out || !status)
    return FOCUS_ERR_INVALID_ARG;
  if (free_cap > 0 && !free_pages) return FOCUS_ERR_INVALID_ARG;
  if (B <= 0 || blk <= 0 || Hkv <= 0 || d <= 0 || S <= 0 || num_pages <= 0 || max_pages <= 0 ||
      free_cap < 0)
    return FOCUS_ERR_INVALID_ARG;
  if (prefix_len_in == prefix_len_out || free_count_in == free_count_out)
    return FOCUS_ERR_INVALID_ARG;
  if (!pow2_in(blk, 16, 64) || !pow2_in(S, 16, 64) || (d != 64 && d != 128) || Hkv > 64 ||
      B > kMaxB || (long long)max_pages * S > (1LL << 24))
    return FOCUS_ERR_UNSUPPORTED;
  if (!aligned16(k_blk) || !aligned16(v_blk) || !aligned16(k_cache) || !aligned16(v_cache))
    return FOCUS_ERR_INVALID_ARG;
  focus::CommitArgs a{};
  a.commit = commit;
  a.k_blk = static_cast<const uint16_t*>(k_blk);
  a.v_blk = static_cast<const uint16_t*>(v_blk);
  a.B = B;
  a.blk = blk;
  a.Hkv = Hkv;
  a.d = d;
  a.S = S;
  a.k_cache = static_cast<uint16_t*>(k_cache);
  a.v_cache = static_cast<uint16_t*>(v_cache);
  a.num_pages = num_pages;
  a.page_table = page_table;
  a.max_pages = max_pages;
  a.prefix_len_in = prefix_len_in;
  a.prefix_len_out = prefix_len_out;
  a.free_pages = free_pages;
  a.free_cap = free_cap;
  a.free_count_in = free_count_in;
  a.free_count_out = free_count_out;
  a.status = status;
  return status_of(focus::launch_commit(a, stream));
}

int focus_kv_pack(const void* k_src, const void* v_src, int layout, int n_blocks, int Hkv, int S,
                  int d, void* k_out, void* v_out, hipStream_t stream) {
  if ((k_src == nullptr) != (k_out == nullptr) || (v_src == nullptr) != (v_out == nullptr))
    return FOCUS_ERR_INVALID_ARG;
  if (k_src == nullptr && v_src == nullptr) return FOCUS_ERR_INVALID_ARG;
  if (n_blocks <= 0 || Hkv <= 0 || S <= 0 || d <= 0) return FOCUS_ERR_INVALID_ARG;
  if (layout != FOCUS_KV_HEAD_MAJOR && layout != FOCUS_KV_TOKEN_MAJOR) return FOCUS_ERR_UNSUPPORTED;
  if (!pow2_in(S, 16, 64) || (d != 64 && d != 128) || Hkv > 64) return FOCUS_ERR_UNSUPPORTED;
  if ((int64_t)n_blocks * Hkv > INT32_MAX) return FOCUS_ERR_UNSUPPORTED;
  const void* ptrs[4] = {k_src, v_src, k_out, v_out};
  for (const void* p : ptrs)
    if (p != nullptr && !aligned16(p)) return FOCUS_ERR_INVALID_ARG;
  // no output may overlap an input or the other output
  const uintptr_t bytes = (uintptr_t)n_blocks * Hkv * S * d * sizeof(uint16_t);
  auto overlap = [&](const void* x, const void* y) {
    if (x == nullptr || y == nullptr) return false;
    const uintptr_t a = reinterpret_cast<uintptr_t>(x), b = reinterpret_cast<uintptr_t>(y);
    return a < b + bytes && b < a + bytes;
  };
  if (overlap(k_out, k_src) || overlap(k_out, v_src) || overlap(v_out, k_src) ||
      overlap(v_out, v_src) || overlap(k_out, v_out))
    return FOCUS_ERR_INVALID_ARG;
  focus::PackArgs a{};
  a.k_src = static_cast<const uint16_t*>(k_src);
  a.v_src = static_cast<const uint16_t*>(v_src);
  a.token_major = layout == FOCUS_KV_TOKEN_MAJOR;
  a.n_blocks = n_blocks;
  a.Hkv = Hkv;
  a.S = S;
  a.d = d;
  a.k_out = static_cast<uint16_t*>(k_out);
  a.v_out = static_cast<uint16_t*>(v_out);
  return status_of(focus::launch_kv_pack(a, stream));
}

}  // extern "C"
