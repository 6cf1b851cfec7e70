// Host-side launchers of the gfx950 kernels (one per .hip file); called by the C ABI after it
// has validated every argument.  Each returns hipSuccess or the launch error.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace focus {

constexpr int kMaxB = 4096;  // largest batch of every call

struct SelectArgs {
  const float* delta;
  const uint8_t* masked;
  const int32_t* budget;
  int adaptive;
  float beta;
  int lo, hi;
  int B, blk;
  uint8_t* keep;
  int32_t* kept_count;
};

hipError_t launch_select(const SelectArgs& a, hipStream_t s);

constexpr int kMaxSets = 2;  // row sets gathered by one compaction launch
struct CompactArgs {
  const uint8_t* keep;
  int B, blk;
  int nsets;                      // 0 (offsets and positions only) .. kMaxSets
  const void* rows[kMaxSets];     // [B, blk, row_bytes[s]]
  int64_t row_bytes[kMaxSets];
  void* gathered[kMaxSets];       // [cap, row_bytes[s]]
  int cap;
  int32_t* offsets;
  int32_t* kept_pos;
};
hipError_t launch_compact(const CompactArgs& a, hipStream_t s);

// Reduction of the score partials + selection with caller budgets + compaction: the second
// launch of the front end (the score launch has written the offsets).
struct SelectCompactArgs {
  const float* part;  // [B, Hkv, blk] score partials
  int Hkv;
  float* delta;       // [B, blk] output
  SelectArgs sel;     // masked, budget, keep, kept_count, B, blk (adaptive = 0)
  CompactArgs cmp;    // row sets, cap, offsets, kept_pos (keep unused)
  int nsplit;         // workgroups per request (each gathers a share of its rows), 1..16
};
hipError_t launch_select_compact(const SelectCompactArgs& a, hipStream_t s);

struct ScoreArgs {
  const void* q0;
  const void* k0;
  const void* q1;
  const void* k1;
  int is_bf16;
  int B, blk, Hq, Hkv, d;
  float scale_log2;  // sm_scale * log2(e)
  const float* lse0; // [B, blk, Hq] full-domain row log-sum-exp of layer 0, or null (block-only)
  const float* lse1; // same for layer 1
  float* delta;      // [B, blk]
  float* part;       // workspace [B, Hkv, blk]
  int fuse_select;   // run the selection of each request right after its delta
  SelectArgs sel;    // (delta unused: the request's delta is in registers)
  int partial_only;  // stop after the per-kv-head partials (a later kernel reduces them)
  // Front end with per-request budgets (block-only domain): the score launch also writes the
  // compacted offsets from sel.masked and sel.budget, which launch_select_compact then reads.
  int scan_offsets;
  int32_t* offsets;  // [B+1]
};
size_t score_workspace_bytes(int B, int blk, int Hkv);
hipError_t launch_score(const ScoreArgs& a, hipStream_t s);

struct AttnArgs {
  const uint16_t* q;       // [cap, Hq, d], or [B, blk, Hq, d] read at q_pos
  const int32_t* q_pos;    // null or [cap] (kept positions)
  const int32_t* offsets;
  int cap;
  const uint16_t* k_cache;
  const uint16_t* v_cache;
  int num_pages;
  const int32_t* page_table;
  int max_pages;
  const int32_t* prefix_len;
  const uint16_t* k_blk;
  const uint16_t* v_blk;
  int B, blk, Hq, Hkv, d, S;
  int max_kept;
  float scale_log2;
  uint16_t* out;
  float* lse;
  void* workspace;
};
struct AttnPlan {
  bool shared;           // the four waves of a workgroup share each tile (several query groups)
  int qt;                // 16-row query tiles per wave (1, 2 or 4)
  int nqg;               // query groups per (request, kv head) at max_kept
  int wgs;               // persistent workgroups (4 waves each)
  int gs;                // waves per column group: one per (kv head, query group)
  int ngroups;           // column groups in the grid (0: Hkv * nqg exceeds the grid)
  long long tiles_bound; // 32-key columns of all requests at the longest possible prefixes
  size_t cnt_bytes;      // arrival counters of cut items (zero between calls)
  size_t ws_o_bytes;     // partial outputs of items cut by slice boundaries
  size_t ws_ml_bytes;    // their running max / sum
  size_t ws_bytes;       // total workspace
};
// lse_only: the plan of the log-sum-exp-only mode (its workspace never exceeds the full one's)
AttnPlan plan_attn(int B, int blk, int Hq, int Hkv, int d, int S, int max_pages, int max_kept,
                   bool lse_only = false);
hipError_t launch_attn(const AttnArgs& a, const AttnPlan& plan, hipStream_t s);

struct WritebackArgs {
  const uint16_t* k_rows;  // [cap, Hkv, d]
  const uint16_t* v_rows;  // [cap, Hkv, d]
  const int32_t* offsets;  // [B+1]
  const int32_t* kept_pos; // [cap]
  int cap, B, blk, Hkv, d;
  uint16_t* k_blk;         // [B, Hkv, d/8, blk, 8]
  uint16_t* v_blk;         // [B, Hkv, blk/8, d, 8]
};
hipError_t launch_writeback(const WritebackArgs& a, hipStream_t s);

struct CommitArgs {
  const uint8_t* commit;   // [B]
  const uint16_t* k_blk;
  const uint16_t* v_blk;
  int B, blk, Hkv, d, S;
  uint16_t* k_cache;
  uint16_t* v_cache;
  int num_pages;
  int32_t* page_table;     // [B, max_pages]
  int max_pages;
  const int32_t* prefix_len_in;
  int32_t* prefix_len_out;
  const int32_t* free_pages;  // [free_cap]
  int free_cap;
  const int32_t* free_count_in;
  int32_t* free_count_out;
  int32_t* status;
};
hipError_t launch_commit(const CommitArgs& a, hipStream_t s);

// Conversion of plain token-row K/V into the MFMA-native layouts above.
struct PackArgs {
  const uint16_t* k_src;   // [n, Hkv, S, d] (token_major = 0) or [n, S, Hkv, d]; null: no K
  const uint16_t* v_src;   // same; null: no V
  int token_major;
  int n_blocks, Hkv, S, d;
  uint16_t* k_out;         // [n, Hkv, d/8, S, 8]
  uint16_t* v_out;         // [n, Hkv, S/8, d, 8]
};
hipError_t launch_kv_pack(const PackArgs& a, hipStream_t s);

}  // namespace focus
