/*
 * focus.h -- C ABI of the focused block-diffusion step on AMD Instinct MI355X (gfx950).
 *
 * The step (FOCUS, "DLLMs Know How to Tame Their Compute Bound", arXiv 2601.23278):
 *   1. focus_score_l01        importance delta of every block token, layer 1 minus layer 0
 *   2. focus_select_budget    keep the k_r masked tokens with the largest delta
 *   3. focus_compact          ragged offsets + kept positions, gather of the kept rows
 *   4. focus_ragged_paged_attn  kept queries against paged prefix KV plus intra-block KV
 *
 * Conventions shared by every entry point
 *   - Every pointer argument is DEVICE memory owned by the caller, unless stated otherwise.
 *     No call allocates, frees or retains memory; the one memory the library owns is the fixed
 *     device array of call 3c, which exists from the moment its code is loaded on a GPU.
 *   - Every call is asynchronous on `stream` (0 = the default stream). No call synchronises
 *     the host; ragged sizes (kept counts, offsets, prefix lengths) never leave the device.
 *   - A negative return value is a host-detected argument error: nothing was launched.
 *     FOCUS_ERR_HIP reports a launch error from the HIP runtime.
 *   - bf16 is IEEE bfloat16 stored as 16-bit words; f32 is IEEE binary32.
 *   - Indices are row-major; shapes are written outermost first.
 *   - All results are deterministic: reductions run in a fixed order, no float atomics.
 */
#ifndef FOCUS_H_
#define FOCUS_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FOCUS_OK = 0,
  FOCUS_ERR_INVALID_ARG = -1, /* null pointer, non-positive size, inconsistent sizes          */
  FOCUS_ERR_UNSUPPORTED = -2, /* a size outside the supported set (listed per call)          */
  FOCUS_ERR_WORKSPACE = -3,   /* workspace missing or smaller than the *_workspace_size value */
  FOCUS_ERR_HIP = -4          /* the HIP runtime reported a launch error                       */
} focus_status;

typedef enum { FOCUS_F32 = 0, FOCUS_BF16 = 1 } focus_dtype;

/* Human-readable name of a status code (static storage; never NULL). */
const char* focus_status_string(int code);

/* Library version, major*10000 + minor*100 + patch. */
int focus_version(void);

/* --------------------------------------------------------------------------------------------
 * 1. Importance scoring.
 *
 * Defined by the project page (focus-inference.github.io), Overview cards "Design" (importance
 * from the early layers' Q/K projections) and "Decodability Signal" (the layer-0 to layer-1
 * change of importance separates decodable tokens), and by the paper's abstract (importance is
 * attention-derived).  For request r, layer l in {0,1}, query head h (kv head g = h / (Hq/Hkv)):
 *     P = softmax_j( sm_scale * q_l[r,i,h,:] . k_l[r,j,g,:] )     (over the blk block keys j)
 *     I_l[r,j] = sum_h sum_i P[i,j]
 *     delta[r,j] = I_1[r,j] - I_0[r,j]                              (every position j)
 *
 *   q0, q1      [B, blk, Hq, d]   layer-0 / layer-1 block queries, dtype `dtype`
 *   k0, k1      [B, blk, Hkv, d]  layer-0 / layer-1 block keys,    dtype `dtype`
 *   dtype       FOCUS_F32 or FOCUS_BF16 (products accumulate in f32)
 *   delta       [B, blk] f32 output
 *   workspace   device scratch of at least focus_score_l01_workspace_size(...) bytes (per-kv-head
 *               partial sums; no initialisation); calls that share a workspace must not run
 *               concurrently
 * Supported: blk in {16,32,64}; d in {64,128}; Hq % Hkv == 0; Hq/Hkv in {1,2,4,8};
 *            1 <= B <= 4096; Hkv <= 64.  Pointers must be 16-byte aligned.
 * ------------------------------------------------------------------------------------------ */
size_t focus_score_l01_workspace_size(int B, int blk, int Hq, int Hkv, int d);
int focus_score_l01(const void* q0, const void* k0, const void* q1, const void* k1, int dtype,
                    int B, int blk, int Hq, int Hkv, int d, float sm_scale, float* delta,
                    void* workspace, size_t workspace_bytes, hipStream_t stream);

/* --------------------------------------------------------------------------------------------
 * 1b. Importance scoring over the full attention domain.
 *
 * The other reading of the importance in call 1 (project page, card "Design": importance from
 * the early layers' attention): the softmax of each block query runs over the layer's whole key
 * set -- the request's prefix tokens and the block -- and a block token's importance is the
 * weight it receives there:
 *     P = exp( sm_scale * q_l[r,i,h,:] . k_l[r,j,g,:] - lse_l[r,i,h] )    (block keys j only)
 *     I_l[r,j] = sum_h sum_i P,   delta[r,j] = I_1[r,j] - I_0[r,j]
 * lse_l[r,i,h] is the natural-log log-sum-exp of sm_scale * q . k over all keys (prefix and
 * block) of layer l, e.g. the `lse` output of focus_ragged_paged_attn run on every block query
 * of that layer (rows r*blk + i).  The prefix keys themselves are not read.
 *
 *   lse0, lse1  [B, blk, Hq] f32 (4-byte aligned), device memory
 *   everything else as in focus_score_l01 (same workspace size and rules, same supported set)
 * ------------------------------------------------------------------------------------------ */
int focus_score_l01_lse(const void* q0, const void* k0, const void* q1, const void* k1,
                        const float* lse0, const float* lse1, int dtype, int B, int blk, int Hq,
                        int Hkv, int d, float sm_scale, float* delta, void* workspace,
                        size_t workspace_bytes, hipStream_t stream);

/* --------------------------------------------------------------------------------------------
 * 2. Budgeted selection (target token selection).
 *
 * Defined by the project page, cards "Design" (keep likely-decodable candidates under an
 * adaptive budget) and "Runtime Action" (dynamic budgeting, token eviction), and by the AI
 * Engineering Academy article's "Arquitetura do FOCUS" section (target token selection).
 * Candidates of request r are its masked positions (masked[r,j] != 0); m_r is their number.
 *   adaptive == 0:  b_r = budget[r]
 *   adaptive != 0:  over the candidates, mu = mean(delta), sigma = population std (both f32),
 *                   c = #{delta > mu + beta*sigma}, b_r = min(max(c, lo), hi)
 *   k_r = min(max(b_r, 0), m_r); the k_r candidates with the largest delta are kept, equal
 *   deltas ordered by lower position first, a delta that is not a number ranked as -infinity
 *   (so exactly k_r are kept).  Decoded positions are never kept.
 *
 *   delta       [B, blk] f32         masked [B, blk] u8      budget [B] i32 (ignored if adaptive)
 *   keep        [B, blk] u8 output (1 = kept)                kept_count [B] i32 output
 * Supported: blk in {16,32,64}; 1 <= B <= 4096.
 * ------------------------------------------------------------------------------------------ */
int focus_select_budget(const float* delta, const uint8_t* masked, const int32_t* budget,
                        int adaptive, float beta, int lo, int hi, int B, int blk, uint8_t* keep,
                        int32_t* kept_count, hipStream_t stream);

/* --------------------------------------------------------------------------------------------
 * 2b. Scoring and selection in one launch.
 *
 * The same results as focus_score_l01 followed by focus_select_budget with the same arguments
 * (delta is written too): the kernel that completes each request's importance runs the request's
 * selection right away, saving a launch and a round trip of delta through memory.
 * Arguments, workspace and supported set: the union of the two calls'.
 * ------------------------------------------------------------------------------------------ */
int focus_score_select(const void* q0, const void* k0, const void* q1, const void* k1,
                       int dtype, int B, int blk, int Hq, int Hkv, int d, float sm_scale,
                       const uint8_t* masked, const int32_t* budget, int adaptive, float beta,
                       int lo, int hi, float* delta, uint8_t* keep, int32_t* kept_count,
                       void* workspace, size_t workspace_bytes, hipStream_t stream);

/* --------------------------------------------------------------------------------------------
 * 3. Compaction + gather (state compaction, ragged execution).
 *
 * Defined by the AI Engineering Academy article's "Arquitetura do FOCUS" section (the state is
 * compacted and evicted tokens dropped) and the project page's "Runtime Action" card (ragged
 * execution over the kept tokens).
 *   offsets[0] = 0, offsets[r+1] = offsets[r] + #{j : keep[r,j] != 0}     (offsets[B] = T)
 *   kept_pos[offsets[r] + t] = t-th kept position of request r, ascending
 *   gathered[n, :] = rows[r, kept_pos[n], :]   (byte copy of row_bytes bytes)
 * Entries n >= cap of kept_pos / gathered are not written; offsets always holds the true totals,
 * so offsets[B] > cap reveals an overflow after the caller synchronises.  cap >= B*blk always
 * suffices.  One workgroup per request writes its positions and gathers its rows; its place in
 * the order is counted by the workgroup itself up to 2048 requests, and above that by a first
 * launch, one workgroup scanning the kept counts into offsets (O(B)).
 *
 *   keep        [B, blk] u8
 *   rows        [B, blk, row_bytes] bytes, or NULL (then gathered must be NULL: offsets only)
 *   offsets     [B+1] i32 output        kept_pos [cap] i32 output (may be NULL)
 *   gathered    [cap, row_bytes] output, or NULL
 * Supported: blk in {16,32,64}; 1 <= B <= 4096; row_bytes > 0, a multiple of 16 and at most
 *            2^24; rows and gathered 16-byte aligned; keep 4-byte aligned.
 * ------------------------------------------------------------------------------------------ */
int focus_compact(const uint8_t* keep, int B, int blk, const void* rows, int64_t row_bytes,
                  int cap, int32_t* offsets, int32_t* kept_pos, void* gathered,
                  hipStream_t stream);

/* Compaction gathering several row sets at once (e.g. the hidden states and the attention
 * queries): the same as focus_compact on each set, offsets/kept_pos written once.
 *   rows[s], row_bytes[s], gathered[s] for s < nsets: HOST arrays of device pointers / sizes
 *   (read during the call only); each set as in focus_compact.
 * Supported: 0 <= nsets <= 2, otherwise as focus_compact. */
int focus_compact_multi(const uint8_t* keep, int B, int blk, int nsets, const void* const* rows,
                        const int64_t* row_bytes, void* const* gathered, int cap,
                        int32_t* offsets, int32_t* kept_pos, hipStream_t stream);

/* --------------------------------------------------------------------------------------------
 * 3b. Scoring, selection with per-request budgets and compaction in two launches.
 *
 * The same results as focus_score_select (adaptive == 0) followed by focus_compact_multi on its
 * keep output: delta, keep, kept_count, offsets, kept_pos and the gathered rows.  With the
 * caller's integer budgets, request r keeps k_r = min(max(budget[r], 0), m_r) tokens, a number
 * known from the mask alone, so each request's place in the compacted order follows from the
 * masks and budgets of the requests before it: one workgroup of the scoring launch scans them
 * into offsets (O(B)), and the second launch reduces the importance, selects and gathers each
 * request without waiting for the others.  (The adaptive rule needs
 * every request's delta first: use focus_score_select and focus_compact_multi for it.)
 * Arguments, workspace and supported set: those of the two calls; masked must be 4-byte
 * aligned.  max_kept (1..blk) is the caller's bound of the kept counts: it sizes the launch
 * (how many workgroups gather a request's rows), the results do not depend on it.
 * ------------------------------------------------------------------------------------------ */
int focus_score_select_compact(const void* q0, const void* k0, const void* q1, const void* k1,
                               int dtype, int B, int blk, int Hq, int Hkv, int d, float sm_scale,
                               const uint8_t* masked, const int32_t* budget, float* delta,
                               uint8_t* keep, int32_t* kept_count, int nsets,
                               const void* const* rows, const int64_t* row_bytes,
                               void* const* gathered, int cap, int32_t* offsets,
                               int32_t* kept_pos, int max_kept, void* workspace,
                               size_t workspace_bytes, hipStream_t stream);

/* --------------------------------------------------------------------------------------------
 * 3c. focus_score_select_compact for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.
 *
 * The same launches and results as focus_score_select_compact, without the workspace
 * arguments: the per-kv-head score partials (B*Hkv*blk*4 bytes) live in a library-owned device
 * array of focus_noalloc_scratch_bytes() bytes (4 MiB), one per GPU, which exists once the
 * library's code is loaded on that GPU and is held until the process ends.  The call allocates
 * nothing; its first call on a GPU looks the array's address up (issue that one before any
 * graph capture).  The partials need no initialisation, so nothing is cleared between calls.
 * All calls on one GPU share the array and it keeps the last call's contents: calls that may
 * overlap in time on the same GPU (several streams or threads) race on it and must not be
 * issued.
 * Returns FOCUS_ERR_UNSUPPORTED when B*Hkv*blk*4 exceeds the array (B = 4096, Hkv = 8, blk = 32
 * fits exactly), FOCUS_ERR_HIP if the array's address cannot be found; everything else as
 * focus_score_select_compact.
 * ------------------------------------------------------------------------------------------ */
size_t focus_noalloc_scratch_bytes(void);
int focus_score_select_compact_noalloc(const void* q0, const void* k0, const void* q1,
                                       const void* k1, int dtype, int B, int blk, int Hq,
                                       int Hkv, int d, float sm_scale, const uint8_t* masked,
                                       const int32_t* budget, float* delta, uint8_t* keep,
                                       int32_t* kept_count, int nsets, const void* const* rows,
                                       const int64_t* row_bytes, void* const* gathered, int cap,
                                       int32_t* offsets, int32_t* kept_pos, int max_kept,
                                       hipStream_t stream);

/* --------------------------------------------------------------------------------------------
 * 4. Ragged paged attention of the kept queries.
 *
 * Defined by the AI Engineering Academy article (ragged paged attention integrated with the
 * KV-cache management) and the project page's "Runtime Action" (ragged execution, intra-block
 * KV caching) and "Motivation" (block diffusion: earlier blocks exactly KV-cached, the block is
 * recomputed bidirectionally) cards.  Row n with offsets[r] <= n < offsets[r+1] is a kept token
 * of request r.  For each such row and query head h (kv head g = h / (Hq/Hkv)) the keys are the
 * request's prefix_len[r] cached tokens followed by all blk block tokens (no mask):
 *   z_t = sm_scale * q[n,h,:] . K_t,   lse[n,h] = log sum_t exp(z_t),
 *   out[n,h,:] = sum_t exp(z_t - lse[n,h]) V_t        (bf16 in, f32 accumulate, bf16 out)
 *
 * Layouts (bf16).  A page holds S consecutive tokens of one request for all kv heads:
 *   k_cache [num_pages, Hkv, d/8, S, 8]  key (page p, slot s, dim c) at [p, g, c/8, s, c%8]
 *   v_cache [num_pages, Hkv, S/8, d, 8]  value (p, s, c) at [p, g, s/8, c, s%8]
 *   k_blk   [B, Hkv, d/8, blk, 8], v_blk [B, Hkv, blk/8, d, 8]: the block KV, same layouts
 *   page_table [B, max_pages] i32: prefix token t of request r is in page page_table[r, t/S]
 *   prefix_len [B] i32
 *   q   [cap, Hq, d] bf16 (compacted queries)   out [cap, Hq, d] bf16   lse [cap, Hq] f32 or NULL
 *   (q and out may be NULL when cap == 0: the call then only checks its arguments)
 *   out == NULL with lse given: log-sum-exp only -- the values are not read (v_cache and v_blk
 *   may then be NULL), which halves the bytes and the matrix work.
 * max_kept is an upper bound of every kept count (offsets[r+1]-offsets[r]); it sizes the
 * launch.  Rows t >= max_kept of a request are not written.  Rows n >= cap are not read or
 * written.  Device data the host cannot check: a request whose prefix_len is negative or above
 * max_pages*S, or whose used page ids fall outside [0, num_pages), gets NaN in all its output
 * rows instead of a memory access.
 *   workspace   at least focus_ragged_paged_attn_workspace_size(...) bytes, ZERO-FILLED before its
 *               first use (it holds arrival counters that every call leaves at zero again, plus
 *               per-wave partial results).  Calls that share a workspace must not run
 *               concurrently; calls of different shapes may share one.  The size depends on the
 *               current device's compute-unit count.
 * Supported: d in {64,128}; S in {16,32,64}; blk in {16,32,64}; Hq/Hkv in {1,2,4,8};
 *            1 <= max_kept <= blk; 1 <= B <= 4096; max_pages*S <= 2^24; num_pages*Hkv < 2^32;
 *            fewer than 2^31 key
 *            tiles of 32 over all (request, kv head, query group) at the longest prefixes;
 *            pointers 16-byte aligned.
 * ------------------------------------------------------------------------------------------ */
size_t focus_ragged_paged_attn_workspace_size(int B, int blk, int Hq, int Hkv, int d, int S,
                                              int max_pages, int max_kept);
int focus_ragged_paged_attn(const void* q, const int32_t* offsets, int cap, const void* k_cache,
                            const void* v_cache, int num_pages, const int32_t* page_table,
                            int max_pages, const int32_t* prefix_len, const void* k_blk,
                            const void* v_blk, int B, int blk, int Hq, int Hkv, int d, int S,
                            int max_kept, float sm_scale, void* out, float* lse, void* workspace,
                            size_t workspace_bytes, hipStream_t stream);

/* --------------------------------------------------------------------------------------------
 * 4b. Ragged paged attention with the queries read in place.
 *
 * The same operation and results as call 4 (same section of the pages: ragged execution of the
 * kept tokens only), with the kept tokens' queries read from the block's query tensor at their
 * positions instead of from a compacted copy, so the compaction need not gather them: row n
 * (offsets[r] <= n < offsets[r+1]) has the query q_block[r, kept_pos[n], h, :].
 *   q_block  [B, blk, Hq, d] bf16;  kept_pos [cap] i32 (as produced by focus_compact or the
 *            fused front ends)
 *   every other argument, layout, workspace and supported size as in call 4, except that out
 *   is required (the log-sum-exp-only mode takes compacted queries: call 4).
 * Device data the host cannot check: a position outside [0, blk) gives NaN in all rows of its
 * request's kv-head group (as an invalid page id does) instead of a memory access.
 * ------------------------------------------------------------------------------------------ */
int focus_ragged_paged_attn_pos(const void* q_block, const int32_t* kept_pos,
                                const int32_t* offsets, int cap, const void* k_cache,
                                const void* v_cache, int num_pages, const int32_t* page_table,
                                int max_pages, const int32_t* prefix_len, const void* k_blk,
                                const void* v_blk, int B, int blk, int Hq, int Hkv, int d, int S,
                                int max_kept, float sm_scale, void* out, float* lse,
                                void* workspace, size_t workspace_bytes, hipStream_t stream);

/* --------------------------------------------------------------------------------------------
 * 5. Intra-block KV write-back.
 *
 * Project page, card "Runtime Action" (intra-block KV caching): the layer's fresh K/V of the kept
 * tokens replace the cached block KV at their positions; evicted positions keep their cached
 * values.  Row n (offsets[r] <= n < offsets[r+1], n < cap) is request r's token kept_pos[n]:
 *   k_blk[r, g, c/8, kept_pos[n], c%8] = k_rows[n, g, c]
 *   v_blk[r, g, kept_pos[n]/8, c, kept_pos[n]%8] = v_rows[n, g, c]
 *
 *   k_rows, v_rows  [cap, Hkv, d] bf16 (compacted order, e.g. from the gathered hidden rows)
 *   offsets [B+1], kept_pos [cap] i32 (as produced by focus_compact)
 *   k_blk [B, Hkv, d/8, blk, 8], v_blk [B, Hkv, blk/8, d, 8] bf16, updated in place
 * A row whose kept_pos is outside [0, blk) is skipped; at most blk rows of a request are read;
 * a position named by several rows of a request takes the last of those rows.
 * Supported: blk in {16,32,64}; d in {64,128}; Hkv <= 64; 1 <= B <= 4096; K/V pointers 16-byte
 * aligned.  cap == 0 does nothing.
 * ------------------------------------------------------------------------------------------ */
int focus_kv_writeback(const void* k_rows, const void* v_rows, const int32_t* offsets,
                       const int32_t* kept_pos, int cap, int B, int blk, int Hkv, int d,
                       void* k_blk, void* v_blk, hipStream_t stream);

/* --------------------------------------------------------------------------------------------
 * 6. Block commit: append finished blocks to the paged prefix.
 *
 * Project page, card "Motivation" (earlier blocks are exactly KV-cached); AI Engineering Academy
 * article, "Arquitetura do FOCUS" (KV-cache management).  For every request with commit[r] != 0
 * its whole block (blk tokens of k_blk/v_blk) becomes prefix positions P_r .. P_r+blk-1, with
 * P_r = prefix_len_in[r]: token t goes to page page_table[r, (P_r+t)/S], slot (P_r+t)%S.  The
 * ceil((P_r+blk)/S) - ceil(P_r/S) pages it needs beyond those it holds are popped from the top
 * of the free-page stack free_pages[0 .. free_count_in-1]: requests in batch order, each
 * request's pages in position order, written into page_table.  prefix_len_out[r] = P_r + blk
 * for committed requests, P_r otherwise; free_count_out = free_count_in - pages taken.
 *   status[0] = 0 done; 1 not enough free pages; 2 a committed request's prefix length is
 *   negative or P_r + blk exceeds max_pages*S; 3 invalid page data (free_count_in outside
 *   [0, free_cap], or a page id to be written outside [0, num_pages)).  On status != 0 nothing
 *   is written except status, prefix_len_out (= prefix_len_in) and free_count_out (= in).
 *
 *   commit [B] u8; k_blk, v_blk as in call 4; k_cache, v_cache, page_table updated in place
 *   prefix_len_in/out [B] i32, free_count_in/out [1] i32, status [1] i32: device memory; the
 *   in and out arrays must be distinct (every workgroup reads all inputs)
 *   free_pages [free_cap] i32 (device), free_cap its length
 * Supported: blk, S in {16,32,64}; d in {64,128}; Hkv <= 64; 1 <= B <= 4096;
 * max_pages*S <= 2^24; K/V pointers 16-byte aligned.
 * ------------------------------------------------------------------------------------------ */
int focus_block_commit(const uint8_t* commit, const void* k_blk, const void* v_blk, int B,
                       int blk, int Hkv, int d, int S, void* k_cache, void* v_cache,
                       int num_pages, int32_t* page_table, int max_pages,
                       const int32_t* prefix_len_in, int32_t* prefix_len_out,
                       const int32_t* free_pages, int free_cap, const int32_t* free_count_in,
                       int32_t* free_count_out, int32_t* status, hipStream_t stream);

/* --------------------------------------------------------------------------------------------
 * 7. KV layout conversion.
 *
 * Calls 4-6 read and write K/V in the MFMA-native layouts given under call 4 (the pages fix no
 * KV layout; they call for a paged prefix cache and an intra-block KV cache: project page,
 * card "Runtime Action" (intra-block KV caching); AI Engineering Academy article, section
 * "Arquitetura do FOCUS" (KV-cache management)).  This call converts K/V stored as plain token
 * rows into them.  For block n (a page of the cache, or a request's block), kv head g, token
 * s < S and dim c < d, the source element is
 *   layout FOCUS_KV_HEAD_MAJOR  (0): src[n, g, s, c]   (src [n_blocks, Hkv, S, d])
 *   layout FOCUS_KV_TOKEN_MAJOR (1): src[n, s, g, c]   (src [n_blocks, S, Hkv, d])
 * and it is written to
 *   k_out[n, g, c/8, s, c%8] = k_src(n, g, s, c)       (k_out [n_blocks, Hkv, d/8, S, 8])
 *   v_out[n, g, s/8, c, s%8] = v_src(n, g, s, c)       (v_out [n_blocks, Hkv, S/8, d, 8])
 * i.e. k_cache / v_cache of call 4 (n = page, S = page size), or k_blk / v_blk (n = request,
 * S = blk).  All bf16, moved bit for bit.  A pair (k_src, k_out) or (v_src, v_out) may be
 * both NULL (that matrix is skipped), not one of the two; at least one pair is given.  No
 * output may overlap an input or the other output (checked on the host).
 * Supported: S in {16,32,64}; d in {64,128}; 1 <= Hkv <= 64; n_blocks * Hkv < 2^31; pointers
 * 16-byte aligned.
 * ------------------------------------------------------------------------------------------ */
typedef enum { FOCUS_KV_HEAD_MAJOR = 0, FOCUS_KV_TOKEN_MAJOR = 1 } focus_kv_layout;

int focus_kv_pack(const void* k_src, const void* v_src, int layout, int n_blocks, int Hkv, int S,
                  int d, void* k_out, void* v_out, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* FOCUS_H_ */
