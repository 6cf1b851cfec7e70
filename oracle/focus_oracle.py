"""Plain fp64 CPU oracle of FOCUS's focused block-diffusion step.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the bench's CPU-baseline leg may
import this module.  The product path (the HIP library and its binding) never calls it and
shares no code with it.

Sources (the web pages describing FOCUS, arXiv 2601.23278):

* [PP]   project page "FOCUS: DLLMs Know How to Tame Their Compute Bound" (focus-inference.github.io):
         the header paragraph, the Overview cards "Design", "Motivation", "Decodability Signal"
         and "Runtime Action".
* [ABS]  the paper's abstract, reproduced on the arXiv-summary pages (shd-paper.top, newx.sg).
* [NEWS] the AI Engineering Academy article on FOCUS, section "Arquitetura do FOCUS" (the three
         components: importance scoring, target token selection, state compaction, plus ragged
         paged attention).

Where the pages leave a step open, the reading taken is stated at the function.  Every function
is the plainest direct computation: loops over requests/heads, one library matmul per product,
no blocking or fusion.  All arithmetic is float64; bf16 inputs are widened exactly.
"""
from __future__ import annotations

import math
from typing import Optional, Sequence

import numpy as np


# --------------------------------------------------------------------------------------------
# input decoding
# --------------------------------------------------------------------------------------------
def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> float64, exactly: a bf16 is the top half of a float32."""
    u32 = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u32.view(np.float32).astype(np.float64)


def to_f64(x: np.ndarray, dtype: str) -> np.ndarray:
    """Widen a stored tensor ("f32" float32 values or "bf16" uint16 bit patterns) to float64."""
    if dtype == "bf16":
        return bf16_to_f64(x)
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32).astype(np.float64)
    raise ValueError(dtype)


# --------------------------------------------------------------------------------------------
# a1: importance scoring
# --------------------------------------------------------------------------------------------
def layer_importance(q: np.ndarray, k: np.ndarray, sm_scale: float) -> np.ndarray:
    """Attention mass each block token receives in one early layer.

    [PP, "Design"]: importance is estimated from the early layers' Q/K projections; [ABS]: the
    importance is derived from attention.  Readings (the pages give no formula):
      * the softmax runs over the block's own keys (block-only domain);
      * every block query (masked or decoded) and every query head contributes;
      * a token's importance is the SUM over heads and queries of the softmax weight it gets.
    q: [B, blk, Hq, d], k: [B, blk, Hkv, d] float64; query head h reads kv head h // (Hq/Hkv).
    Returns I [B, blk] with I[r, j] = sum_h sum_i softmax_j(sm_scale * q[r,i,h] . k[r,j,g(h)]).
    """
    B, blk, Hq, d = q.shape
    Hkv = k.shape[2]
    G = Hq // Hkv
    imp = np.zeros((B, blk), dtype=np.float64)
    for h in range(Hq):
        g = h // G
        s = sm_scale * (q[:, :, h, :] @ k[:, :, g, :].transpose(0, 2, 1))    # [B, i, j]
        s = s - s.max(axis=2, keepdims=True)
        p = np.exp(s)
        p = p / p.sum(axis=2, keepdims=True)       # row softmax over the keys j
        imp += p.sum(axis=1)                        # mass received by key j, summed over queries
    return imp


def score_l01(q0, k0, q1, k1, sm_scale: float, dtype: str = "bf16") -> np.ndarray:
    """Decodability score of every block token: layer-1 importance minus layer-0 importance.

    [PP, "Decodability Signal"]: the change of importance from layer 0 to layer 1 is the signal
    that separates decodable tokens from the rest.  Reported for every position (decoded ones
    too); selection ignores decoded positions.  Returns delta [B, blk] float64.
    """
    i0 = layer_importance(to_f64(q0, dtype), to_f64(k0, dtype), sm_scale)
    i1 = layer_importance(to_f64(q1, dtype), to_f64(k1, dtype), sm_scale)
    return i1 - i0


def prefix_keys(r: int, g: int, k_cache, page_table, prefix_len) -> np.ndarray:
    """The prefix keys of request r for kv head g, in token order: [P, d] float64.  Token t is
    in page page_table[r, t // S] at slot t % S; paged K layout [pages, Hkv, d/8, S, 8]."""
    S = k_cache.shape[3]
    d = k_cache.shape[2] * 8
    P = int(prefix_len[r])
    t = np.arange(P)
    page = np.asarray(page_table[r], dtype=np.int64)[t // S]
    return k_cache[page, g, :, t % S, :].reshape(P, d)


def layer_importance_full(q: np.ndarray, k: np.ndarray, k_cache, page_table, prefix_len,
                          sm_scale: float) -> np.ndarray:
    """Attention mass each block token receives in one early layer, full attention domain.

    The other reading of [PP, "Design"] (importance from the early layers' attention): a block
    query's softmax runs over all keys it attends to in that layer -- the request's prefix keys
    (from the paged cache of that layer) followed by the block keys -- and block token j's
    importance is the weight it receives there, summed over query heads and block queries.
    q: [B, blk, Hq, d], k: [B, blk, Hkv, d] float64 (the layer's block Q/K); k_cache float64 in
    the paged layout.  Returns I [B, blk].
    """
    B, blk, Hq, d = q.shape
    Hkv = k.shape[2]
    G = Hq // Hkv
    imp = np.zeros((B, blk), dtype=np.float64)
    for r in range(B):
        for h in range(Hq):
            g = h // G
            keys = np.concatenate([prefix_keys(r, g, k_cache, page_table, prefix_len),
                                   k[r, :, g, :]], axis=0)                  # [P + blk, d]
            s = sm_scale * (q[r, :, h, :] @ keys.T)                          # [blk, P + blk]
            s = s - s.max(axis=1, keepdims=True)
            p = np.exp(s)
            p = p / p.sum(axis=1, keepdims=True)                             # over all keys
            imp[r] += p[:, keys.shape[0] - blk:].sum(axis=0)                 # block columns
    return imp


def score_l01_full(q0, k0, q1, k1, k_cache0, k_cache1, page_table, prefix_len,
                   sm_scale: float) -> np.ndarray:
    """delta = I_1 - I_0 with the full-domain importance of each layer (layer l's prefix keys
    in k_cache_l).  Inputs float64 (bf16 widened exactly)."""
    return (layer_importance_full(q1, k1, k_cache1, page_table, prefix_len, sm_scale)
            - layer_importance_full(q0, k0, k_cache0, page_table, prefix_len, sm_scale))


# --------------------------------------------------------------------------------------------
# a2: budgeted selection
# --------------------------------------------------------------------------------------------
def request_budget(delta_r: np.ndarray, masked_r: np.ndarray, budget_r: Optional[int],
                   rule: Sequence) -> int:
    """Budget b_r of one request before clipping to the masked count.

    [PP, "Design"] keeps likely-decodable candidates under an adaptive budget; [PP, "Runtime
    Action"] names dynamic budgeting.  The pages give no formula, so the caller chooses:
      * rule ("fixed",): b_r = budget_r (fixed counts and fractions of the masked count are
        turned into per-request integers by the caller);
      * rule ("adaptive", beta, lo, hi): over the masked candidates, mu = mean(delta),
        sigma = population std, c = #{delta > mu + beta*sigma} (strict), b_r = clamp(c, lo, hi).
    """
    if rule[0] == "fixed":
        return int(budget_r)
    _, beta, lo, hi = rule
    cand = [float(delta_r[j]) for j in range(len(delta_r)) if masked_r[j]]
    if not cand:
        return int(min(max(0, lo), hi))
    mu = sum(cand) / len(cand)
    var = sum((x - mu) ** 2 for x in cand) / len(cand)
    thr = mu + beta * math.sqrt(var)
    c = sum(1 for x in cand if x > thr)
    return int(min(max(c, lo), hi))


def adaptive_threshold(delta_r: np.ndarray, masked_r: np.ndarray, beta: float) -> float:
    """mu + beta*sigma over a request's masked candidates (used by the tests' near-tie rule)."""
    cand = np.asarray([delta_r[j] for j in range(len(delta_r)) if masked_r[j]], dtype=np.float64)
    if cand.size == 0:
        return float("nan")
    mu = cand.sum() / cand.size
    return float(mu + beta * math.sqrt(((cand - mu) ** 2).sum() / cand.size))


def select_budget(delta: np.ndarray, masked: np.ndarray, budget: Optional[np.ndarray],
                  rule: Sequence = ("fixed",)):
    """Target token selection: keep the k_r masked tokens with the largest score.

    [NEWS, "Arquitetura do FOCUS"]: target token selection picks the tokens to process;
    [PP header]: non-decodable tokens are evicted.  Readings: a larger delta means more likely
    decodable; only masked tokens are candidates (decoded ones are never kept);
    k_r = min(max(b_r, 0), m_r); equal scores are ordered by block position, lower first.
    A score that is not a number ranks as minus infinity (the pages never meet one; this keeps
    the order total, so exactly k_r tokens are kept).
    Returns keep [B, blk] uint8 and kept_count [B] int32.
    """
    B, blk = delta.shape
    keep = np.zeros((B, blk), dtype=np.uint8)
    kept = np.zeros(B, dtype=np.int32)
    for r in range(B):
        cand = [j for j in range(blk) if masked[r, j]]
        b = request_budget(delta[r], masked[r], None if budget is None else budget[r], rule)
        k = min(max(b, 0), len(cand))
        order = sorted(cand, key=lambda j: (-rank_key(delta[r, j]), j))
        for j in order[:k]:
            keep[r, j] = 1
        kept[r] = k
    return keep, kept


def rank_key(x) -> float:
    """The value a score is ranked by: itself, or minus infinity if it is not a number."""
    x = float(x)
    return -math.inf if math.isnan(x) else x


def kth_boundary(delta_r: np.ndarray, masked_r: np.ndarray, k: int) -> float:
    """The k-th largest masked score of a request (its rank key), clipped to the last
    candidate when k exceeds their number; nan if k <= 0 or nothing is masked.  This is the
    selection boundary: the smallest kept score."""
    cand = sorted((rank_key(delta_r[j]) for j in range(len(delta_r)) if masked_r[j]),
                  reverse=True)
    if k <= 0 or not cand:
        return float("nan")
    return cand[min(k, len(cand)) - 1]


# --------------------------------------------------------------------------------------------
# a3: compaction
# --------------------------------------------------------------------------------------------
def compact(keep: np.ndarray, rows: Optional[np.ndarray] = None, cap: Optional[int] = None):
    """State compaction into ragged lists.

    [NEWS, "Arquitetura do FOCUS"]: the inference state is compacted, dropping evicted tokens;
    [PP, "Runtime Action"]: later layers run ragged over what is kept.  offsets is the exclusive
    running total of kept counts (offsets[B] = T); kept_pos lists each request's kept positions
    in ascending order, requests in batch order; gathered[n] = rows[r, kept_pos[n]].  Entries
    n >= cap are not produced (offsets still hold the true totals).
    """
    B, blk = keep.shape
    offsets = np.zeros(B + 1, dtype=np.int32)
    kept_pos = []
    owner = []
    for r in range(B):
        n_r = 0
        for j in range(blk):
            if keep[r, j]:
                kept_pos.append(j)
                owner.append(r)
                n_r += 1
        offsets[r + 1] = offsets[r] + n_r
    T = int(offsets[B])
    lim = T if cap is None else min(T, cap)
    kept_pos = np.asarray(kept_pos[:lim], dtype=np.int32)
    gathered = None
    if rows is not None:
        gathered = np.stack([rows[owner[n], kept_pos[n]] for n in range(lim)]) if lim else \
            np.zeros((0,) + rows.shape[2:], dtype=rows.dtype)
    return offsets, kept_pos, gathered


# --------------------------------------------------------------------------------------------
# a4: ragged paged attention
# --------------------------------------------------------------------------------------------
def request_kv(r: int, g: int, k_cache, v_cache, page_table, prefix_len, k_blk, v_blk):
    """Keys/values visible to request r through kv head g, in order: prefix then block.

    Prefix token t lives in page page_table[r, t // S] at slot t % S.  Paged K layout
    [pages, Hkv, d/8, S, 8]: element (t, c) is k_cache[page, g, c // 8, slot, c % 8].  Paged V
    layout [pages, Hkv, S/8, d, 8]: element (t, c) is v_cache[page, g, slot // 8, c, slot % 8].
    The block KV uses the same layouts with one page of blk tokens per request.
    Inputs are float64 arrays in those shapes.  Returns K [n, d], V [n, d].
    """
    S = k_cache.shape[3]
    d = k_cache.shape[2] * 8
    P = int(prefix_len[r])
    t = np.arange(P)
    page = np.asarray(page_table[r], dtype=np.int64)[t // S]
    slot = t % S
    kp = k_cache[page, g, :, slot, :].reshape(P, d)               # [P, d]
    vp = v_cache[page, g, slot // 8, :, slot % 8]                 # [P, d]
    blk = k_blk.shape[3]
    j = np.arange(blk)
    kb = k_blk[r, g, :, j, :].reshape(blk, d)
    vb = v_blk[r, g, j // 8, :, j % 8]
    return np.concatenate([kp, kb], axis=0), np.concatenate([vp, vb], axis=0)


def ragged_paged_attn(q: np.ndarray, offsets: np.ndarray, k_cache, v_cache, page_table,
                      prefix_len, k_blk, v_blk, sm_scale: float, cap: Optional[int] = None):
    """Attention of the kept queries over each request's paged prefix KV plus its block KV.

    [NEWS]: ragged paged attention; [PP, "Runtime Action"]: ragged execution with intra-block KV
    caching; [PP, "Motivation"]: block diffusion keeps earlier blocks exactly KV-cached and the
    block is processed bidirectionally.  Readings: no mask -- each kept query sees the whole
    prefix and every block position (evicted ones stay visible through the cached block KV).
    q: [cap, Hq, d] float64 (row n belongs to the request r with offsets[r] <= n < offsets[r+1]).
    Returns out [rows, Hq, d] and lse [rows, Hq] (natural log) for rows n < min(T, cap).
    """
    B = len(prefix_len)
    Hq, d = q.shape[1], q.shape[2]
    Hkv = k_cache.shape[1]
    G = Hq // Hkv
    T = int(offsets[B])
    rows = T if cap is None else min(T, cap)
    out = np.zeros((rows, Hq, d), dtype=np.float64)
    lse = np.zeros((rows, Hq), dtype=np.float64)
    for r in range(B):
        lo, hi = int(offsets[r]), min(int(offsets[r + 1]), rows)
        if hi <= lo:
            continue
        for g in range(Hkv):
            K, V = request_kv(r, g, k_cache, v_cache, page_table, prefix_len, k_blk, v_blk)
            for h in range(g * G, (g + 1) * G):
                z = sm_scale * (q[lo:hi, h, :] @ K.T)              # [rows_r, n]
                m = z.max(axis=1, keepdims=True)
                l = m[:, 0] + np.log(np.exp(z - m).sum(axis=1))
                lse[lo:hi, h] = l
                out[lo:hi, h, :] = np.exp(z - l[:, None]) @ V
    return out, lse


# --------------------------------------------------------------------------------------------
# f3: intra-block KV write-back and block commit
# --------------------------------------------------------------------------------------------
def kv_pack(k=None, v=None, token_major: bool = False):
    """Plain K/V token rows -> the paged layouts `request_kv` reads (the prefix cache of [PP,
    "Motivation"] and the intra-block cache of [PP, "Runtime Action"] store K/V; the pages fix
    no layout, these are the library's).

    k, v: [n, Hkv, S, d] (head-major) or [n, S, Hkv, d] (token_major), either may be None; any
    dtype (a move).  Returns (K [n, Hkv, d/8, S, 8], V [n, Hkv, S/8, d, 8]), None where the input
    was None: key (s, c) of (block b, head g) at [b, g, c // 8, s, c % 8], value (s, c) at
    [b, g, s // 8, c, s % 8].
    """
    def rows(x):  # [n, Hkv, S, d]
        x = np.asarray(x)
        return x.transpose(0, 2, 1, 3) if token_major else x

    kp = vp = None
    if k is not None:
        kx = rows(k)
        n, H, S, d = kx.shape
        kp = np.zeros((n, H, d // 8, S, 8), dtype=kx.dtype)
        for b in range(n):
            for g in range(H):
                for s in range(S):
                    kp[b, g, :, s, :] = kx[b, g, s].reshape(d // 8, 8)
    if v is not None:
        vx = rows(v)
        n, H, S, d = vx.shape
        vp = np.zeros((n, H, S // 8, d, 8), dtype=vx.dtype)
        for b in range(n):
            for g in range(H):
                for s in range(S):
                    vp[b, g, s // 8, :, s % 8] = vx[b, g, s]
    return kp, vp


def kv_writeback(k_rows, v_rows, offsets, kept_pos, k_blk, v_blk, cap: Optional[int] = None):
    """The kept tokens' fresh K/V replace the cached block KV at their positions; evicted
    positions keep their cached values ([PP, "Runtime Action"]: intra-block KV caching; [NEWS,
    "Arquitetura do FOCUS"]: compacted state).

    k_rows, v_rows: [T, Hkv, d], row n being request r's token kept_pos[n] for
    offsets[r] <= n < offsets[r+1]; rows n >= cap are absent.  k_blk [B, Hkv, d/8, blk, 8] and
    v_blk [B, Hkv, blk/8, d, 8] (any dtype: a byte move).  Returns new (k_blk, v_blk).
    """
    kb, vb = k_blk.copy(), v_blk.copy()
    Hkv, d = k_rows.shape[1], k_rows.shape[2]
    T = int(offsets[-1]) if cap is None else min(int(offsets[-1]), cap)
    for r in range(len(offsets) - 1):
        for n in range(int(offsets[r]), min(int(offsets[r + 1]), T)):
            j = int(kept_pos[n])
            kb[r, :, :, j, :] = k_rows[n].reshape(Hkv, d // 8, 8)   # key (j, c) at [c//8, j, c%8]
            vb[r, :, j // 8, :, j % 8] = v_rows[n]                  # value (j, c) at [j//8, c, j%8]
    return kb, vb


def block_commit(commit, k_blk, v_blk, k_cache, v_cache, page_table, prefix_len, free_pages,
                 free_count: int):
    """Appends each committed request's finished block (all blk tokens) to its paged prefix
    ([PP, "Motivation"]: finished blocks are exactly KV-cached; [NEWS]: KV-cache management).

    Request r's block token t goes to prefix position P_r + t.  The pages this needs beyond the
    ceil(P_r / S) it holds are taken from the top of the free-page stack
    free_pages[0 .. free_count-1], requests in batch order, each request's pages in position
    order.  Status 0: done.  Status 2: a committed request would outgrow its page table row.
    Status 1: not enough free pages.  On a non-zero status nothing changes.
    Returns (k_cache, v_cache, page_table, prefix_len, free_count, status) as new arrays.
    """
    S = k_cache.shape[3]
    blk = k_blk.shape[3]
    max_pages = page_table.shape[1]
    kc, vc = k_cache.copy(), v_cache.copy()
    table, plen = page_table.copy(), np.asarray(prefix_len).copy()
    B = len(plen)
    need = np.zeros(B, dtype=np.int64)
    for r in range(B):
        if commit[r]:
            P = int(plen[r])
            if P + blk > max_pages * S:
                return k_cache.copy(), v_cache.copy(), page_table.copy(), plen, free_count, 2
            need[r] = -(-(P + blk) // S) - (-(-P // S))
    if need.sum() > free_count:
        return kc, vc, table, plen, free_count, 1
    top = int(free_count)
    for r in range(B):
        if not commit[r]:
            continue
        P = int(plen[r])
        first_new = -(-P // S)
        for i in range(int(need[r])):
            top -= 1
            table[r, first_new + i] = free_pages[top]
        for t in range(blk):
            p = P + t
            page, slot = int(table[r, p // S]), p % S
            kc[page, :, :, slot, :] = k_blk[r, :, :, t, :]
            vc[page, :, slot // 8, :, slot % 8] = v_blk[r, :, t // 8, :, t % 8]
        plen[r] = P + blk
    return kc, vc, table, plen, top, 0


# --------------------------------------------------------------------------------------------
# the whole step
# --------------------------------------------------------------------------------------------
def step(st, hidden: bool = True):
    """Run score -> select -> compact -> attend on a ``workloads.Step`` (all fp64).

    The attention stands in for a later layer using the layer-1 tensors: the kept tokens'
    layer-1 queries, the layer-1 block K/V as intra-block KV and the step's prefix cache.
    """
    delta = score_l01(st.q0, st.k0, st.q1, st.k1, st.sm_scale, st.score_dtype)
    keep, kept = select_budget(delta, st.masked, st.budget, st.rule)
    offsets, kept_pos, q_rows = compact(keep, bf16_to_f64(st.q_att))
    res = {"delta": delta, "keep": keep, "kept_count": kept, "offsets": offsets,
           "kept_pos": kept_pos}
    if hidden and st.hidden is not None:
        _, _, g = compact(keep, st.hidden)
        res["gathered_hidden"] = g
    out, lse = ragged_paged_attn(q_rows, offsets, bf16_to_f64(st.k_cache), bf16_to_f64(st.v_cache),
                                 st.page_table, st.prefix_len, bf16_to_f64(st.k_blk),
                                 bf16_to_f64(st.v_blk), st.sm_scale)
    res["out"] = out
    res["lse"] = lse
    return res
