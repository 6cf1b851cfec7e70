"""Seeded synthetic inputs for one focused block-diffusion step.

This is the only module shared by the oracle's tests and the HIP path's tests and bench.  It
draws random numbers, rounds them to bfloat16 storage and lays them out in the C-ABI's memory
layouts; it computes nothing of the method itself (no scores, budgets of kept tokens, offsets or
attention).

Draw order: the small draws come from one ``numpy.random.Generator(PCG64(seed))`` in a fixed
order (masked counts, masked positions, prefix lengths, page tables, bias positions); each large
tensor has its own stream (Q0=1, K0=2, V0=3 (unused), Q1=4, K1=5, V1=6, prefix K=7, prefix V=8,
hidden=9), drawn in fixed-size chunks seeded by ``SeedSequence([seed, stream, chunk])``.  All
projections are N(0,1)/sqrt(d) drawn in float32; bf16 tensors are rounded to nearest-even from
those draws.

Memory layouts (all row-major numpy arrays; bf16 is carried as uint16 bit patterns):

* scoring inputs  q0, q1: [B, blk, Hq, d];  k0, k1: [B, blk, Hkv, d]   (float32 or bf16)
* attention query q_att:  [B, blk, Hq, d]  bf16 (the layer-1 query, rounded to bf16)
* paged K cache   k_cache: [num_pages, Hkv, d/8, S, 8]  -- for each 8-wide slice of the head
  dimension the page's S keys are contiguous, 16 bytes per key
* paged V cache   v_cache: [num_pages, Hkv, S/8, d, 8]  -- for each group of 8 keys the head
  dimension is contiguous, with the 8 keys' values interleaved (16 bytes per dim)
* block K/V       k_blk: [B, Hkv, d/8, blk, 8], v_blk: [B, Hkv, blk/8, d, 8] (the same layouts with
  the block as one page of blk tokens)
* page_table [B, max_pages] int32 (entries past a request's last page are -1), prefix_len [B]
* masked [B, blk] uint8 (1 = still masked), budget [B] int32 (None for the adaptive rule)
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

from .configs import Recipe

BF16_NAN = np.uint16(0x7FC0)
PAGE_POISON = np.int32(0x3FFFFFFF)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); returns the uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns to float32 (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def pack_k(tokens: np.ndarray, S: int) -> np.ndarray:
    """Logical keys [n_pages*S, Hkv, d] -> paged K layout [n_pages, Hkv, d/8, S, 8]."""
    n = tokens.shape[0] // S
    Hkv, d = tokens.shape[1], tokens.shape[2]
    return np.ascontiguousarray(tokens.reshape(n, S, Hkv, d // 8, 8).transpose(0, 2, 3, 1, 4))


def pack_v(tokens: np.ndarray, S: int) -> np.ndarray:
    """Logical values [n_pages*S, Hkv, d] -> paged V layout [n_pages, Hkv, S/8, d, 8]."""
    n = tokens.shape[0] // S
    Hkv, d = tokens.shape[1], tokens.shape[2]
    return np.ascontiguousarray(tokens.reshape(n, S // 8, 8, Hkv, d).transpose(0, 3, 1, 4, 2))


@dataclass
class Step:
    recipe: Recipe
    B: int
    blk: int
    Hq: int
    Hkv: int
    d: int
    S: int
    sm_scale: float
    score_dtype: str
    masked: np.ndarray            # [B, blk] uint8
    masked_count: np.ndarray      # [B] int32
    budget: Optional[np.ndarray]  # [B] int32 or None
    rule: tuple                   # ("fixed",) or ("adaptive", beta, lo, hi)
    max_kept: int
    prefix_len: np.ndarray        # [B] int32
    page_table: np.ndarray        # [B, max_pages] int32
    num_pages: int
    q0: np.ndarray
    k0: np.ndarray
    q1: np.ndarray
    k1: np.ndarray
    q_att: np.ndarray             # [B, blk, Hq, d] uint16 (bf16)
    k_blk: np.ndarray             # [B, Hkv, d/8, blk, 8] uint16
    v_blk: np.ndarray             # [B, Hkv, blk/8, d, 8] uint16
    k_cache: np.ndarray           # [num_pages, Hkv, d/8, S, 8] uint16
    v_cache: np.ndarray           # [num_pages, Hkv, S/8, d, 8] uint16
    hidden: Optional[np.ndarray]  # [B, blk, W] uint16 or None
    bias_pos: Optional[np.ndarray] = None
    k_cache0: Optional[np.ndarray] = None  # layer-0 prefix keys, paged like k_cache (optional)
    k_blk0: Optional[np.ndarray] = None    # layer-0 block keys, packed like k_blk (optional)
    extra: dict = field(default_factory=dict)

    @property
    def max_pages(self) -> int:
        return self.page_table.shape[1]


_CHUNK = 1 << 22  # elements per independently seeded chunk of a large tensor
_POOL = None


def _pool():
    global _POOL
    if _POOL is None:
        import concurrent.futures
        import os
        _POOL = concurrent.futures.ThreadPoolExecutor(max_workers=min(16, os.cpu_count() or 1))
    return _POOL


def _draw_normal(seed: int, stream: int, shape, scale: float, bf16: bool) -> np.ndarray:
    """N(0,1)*scale of ``shape`` from stream ``stream`` of ``seed``.

    The flat tensor is cut into chunks of ``_CHUNK`` elements; chunk c is drawn from
    ``PCG64(SeedSequence([seed, stream, c]))``, so the values do not depend on how many threads
    draw them.  With ``bf16`` the float32 draws are rounded to bf16 bit patterns.
    """
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16 if bf16 else np.float32)

    def work(c):
        lo, hi = c * _CHUNK, min(n, (c + 1) * _CHUNK)
        g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, stream, c])))
        x = g.standard_normal(size=hi - lo, dtype=np.float32)
        if scale != 1.0:
            x *= np.float32(scale)
        out[lo:hi] = f32_to_bf16_bits(x) if bf16 else x

    list(_pool().map(work, range((n + _CHUNK - 1) // _CHUNK)))
    return out.reshape(shape)


def make_step(recipe: Recipe, seed: Optional[int] = None, poison: bool = False,
              prefix_override: Optional[np.ndarray] = None,
              masked_override: Optional[np.ndarray] = None, layer0_prefix: bool = False) -> Step:
    """Draw one synthetic step for ``recipe``.

    ``poison`` fills every memory location the step must never read (cache slots past a prefix,
    spare pool pages, page-table entries past a request's last page) with NaN / out-of-range ids.
    ``prefix_override`` / ``masked_override`` replace the drawn prefix lengths / masked counts
    (edge-case tests); the random stream is consumed identically either way.
    ``layer0_prefix`` also draws the layer-0 prefix keys (stream 10) into their own paged cache
    with the same page table, and packs the layer-0 block keys, for the full-domain importance.
    """
    r = recipe
    rng = np.random.Generator(np.random.PCG64(r.seed if seed is None else seed))
    B, blk, Hq, Hkv, d, S = r.B, r.blk, r.Hq, r.Hkv, r.d, r.S
    if Hq % Hkv or d % 8 or S % 8 or blk % 8:
        raise ValueError("recipe shape not representable in the paged layouts")

    # 1. masked counts
    if r.masked[0] == "fixed":
        mcount = np.full(B, int(r.masked[1]), dtype=np.int64)
    else:
        lo = math.ceil(r.masked[1] * blk)
        mcount = rng.integers(lo, blk + 1, size=B)
    if masked_override is not None:
        mcount = np.asarray(masked_override, dtype=np.int64).copy()
    # 2. masked positions: a seeded random subset of the block per request
    masked = np.zeros((B, blk), dtype=np.uint8)
    for b in range(B):
        perm = rng.permutation(blk)
        masked[b, perm[: int(mcount[b])]] = 1
    # 3. prefix lengths
    kind = r.prefix[0]
    if kind == "fixed":
        plen = np.full(B, int(r.prefix[1]), dtype=np.int64)
    elif kind == "uniform":
        plen = rng.integers(int(r.prefix[1]), int(r.prefix[2]) + 1, size=B)
    elif kind == "lognormal":
        med, sig, cap = r.prefix[1], r.prefix[2], int(r.prefix[3])
        z = rng.standard_normal(size=B)
        plen = np.minimum(cap, np.maximum(1, np.rint(med * np.exp(sig * z)))).astype(np.int64)
    else:
        raise ValueError(kind)
    if prefix_override is not None:
        plen = np.asarray(prefix_override, dtype=np.int64).copy()
    if plen.max(initial=0) > r.max_pages * S:
        raise ValueError("prefix longer than the page table allows")
    # 4. page tables
    npg = (plen + S - 1) // S
    used = int(npg.sum())
    if r.table == "sequential":
        pool = used
        order = np.arange(pool, dtype=np.int64)
    else:
        pool = int(math.ceil(used * (1.0 + r.spare_frac)))
        order = rng.permutation(pool)
    pool = max(pool, 1)
    table = np.full((B, r.max_pages), PAGE_POISON if poison else -1, dtype=np.int32)
    base = np.concatenate([[0], np.cumsum(npg)])
    for b in range(B):
        table[b, : npg[b]] = order[base[b]: base[b + 1]]

    # 5. block projections for layers 0 and 1 (stream ids 1..6), prefix K/V (7, 8), hidden (9)
    seed_ = r.seed if seed is None else seed
    sc = 1.0 / math.sqrt(d)
    f32 = r.score_dtype == "f32"
    q0 = _draw_normal(seed_, 1, (B, blk, Hq, d), sc, not f32)
    k0 = _draw_normal(seed_, 2, (B, blk, Hkv, d), sc, not f32)
    # stream 3 would hold the layer-0 values, which the step never reads
    q1 = _draw_normal(seed_, 4, (B, blk, Hq, d), sc, not f32)
    k1 = _draw_normal(seed_, 5, (B, blk, Hkv, d), sc, not f32)
    v1 = _draw_normal(seed_, 6, (B, blk, Hkv, d), sc, True)
    total = int(plen.sum())
    pk = _draw_normal(seed_, 7, (total, Hkv, d), sc, True)
    pv = _draw_normal(seed_, 8, (total, Hkv, d), sc, True)
    hidden = _draw_normal(seed_, 9, (B, blk, r.hidden), 1.0, True) if r.hidden else None

    # 6. skewed attention: key coordinate 0 carries the bias, query coordinate 0 is one.  The
    # values written (1.0, 0.0, bias_value) are exact in bf16, so editing the bf16 bit patterns
    # equals rounding the edited float32 draws.
    bias_pos = None
    if r.bias_positions:
        if f32:
            raise ValueError("biased recipes use bf16 scoring inputs")
        one = f32_to_bf16_bits(np.float32([1.0]))[0]
        bval = f32_to_bf16_bits(np.float32([r.bias_value]))[0]
        bias_pos = np.zeros((B, r.bias_positions), dtype=np.int64)
        pstart = np.concatenate([[0], np.cumsum(plen)])
        q1[..., 0] = one
        k1[..., 0] = 0
        pk[..., 0] = 0
        for b in range(B):
            nb = min(r.bias_positions, int(plen[b]))
            sel = rng.choice(int(plen[b]), size=nb, replace=False)
            bias_pos[b, :nb] = sel
            pk[pstart[b] + sel, :, 0] = bval

    q_att = f32_to_bf16_bits(q1) if f32 else q1.copy()
    k1_16 = f32_to_bf16_bits(k1) if f32 else k1
    k_blk = pack_k(k1_16.reshape(B * blk, Hkv, d), blk)
    v_blk = pack_v(v1.reshape(B * blk, Hkv, d), blk)

    # 7. scatter prefix tokens into pages (slots past a prefix are zero, or NaN when poisoned)
    fill = BF16_NAN if poison else np.uint16(0)
    tstart = np.concatenate([[0], np.cumsum(plen)])

    def paged(tokens, shape, pack):
        cache = np.full((pool,) + shape, fill, dtype=np.uint16)
        for b in range(B):
            n = int(plen[b])
            if n == 0:
                continue
            nfull = n // S
            ids = table[b, : npg[b]].astype(np.int64)
            if nfull:
                cache[ids[:nfull]] = pack(tokens[tstart[b]: tstart[b] + nfull * S], S)
            rem = n - nfull * S
            if rem:
                tail = np.full((S, Hkv, d), fill, dtype=np.uint16)
                tail[:rem] = tokens[tstart[b] + nfull * S: tstart[b] + n]
                cache[ids[nfull]] = pack(tail, S)[0]
        return cache

    k_cache = paged(pk, (Hkv, d // 8, S, 8), pack_k)
    v_cache = paged(pv, (Hkv, S // 8, d, 8), pack_v)
    del pk, pv
    k_cache0 = k_blk0 = None
    if layer0_prefix:
        pk0 = _draw_normal(seed_, 10, (total, Hkv, d), sc, True)
        k_cache0 = paged(pk0, (Hkv, d // 8, S, 8), pack_k)
        del pk0
        k0_16 = f32_to_bf16_bits(k0) if f32 else k0
        k_blk0 = pack_k(k0_16.reshape(B * blk, Hkv, d), blk)
    s_q0, s_k0, s_q1, s_k1 = q0, k0, q1, k1

    rule = ("fixed",)
    budget = None
    bk = r.budget[0]
    if bk == "fixed":
        budget = np.full(B, int(r.budget[1]), dtype=np.int32)
    elif bk == "frac":
        budget = np.ceil(r.budget[1] * mcount).astype(np.int32)
    else:
        rule = ("adaptive", float(r.budget[1]), int(r.budget[2]), int(r.budget[3]))

    return Step(recipe=r, B=B, blk=blk, Hq=Hq, Hkv=Hkv, d=d, S=S, sm_scale=sc,
                score_dtype=r.score_dtype, masked=masked, masked_count=mcount.astype(np.int32),
                budget=budget, rule=rule, max_kept=r.max_kept(),
                prefix_len=plen.astype(np.int32), page_table=table, num_pages=pool,
                q0=s_q0, k0=s_k0, q1=s_q1, k1=s_k1, q_att=q_att, k_blk=k_blk, v_blk=v_blk,
                k_cache=k_cache, v_cache=v_cache, hidden=hidden, bias_pos=bias_pos,
                k_cache0=k_cache0, k_blk0=k_blk0)
