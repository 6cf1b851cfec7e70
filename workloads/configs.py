"""Workload recipes for the focused block-diffusion step.

Each recipe describes one synthetic decoding step: a batch of requests, each with a block of
``blk`` tokens (some still masked, the rest already decoded), a prefix held in a paged KV cache,
the layer-0/layer-1 query/key projections of the block, and an eviction budget rule.

The shapes follow the FOCUS project page ("FOCUS: DLLMs Know How to Tame Their Compute Bound",
focus-inference.github.io): block sizes of 16/32/64 tokens (Efficiency summary, "block size
B=64"), about one token in ten decoded per step (page header), batches up to 256 (throughput
chart x-axis).  Head counts mimic an 8B block-diffusion model (32 query heads, 8 kv heads,
head dim 128).  The pages' throughput datasets (ShareGPT, WildChat, MATH) are not available;
these seeded distributions of batch, block, masked count and prefix length stand in for them.

This module holds no part of the method's arithmetic: it only names sizes and distributions.
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass


@dataclass(frozen=True)
class Recipe:
    name: str
    seed: int                 # numpy PCG64 seed
    B: int                    # requests in the batch
    blk: int                  # block size (tokens)
    Hq: int                   # query heads
    Hkv: int                  # kv heads
    d: int                    # head dim
    S: int                    # page size (tokens per page)
    masked: tuple             # ("fixed", m) or ("uniform", frac_lo): m ~ U{ceil(frac_lo*blk) .. blk}
    prefix: tuple             # ("fixed", P) | ("uniform", lo, hi) | ("lognormal", median, sigma, cap)
    max_prefix: int           # upper bound of the prefix distribution (sizes the page table)
    table: str = "sequential"  # "sequential" or "fragmented" (random permutation of a pool)
    spare_frac: float = 0.0   # extra pool pages (fragmented tables)
    score_dtype: str = "bf16"  # dtype of the layer-0/1 Q/K handed to scoring: "f32" or "bf16"
    budget: tuple = ("fixed", 4)  # ("fixed", b) | ("frac", f) | ("adaptive", beta, lo, hi)
    hidden: int = 0           # width of the hidden states gathered by compaction (0: none)
    bias_positions: int = 0   # prefix positions per request whose keys get a logit bias
    bias_value: float = 45.25  # value written into key coordinate 0 at those positions

    def scaled(self, **kw) -> "Recipe":
        return dataclasses.replace(self, **kw)

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @property
    def max_pages(self) -> int:
        return -(-self.max_prefix // self.S)

    def max_kept(self) -> int:
        """Upper bound of any request's kept count under this recipe's budget rule."""
        kind = self.budget[0]
        if kind == "fixed":
            return min(self.blk, int(self.budget[1]))
        if kind == "frac":
            import math
            return min(self.blk, math.ceil(self.budget[1] * self.blk))
        return min(self.blk, int(self.budget[3]))


# Tiny step the oracle finishes instantly: 2 requests, block 16 with 10 masked, 64-token prefix
# in 16-token pages, 4 heads without grouping, head dim 64, fp32 scoring inputs, keep 4.
TINY = Recipe(name="tiny_b2_blk16", seed=1000, B=2, blk=16, Hq=4, Hkv=4, d=64, S=16,
              masked=("fixed", 10), prefix=("fixed", 64), max_prefix=64,
              score_dtype="f32", budget=("fixed", 4))

# Block-diffusion 8B-like step at batch 32: 60-100% masked, prefix U[256,1024], keep 25%.
SDAR_B32 = Recipe(name="sdar_b32_blk32", seed=1001, B=32, blk=32, Hq=32, Hkv=8, d=128, S=64,
                  masked=("uniform", 0.6), prefix=("uniform", 256, 1024), max_prefix=1024,
                  budget=("frac", 0.25))

# The headline step: batch 256, block 32, lognormal prefixes (median 600, sigma 0.8, cap 4096),
# keep 12.5% of the masked tokens, 4096-wide hidden states gathered by compaction.
SDAR_B256 = Recipe(name="sdar_b256_blk32", seed=1002, B=256, blk=32, Hq=32, Hkv=8, d=128, S=64,
                   masked=("uniform", 0.6), prefix=("lognormal", 600.0, 0.8, 4096),
                   max_prefix=4096, budget=("frac", 0.125), hidden=4096)

# Block-size sweep with the adaptive budget clamp(#{delta > mean + 0.5 std}, 2, 16).
BLK64 = Recipe(name="sweep_b128_blk64", seed=1003, B=128, blk=64, Hq=32, Hkv=8, d=128, S=64,
               masked=("uniform", 0.6), prefix=("uniform", 512, 2048), max_prefix=2048,
               budget=("adaptive", 0.5, 2, 16))
BLK16 = BLK64.scaled(name="sweep_b128_blk16", blk=16)

# Long-context stress: prefixes U[4096,8192] in 16-token pages scattered over a pool with 25%
# spare pages, 16/4 heads, 8 prefix positions per request carry a +4 logit bias, keep 4.
LONG_CTX = Recipe(name="longctx_b64_blk32", seed=1004, B=64, blk=32, Hq=16, Hkv=4, d=128, S=16,
                  masked=("uniform", 0.6), prefix=("uniform", 4096, 8192), max_prefix=8192,
                  table="fragmented", spare_frac=0.25, budget=("fixed", 4), bias_positions=8)

ALL = (TINY, SDAR_B32, SDAR_B256, BLK64, BLK16, LONG_CTX)
BY_NAME = {r.name: r for r in ALL}

# The step that throughput is quoted on.
HEADLINE = SDAR_B256
