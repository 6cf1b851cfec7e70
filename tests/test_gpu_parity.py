"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle on seeded inputs.

Every recipe runs end to end at a reduced batch (every element compared) and at its full size
(scores, selections, offsets and gathers compared everywhere; attention on sampled requests,
whose rows the oracle computes one by one).  Isolated tests cover each call's edge cases.
"""
import zlib

import numpy as np
import pytest
import torch

import oracle as O
from decodability_aware_token_amd import FocusStep
from decodability_aware_token_amd import binding as F
from parity_helpers import (DELTA_TOL, LSE_TOL, OUT_TOL, attn_case_inputs, bf16_to_np,
                            check_keep, check_ragged, compare_attention, gathered_sets,
                            oracle_attention, run_gpu_step, step_inputs)
from workloads import BY_NAME, make_step
from workloads.torch_io import bf16_tensor

pytestmark = pytest.mark.gpu

DEV = "cuda"

# reduced batches of every recipe: oracle runs in seconds, still several tiles and ragged tails
SMALL = {
    "tiny_b2_blk16": {},
    "sdar_b32_blk32": {"B": 12},
    "sdar_b256_blk32": {"B": 24},
    "sweep_b128_blk64": {"B": 10},
    "sweep_b128_blk16": {"B": 12},
    "longctx_b64_blk32": {"B": 4},
}


def _announce(msg):
    print(f"\n[case] {msg}", flush=True)


def _end_to_end(st, cap=None):
    ref = O.step(st)
    fs, gpu = run_gpu_step(st, cap=cap)
    derr = np.abs(gpu["delta"] - ref["delta"]).max()
    assert derr <= DELTA_TOL, f"delta error {derr}"
    excused = check_keep(gpu["keep"], ref["keep"], ref["delta"], st.masked, st.rule,
                         gpu["kept_count"])
    # offsets, kept positions and the gathered hidden rows request by request (an excused
    # request only shifts the offsets after it)
    check_ragged(gpu, ref, st.B, excused, st.rule, gathered_sets(gpu, st, ref["keep"]))
    oerr, lerr = compare_attention(gpu, ref, st.B, excused)
    return derr, oerr, lerr, len(excused)


@pytest.mark.parametrize("name", list(SMALL))
def test_step_reduced_batch(name):
    st = make_step(BY_NAME[name].scaled(**SMALL[name]))
    _announce(f"step {name} reduced {SMALL[name]}")
    derr, oerr, lerr, nex = _end_to_end(st)
    print(f"delta err {derr:.2e} out err {oerr:.2e} lse err {lerr:.2e} excused {nex}")


@pytest.mark.parametrize("name", ["sdar_b32_blk32", "sdar_b256_blk32", "sweep_b128_blk64",
                                  "sweep_b128_blk16", "longctx_b64_blk32"])
def test_step_full_size(name):
    st = make_step(BY_NAME[name])
    _announce(f"step {name} full size B={st.B}")
    delta = O.score_l01(st.q0, st.k0, st.q1, st.k1, st.sm_scale, st.score_dtype)
    keep, kept = O.select_budget(delta, st.masked, st.budget, st.rule)
    offsets, kept_pos, _ = O.compact(keep)
    fs, gpu = run_gpu_step(st)
    derr = np.abs(gpu["delta"] - delta).max()
    assert derr <= DELTA_TOL, f"delta error {derr}"
    excused = check_keep(gpu["keep"], keep, delta, st.masked, st.rule, gpu["kept_count"])
    check_ragged(gpu, {"offsets": offsets, "kept_pos": kept_pos}, st.B, excused, st.rule,
                 gathered_sets(gpu, st, keep))
    # attention on sampled requests: the oracle computes those rows one request at a time,
    # from the GPU-independent oracle-selected queries compared against the same GPU rows
    rng = np.random.default_rng(7)
    sample = rng.choice(st.B, size=min(st.B, 24), replace=False)
    sample = [r for r in sample if r not in excused]
    sample.append(int(np.argmax(st.prefix_len)))           # the longest prefix
    sample = sorted(set(sample))
    q64 = O.bf16_to_f64(st.q_att)
    owner = np.repeat(np.arange(st.B), np.diff(offsets))
    _, out, lse = oracle_attention(st, q64[owner, kept_pos], offsets, requests=sample)
    goff = gpu["offsets"]
    grows = np.concatenate([np.arange(goff[r], goff[r + 1]) for r in sample]).astype(np.int64)
    gidx = torch.as_tensor(grows, device=DEV)
    gout = fs.out[gidx].float().cpu().numpy()
    glse = fs.lse[gidx].cpu().numpy()
    oerr = np.abs(gout - out).max()
    lerr = np.abs(glse - lse).max()
    assert oerr <= OUT_TOL and lerr <= LSE_TOL, (oerr, lerr)
    print(f"delta err {derr:.2e} out err {oerr:.2e} lse err {lerr:.2e} excused {len(excused)}")


# ------------------------------------------------------------------------------- selection
@pytest.mark.parametrize("blk", [16, 32, 64])
@pytest.mark.parametrize("adaptive", [False, True])
def test_select_isolated(blk, adaptive):
    _announce(f"select blk={blk} adaptive={adaptive}")
    rng = np.random.default_rng(100 + blk)
    B = 300
    delta = np.round(rng.standard_normal((B, blk)) * 4) / 8  # many exact ties
    delta = delta.astype(np.float32)
    masked = (rng.random((B, blk)) < 0.6).astype(np.uint8)
    masked[0] = 0                                            # a request with nothing masked
    masked[1] = 1
    budget = rng.integers(-2, blk + 3, size=B).astype(np.int32)
    rule = ("adaptive", 0.5, 2, 16) if adaptive else ("fixed",)
    keep, kept = O.select_budget(delta.astype(np.float64), masked,
                                 None if adaptive else budget, rule)
    gk, gc = F.select_budget(torch.from_numpy(delta).to(DEV), torch.from_numpy(masked).to(DEV),
                             None if adaptive else torch.from_numpy(budget).to(DEV),
                             adaptive=rule[1:] if adaptive else None)
    gk, gc = gk.cpu().numpy(), gc.cpu().numpy()
    if adaptive:
        check_keep(gk, keep, delta.astype(np.float64), masked, rule, gc)
    else:
        assert np.array_equal(gk, keep) and np.array_equal(gc, kept)


@pytest.mark.parametrize("blk", [16, 32, 64])
@pytest.mark.parametrize("adaptive", [False, True])
def test_select_nonfinite_scores(blk, adaptive):
    # NaN ranks as -inf (ties by position), so exactly kept_count tokens are kept; a request
    # with a non-finite candidate has a NaN mean + beta*std under the adaptive rule, which
    # counts nothing: it keeps lo.  Then the compaction of that selection, whose neighbouring
    # requests must keep their own positions.
    _announce(f"select non-finite blk={blk} adaptive={adaptive}")
    rng = np.random.default_rng(300 + blk)
    B = 200
    delta = (np.round(rng.standard_normal((B, blk)) * 4) / 8).astype(np.float32)
    special = np.array([np.nan, np.inf, -np.inf], dtype=np.float32)
    hit = rng.random((B, blk)) < 0.15
    delta[hit] = special[rng.integers(0, 3, size=int(hit.sum()))]
    delta[5] = np.nan                                        # a request of NaNs only
    masked = (rng.random((B, blk)) < 0.6).astype(np.uint8)
    budget = rng.integers(0, blk + 2, size=B).astype(np.int32)
    rule = ("adaptive", 0.5, 2, 16) if adaptive else ("fixed",)
    keep, kept = O.select_budget(delta.astype(np.float64), masked,
                                 None if adaptive else budget, rule)
    gk, gc = F.select_budget(torch.from_numpy(delta).to(DEV), torch.from_numpy(masked).to(DEV),
                             None if adaptive else torch.from_numpy(budget).to(DEV),
                             adaptive=rule[1:] if adaptive else None)
    gk, gc = gk.cpu().numpy(), gc.cpu().numpy()
    assert np.array_equal(gc, gk.astype(np.int64).sum(axis=1)), "kept count != kept tokens"
    nonfinite = ~np.isfinite(np.where(masked == 1, delta, 0.0)).all(axis=1)
    assert np.array_equal(gk[nonfinite], keep[nonfinite])    # no tie excusal for these
    if adaptive:
        check_keep(gk, keep, delta.astype(np.float64), masked, rule, gc)
    else:
        assert np.array_equal(gk, keep) and np.array_equal(gc, kept)
    go, gp, _ = F.compact(torch.from_numpy(gk).to(DEV), None, cap=B * blk)
    off, pos, _ = O.compact(gk)
    assert np.array_equal(go.cpu().numpy(), off)
    assert np.array_equal(gp[: int(off[-1])].cpu().numpy(), pos)


def _nan_equal_close(a, b, tol):
    """Same NaN positions, finite entries within tol."""
    na, nb = np.isnan(a), np.isnan(b)
    assert np.array_equal(na, nb), "NaN positions differ"
    return np.abs(a[~na] - b[~na]).max() if (~na).any() else 0.0


@pytest.mark.parametrize("name,over", [("sdar_b32_blk32", {"B": 8}),
                                       ("sdar_b256_blk32", {"B": 10}),
                                       ("sweep_b128_blk16", {"B": 8})])
def test_front_end_nonfinite_inputs(name, over):
    # a NaN or an infinity in a layer-1 query turns every score of its request into NaN; the
    # selection then keeps the request's first k_r masked positions on both sides, and the
    # offsets and gathered rows of every other request stay as the oracle's
    st = make_step(BY_NAME[name].scaled(**over))
    _announce(f"front end non-finite {name} {over}")
    bad = {1: 0x7FC0, 4: 0x7F80, 6: 0xFF80}                   # NaN, +inf, -inf (bf16 bits)
    for r, bits in bad.items():
        if st.score_dtype == "bf16":
            st.q1[r, 3, 2, 5] = bits
        else:
            st.q1[r, 3, 2, 5] = {0x7FC0: np.nan, 0x7F80: np.inf, 0xFF80: -np.inf}[bits]
    ref = O.step(st, hidden=True)
    fs, gpu = run_gpu_step(st)
    for r in bad:
        assert np.isnan(ref["delta"][r]).all() and np.isnan(gpu["delta"][r]).all()
    derr = _nan_equal_close(gpu["delta"], ref["delta"], DELTA_TOL)
    assert derr <= DELTA_TOL, derr
    excused = check_keep(gpu["keep"], ref["keep"], ref["delta"], st.masked, st.rule,
                         gpu["kept_count"])
    assert not set(excused) & set(bad)
    check_ragged(gpu, ref, st.B, excused, st.rule, gathered_sets(gpu, st, ref["keep"]))


def test_step_never_gathers_decoded_rows():
    # rows at decoded positions of the hidden states and queries hold a sentinel: decoded
    # positions are never kept, so no gathered row may hold it and every gathered row equals
    # the oracle's (the fused score + select + compact path and the attention after it)
    st = make_step(BY_NAME["sdar_b256_blk32"].scaled(B=16))
    _announce("step sentinel rows at decoded positions")
    sentinel = np.uint16(0xA5A5)
    dec = st.masked == 0
    st.hidden[dec] = sentinel
    st.q_att[dec] = sentinel
    ref = O.step(st)
    for gather_q in (True, False):
        fs, gpu = run_gpu_step(st, gather_q=gather_q)
        excused = check_keep(gpu["keep"], ref["keep"], ref["delta"], st.masked, st.rule,
                             gpu["kept_count"])
        check_ragged(gpu, ref, st.B, excused, st.rule, gathered_sets(gpu, st, ref["keep"]))
        assert not (gpu["hidden_rows"] == sentinel).all(axis=1).any()
        if gather_q:
            assert not (gpu["q_rows"] == sentinel).all(axis=(1, 2)).any()
        compare_attention(gpu, ref, st.B, excused)


@pytest.mark.parametrize("nsets", [1, 2])
def test_compact_sentinel_rows_at_unkept_positions(nsets):
    # every unkept row of the gather sources holds a sentinel: a gather reading a wrong row
    # shows it (through compact and compact_multi)
    _announce(f"compact sentinel rows nsets={nsets}")
    rng = np.random.default_rng(41 + nsets)
    B, blk = 300, 32
    keep = (rng.random((B, blk)) < 0.12).astype(np.uint8)
    srcs = []
    for w in (4096, 256)[:nsets]:
        rows = rng.integers(0, 0xA5A4, size=(B, blk, w), dtype=np.uint16)
        rows[keep == 0] = 0xA5A5
        srcs.append(rows)
    off, pos, _ = O.compact(keep)
    T = int(off[-1])
    dk = torch.from_numpy(keep).to(DEV)
    dsrc = [bf16_tensor(x, DEV) for x in srcs]
    if nsets == 1:
        go, gp, gg = F.compact(dk, dsrc[0], cap=T)
        outs = [gg]
    else:
        go, gp, outs = F.compact_multi(dk, dsrc, cap=T)
    torch.cuda.synchronize()
    assert np.array_equal(go.cpu().numpy(), off)
    assert np.array_equal(gp[:T].cpu().numpy(), pos)
    for x, g in zip(srcs, outs):
        gb = bf16_to_np(g[:T])
        assert np.array_equal(gb, O.compact(keep, x)[2])
        assert not (gb == 0xA5A5).any()


# ------------------------------------------------------------------------------- compaction
@pytest.mark.parametrize("blk,B,row_bytes,capfrac", [(16, 7, 16, 1.0), (32, 256, 8192, 1.0),
                                                     (64, 33, 96, 0.3), (32, 1, 256, 0.0),
                                                     (64, 1500, 32, 1.0), (32, 2048, 48, 1.0),
                                                     (16, 2049, 16, 0.5), (64, 4096, 32, 1.0)])
def test_compact_isolated(blk, B, row_bytes, capfrac):
    # up to 2048 requests every workgroup counts its predecessors' kept tokens; above, a
    # one-workgroup scan of the kept counts runs first
    _announce(f"compact blk={blk} B={B} row_bytes={row_bytes} cap={capfrac}")
    rng = np.random.default_rng(blk * 1000 + B)
    keep = (rng.random((B, blk)) < 0.15).astype(np.uint8)
    keep[rng.random(B) < 0.2] = 0                            # requests keeping nothing
    rows = rng.integers(0, 256, size=(B, blk, row_bytes), dtype=np.uint8)
    T = int(keep.sum())
    cap = int(T * capfrac)
    offsets, kept_pos, gathered = O.compact(keep, rows, cap=cap)
    go, gp, gg = F.compact(torch.from_numpy(keep).to(DEV), torch.from_numpy(rows).to(DEV), cap=cap)
    assert np.array_equal(go.cpu().numpy(), offsets)
    assert np.array_equal(gp[:cap].cpu().numpy(), kept_pos)
    assert np.array_equal(gg[:cap].cpu().numpy(), gathered)
    # offsets only
    go2, _, _ = F.compact(torch.from_numpy(keep).to(DEV), None, cap=cap, with_pos=False)
    assert np.array_equal(go2.cpu().numpy(), offsets)


# ------------------------------------------------------------------------------- attention
def _random_keep(rng, B, blk, max_kept, empty_frac=0.1):
    keep = np.zeros((B, blk), dtype=np.uint8)
    for r in range(B):
        if rng.random() < empty_frac:
            continue
        k = int(rng.integers(1, max_kept + 1))
        keep[r, rng.choice(blk, size=k, replace=False)] = 1
    return keep


ATTN_CASES = {
    # name: (recipe, overrides, max_kept)
    "g4_d128_s64": ("sdar_b32_blk32", {"B": 9}, 4),
    "g4_q32rows": ("sdar_b32_blk32", {"B": 6}, 8),
    "g4_q64rows_blk64": ("sweep_b128_blk64", {"B": 5}, 16),
    "blk16_s64": ("sweep_b128_blk16", {"B": 7}, 4),
    "g1_d64_s16": ("tiny_b2_blk16", {"B": 5, "prefix": ("uniform", 0, 64)}, 4),
    "g2_d64_s32": ("tiny_b2_blk16", {"B": 6, "Hq": 8, "Hkv": 4, "S": 32,
                                     "prefix": ("uniform", 1, 300), "max_prefix": 320}, 8),
    "g8_d128_s16_split": ("longctx_b64_blk32", {"B": 3, "Hq": 16, "Hkv": 2,
                                                "prefix": ("uniform", 3000, 5000),
                                                "max_prefix": 5000}, 2),
    "g4_long_split": ("longctx_b64_blk32", {"B": 4}, 4),
    # two long requests with 32 and 64 rows per item: each item is cut into more pieces than
    # the 32-row kernel merges in one batch, so the piece-by-piece merge runs as well
    "g4_q32rows_many_pieces": ("longctx_b64_blk32", {"B": 2}, 8),
    "g4_q64rows_many_pieces": ("longctx_b64_blk32", {"B": 2}, 16),
    # launch bound above every request's kept count (as with adaptive budgets): four 64-row
    # query groups per kv head, of which two, or one, hold rows (the others compute nothing)
    "g4_q64rows_bound_2_of_4_groups": ("sweep_b128_blk64", {"B": 6}, 20, 64),
    "g4_q64rows_bound_1_of_4_groups": ("sweep_b128_blk64", {"B": 6}, 12, 64),
    # head dim 64 with shared tiles: 48 rows (16 per wave) and 96 rows (32 per wave)
    "g4_d64_q48rows_shared": ("tiny_b2_blk16", {"B": 5, "blk": 32, "Hq": 8, "Hkv": 2, "S": 32,
                                                "prefix": ("uniform", 1, 300),
                                                "max_prefix": 320}, 12),
    "g4_d64_q96rows_shared": ("tiny_b2_blk16", {"B": 5, "blk": 32, "Hq": 8, "Hkv": 2, "S": 32,
                                                "prefix": ("uniform", 1, 300),
                                                "max_prefix": 320}, 24),
    # shared 16-row waves over 16-token pages: a 32-key tile spans two pages, each thread's
    # share taking its keys and values from either
    "g4_d128_s16_q48rows_shared": ("longctx_b64_blk32", {"B": 4, "prefix": ("uniform", 1, 700),
                                                         "max_prefix": 800}, 12),
    "g4_d64_s16_q48rows_shared": ("tiny_b2_blk16", {"B": 5, "blk": 32, "Hq": 8, "Hkv": 2,
                                                    "prefix": ("uniform", 1, 300),
                                                    "max_prefix": 320}, 12),
    # the largest batches: 16 requests per thread in every workgroup's metadata scan and the
    # widest search rounds; one wave per item, and shared tiles with 4096 requests' metadata
    # beside the tile ring in LDS
    "g1_d64_b4096": ("tiny_b2_blk16", {"B": 4096, "prefix": ("uniform", 0, 64)}, 4),
    "g4_d64_b2500_shared": ("tiny_b2_blk16", {"B": 2500, "blk": 32, "Hq": 8, "Hkv": 2, "S": 32,
                                              "prefix": ("uniform", 1, 100),
                                              "max_prefix": 128}, 12),
    # shared tiles at head dim 128 with empty prefixes (block tiles only: one tile per item, a
    # new piece at every step) and a request without kept tokens among the others (the 19th
    # for this case's seed)
    "g4_d128_q64rows_prefix0_shared": ("tiny_b2_blk16", {"B": 24, "blk": 32, "Hq": 8, "Hkv": 2,
                                                         "d": 128, "S": 64,
                                                         "prefix": ("uniform", 0, 0),
                                                         "max_prefix": 64}, 16),
    # 384 rows per item (G = 8, 48 kept): three shared-tile workgroups per item, whose column
    # groups (six workgroups) do not divide the grid's XCD rounds evenly
    "g8_q384rows_shared": ("sweep_b128_blk64", {"B": 3, "Hq": 16, "Hkv": 2,
                                                "prefix": ("uniform", 1, 900),
                                                "max_prefix": 1024}, 48),
    # 4096 requests' metadata and the tile ring at head dim 128: the LDS holds one shared-tile
    # workgroup per CU, so the grid has one per CU
    "g4_d128_b4096_shared": ("tiny_b2_blk16", {"B": 4096, "blk": 32, "Hq": 8, "Hkv": 2, "d": 128,
                                               "S": 32, "prefix": ("uniform", 1, 70),
                                               "max_prefix": 96}, 12),
}


@pytest.mark.parametrize("case", list(ATTN_CASES))
def test_attn_isolated(case):
    name, over, max_kept = ATTN_CASES[case][:3]
    bound = ATTN_CASES[case][3] if len(ATTN_CASES[case]) > 3 else max_kept
    over = dict(over)
    over.setdefault("budget", ("fixed", max_kept))
    over["score_dtype"] = "bf16"
    st = make_step(BY_NAME[name].scaled(**over))
    _announce(f"attn {case} B={st.B} G={st.Hq // st.Hkv} d={st.d} S={st.S} blk={st.blk} "
              f"max_kept={max_kept} bound={bound} prefix_max={int(st.prefix_len.max())}")
    rng = np.random.default_rng(zlib.crc32(case.encode()) % 1000)
    keep = _random_keep(rng, st.B, st.blk, max_kept)
    c = attn_case_inputs(st, keep)
    ref_out, ref_lse = oracle_attention(st, c["q_rows64"], c["offsets"])
    t = step_inputs(st)
    out, lse = F.ragged_paged_attn(c["d_q"], c["d_offsets"], t.k_cache, t.v_cache, t.page_table,
                                   t.prefix_len, t.k_blk, t.v_blk, bound, st.sm_scale)
    torch.cuda.synchronize()
    T = int(c["offsets"][-1])
    go = out[:T].float().cpu().numpy()
    gl = lse[:T].cpu().numpy()
    oerr = np.abs(go - ref_out).max() if T else 0.0
    lerr = np.abs(gl - ref_lse).max() if T else 0.0
    assert oerr <= OUT_TOL and lerr <= LSE_TOL, (oerr, lerr)
    # the same rows with the queries read in place at the kept positions: the same bits
    pout, plse = F.ragged_paged_attn_pos(t.q_att, torch.from_numpy(c["kept_pos"]).to(DEV),
                                         c["d_offsets"], t.k_cache, t.v_cache, t.page_table,
                                         t.prefix_len, t.k_blk, t.v_blk, bound, st.sm_scale)
    torch.cuda.synchronize()
    assert torch.equal(pout[:T].view(torch.int16), out[:T].view(torch.int16))
    assert torch.equal(plse[:T].view(torch.int32), lse[:T].view(torch.int32))
    print(f"T={T} out err {oerr:.2e} lse err {lerr:.2e}")


def test_attn_peaky_inputs_and_cap():
    # unscaled N(0,1) queries make the softmax peaky (rescaling of the running max matters);
    # cap below T leaves the rows past cap untouched
    st = make_step(BY_NAME["sdar_b32_blk32"].scaled(B=8))
    _announce("attn peaky + cap")
    rng = np.random.default_rng(3)
    keep = _random_keep(rng, st.B, st.blk, 4, empty_frac=0.0)
    c = attn_case_inputs(st, keep)
    from workloads import f32_to_bf16_bits
    qbits = f32_to_bf16_bits(rng.standard_normal(c["q_bits"].shape).astype(np.float32) * 3.0)
    q64 = O.bf16_to_f64(qbits)
    T = int(c["offsets"][-1])
    cap = T - 5
    ref_out, ref_lse = oracle_attention(st, q64, c["offsets"], cap=cap)
    t = step_inputs(st)
    sentinel = torch.full((T, st.Hq, st.d), 7.0, dtype=torch.bfloat16, device=DEV)
    dq = bf16_tensor(qbits[:cap], DEV)
    out, lse = F.ragged_paged_attn(dq, c["d_offsets"], t.k_cache, t.v_cache, t.page_table,
                                   t.prefix_len, t.k_blk, t.v_blk, 4, st.sm_scale,
                                   out=sentinel[:cap])
    torch.cuda.synchronize()
    oerr = np.abs(out.float().cpu().numpy() - ref_out).max()
    lerr = np.abs(lse.cpu().numpy() - ref_lse).max()
    assert oerr <= OUT_TOL and lerr <= LSE_TOL, (oerr, lerr)
    assert torch.all(sentinel[cap:] == 7.0)


@pytest.mark.parametrize("max_kept", [4, 12, 24])
def test_attn_growing_logits_rescale(max_kept):
    # keys scaled up page by page along each prefix (and the block keys most): the running max
    # of a row keeps jumping by many log2 units inside an item, so the output is rescaled
    # several times per item and its weights span a wide range (one wave per item, and shared
    # tiles with 16- and 32-row waves)
    st = make_step(BY_NAME["sdar_b32_blk32"].scaled(B=6))
    _announce(f"attn growing logits, max_kept={max_kept}")
    from workloads import f32_to_bf16_bits, bf16_bits_to_f32
    kc = bf16_bits_to_f32(st.k_cache)
    seen = set()
    for r in range(st.B):
        for i in range(int(np.ceil(st.prefix_len[r] / st.S))):
            pid = int(st.page_table[r, i])
            if pid not in seen:
                seen.add(pid)
                kc[pid] *= 1.0 + 3.0 * i
    st.k_cache = f32_to_bf16_bits(kc)
    st.k_blk = f32_to_bf16_bits(bf16_bits_to_f32(st.k_blk) * 24.0)
    rng = np.random.default_rng(8)
    keep = _random_keep(rng, st.B, st.blk, max_kept, empty_frac=0.0)
    c = attn_case_inputs(st, keep)
    qbits = f32_to_bf16_bits(rng.standard_normal(c["q_bits"].shape).astype(np.float32) * 2.0)
    ref_out, ref_lse = oracle_attention(st, O.bf16_to_f64(qbits), c["offsets"])
    # the logits really span a wide range: several times the kernel's rescale step (8 log2
    # units, about 5.5 natural-log units)
    assert np.ptp(ref_lse) > 15.0
    t = step_inputs(st)
    out, lse = F.ragged_paged_attn(bf16_tensor(qbits, DEV), c["d_offsets"], t.k_cache, t.v_cache,
                                   t.page_table, t.prefix_len, t.k_blk, t.v_blk, max_kept,
                                   st.sm_scale)
    torch.cuda.synchronize()
    T = int(c["offsets"][-1])
    oerr = np.abs(out[:T].float().cpu().numpy() - ref_out).max()
    lerr = np.abs(lse[:T].cpu().numpy() - ref_lse).max()
    print(f"T={T} out err {oerr:.2e} lse err {lerr:.2e} max |lse| {np.abs(ref_lse).max():.1f}")
    assert oerr <= OUT_TOL and lerr <= LSE_TOL, (oerr, lerr)


@pytest.mark.parametrize("max_kept", [4, 12, 24])
def test_attn_poisoned_unused_memory_is_never_read(max_kept):
    # NaN in every cache slot past a prefix and in spare pages, out-of-range ids past each
    # request's last page: the result must equal the clean run bit for bit (one wave per item,
    # and shared tiles with 16- and 32-row waves over 16-token pages)
    _announce(f"attn poison, max_kept={max_kept}")
    rec = BY_NAME["longctx_b64_blk32"].scaled(B=4)
    clean = make_step(rec)
    pois = make_step(rec, poison=True)
    keep = _random_keep(np.random.default_rng(5), rec.B, rec.blk, max_kept, empty_frac=0.0)
    outs = []
    for st in (clean, pois):
        c = attn_case_inputs(st, keep)
        t = step_inputs(st)
        out, lse = F.ragged_paged_attn(c["d_q"], c["d_offsets"], t.k_cache, t.v_cache,
                                       t.page_table, t.prefix_len, t.k_blk, t.v_blk, max_kept,
                                       st.sm_scale)
        torch.cuda.synchronize()
        outs.append((bf16_to_np(out), lse.cpu().numpy()))
    assert np.isfinite(outs[1][1][: int(keep.sum())]).all()
    assert np.array_equal(outs[0][0], outs[1][0]) and np.array_equal(outs[0][1], outs[1][1])


@pytest.mark.parametrize("max_kept", [4, 12, 24])
def test_attn_invalid_device_data_gives_nan_rows(max_kept):
    # 4 kept tokens x G = 4: one wave per item; 12 and 24: shared tiles with 16- and 32-row
    # waves, where the invalid page id is seen by one thread's share and must reach every wave
    _announce(f"attn invalid page id / prefix length, max_kept={max_kept}")
    st = make_step(BY_NAME["sdar_b32_blk32"].scaled(B=6))
    keep = _random_keep(np.random.default_rng(9), st.B, st.blk, max_kept, empty_frac=0.0)
    c = attn_case_inputs(st, keep)
    t = step_inputs(st)
    ref, ref_lse = F.ragged_paged_attn(c["d_q"], c["d_offsets"], t.k_cache, t.v_cache,
                                       t.page_table, t.prefix_len, t.k_blk, t.v_blk, max_kept,
                                       st.sm_scale)
    pt = t.page_table.clone()
    pt[1, 0] = st.num_pages + 5          # request 1: a used page id out of range
    pl = t.prefix_len.clone()
    pl[3] = -4                           # request 3: negative prefix length
    out, lse = F.ragged_paged_attn(c["d_q"], c["d_offsets"], t.k_cache, t.v_cache, pt, pl,
                                   t.k_blk, t.v_blk, max_kept, st.sm_scale)
    torch.cuda.synchronize()
    off = c["offsets"]
    for r in range(st.B):
        rows = slice(int(off[r]), int(off[r + 1]))
        if r in (1, 3):
            assert torch.isnan(out[rows].float()).all() and torch.isnan(lse[rows]).all()
        else:
            # the other requests keep their results; not bit for bit, since a request's key
            # range may be cut at other places once the columns of requests 1 and 3 change
            assert torch.isfinite(out[rows].float()).all()
            oerr = (out[rows].float() - ref[rows].float()).abs().max().item()
            lerr = (lse[rows] - ref_lse[rows]).abs().max().item()
            assert oerr <= OUT_TOL and lerr <= LSE_TOL, (r, oerr, lerr)


@pytest.mark.parametrize("max_kept", [4, 12, 24])
def test_attn_pos_invalid_position_gives_nan_rows(max_kept):
    # queries read in place: a kept position outside the block reads no memory outside the
    # query tensor and turns its row (with the rows computed together with it) into NaN; the
    # other requests' rows keep their bits (the columns, and so the cuts, do not change)
    _announce(f"attn_pos invalid kept position, max_kept={max_kept}")
    st = make_step(BY_NAME["sdar_b32_blk32"].scaled(B=6))
    keep = _random_keep(np.random.default_rng(11), st.B, st.blk, max_kept, empty_frac=0.0)
    c = attn_case_inputs(st, keep)
    t = step_inputs(st)
    pos = torch.from_numpy(c["kept_pos"]).to(DEV)
    args = (t.k_cache, t.v_cache, t.page_table, t.prefix_len, t.k_blk, t.v_blk, max_kept,
            st.sm_scale)
    ref, ref_lse = F.ragged_paged_attn_pos(t.q_att, pos, c["d_offsets"], *args)
    off = c["offsets"]
    bad_rows = {int(off[2]): st.blk + 5, int(off[5]) - 1: -1}  # requests 2 and 4
    bpos = pos.clone()
    for n, v in bad_rows.items():
        bpos[n] = v
    out, lse = F.ragged_paged_attn_pos(t.q_att, bpos, c["d_offsets"], *args)
    torch.cuda.synchronize()
    for n in bad_rows:
        assert torch.isnan(out[n].float()).all() and torch.isnan(lse[n]).all(), n
    for r in range(st.B):
        for n in range(int(off[r]), int(off[r + 1])):
            same = torch.equal(out[n].view(torch.int16), ref[n].view(torch.int16)) and \
                torch.equal(lse[n].view(torch.int32), ref_lse[n].view(torch.int32))
            if r in (2, 4):
                assert same or (torch.isnan(out[n].float()).all() and
                                torch.isnan(lse[n]).all()), (r, n)
            else:
                assert same, (r, n)


@pytest.mark.parametrize("max_kept", [4, 12])
def test_attn_pos_capacity_cut(max_kept):
    # a capacity below the kept rows: the in-place call reads positions and writes rows only
    # below cap, with the bits of the compacted call under the same cap
    _announce(f"attn_pos capacity cut, max_kept={max_kept}")
    st = make_step(BY_NAME["sdar_b32_blk32"].scaled(B=8))
    keep = _random_keep(np.random.default_rng(13), st.B, st.blk, max_kept, empty_frac=0.0)
    c = attn_case_inputs(st, keep)
    t = step_inputs(st)
    T = int(c["offsets"][-1])
    cap = T - 7
    args = (t.k_cache, t.v_cache, t.page_table, t.prefix_len, t.k_blk, t.v_blk, max_kept,
            st.sm_scale)
    ref, ref_lse = F.ragged_paged_attn(c["d_q"][:cap].contiguous(), c["d_offsets"], *args)
    sentinel = torch.full((T, st.Hq, st.d), 7.0, dtype=torch.bfloat16, device=DEV)
    pos = torch.from_numpy(c["kept_pos"][:cap].copy()).to(DEV)
    out, lse = F.ragged_paged_attn_pos(t.q_att, pos, c["d_offsets"], *args, out=sentinel[:cap])
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
    assert torch.equal(lse.view(torch.int32), ref_lse.view(torch.int32))
    assert torch.all(sentinel[cap:] == 7.0)


def test_step_edge_cases_empty_prefix_and_nothing_masked():
    _announce("step edge cases")
    rec = BY_NAME["sdar_b32_blk32"].scaled(B=6, prefix=("uniform", 0, 200), budget=("fixed", 3))
    plen = np.array([0, 1, 31, 32, 33, 200])
    mcount = np.array([20, 0, 32, 25, 1, 20])    # request 1 has nothing masked: keeps nothing
    st = make_step(rec, prefix_override=plen, masked_override=mcount)
    derr, oerr, lerr, nex = _end_to_end(st)
    print(f"delta err {derr:.2e} out err {oerr:.2e} lse err {lerr:.2e}")


def test_deterministic_bitwise():
    _announce("determinism")
    st = make_step(BY_NAME["longctx_b64_blk32"].scaled(B=8))
    fs, a = run_gpu_step(st)
    fs.run()
    torch.cuda.synchronize()
    from parity_helpers import fetch
    b = fetch(fs)
    assert np.array_equal(a["delta"], b["delta"])
    assert np.array_equal(a["out_bits"], b["out_bits"])
    assert np.array_equal(a["lse"], b["lse"])


def test_attn_output_rounds_to_nearest_even():
    # q = 0 gives every key weight exactly 1, so with 63 values of 1.0 and one of 1.75 over 64
    # keys (32 prefix + 32 block) the f32 result is exactly 1 + 3/256, the midpoint between the
    # bf16 neighbours 1 + 1/128 (odd mantissa) and 1 + 1/64 (even): nearest-even gives 1 + 1/64.
    _announce("attn output rounding")
    from workloads import f32_to_bf16_bits, pack_v
    rec = BY_NAME["sdar_b32_blk32"].scaled(B=1)
    st = make_step(rec, prefix_override=np.array([32]))
    Hkv, d, S, blk = st.Hkv, st.d, st.S, st.blk
    vals = np.ones((64, Hkv, d), dtype=np.float32)
    vals[5] = 1.75                                          # one prefix key
    vbits = f32_to_bf16_bits(vals)
    pv = np.zeros((S, Hkv, d), dtype=np.uint16)
    pv[:32] = vbits[:32]
    st.v_cache[st.page_table[0, 0]] = pack_v(pv, S)[0]
    st.v_blk[0] = pack_v(vbits[32:], blk)[0]
    keep = np.zeros((1, blk), dtype=np.uint8)
    keep[0, 3] = 1
    c = attn_case_inputs(st, keep)
    t = step_inputs(st)
    dq = torch.zeros_like(c["d_q"])
    out, lse = F.ragged_paged_attn(dq, c["d_offsets"], t.k_cache, t.v_cache, t.page_table,
                                   t.prefix_len, t.k_blk, t.v_blk, 1, st.sm_scale)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy()
    assert np.all(got == 1.0 + 1.0 / 64), np.unique(got)
    assert np.allclose(lse.cpu().numpy(), np.log(64.0), atol=1e-6)


@pytest.mark.parametrize("case", ["g4_d128_s64", "g4_q64rows_blk64", "g8_d128_s16_split",
                                  "g1_d64_s16", "g4_q64rows_many_pieces"])
def test_attn_lse_only_equals_full_call(case):
    # without an output the kernel reads no values (none are given here) and its log-sum-exp
    # is the one of the full call: bit for bit with one query tile per item; with larger query
    # tiles the mode runs twice the workgroups, so items are cut elsewhere and the merges round
    # differently (f32 rounding only)
    name, over, max_kept = ATTN_CASES[case]
    over = dict(over)
    over.setdefault("budget", ("fixed", max_kept))
    over["score_dtype"] = "bf16"
    st = make_step(BY_NAME[name].scaled(**over))
    _announce(f"attn lse only {case}")
    keep = _random_keep(np.random.default_rng(21), st.B, st.blk, max_kept)
    c = attn_case_inputs(st, keep)
    t = step_inputs(st)
    _, lse_full = F.ragged_paged_attn(c["d_q"], c["d_offsets"], t.k_cache, t.v_cache,
                                      t.page_table, t.prefix_len, t.k_blk, t.v_blk, max_kept,
                                      st.sm_scale)
    out, lse = F.ragged_paged_attn(c["d_q"], c["d_offsets"], t.k_cache, None, t.page_table,
                                   t.prefix_len, t.k_blk, None, max_kept, st.sm_scale,
                                   want_out=False)
    torch.cuda.synchronize()
    T = int(c["offsets"][-1])
    assert out is None
    a_, b_ = lse[:T].cpu().numpy(), lse_full[:T].cpu().numpy()
    if max_kept * st.Hq // st.Hkv <= 16:
        assert np.array_equal(a_, b_)
    else:
        assert np.allclose(a_, b_, rtol=0, atol=4e-6 * max(1.0, np.abs(b_).max()))


def test_attn_nothing_kept():
    # every request keeps nothing: zero rows in, zero rows out, and the call succeeds
    _announce("attn nothing kept")
    st = make_step(BY_NAME["sdar_b32_blk32"].scaled(B=5, budget=("fixed", 4), score_dtype="bf16"))
    keep = np.zeros((st.B, st.blk), dtype=np.uint8)
    c = attn_case_inputs(st, keep)
    t = step_inputs(st)
    out, lse = F.ragged_paged_attn(c["d_q"], c["d_offsets"], t.k_cache, t.v_cache, t.page_table,
                                   t.prefix_len, t.k_blk, t.v_blk, 4, st.sm_scale)
    torch.cuda.synchronize()
    assert out.shape == (0, st.Hq, st.d) and lse.shape == (0, st.Hq)


def test_attn_shared_workspace_across_calls():
    # one zero-filled workspace serves a sequence of calls of different shapes, each with many
    # cut items (few requests, long prefixes): the arrival counters must come back to zero after
    # every call, or a later call would merge the wrong pieces
    _announce("attn shared workspace")
    seq = ["g8_d128_s16_split", "g4_d128_s64", "g4_q64rows_blk64", "g4_long_split",
           "g4_d64_q96rows_shared", "g8_d128_s16_split", "g4_q64rows_blk64"]
    steps = {}
    for case in set(seq):
        name, over, max_kept = ATTN_CASES[case]
        over = dict(over)
        over.setdefault("budget", ("fixed", max_kept))
        over["score_dtype"] = "bf16"
        st = make_step(BY_NAME[name].scaled(**over))
        steps[case] = (st, max_kept, F.attn_workspace_bytes(
            st.B, st.blk, st.Hq, st.Hkv, st.d, st.S, st.page_table.shape[1], max_kept))
    ws = torch.zeros(max(v[2] for v in steps.values()), dtype=torch.uint8, device=DEV)
    for case in seq:
        st, max_kept, need = steps[case]
        keep = _random_keep(np.random.default_rng(11), st.B, st.blk, max_kept, empty_frac=0.0)
        c = attn_case_inputs(st, keep)
        ref_out, ref_lse = oracle_attention(st, c["q_rows64"], c["offsets"])
        t = step_inputs(st)
        assert need <= ws.numel()
        for _ in range(2):
            out, lse = F.ragged_paged_attn(c["d_q"], c["d_offsets"], t.k_cache, t.v_cache,
                                           t.page_table, t.prefix_len, t.k_blk, t.v_blk,
                                           max_kept, st.sm_scale, workspace=ws)
            torch.cuda.synchronize()
            T = int(c["offsets"][-1])
            oerr = np.abs(out[:T].float().cpu().numpy() - ref_out).max()
            lerr = np.abs(lse[:T].cpu().numpy() - ref_lse).max()
            assert oerr <= OUT_TOL and lerr <= LSE_TOL, (case, oerr, lerr)


def test_step_graph_replay_matches_eager():
    # the whole step captured in a HIP graph: every replay, with eager work of the program in
    # between, must reproduce the eager step bit for bit (the kernels reset their own counters)
    _announce("graph replay")
    st = make_step(BY_NAME["sdar_b256_blk32"].scaled(B=24))
    fs, ref = run_gpu_step(st)
    from parity_helpers import fetch
    fs.capture()
    for rep in range(3):
        for name in ("out", "lse", "delta", "q_rows", "hidden_rows"):
            t = getattr(fs, name)
            if t is not None:
                t.fill_(0)
        torch.cuda.synchronize()
        fs.replay()
        torch.cuda.synchronize()
        got = fetch(fs)
        for key in ("delta", "keep", "offsets", "kept_pos", "out_bits", "lse", "hidden_rows"):
            assert np.array_equal(got[key], ref[key]), (rep, key)
        fs.run()  # eager work between replays
        torch.cuda.synchronize()


@pytest.mark.parametrize("name,over", [("sdar_b256_blk32", {"B": 6}),
                                       ("sweep_b128_blk64", {"B": 3}),
                                       ("longctx_b64_blk32", {"B": 2})])
def test_full_block_step(name, over):
    # the unfocused baseline: every block token is a query (k_r = blk), rows = G * blk per kv
    # head, so several query groups per item
    from decodability_aware_token_amd import FullBlockStep
    st = make_step(BY_NAME[name].scaled(**over))
    _announce(f"full-block step {name} {over}")
    keep = np.ones((st.B, st.blk), dtype=np.uint8)
    c = attn_case_inputs(st, keep)
    ref_out, ref_lse = oracle_attention(st, c["q_rows64"], c["offsets"])
    fb = FullBlockStep(step_inputs(st))
    fb.run()
    torch.cuda.synchronize()
    assert np.array_equal(fb.offsets.cpu().numpy(), c["offsets"])
    oerr = np.abs(fb.out.float().cpu().numpy() - ref_out).max()
    lerr = np.abs(fb.lse.cpu().numpy() - ref_lse).max()
    assert oerr <= OUT_TOL and lerr <= LSE_TOL, (oerr, lerr)
    print(f"rows={st.B * st.blk} out err {oerr:.2e} lse err {lerr:.2e}")


def _sample_requests(st, n, seed):
    rng = np.random.default_rng(seed)
    sample = set(int(r) for r in rng.choice(st.B, size=min(st.B, n), replace=False))
    sample.add(int(np.argmax(st.prefix_len)))  # the longest prefix
    return sorted(sample)


def test_full_block_step_full_size_sampled():
    # the unfocused baseline at the headline size, in the bench's launch configuration (all
    # 8192 block rows in one call), checked on sampled requests against the oracle
    from decodability_aware_token_amd import FullBlockStep
    st = make_step(BY_NAME["sdar_b256_blk32"])
    _announce(f"full-block step full size B={st.B}")
    fb = FullBlockStep(step_inputs(st))
    fb.run()
    torch.cuda.synchronize()
    sample = _sample_requests(st, 5, 31)
    keep = np.ones((st.B, st.blk), dtype=np.uint8)
    c = attn_case_inputs(st, keep)
    rows, out, lse = oracle_attention(st, c["q_rows64"], c["offsets"], requests=sample)
    gidx = torch.as_tensor(rows, device=DEV)
    oerr = np.abs(fb.out[gidx].float().cpu().numpy() - out).max()
    lerr = np.abs(fb.lse[gidx].cpu().numpy() - lse).max()
    assert oerr <= OUT_TOL and lerr <= LSE_TOL, (oerr, lerr)
    print(f"sampled {sample}: out err {oerr:.2e} lse err {lerr:.2e}")


def test_full_domain_score_full_size_sampled():
    # full-domain importance at the headline size (both layers' log-sum-exp-only attentions over
    # all 8192 block rows, then the score), checked on sampled requests against the oracle
    from decodability_aware_token_amd import FullDomainScore
    st = make_step(BY_NAME["sdar_b256_blk32"], layer0_prefix=True)
    _announce(f"full-domain score full size B={st.B}")
    from workloads.torch_io import upload
    t = upload(st)
    fd = FullDomainScore(step_inputs(st), t["k_cache0"], t["k_blk0"])
    got = fd.run().cpu().numpy()
    torch.cuda.synchronize()
    sample = _sample_requests(st, 4, 32)
    f64 = O.bf16_to_f64
    ref = O.score_l01_full(f64(st.q0[sample]), f64(st.k0[sample]), f64(st.q1[sample]),
                           f64(st.k1[sample]), f64(st.k_cache0), f64(st.k_cache),
                           st.page_table[sample], st.prefix_len[sample], st.sm_scale)
    err = np.abs(got[sample] - ref).max()
    assert err <= DELTA_TOL, err
    print(f"sampled {sample}: delta err {err:.2e}")


FULL_DOMAIN_CASES = {"sdar_b32_blk32": {"B": 4}, "longctx_b64_blk32": {"B": 2},
                     "sweep_b128_blk16": {"B": 3}}


@pytest.mark.parametrize("name", list(FULL_DOMAIN_CASES))
def test_full_domain_score(name):
    # layer-0/1 attentions over every block query give the row LSEs; the score variant then
    # weights block keys by exp(z - lse): compared with the oracle's softmax over prefix+block
    from decodability_aware_token_amd import FullDomainScore
    st = make_step(BY_NAME[name].scaled(**FULL_DOMAIN_CASES[name]), layer0_prefix=True)
    _announce(f"full-domain score {name} B={st.B} S={st.S}")
    f64 = O.bf16_to_f64
    ref = O.score_l01_full(f64(st.q0), f64(st.k0), f64(st.q1), f64(st.k1), f64(st.k_cache0),
                           f64(st.k_cache), st.page_table, st.prefix_len, st.sm_scale)
    from workloads.torch_io import upload
    t = upload(st)
    fd = FullDomainScore(step_inputs(st), t["k_cache0"], t["k_blk0"])
    got = fd.run()
    torch.cuda.synchronize()
    err = np.abs(got.cpu().numpy() - ref).max()
    assert err <= DELTA_TOL, err
    # the score call alone, fed the oracle's own row LSEs
    offs = np.arange(st.B + 1, dtype=np.int32) * st.blk
    rows0 = f64(st.q0).reshape(-1, st.Hq, st.d)
    rows1 = f64(st.q1).reshape(-1, st.Hq, st.d)
    _, l0 = O.ragged_paged_attn(rows0, offs, f64(st.k_cache0), f64(st.v_cache), st.page_table,
                                st.prefix_len, f64(st.k_blk0), f64(st.v_blk), st.sm_scale)
    _, l1 = O.ragged_paged_attn(rows1, offs, f64(st.k_cache), f64(st.v_cache), st.page_table,
                                st.prefix_len, f64(st.k_blk), f64(st.v_blk), st.sm_scale)
    lse0 = torch.from_numpy(l0.astype(np.float32).reshape(st.B, st.blk, st.Hq)).cuda()
    lse1 = torch.from_numpy(l1.astype(np.float32).reshape(st.B, st.blk, st.Hq)).cuda()
    got2 = F.score_l01_lse(t["q0"], t["k0"], t["q1"], t["k1"], lse0, lse1, st.sm_scale)
    torch.cuda.synchronize()
    err2 = np.abs(got2.cpu().numpy() - ref).max()
    assert err2 <= DELTA_TOL, err2
    print(f"delta err {err:.2e} (own LSE), {err2:.2e} (oracle LSE)")


# ------------------------------------------------------------------ KV write-back / commit
def _bits(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("name,over", [("sdar_b32_blk32", {"B": 6}),
                                       ("sweep_b128_blk64", {"B": 4, "d": 64}),
                                       ("sweep_b128_blk16", {"B": 5})])
def test_kv_writeback(name, over):
    from workloads import f32_to_bf16_bits
    st = make_step(BY_NAME[name].scaled(**over))
    _announce(f"kv writeback {name} {over}")
    rng = np.random.default_rng(41)
    keep = _random_keep(rng, st.B, st.blk, st.blk // 2)
    offsets, kept_pos, _ = O.compact(keep)
    T = int(offsets[-1])
    k_rows = f32_to_bf16_bits(rng.standard_normal((T, st.Hkv, st.d)).astype(np.float32))
    v_rows = f32_to_bf16_bits(rng.standard_normal((T, st.Hkv, st.d)).astype(np.float32))
    ref_k, ref_v = O.kv_writeback(k_rows, v_rows, offsets, kept_pos, st.k_blk, st.v_blk)
    kb, vb = bf16_tensor(st.k_blk, DEV), bf16_tensor(st.v_blk, DEV)
    F.kv_writeback(bf16_tensor(k_rows, DEV), bf16_tensor(v_rows, DEV),
                   torch.from_numpy(offsets).to(DEV), torch.from_numpy(kept_pos).to(DEV), kb, vb)
    torch.cuda.synchronize()
    assert np.array_equal(_bits(kb), ref_k) and np.array_equal(_bits(vb), ref_v)


def test_kv_writeback_repeated_and_invalid_positions():
    # a position named by several rows of a request takes the last of them (as the oracle's
    # row-order writes do); rows whose position is outside the block are skipped, so the
    # reference is the oracle on the other rows.  Request 1 writes a whole 8-position group.
    from workloads import f32_to_bf16_bits
    _announce("kv writeback repeated / invalid positions")
    rng = np.random.default_rng(43)
    B, blk, Hkv, d = 3, 32, 2, 64
    pos = [[3, 7, 3, 40, -1, 31, 7], list(range(8, 16)) + [20], []]
    offsets = np.concatenate([[0], np.cumsum([len(x) for x in pos])]).astype(np.int32)
    kept_pos = np.array(sum(pos, []), dtype=np.int32)
    T = int(offsets[-1])
    k_rows = f32_to_bf16_bits(rng.standard_normal((T, Hkv, d)).astype(np.float32))
    v_rows = f32_to_bf16_bits(rng.standard_normal((T, Hkv, d)).astype(np.float32))
    k_blk = f32_to_bf16_bits(rng.standard_normal((B, Hkv, d // 8, blk, 8)).astype(np.float32))
    v_blk = f32_to_bf16_bits(rng.standard_normal((B, Hkv, blk // 8, d, 8)).astype(np.float32))
    ok = (kept_pos >= 0) & (kept_pos < blk)
    owner = np.repeat(np.arange(B), np.diff(offsets))
    ref_off = np.concatenate([[0], np.cumsum(np.bincount(owner[ok], minlength=B))])
    ref_k, ref_v = O.kv_writeback(k_rows[ok], v_rows[ok], ref_off, kept_pos[ok], k_blk, v_blk)
    kb, vb = bf16_tensor(k_blk, DEV), bf16_tensor(v_blk, DEV)
    F.kv_writeback(bf16_tensor(k_rows, DEV), bf16_tensor(v_rows, DEV),
                   torch.from_numpy(offsets).to(DEV), torch.from_numpy(kept_pos).to(DEV), kb, vb)
    torch.cuda.synchronize()
    assert np.array_equal(_bits(kb), ref_k) and np.array_equal(_bits(vb), ref_v)


@pytest.mark.parametrize("n,Hkv,S,d,token_major", [(5, 8, 64, 128, False), (7, 4, 16, 128, True),
                                                   (3, 1, 32, 64, False), (9, 8, 16, 64, True),
                                                   (33, 3, 64, 64, True),
                                                   (520, 8, 64, 128, False)])
def test_kv_pack(n, Hkv, S, d, token_major):
    # arbitrary 16-bit patterns (NaN payloads included): the conversion is a move
    _announce(f"kv pack n={n} Hkv={Hkv} S={S} d={d} token_major={token_major}")
    rng = np.random.default_rng(n * 131 + S)
    shape = (n, S, Hkv, d) if token_major else (n, Hkv, S, d)
    k = rng.integers(0, 1 << 16, size=shape, dtype=np.uint16)
    v = rng.integers(0, 1 << 16, size=shape, dtype=np.uint16)
    ref_k, ref_v = O.kv_pack(k, v, token_major=token_major)
    gk, gv = F.kv_pack(bf16_tensor(k, DEV), bf16_tensor(v, DEV), token_major=token_major)
    torch.cuda.synchronize()
    assert np.array_equal(_bits(gk), ref_k) and np.array_equal(_bits(gv), ref_v)
    # one matrix alone; the other output is not written
    sentinel = torch.full(tuple(gv.shape), 7.0, dtype=torch.bfloat16, device=DEV)
    gk2, none = F.kv_pack(bf16_tensor(k, DEV), None, token_major=token_major)
    _, gv2 = F.kv_pack(None, bf16_tensor(v, DEV), token_major=token_major, v_out=sentinel)
    torch.cuda.synchronize()
    assert none is None and gv2 is sentinel
    assert np.array_equal(_bits(gk2), ref_k) and np.array_equal(_bits(gv2), ref_v)


def test_kv_pack_rebuilds_the_step_caches():
    # the generator's paged caches, unpacked to plain head-major rows, and its block KV from the
    # token-major layer-1 keys (and the block values unpacked to token-major rows), come back
    # bit for bit from focus_kv_pack
    st = make_step(BY_NAME["longctx_b64_blk32"].scaled(B=3))
    _announce("kv pack of the step caches (longctx, B=3)")
    pages, Hkv, D8, S, _ = st.k_cache.shape
    d = 8 * D8
    k_rows = st.k_cache.transpose(0, 1, 3, 2, 4).reshape(pages, Hkv, S, d)
    v_rows = st.v_cache.transpose(0, 1, 2, 4, 3).reshape(pages, Hkv, S, d)
    B, blk = st.k1.shape[0], st.k1.shape[1]
    v1 = st.v_blk.transpose(0, 2, 4, 1, 3).reshape(B, blk, Hkv, d)  # [B, blk, Hkv, d]
    gk, gv = F.kv_pack(bf16_tensor(k_rows, DEV), bf16_tensor(v_rows, DEV))
    bk, bv = F.kv_pack(bf16_tensor(st.k1, DEV), bf16_tensor(v1, DEV), token_major=True)
    torch.cuda.synchronize()
    assert np.array_equal(_bits(gk), st.k_cache) and np.array_equal(_bits(gv), st.v_cache)
    assert np.array_equal(_bits(bk), st.k_blk) and np.array_equal(_bits(bv), st.v_blk)


def _commit_case(st, rng, nfree, commit, shuffle=True):
    """Device state for a commit: the step's caches plus nfree free pages (the stack)."""
    pool = st.k_cache.shape[0]
    kc = np.concatenate([st.k_cache, np.zeros((nfree,) + st.k_cache.shape[1:], np.uint16)])
    vc = np.concatenate([st.v_cache, np.zeros((nfree,) + st.v_cache.shape[1:], np.uint16)])
    free = np.arange(pool, pool + nfree, dtype=np.int32)
    if shuffle:
        free = rng.permutation(free).astype(np.int32)
    return kc, vc, free


def _run_commit(st, kc, vc, table, plen, free, fc, commit):
    d = {"kc": bf16_tensor(kc, DEV), "vc": bf16_tensor(vc, DEV),
         "pt": torch.from_numpy(table.copy()).to(DEV),
         "pi": torch.from_numpy(plen.copy()).to(DEV),
         "po": torch.full((st.B,), -7, dtype=torch.int32, device=DEV),
         "fp": torch.from_numpy(free).to(DEV),
         "fi": torch.tensor([fc], dtype=torch.int32, device=DEV),
         "fo": torch.full((1,), -7, dtype=torch.int32, device=DEV),
         "st": torch.full((1,), -7, dtype=torch.int32, device=DEV)}
    F.block_commit(torch.from_numpy(commit).to(DEV), bf16_tensor(st.k_blk, DEV),
                   bf16_tensor(st.v_blk, DEV), d["kc"], d["vc"], d["pt"], d["pi"], d["po"],
                   d["fp"], d["fi"], d["fo"], d["st"])
    torch.cuda.synchronize()
    return d


@pytest.mark.parametrize("name,over", [("sdar_b32_blk32", {"B": 6}),
                                       ("longctx_b64_blk32", {"B": 3}),
                                       ("sweep_b128_blk16", {"B": 4, "S": 32}),
                                       ("tiny_b2_blk16", {"B": 5, "prefix": ("uniform", 0, 40),
                                                          "score_dtype": "bf16"})])
def test_block_commit(name, over):
    st = make_step(BY_NAME[name].scaled(**over))
    _announce(f"block commit {name} {over} plen={st.prefix_len.tolist()}")
    rng = np.random.default_rng(43)
    commit = (rng.random(st.B) < 0.7).astype(np.uint8)
    commit[0] = 1
    nfree = int(np.ceil(st.blk / st.S) + 1) * st.B + 3
    # the table rows must have room for one more block
    table = st.page_table
    need_cols = int((st.prefix_len.max() + st.blk + st.S - 1) // st.S)
    if table.shape[1] < need_cols:
        table = np.concatenate([table, np.full((st.B, need_cols - table.shape[1]), -1,
                                               np.int32)], axis=1)
    kc, vc, free = _commit_case(st, rng, nfree, commit)
    ref = O.block_commit(commit, st.k_blk, st.v_blk, kc, vc, table, st.prefix_len, free, nfree)
    d = _run_commit(st, kc, vc, table, st.prefix_len, free, nfree, commit)
    assert int(d["st"][0]) == ref[5] == 0
    assert int(d["fo"][0]) == ref[4]
    assert np.array_equal(d["po"].cpu().numpy(), ref[3])
    assert np.array_equal(d["pt"].cpu().numpy(), ref[2])
    assert np.array_equal(_bits(d["kc"]), ref[0]) and np.array_equal(_bits(d["vc"]), ref[1])
    # the committed state is attended like any prefix: the attention over it equals the
    # oracle's over the oracle's committed state
    keep = _random_keep(rng, st.B, st.blk, 4, empty_frac=0.0)
    c = attn_case_inputs(st, keep)
    o_out, o_lse = O.ragged_paged_attn(c["q_rows64"], c["offsets"], O.bf16_to_f64(ref[0]),
                                       O.bf16_to_f64(ref[1]), ref[2], ref[3],
                                       O.bf16_to_f64(st.k_blk), O.bf16_to_f64(st.v_blk),
                                       st.sm_scale)
    out, lse = F.ragged_paged_attn(c["d_q"], c["d_offsets"], d["kc"], d["vc"], d["pt"], d["po"],
                                   bf16_tensor(st.k_blk, DEV), bf16_tensor(st.v_blk, DEV), 4,
                                   st.sm_scale)
    torch.cuda.synchronize()
    T = int(c["offsets"][-1])
    assert np.abs(out[:T].float().cpu().numpy() - o_out).max() <= OUT_TOL
    assert np.abs(lse[:T].cpu().numpy() - o_lse).max() <= LSE_TOL


def test_block_commit_failures_change_nothing():
    st = make_step(BY_NAME["sdar_b32_blk32"].scaled(B=4))
    _announce("block commit failures")
    rng = np.random.default_rng(44)
    commit = np.ones(st.B, np.uint8)
    table = np.concatenate([st.page_table, np.full((st.B, 2), -1, np.int32)], axis=1)
    kc, vc, free = _commit_case(st, rng, 2, commit)
    aligned = (st.S * np.arange(1, st.B + 1)).astype(np.int32)   # one new page each
    for plen, fc, want in ((aligned, 2, 1),                                        # out of pages
                           (np.where(np.arange(st.B) == 2, table.shape[1] * st.S - 3,
                                     st.prefix_len).astype(np.int32), 2, 2),       # row overflow
                           (st.prefix_len, 5, 3)):                                 # count > stack
        d = _run_commit(st, kc, vc, table, plen, free, fc, commit)
        assert int(d["st"][0]) == want
        assert int(d["fo"][0]) == fc
        assert np.array_equal(d["po"].cpu().numpy(), plen)
        assert np.array_equal(d["pt"].cpu().numpy(), table)
        assert np.array_equal(_bits(d["kc"]), kc) and np.array_equal(_bits(d["vc"]), vc)


@pytest.mark.parametrize("name,over", [("sdar_b256_blk32", {"B": 24}),
                                       ("sweep_b128_blk64", {"B": 10}),
                                       ("tiny_b2_blk16", {})])
def test_fused_step_equals_separate_calls(name, over):
    # score+select in one launch and both gathers in one compaction launch give exactly the
    # results of the five separate entry points
    st = make_step(BY_NAME[name].scaled(**over))
    _announce(f"fused vs separate {name} {over}")
    from parity_helpers import fetch
    inp = step_inputs(st)
    runs = []
    for gather_q in (True, False):
        fs = FocusStep(inp, gather_q=gather_q)
        fs.run_unfused()
        torch.cuda.synchronize()
        a = fetch(fs)
        for nm in ("out", "delta", "q_rows", "hidden_rows", "keep", "kept_count", "offsets"):
            t = getattr(fs, nm)
            if t is not None:
                t.fill_(0)
        fs.run()
        torch.cuda.synchronize()
        b = fetch(fs)
        for key in ("delta", "keep", "kept_count", "offsets", "kept_pos", "out_bits", "lse",
                    "hidden_rows", "q_rows"):
            if key in a:
                assert np.array_equal(a[key], b[key]), (gather_q, key)
        runs.append(b)
    # queries read in place give the bits of the attention over the gathered queries
    for key in ("delta", "keep", "offsets", "kept_pos", "out_bits", "lse", "hidden_rows"):
        if key in runs[0]:
            assert np.array_equal(runs[0][key], runs[1][key]), key


@pytest.mark.parametrize("name,over,cap_frac", [
    ("tiny_b2_blk16", {}, 1.0),
    ("sdar_b32_blk32", {"B": 300, "prefix": ("fixed", 64), "max_prefix": 64}, 1.0),
    ("sdar_b32_blk32", {"B": 40, "prefix": ("fixed", 64), "max_prefix": 64}, 0.05),  # overflow
    ("sweep_b128_blk16", {"B": 33, "prefix": ("fixed", 64), "max_prefix": 64}, 1.0),
    ("sweep_b128_blk64", {"B": 21, "prefix": ("fixed", 64), "max_prefix": 64}, 1.0),
    ("tiny_b2_blk16", {"B": 4096}, 1.0),    # the largest batch: 16 requests per scan thread
    ("tiny_b2_blk16", {"B": 2500}, 0.3),    # the compaction's scan launch, with overflow
])
def test_score_select_compact_equals_two_calls(name, over, cap_frac):
    # the two-launch front end with per-request budgets (including budgets below zero and above
    # the masked count) gives exactly what score + select and the compaction give, also past
    # the first 256 predecessors and when the kept rows overflow cap
    st = make_step(BY_NAME[name].scaled(**over))
    _announce(f"score_select_compact {name} {over} cap_frac={cap_frac}")
    t = step_inputs(st)
    rng = np.random.default_rng(zlib.crc32(name.encode()) + st.B)
    budget = torch.from_numpy(rng.integers(-2, st.blk + 3, size=st.B).astype(np.int32)).cuda()
    sets = [t.q_att] if t.hidden is None else [t.hidden, t.q_att]
    cap = max(1, int(cap_frac * st.B * st.blk))
    d1, k1, c1 = F.score_select(t.q0, t.k0, t.q1, t.k1, t.sm_scale, t.masked, budget)
    o1, p1, g1 = F.compact_multi(k1, sets, cap)
    torch.cuda.synchronize()
    T = min(int(o1[-1]), cap)
    # the launch bound max_kept changes how many workgroups gather, never the results (even when
    # the budgets exceed it); repeated calls may share one workspace
    ws = torch.zeros(F.lib().focus_score_l01_workspace_size(st.B, st.blk, st.Hq, st.Hkv, st.d),
                     dtype=torch.uint8, device="cuda")
    for mk in (1, 1, 3, st.blk, 2):
        d2, k2, c2, o2, p2, g2 = F.score_select_compact(t.q0, t.k0, t.q1, t.k1, t.sm_scale,
                                                        t.masked, budget, sets, cap, max_kept=mk,
                                                        workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(d1, d2) and torch.equal(k1, k2) and torch.equal(c1, c2)
        assert torch.equal(o1, o2)
        assert torch.equal(p1[:T], p2[:T])
        for a, b in zip(g1, g2):
            assert torch.equal(a[:T].view(torch.int16), b[:T].view(torch.int16))
    # the kept counts follow the budgets: min(max(b, 0), masked count)
    m = t.masked.ne(0).sum(1).to(torch.int32)
    assert torch.equal(c2, torch.minimum(budget.clamp(min=0), m))


def test_score_select_compact_workspace_shared_across_shapes():
    # one workspace serves repeated calls of two shapes with a scoring call of a third shape in
    # between
    cases = [make_step(BY_NAME["sdar_b32_blk32"].scaled(B=300, prefix=("fixed", 64),
                                                        max_prefix=64)),
             make_step(BY_NAME["sweep_b128_blk16"].scaled(B=260, prefix=("fixed", 64),
                                                          max_prefix=64))]
    other_st = make_step(BY_NAME["sweep_b128_blk64"].scaled(B=9, prefix=("fixed", 64),
                                                            max_prefix=64))
    other = step_inputs(other_st)
    _announce("score_select_compact shared workspace")
    size = max(F.lib().focus_score_l01_workspace_size(c.B, c.blk, c.Hq, c.Hkv, c.d)
               for c in cases + [other_st])
    ws = torch.zeros(size, dtype=torch.uint8, device="cuda")
    refs = []
    for st in cases:
        t = step_inputs(st)
        rng = np.random.default_rng(st.B)
        budget = torch.from_numpy(rng.integers(0, st.blk + 1, size=st.B).astype(np.int32)).cuda()
        sets = [t.q_att] if t.hidden is None else [t.hidden, t.q_att]
        cap = st.B * st.blk
        d1, k1, c1 = F.score_select(t.q0, t.k0, t.q1, t.k1, t.sm_scale, t.masked, budget)
        o1, p1, g1 = F.compact_multi(k1, sets, cap)
        refs.append((t, budget, sets, cap, (d1, k1, c1, o1, p1, g1)))
    for rnd in range(2):
        for t, budget, sets, cap, ref in refs:
            got = F.score_select_compact(t.q0, t.k0, t.q1, t.k1, t.sm_scale, t.masked, budget,
                                         sets, cap, max_kept=1, workspace=ws)
            F.score_l01(other.q0, other.k0, other.q1, other.k1, other.sm_scale, workspace=ws)
            torch.cuda.synchronize()
            T = int(ref[3][-1])  # rows kept (below cap): the rest of the outputs is not written
            for x, y in zip(ref[:4], got[:4]):
                assert torch.equal(x, y), rnd
            assert torch.equal(ref[4][:T], got[4][:T]), rnd
            for x, y in zip(ref[5], got[5]):
                assert torch.equal(x[:T].view(torch.int16), y[:T].view(torch.int16)), rnd
