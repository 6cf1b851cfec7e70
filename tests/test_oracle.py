"""Pins for the fp64 oracle: closed forms, invariants, hand-derived cases and independent library
routines on tiny inputs.  CPU only.

Each pin is chosen so that a plausible mistake in the oracle fails it: a softmax over the wrong
axis, a transposed product, a wrong GQA head mapping, a flipped layer difference, a missing
sm_scale, a non-strict threshold, a sample instead of population std, a wrong tie order, a wrong
paged-layout index, a dropped block or prefix term, a missing normalisation.
"""
import math

import numpy as np
import pytest

import oracle as O
from workloads import BY_NAME, make_step, pack_k, pack_v, f32_to_bf16_bits

torch = pytest.importorskip("torch")


def _sig(x):
    return 1.0 / (1.0 + math.exp(-x))


# ------------------------------------------------------------------ scoring
def test_importance_uniform_when_queries_zero():
    # Q == 0 makes every softmax row uniform: each key receives 1/blk from each of the blk queries
    # of each of the Hq heads, so I(j) = Hq exactly.
    rng = np.random.default_rng(0)
    B, blk, Hq, Hkv, d = 2, 16, 6, 3, 8
    q = np.zeros((B, blk, Hq, d))
    k = rng.standard_normal((B, blk, Hkv, d))
    imp = O.layer_importance(q, k, 0.3)
    np.testing.assert_allclose(imp, Hq, rtol=0, atol=1e-12)


def test_importance_two_token_closed_form():
    # blk = 2, d = 1: row i's softmax weight on key 0 is sigmoid(c * q_i * (k0 - k1)), so
    # I(0) = sum_h sum_i sigmoid(c q_ih (k0_g - k1_g)) and I(1) = 2*Hq - I(0).
    c = 0.7
    q = np.array([[[[1.5], [-0.25]], [[0.5], [2.0]]]])          # [1, 2, Hq=2, 1]
    k = np.array([[[[0.8], [-1.0]], [[-0.4], [0.3]]]])          # [1, 2, Hkv=2, 1]
    imp = O.layer_importance(q, k, c)
    want0 = 0.0
    for h in range(2):
        g = h  # G = 1
        for i in range(2):
            want0 += _sig(c * q[0, i, h, 0] * (k[0, 0, g, 0] - k[0, 1, g, 0]))
    assert imp[0, 0] == pytest.approx(want0, abs=1e-14)
    assert imp[0, 1] == pytest.approx(4.0 - want0, abs=1e-14)


def test_importance_one_hot_attention_counts_and_gqa_mapping():
    # Orthonormal keys e_j and queries 40*e_pi(i): row i puts weight w = e^40/(e^40 + blk - 1) on
    # key pi(i) and (1-w)/(blk-1) on every other key, so
    #   I(j) = sum_h [ n_h(j) * w + (blk - n_h(j)) * (1 - w)/(blk - 1) ],  n_h(j) = #{i: pi_h(i) = j}.
    # Query heads 0,1 read kv head 0 and heads 2,3 read kv head 1 (h // G); the kv heads hold
    # different key orders, so a head-to-kv mapping of h % Hkv changes the counts.
    blk, d, Hq, Hkv = 8, 8, 4, 2
    eye = np.eye(d)
    k = np.zeros((1, blk, Hkv, d))
    k[0, :, 0, :] = eye                          # kv head 0: key j = e_j
    k[0, :, 1, :] = eye[::-1]                    # kv head 1: key j = e_{7-j}
    pi = [0, 0, 0, 3, 3, 5, 6, 1]                # target key of query i, for every head
    q = np.zeros((1, blk, Hq, d))
    for h in range(Hq):
        g = h // 2
        for i in range(blk):
            q[0, i, h, :] = 40.0 * k[0, pi[i], g, :]
    imp = O.layer_importance(q, k, 1.0)
    w = math.exp(40.0) / (math.exp(40.0) + blk - 1)
    counts = np.bincount(pi, minlength=blk)
    want = Hq * (counts * w + (blk - counts) * (1 - w) / (blk - 1))
    np.testing.assert_allclose(imp[0], want, rtol=0, atol=1e-12)


def test_delta_sign_and_sum_invariants():
    # Layer 0 with Q = 0 gives I0 = Hq; layer 1 one-hot attention onto key 2 gives
    # I1(2) ~= Hq*blk, so delta = I1 - I0 is positive at key 2 (layer 1 minus layer 0).
    blk, d, Hq = 8, 8, 2
    k = np.zeros((1, blk, 1, d)); k[0, :, 0, :] = np.eye(d)
    q1 = np.zeros((1, blk, Hq, d)); q1[0, :, :, 2] = 60.0
    q0 = np.zeros_like(q1)
    f = lambda a: a.astype(np.float32)
    delta = O.score_l01(f(q0), f(k), f(q1), f(k), 1.0, "f32")
    assert delta[0, 2] == pytest.approx(Hq * blk - Hq, abs=1e-9)
    assert abs(delta.sum()) < 1e-9
    # random inputs: rows sum to one => sum_j I_l(j) = Hq*blk and sum_j delta_j = 0
    st = make_step(BY_NAME["tiny_b2_blk16"])
    d2 = O.score_l01(st.q0, st.k0, st.q1, st.k1, st.sm_scale, "f32")
    i1 = O.layer_importance(O.to_f64(st.q1, "f32"), O.to_f64(st.k1, "f32"), st.sm_scale)
    np.testing.assert_allclose(i1.sum(axis=1), st.Hq * st.blk, atol=1e-9)
    np.testing.assert_allclose(d2.sum(axis=1), 0.0, atol=1e-9)


def test_identical_layers_give_zero_delta_and_permutation_equivariance():
    st = make_step(BY_NAME["tiny_b2_blk16"])
    d0 = O.score_l01(st.q1, st.k1, st.q1, st.k1, st.sm_scale, "f32")
    assert np.abs(d0).max() == 0.0
    perm = np.random.default_rng(3).permutation(st.blk)
    d = O.score_l01(st.q0, st.k0, st.q1, st.k1, st.sm_scale, "f32")
    dp = O.score_l01(st.q0[:, perm], st.k0[:, perm], st.q1[:, perm], st.k1[:, perm],
                     st.sm_scale, "f32")
    np.testing.assert_allclose(dp, d[:, perm], atol=1e-12)


def test_importance_against_torch_softmax():
    # independent library: torch float64 softmax over the key axis of (q k^T)*scale
    rng = np.random.default_rng(5)
    B, blk, Hq, Hkv, d = 2, 16, 8, 2, 16
    q = rng.standard_normal((B, blk, Hq, d))
    k = rng.standard_normal((B, blk, Hkv, d))
    imp = O.layer_importance(q, k, 0.4)
    tq = torch.from_numpy(q).permute(0, 2, 1, 3)                       # [B, Hq, blk, d]
    tk = torch.from_numpy(k).permute(0, 2, 1, 3).repeat_interleave(Hq // Hkv, dim=1)
    p = torch.softmax(0.4 * tq @ tk.transpose(-1, -2), dim=-1)          # [B, Hq, i, j]
    np.testing.assert_allclose(imp, p.sum(dim=(1, 2)).numpy(), atol=1e-12)


# ------------------------------------------------------------------ full-domain scoring
def _paged_prefix(rng, B, Hkv, d, S, plen, scale=1.0):
    """Random prefix keys per request, stored sequentially in pages; returns (k_cache float64
    in the paged layout, page_table, dense keys per request [P, Hkv, d])."""
    npg = [(-(-int(P) // S)) for P in plen]
    tot = max(sum(npg), 1)
    dense = rng.standard_normal((tot * S, Hkv, d)) * scale
    table = np.full((B, max(max(npg), 1)), -1, dtype=np.int32)
    base, keys = 0, []
    for r in range(B):
        table[r, : npg[r]] = np.arange(base, base + npg[r])
        keys.append(dense[base * S: base * S + int(plen[r])])
        base += npg[r]
    return pack_k(dense, S), table, keys


def test_full_domain_importance_without_prefix_is_block_only():
    # with no prefix key the full domain is the block: the two readings coincide
    rng = np.random.default_rng(21)
    B, blk, Hq, Hkv, d, S = 3, 16, 4, 2, 8, 16
    q = rng.standard_normal((B, blk, Hq, d))
    k = rng.standard_normal((B, blk, Hkv, d))
    kc, table, _ = _paged_prefix(rng, B, Hkv, d, S, [0, 0, 0])
    full = O.layer_importance_full(q, k, kc, table, np.zeros(B, np.int32), 0.4)
    np.testing.assert_allclose(full, O.layer_importance(q, k, 0.4), rtol=0, atol=1e-12)


def test_full_domain_importance_matches_torch_softmax_over_prefix_and_block():
    # an independent float64 torch.softmax over [prefix keys; block keys] per (r, h), read
    # through the page table, then the block columns summed over the queries
    rng = np.random.default_rng(22)
    B, blk, Hq, Hkv, d, S = 2, 16, 4, 2, 8, 16
    plen = np.array([37, 5], dtype=np.int32)
    q = rng.standard_normal((B, blk, Hq, d))
    k = rng.standard_normal((B, blk, Hkv, d))
    kc, table, keys = _paged_prefix(rng, B, Hkv, d, S, plen)
    got = O.layer_importance_full(q, k, kc, table, plen, 0.35)
    ref = np.zeros((B, blk))
    for r in range(B):
        for h in range(Hq):
            g = h // (Hq // Hkv)
            allk = torch.from_numpy(np.concatenate([keys[r][:, g, :], k[r, :, g, :]]))
            z = 0.35 * torch.from_numpy(q[r, :, h, :]) @ allk.T
            ref[r] += torch.softmax(z, dim=1)[:, plen[r]:].sum(dim=0).numpy()
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


def test_full_domain_importance_duplicate_prefix_key_closed_form():
    # one prefix token equal to block key 0: row i's full-domain weights are the block-only
    # ones divided by 1 + p_i0 (the duplicate adds the weight of key 0 to the denominator)
    rng = np.random.default_rng(23)
    blk, Hq, Hkv, d, S = 16, 2, 1, 8, 16
    q = rng.standard_normal((1, blk, Hq, d))
    k = rng.standard_normal((1, blk, Hkv, d))
    dense = np.zeros((S, Hkv, d))
    dense[0] = k[0, 0]
    kc = pack_k(dense, S)
    got = O.layer_importance_full(q, k, kc, np.array([[0]], np.int32), np.array([1]), 0.5)
    exp = np.zeros(blk)
    for h in range(Hq):
        z = 0.5 * q[0, :, h, :] @ k[0, :, 0, :].T
        p = np.exp(z - z.max(axis=1, keepdims=True))
        p = p / p.sum(axis=1, keepdims=True)
        exp += (p / (1.0 + p[:, :1])).sum(axis=0)
    np.testing.assert_allclose(got[0], exp, rtol=1e-12, atol=1e-12)


def test_full_domain_importance_is_below_block_only_and_mass_adds_up():
    # a superset of keys only grows each row's denominator: every block key's weight shrinks;
    # the block mass plus the prefix mass is Hq * blk
    rng = np.random.default_rng(24)
    B, blk, Hq, Hkv, d, S = 2, 32, 4, 4, 8, 16
    plen = np.array([50, 17], dtype=np.int32)
    q = rng.standard_normal((B, blk, Hq, d))
    k = rng.standard_normal((B, blk, Hkv, d))
    kc, table, keys = _paged_prefix(rng, B, Hkv, d, S, plen)
    full = O.layer_importance_full(q, k, kc, table, plen, 0.3)
    assert np.all(full <= O.layer_importance(q, k, 0.3) + 1e-12)
    for r in range(B):
        pm = 0.0
        for h in range(Hq):
            allk = np.concatenate([keys[r][:, h, :], k[r, :, h, :]])
            z = 0.3 * q[r, :, h, :] @ allk.T
            p = np.exp(z - z.max(axis=1, keepdims=True))
            p = p / p.sum(axis=1, keepdims=True)
            pm += p[:, : plen[r]].sum()
        assert abs(full[r].sum() + pm - Hq * blk) < 1e-9


def test_full_domain_score_is_layer_difference_with_own_caches():
    # delta takes layer 1 minus layer 0, each with its own prefix cache: swapping the layers
    # (inputs and caches together) negates it
    rng = np.random.default_rng(25)
    B, blk, Hq, Hkv, d, S = 2, 16, 4, 2, 8, 16
    plen = np.array([20, 9], dtype=np.int32)
    q0, q1 = rng.standard_normal((2, B, blk, Hq, d))
    k0, k1 = rng.standard_normal((2, B, blk, Hkv, d))
    kc0, table, _ = _paged_prefix(rng, B, Hkv, d, S, plen)
    kc1 = pack_k(rng.standard_normal((kc0.shape[0] * S, Hkv, d)), S)
    a = O.score_l01_full(q0, k0, q1, k1, kc0, kc1, table, plen, 0.3)
    b = O.score_l01_full(q1, k1, q0, k0, kc1, kc0, table, plen, 0.3)
    np.testing.assert_allclose(a, -b, rtol=0, atol=1e-12)
    assert abs(a.sum()) > 1e-6


def test_full_domain_score_orientation_closed_form():
    # Layer 0: Q == 0, so each block query spreads its weight evenly over all P + blk keys of
    # that layer (prefix and block): I0(j) = Hq * blk / (P + blk).  Layer 1: block key j is e_j,
    # its prefix keys are zero, and every query is c * e_t: a row gives key t the weight
    # e^c / (e^c + P + blk - 1) and every other key 1 / (e^c + P + blk - 1).  So
    #   delta(t) = Hq*blk*e^c/(e^c+n-1) - Hq*blk/n > 0,  delta(j != t) = Hq*blk/(e^c+n-1) - Hq*blk/n < 0
    # with n = P + blk.  A flipped difference, a dropped prefix or the layers' caches swapped
    # (layer 0's random prefix keys in layer 1) all change these values.
    rng = np.random.default_rng(26)
    B, blk, Hq, Hkv, d, S = 1, 8, 2, 1, 8, 16
    P, t, c = 21, 5, 3.0
    plen = np.array([P], dtype=np.int32)
    kc0, table, _ = _paged_prefix(rng, B, Hkv, d, S, plen)                 # random, unused by Q0 = 0
    kc1, table1, _ = _paged_prefix(rng, B, Hkv, d, S, plen, scale=0.0)     # zero prefix keys
    assert np.array_equal(table, table1)
    kb = np.zeros((B, blk, Hkv, d)); kb[0, :, 0, :] = np.eye(d)
    q0 = np.zeros((B, blk, Hq, d))
    q1 = np.zeros((B, blk, Hq, d)); q1[0, :, :, t] = c
    delta = O.score_l01_full(q0, kb, q1, kb, kc0, kc1, table, plen, 1.0)
    n = P + blk
    i0 = Hq * blk / n
    want = np.full(blk, Hq * blk / (math.exp(c) + n - 1) - i0)
    want[t] = Hq * blk * math.exp(c) / (math.exp(c) + n - 1) - i0
    np.testing.assert_allclose(delta[0], want, rtol=0, atol=1e-12)
    assert delta[0, t] > 0 and np.all(np.delete(delta[0], t) < 0)


# ------------------------------------------------------------------ selection
def test_kth_boundary_hand_cases():
    # masked scores, largest first: 0.9, 0.9, 0.5, 0.3, -0.1; the decoded 2.0 never counts.
    # An ascending order, an off-by-one index or counting decoded positions changes one of these.
    delta = np.array([0.3, 0.9, 2.0, 0.9, -0.1, 0.5])
    masked = np.array([1, 1, 0, 1, 1, 1], dtype=np.uint8)
    got = [O.kth_boundary(delta, masked, k) for k in range(1, 8)]
    assert got == [0.9, 0.9, 0.5, 0.3, -0.1, -0.1, -0.1]     # k = 5 = m; k > m clips to m
    assert math.isnan(O.kth_boundary(delta, masked, 0))
    assert math.isnan(O.kth_boundary(delta, masked, -2))
    assert math.isnan(O.kth_boundary(delta, np.zeros(6, np.uint8), 3))
    # a score that is not a number ranks as minus infinity
    dn = np.array([np.nan, 0.2, -np.inf, 0.1])
    assert O.kth_boundary(dn, np.ones(4, np.uint8), 2) == 0.1
    assert O.kth_boundary(dn, np.ones(4, np.uint8), 3) == -math.inf


def test_kth_boundary_is_the_smallest_kept_score():
    # against the selection (itself pinned by the lexsort brute force below): for every request
    # with 0 < k, the boundary equals the smallest kept score and no unkept candidate is above it
    rng = np.random.default_rng(12)
    B, blk = 60, 16
    delta = np.round(rng.standard_normal((B, blk)), 1)
    masked = (rng.random((B, blk)) < 0.7).astype(np.uint8)
    budget = rng.integers(0, blk + 3, size=B)
    keep, kept = O.select_budget(delta, masked, budget)
    for r in range(B):
        t = O.kth_boundary(delta[r], masked[r], int(kept[r]))
        if kept[r] == 0:
            assert math.isnan(t)
            continue
        assert t == delta[r][keep[r] == 1].min()
        rest = delta[r][(masked[r] == 1) & (keep[r] == 0)]
        assert rest.size == 0 or rest.max() <= t


def test_select_nan_ranks_below_every_number():
    # NaN ranks as -inf: below every number, tied with -inf (lower position first), so exactly
    # k tokens are kept and the mean/std of the adaptive rule turn NaN (no count above it)
    delta = np.array([[np.nan, 0.5, -np.inf, np.nan, -3.0, np.inf]])
    masked = np.ones((1, 6), dtype=np.uint8)
    for k, want in [(1, [0, 0, 0, 0, 0, 1]), (2, [0, 1, 0, 0, 0, 1]), (3, [0, 1, 0, 0, 1, 1]),
                    (4, [1, 1, 0, 0, 1, 1]), (5, [1, 1, 1, 0, 1, 1]), (6, [1] * 6)]:
        keep, kept = O.select_budget(delta, masked, np.array([k]))
        assert keep[0].tolist() == want and kept[0] == k, k
    assert O.request_budget(delta[0], masked[0], None, ("adaptive", 0.5, 2, 16)) == 2
    keep, kept = O.select_budget(delta, masked, None, ("adaptive", 0.5, 2, 16))
    assert keep[0].tolist() == [0, 1, 0, 0, 0, 1] and kept[0] == 2


def test_select_hand_example():
    delta = np.array([[0.1, 0.9, 0.5, 0.9, -0.2, 0.7, 0.0, 0.3]])
    masked = np.array([[1, 1, 1, 1, 1, 0, 1, 1]], dtype=np.uint8)
    keep, kept = O.select_budget(delta, masked, np.array([3]))
    # position 5 (0.7) is decoded and may not be kept; ranking 1,3 (0.9 tie: lower first), 2
    assert keep[0].tolist() == [0, 1, 1, 1, 0, 0, 0, 0]
    assert kept.tolist() == [3]


def test_select_ties_lower_position_wins_and_budget_clipping():
    delta = np.array([[0.5, 0.5, 0.5, 0.5], [0.5, 0.5, 0.5, 0.5], [1, 2, 3, 4.0]])
    masked = np.array([[1, 1, 1, 1], [0, 1, 0, 1], [1, 0, 1, 0]], dtype=np.uint8)
    keep, kept = O.select_budget(delta, masked, np.array([2, 10, -3]))
    assert keep.tolist() == [[1, 1, 0, 0], [0, 1, 0, 1], [0, 0, 0, 0]]
    assert kept.tolist() == [2, 2, 0]          # min(b, m), negative budget keeps nothing


def test_adaptive_rule_strict_threshold():
    # beta = 0: threshold = mean = 0.5; the value equal to it is NOT counted (strict >)
    delta = np.array([[1.0, 0.5, 0.0, 0.5]])
    masked = np.ones((1, 4), dtype=np.uint8)
    assert O.request_budget(delta[0], masked[0], None, ("adaptive", 0.0, 0, 16)) == 1
    keep, kept = O.select_budget(delta, masked, None, ("adaptive", 0.0, 0, 16))
    assert keep[0].tolist() == [1, 0, 0, 0]


def test_adaptive_rule_population_std_and_clamp():
    # candidates [0,0,0,0,0,0,3.25,5.75], beta=1: mean = 9/8, sum of squared deviations = 33.5,
    # population sigma = sqrt(33.5/8) = 2.0463 -> threshold 3.1713 -> c = 2 (3.25 and 5.75);
    # a sample sigma sqrt(33.5/7) would give threshold 3.3126 and c = 1.
    delta = np.array([[0, 0, 3.25, 0, 0, 0, 5.75, 0, 9.0]])
    masked = np.array([[1, 1, 1, 1, 1, 1, 1, 1, 0]], dtype=np.uint8)   # 9.0 is decoded
    assert O.request_budget(delta[0], masked[0], None, ("adaptive", 1.0, 1, 16)) == 2
    assert O.adaptive_threshold(delta[0], masked[0], 1.0) == pytest.approx(
        1.125 + math.sqrt(33.5 / 8), abs=1e-12)
    # clamp: lo raises the count, hi lowers it
    assert O.request_budget(delta[0], masked[0], None, ("adaptive", 1.0, 5, 16)) == 5
    assert O.request_budget(delta[0], masked[0], None, ("adaptive", 1.0, 0, 1)) == 1
    keep, kept = O.select_budget(delta, masked, None, ("adaptive", 1.0, 3, 16))
    # three kept: 5.75 (6), 3.25 (2), then the lowest-position zero (0)
    assert keep[0].tolist() == [1, 0, 1, 0, 0, 0, 1, 0, 0] and kept[0] == 3


def test_select_matches_lexsort_brute_force_and_invariants():
    rng = np.random.default_rng(11)
    B, blk = 40, 32
    delta = np.round(rng.standard_normal((B, blk)), 1)          # many exact ties
    masked = (rng.random((B, blk)) < 0.7).astype(np.uint8)
    budget = rng.integers(-1, 12, size=B)
    keep, kept = O.select_budget(delta, masked, budget)
    for r in range(B):
        cand = np.nonzero(masked[r])[0]
        order = cand[np.lexsort((cand, -delta[r, cand]))]
        k = min(max(int(budget[r]), 0), cand.size)
        assert set(np.nonzero(keep[r])[0]) == set(order[:k])
        assert kept[r] == k and not np.any(keep[r] & (1 - masked[r]))
        if 0 < k < cand.size:
            kd = delta[r][keep[r] == 1]
            rest = delta[r][(masked[r] == 1) & (keep[r] == 0)]
            assert kd.min() >= rest.max()


# ------------------------------------------------------------------ compaction
def test_compact_hand_example_and_cap():
    keep = np.array([[0, 1, 1, 0], [0, 0, 0, 0], [1, 0, 0, 1]], dtype=np.uint8)
    rows = np.arange(3 * 4 * 2).reshape(3, 4, 2)
    off, pos, gat = O.compact(keep, rows)
    assert off.tolist() == [0, 2, 2, 4]
    assert pos.tolist() == [1, 2, 0, 3]
    assert gat.tolist() == [[2, 3], [4, 5], [16, 17], [22, 23]]
    off, pos, gat = O.compact(keep, rows, cap=3)
    assert off.tolist() == [0, 2, 2, 4] and pos.tolist() == [1, 2, 0] and len(gat) == 3


def test_compact_matches_cumsum_and_nonzero():
    rng = np.random.default_rng(2)
    keep = (rng.random((50, 64)) < 0.2).astype(np.uint8)
    off, pos, _ = O.compact(keep)
    assert off.tolist() == [0] + np.cumsum(keep.sum(axis=1)).tolist()
    assert pos.tolist() == np.concatenate([np.nonzero(row)[0] for row in keep]).tolist()


# ------------------------------------------------------------------ attention
def _tiny_attn_case(B=3, blk=16, Hq=4, Hkv=2, d=16, S=16, plen=(20, 0, 37), seed=0,
                    fragmented=True):
    """Logical per-request K/V plus the same data in the paged layouts (built with the input
    generator's packers, which are independent of the oracle)."""
    rng = np.random.default_rng(seed)
    plen = np.asarray(plen)
    maxp = int(-(-plen.max() // S)) or 1
    npg = -(-plen // S)
    pool = int(npg.sum()) + 3
    ids = rng.permutation(pool) if fragmented else np.arange(pool)
    table = np.full((B, maxp), -1, dtype=np.int32)
    logical_k, logical_v = [], []
    kc = np.zeros((pool, Hkv, d // 8, S, 8)); vc = np.zeros((pool, Hkv, S // 8, d, 8))
    pos = 0
    for r in range(B):
        P = int(plen[r])
        table[r, : npg[r]] = ids[pos: pos + npg[r]]; pos += npg[r]
        kk = rng.standard_normal((P, Hkv, d)); vv = rng.standard_normal((P, Hkv, d))
        logical_k.append(kk); logical_v.append(vv)
        padk = np.zeros((npg[r] * S, Hkv, d)); padk[:P] = kk
        padv = np.zeros((npg[r] * S, Hkv, d)); padv[:P] = vv
        if npg[r]:
            kc[table[r, : npg[r]]] = pack_k(padk, S)
            vc[table[r, : npg[r]]] = pack_v(padv, S)
    kb = rng.standard_normal((B, blk, Hkv, d)); vb = rng.standard_normal((B, blk, Hkv, d))
    kblk = pack_k(kb.reshape(B * blk, Hkv, d), blk); vblk = pack_v(vb.reshape(B * blk, Hkv, d), blk)
    return dict(B=B, blk=blk, Hq=Hq, Hkv=Hkv, d=d, S=S, plen=plen.astype(np.int32), table=table,
                kc=kc, vc=vc, kblk=kblk, vblk=vblk, lk=logical_k, lv=logical_v, kb=kb, vb=vb)


def _run(c, q, offsets, scale=0.25):
    return O.ragged_paged_attn(q, offsets, c["kc"], c["vc"], c["table"], c["plen"], c["kblk"],
                               c["vblk"], scale)


def test_attn_against_torch_sdpa_on_dense_kv():
    # independent library on the dense (unpaged) KV: prefix tokens then block tokens
    c = _tiny_attn_case()
    rng = np.random.default_rng(1)
    offsets = np.array([0, 2, 3, 7], dtype=np.int32)
    q = rng.standard_normal((7, c["Hq"], c["d"]))
    out, lse = _run(c, q, offsets)
    G = c["Hq"] // c["Hkv"]
    for r in range(c["B"]):
        lo, hi = offsets[r], offsets[r + 1]
        K = np.concatenate([c["lk"][r], c["kb"][r]], axis=0)       # [n, Hkv, d]
        V = np.concatenate([c["lv"][r], c["vb"][r]], axis=0)
        tq = torch.from_numpy(q[lo:hi]).permute(1, 0, 2)           # [Hq, rows, d]
        tk = torch.from_numpy(K).permute(1, 0, 2).repeat_interleave(G, 0)
        tv = torch.from_numpy(V).permute(1, 0, 2).repeat_interleave(G, 0)
        ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, scale=0.25)
        np.testing.assert_allclose(out[lo:hi], ref.permute(1, 0, 2).numpy(), atol=1e-12)
        ref_lse = torch.logsumexp(0.25 * tq @ tk.transpose(-1, -2), dim=-1).T.numpy()
        np.testing.assert_allclose(lse[lo:hi], ref_lse, atol=1e-12)


def test_attn_zero_query_is_mean_of_values():
    # q == 0: uniform weights over all P_r + blk keys -> O = mean(V), LSE = log(P_r + blk)
    c = _tiny_attn_case()
    offsets = np.array([0, 1, 2, 3], dtype=np.int32)
    out, lse = _run(c, np.zeros((3, c["Hq"], c["d"])), offsets)
    G = c["Hq"] // c["Hkv"]
    for r in range(3):
        V = np.concatenate([c["lv"][r], c["vb"][r]], axis=0)
        for h in range(c["Hq"]):
            np.testing.assert_allclose(out[r, h], V[:, h // G, :].mean(axis=0), atol=1e-12)
            assert lse[r, h] == pytest.approx(math.log(c["plen"][r] + c["blk"]), abs=1e-12)


def test_attn_constant_values_and_dominant_key():
    c = _tiny_attn_case()
    offsets = np.array([0, 1, 1, 2], dtype=np.int32)
    rng = np.random.default_rng(4)
    q = rng.standard_normal((2, c["Hq"], c["d"]))
    # V == 1 -> O == 1 (weights are normalised)
    c1 = dict(c); c1["vc"] = np.ones_like(c["vc"]); c1["vblk"] = np.ones_like(c["vblk"])
    out, _ = _run(c1, q, offsets)
    np.testing.assert_allclose(out, 1.0, atol=1e-12)
    # a query aligned with prefix token 33 of request 2 (page 2, slot 1) at scale 50 takes
    # that token's value: exp(-gap) of the others is below 1e-12
    r, t, g = 2, 33, 1
    kvec = c["lk"][r][t, g]
    q2 = np.zeros((2, c["Hq"], c["d"]))
    q2[1, 2] = 50.0 * kvec / (kvec @ kvec)
    out, lse = _run(c, q2, offsets, scale=1.0)
    np.testing.assert_allclose(out[1, 2], c["lv"][r][t, g], atol=1e-10)


def test_attn_two_groups_sigmoid_closed_form():
    # all keys equal to a (n_a of them: prefix) or b (n_b: block); values vA / vB.  With
    # z_a = s q.a, z_b = s q.b: O = sigmoid(z_a - z_b + log(n_a/n_b)) vA + (1 - that) vB.
    c = _tiny_attn_case(B=1, plen=(21,), fragmented=False)
    d, Hkv, S = c["d"], c["Hkv"], c["S"]
    rng = np.random.default_rng(7)
    a, b = rng.standard_normal(d), rng.standard_normal(d)
    vA, vB = rng.standard_normal(d), rng.standard_normal(d)
    c["kc"][:] = pack_k(np.broadcast_to(a, (c["kc"].shape[0] * S, Hkv, d)).copy(), S)
    c["vc"][:] = pack_v(np.broadcast_to(vA, (c["vc"].shape[0] * S, Hkv, d)).copy(), S)
    c["kblk"][:] = pack_k(np.broadcast_to(b, (c["blk"], Hkv, d)).copy(), c["blk"])
    c["vblk"][:] = pack_v(np.broadcast_to(vB, (c["blk"], Hkv, d)).copy(), c["blk"])
    q = rng.standard_normal((1, c["Hq"], d))
    out, _ = _run(c, q, np.array([0, 1], dtype=np.int32), scale=0.3)
    for h in range(c["Hq"]):
        x = 0.3 * (q[0, h] @ a) - 0.3 * (q[0, h] @ b) + math.log(21 / c["blk"])
        w = _sig(x)
        np.testing.assert_allclose(out[0, h], w * vA + (1 - w) * vB, atol=1e-12)


def test_attn_gqa_mapping_and_page_permutation_invariance():
    c = _tiny_attn_case(Hq=6, Hkv=3)
    offsets = np.array([0, 2, 2, 4], dtype=np.int32)
    rng = np.random.default_rng(8)
    q = rng.standard_normal((4, 6, c["d"]))
    # value of kv head g == g + 1 everywhere -> every query head h sees h // 2 + 1
    cg = dict(c)
    vc = np.zeros_like(c["vc"]); vb = np.zeros_like(c["vblk"])
    for g in range(3):
        vc[:, g] = g + 1; vb[:, g] = g + 1
    cg["vc"], cg["vblk"] = vc, vb
    out, _ = _run(cg, q, offsets)
    for h in range(6):
        np.testing.assert_allclose(out[:, h], h // 2 + 1, atol=1e-12)
    # physically permuting the pool while remapping the table leaves the result unchanged
    out0, lse0 = _run(c, q, offsets)
    perm = rng.permutation(c["kc"].shape[0])
    inv = np.argsort(perm)
    cp = dict(c)
    cp["kc"], cp["vc"] = c["kc"][perm], c["vc"][perm]
    cp["table"] = np.where(c["table"] >= 0, inv[np.maximum(c["table"], 0)], -1).astype(np.int32)
    out1, lse1 = _run(cp, q, offsets)
    np.testing.assert_array_equal(out0, out1)
    np.testing.assert_array_equal(lse0, lse1)


def test_attn_respects_cap():
    c = _tiny_attn_case()
    offsets = np.array([0, 2, 3, 7], dtype=np.int32)
    q = np.random.default_rng(9).standard_normal((7, c["Hq"], c["d"]))
    full, _ = _run(c, q, offsets)
    part, _ = O.ragged_paged_attn(q, offsets, c["kc"], c["vc"], c["table"], c["plen"],
                                  c["kblk"], c["vblk"], 0.25, cap=5)
    assert part.shape[0] == 5
    np.testing.assert_array_equal(part, full[:5])


# ------------------------------------------------------------------ end to end on the tiny step
def test_tiny_step_invariants():
    st = make_step(BY_NAME["tiny_b2_blk16"])
    res = O.step(st)
    assert res["kept_count"].tolist() == [4, 4]
    assert res["offsets"].tolist() == [0, 4, 8]
    assert not np.any(res["keep"] & (1 - st.masked))
    assert res["out"].shape == (8, st.Hq, st.d)
    assert np.isfinite(res["out"]).all() and np.isfinite(res["lse"]).all()


def test_bf16_decoder_exact():
    x = np.array([1.0, -2.5, 45.25, 3.0e-3, 1.0 / 3.0], dtype=np.float32)
    bits = f32_to_bf16_bits(x)
    back = O.bf16_to_f64(bits)
    assert back[0] == 1.0 and back[1] == -2.5 and back[2] == 45.25
    # 1/3 rounds to the nearest bf16: 0x3EAB = 0.333984375
    assert bits[4] == 0x3EAB and back[4] == 0.333984375


# ------------------------------------------------------------------ KV write-back / block commit
def _logical_block(k_blk, v_blk, r, g):
    # the block's keys/values of request r, kv head g, read through request_kv's layout reader
    # (an empty prefix leaves just the block)
    B, Hkv = k_blk.shape[0], k_blk.shape[1]
    d = k_blk.shape[2] * 8
    kc = np.zeros((1, Hkv, d // 8, 16, 8))
    vc = np.zeros((1, Hkv, 2, d, 8))
    return O.request_kv(r, g, kc, vc, np.zeros((B, 1), np.int32), np.zeros(B, np.int32),
                        k_blk, v_blk)


def test_kv_pack_reads_back_through_the_layout_reader():
    # Pages packed from plain head-major rows and read through request_kv (the layout reader the
    # attention pins check against SDPA) give back the rows in order, prefix then block; the
    # token-major source is the same data transposed.
    rng = np.random.default_rng(41)
    B, Hkv, S, d, blk, npg = 2, 3, 16, 16, 16, 3
    kc_rows = rng.standard_normal((B * npg, Hkv, S, d))
    vc_rows = rng.standard_normal((B * npg, Hkv, S, d))
    kb_rows = rng.standard_normal((B, Hkv, blk, d))
    vb_rows = rng.standard_normal((B, Hkv, blk, d))
    kc, vc = O.kv_pack(kc_rows, vc_rows)
    kb, vb = O.kv_pack(kb_rows, vb_rows)
    table = np.arange(B * npg, dtype=np.int32).reshape(B, npg)[:, ::-1].copy()  # reversed order
    plen = np.array([npg * S, npg * S - 5], dtype=np.int32)
    for r in range(B):
        for g in range(Hkv):
            K, V = O.request_kv(r, g, kc, vc, table, plen, kb, vb)
            ek = np.concatenate([kc_rows[table[r], g].reshape(-1, d)[: plen[r]], kb_rows[r, g]])
            ev = np.concatenate([vc_rows[table[r], g].reshape(-1, d)[: plen[r]], vb_rows[r, g]])
            np.testing.assert_array_equal(K, ek)
            np.testing.assert_array_equal(V, ev)
    tk, tv = O.kv_pack(kc_rows.transpose(0, 2, 1, 3), vc_rows.transpose(0, 2, 1, 3),
                       token_major=True)
    np.testing.assert_array_equal(tk, kc)
    np.testing.assert_array_equal(tv, vc)
    only_v = O.kv_pack(None, vc_rows)
    assert only_v[0] is None
    np.testing.assert_array_equal(only_v[1], vc)


def test_kv_pack_matches_the_generator_packers():
    # The input generator packs its caches with its own reshapes (pack_k / pack_v, token rows
    # [pages*S, Hkv, d]); the oracle's per-token loops agree with them.
    rng = np.random.default_rng(43)
    n, S, Hkv, d = 3, 32, 2, 64
    tok_k = rng.standard_normal((n * S, Hkv, d))
    tok_v = rng.standard_normal((n * S, Hkv, d))
    k, v = O.kv_pack(tok_k.reshape(n, S, Hkv, d), tok_v.reshape(n, S, Hkv, d), token_major=True)
    np.testing.assert_array_equal(k, pack_k(tok_k, S))
    np.testing.assert_array_equal(v, pack_v(tok_v, S))


def test_kv_writeback_replaces_kept_positions_only():
    rng = np.random.default_rng(31)
    B, blk, Hkv, d = 3, 16, 2, 16
    k_blk = rng.standard_normal((B, Hkv, d // 8, blk, 8))
    v_blk = rng.standard_normal((B, Hkv, blk // 8, d, 8))
    keep = np.zeros((B, blk), dtype=np.uint8)
    keep[0, [1, 7, 15]] = 1
    keep[2, [0]] = 1
    offsets, kept_pos, _ = O.compact(keep)
    T = int(offsets[-1])
    k_rows = rng.standard_normal((T, Hkv, d))
    v_rows = rng.standard_normal((T, Hkv, d))
    kb, vb = O.kv_writeback(k_rows, v_rows, offsets, kept_pos, k_blk, v_blk)
    for r in range(B):
        for g in range(Hkv):
            K0, V0 = _logical_block(k_blk, v_blk, r, g)
            K1, V1 = _logical_block(kb, vb, r, g)
            for j in range(blk):
                n = [m for m in range(offsets[r], offsets[r + 1]) if kept_pos[m] == j]
                if n:
                    np.testing.assert_array_equal(K1[j], k_rows[n[0], g])
                    np.testing.assert_array_equal(V1[j], v_rows[n[0], g])
                else:
                    np.testing.assert_array_equal(K1[j], K0[j])
                    np.testing.assert_array_equal(V1[j], V0[j])
    # a capacity below T drops the rows at or past it
    kb2, _ = O.kv_writeback(k_rows, v_rows, offsets, kept_pos, k_blk, v_blk, cap=2)
    K2, _ = _logical_block(kb2, vb, 0, 0)
    np.testing.assert_array_equal(K2[15], _logical_block(k_blk, v_blk, 0, 0)[0][15])


def _pool(rng, B, Hkv, d, S, plen, spare):
    npg = [-(-int(P) // S) for P in plen]
    used = sum(npg)
    pool = used + spare
    kc = rng.standard_normal((pool, Hkv, d // 8, S, 8))
    vc = rng.standard_normal((pool, Hkv, S // 8, d, 8))
    table = np.full((B, 8), -1, dtype=np.int32)
    base = 0
    for r in range(B):
        table[r, : npg[r]] = np.arange(base, base + npg[r])
        base += npg[r]
    free = np.arange(used, pool, dtype=np.int32)
    return kc, vc, table, free


def test_block_commit_appends_block_to_prefix():
    # after the commit, the request's keys/values read through its page table are the old
    # prefix followed by the whole block (request_kv is the independent layout reader)
    rng = np.random.default_rng(32)
    B, blk, Hkv, d, S = 3, 16, 2, 16, 16
    plen = np.array([16, 5, 40], dtype=np.int32)
    kc, vc, table, free = _pool(rng, B, Hkv, d, S, plen, spare=6)
    k_blk = rng.standard_normal((B, Hkv, d // 8, blk, 8))
    v_blk = rng.standard_normal((B, Hkv, blk // 8, d, 8))
    commit = np.array([1, 1, 0], dtype=np.uint8)
    kc2, vc2, table2, plen2, fc, status = O.block_commit(commit, k_blk, v_blk, kc, vc, table,
                                                         plen, free, len(free))
    assert status == 0
    np.testing.assert_array_equal(plen2, [32, 21, 40])
    for r in range(B):
        for g in range(Hkv):
            Kold, Vold = O.request_kv(r, g, kc, vc, table, plen, k_blk, v_blk)
            Knew, Vnew = O.request_kv(r, g, kc2, vc2, table2, plen2, k_blk, v_blk)
            if commit[r]:
                # [old prefix, block] then the block again (request_kv appends k_blk)
                np.testing.assert_array_equal(Knew[: plen[r] + blk], Kold)
                np.testing.assert_array_equal(Vnew[: plen[r] + blk], Vold)
            else:
                np.testing.assert_array_equal(Knew, Kold)


def test_block_commit_page_allocation_order_and_failures():
    # S = blk = 16: request 0 (P=16) needs one page, request 1 (P=5 -> 21 tokens) one more,
    # request 2 is not committed: pages come off the top of the stack in request order
    rng = np.random.default_rng(33)
    B, blk, Hkv, d, S = 3, 16, 1, 8, 16
    plen = np.array([16, 5, 3], dtype=np.int32)
    kc, vc, table, _ = _pool(rng, B, Hkv, d, S, plen, spare=0)
    kc = np.concatenate([kc, np.zeros((14,) + kc.shape[1:])])
    vc = np.concatenate([vc, np.zeros((14,) + vc.shape[1:])])
    free = np.array([10, 11, 12, 13], dtype=np.int32)
    k_blk = rng.standard_normal((B, Hkv, d // 8, blk, 8))
    v_blk = rng.standard_normal((B, Hkv, blk // 8, d, 8))
    commit = np.array([1, 1, 0], dtype=np.uint8)
    _, _, t2, p2, fc, st = O.block_commit(commit, k_blk, v_blk, kc, vc, table, plen, free, 4)
    assert st == 0 and fc == 2
    assert t2[0, 1] == 13 and t2[1, 1] == 12 and t2[2, 1] == -1
    # two free pages are not enough for three committed requests needing one each
    _, _, t3, p3, fc3, st3 = O.block_commit(np.ones(3, np.uint8), k_blk, v_blk, kc, vc, table,
                                            plen, free, 2)
    assert st3 == 1 and fc3 == 2 and np.array_equal(t3, table) and np.array_equal(p3, plen)
    # a request that would outgrow its table row fails the whole commit
    plen_full = np.array([16, 5, 8 * S - 4], dtype=np.int32)
    _, _, t4, p4, fc4, st4 = O.block_commit(np.ones(3, np.uint8), k_blk, v_blk, kc, vc, table,
                                            plen_full, free, 4)
    assert st4 == 2 and fc4 == 4 and np.array_equal(p4, plen_full)
