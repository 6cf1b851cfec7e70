"""Helpers for the GPU parity tests: run the HIP path on a generated step and compare it with
the fp64 oracle under the published tolerances.

Tolerances (fixed by the task's target, restated):
  * importance delta: max abs error <= 1e-4 on every block position;
  * kept positions and offsets: bit-exact, except that a request may differ when every position
    in the symmetric difference of the two kept sets lies within 1e-5 of the selection boundary
    (the oracle's k-th largest masked delta, or mu + beta*sigma for the adaptive rule);
  * attention output: max abs error <= 2e-2 against fp64 on the same bf16 inputs; LSE <= 1e-3.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle as O
from decodability_aware_token_amd import FocusStep, StepInputs
from workloads.torch_io import bf16_tensor, upload

DELTA_TOL = 1e-4
TIE_TOL = 1e-5
OUT_TOL = 2e-2
LSE_TOL = 1e-3

_FIELDS = ("q0", "k0", "q1", "k1", "masked", "budget", "adaptive", "max_kept", "q_att",
           "k_cache", "v_cache", "page_table", "prefix_len", "k_blk", "v_blk", "sm_scale",
           "hidden")


def step_inputs(st, device="cuda") -> StepInputs:
    t = upload(st, device)
    return StepInputs(**{k: t[k] for k in _FIELDS})


def run_gpu_step(st, cap=None, device="cuda", gather_q=False):
    fs = FocusStep(step_inputs(st, device), cap=cap, gather_q=gather_q)
    fs.run()
    torch.cuda.synchronize()
    return fs, fetch(fs)


def bf16_to_np(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def fetch(fs: FocusStep) -> dict:
    off = fs.offsets.cpu().numpy()
    T = min(int(off[-1]), fs.cap)
    res = {
        "delta": fs.delta.cpu().numpy().astype(np.float64),
        "keep": fs.keep.cpu().numpy(),
        "kept_count": fs.kept_count.cpu().numpy(),
        "offsets": off,
        "kept_pos": fs.kept_pos[:T].cpu().numpy(),
        "out": fs.out[:T].float().cpu().numpy().astype(np.float64),
        "out_bits": bf16_to_np(fs.out[:T]),
        "lse": None if fs.lse is None else fs.lse[:T].cpu().numpy().astype(np.float64),
    }
    if fs.q_rows is not None:
        res["q_rows"] = bf16_to_np(fs.q_rows[:T])
    if fs.hidden_rows is not None:
        res["hidden_rows"] = bf16_to_np(fs.hidden_rows[:T])
    return res


def boundary(ref_delta_r, masked_r, k_ref, rule):
    if rule[0] == "adaptive":
        return O.adaptive_threshold(ref_delta_r, masked_r, rule[1])
    return O.kth_boundary(ref_delta_r, masked_r, k_ref)


def check_keep(gpu_keep, ref_keep, ref_delta, masked, rule, gpu_kept=None, ref_kept=None):
    """Bit-exact kept sets except near-boundary excusals; returns the excused request ids."""
    excused = []
    for r in range(gpu_keep.shape[0]):
        if np.array_equal(gpu_keep[r], ref_keep[r]):
            continue
        diff = np.nonzero(gpu_keep[r] != ref_keep[r])[0]
        t = boundary(ref_delta[r], masked[r], int(ref_keep[r].sum()), rule)
        gaps = np.abs(ref_delta[r, diff] - t)
        assert np.all(gaps <= TIE_TOL), (
            f"request {r}: kept sets differ at {diff.tolist()} with gaps {gaps.tolist()}")
        excused.append(r)
    if gpu_kept is not None:
        assert np.array_equal(gpu_kept, gpu_keep.sum(axis=1))
    assert not np.any(gpu_keep & (1 - masked)), "a decoded token was kept"
    return excused


def check_ragged(gpu, ref, B, excused, rule, gathered=None):
    """Offsets, kept positions and (optionally) gathered rows of the GPU against the oracle's,
    request by request.

    gpu: dict with offsets, kept_pos (rows below min(T, cap)), keep; ref: dict with offsets,
    kept_pos, keep (the oracle's).  excused: requests whose kept sets may differ (near-ties).
      * the GPU's offsets are the running total of its own kept counts;
      * offsets are bit-exact up to the first excused request (all of them for budgets that do
        not depend on the scores: the counts then never differ);
      * every request that is not excused has exactly the oracle's kept positions; an excused
        one lists its own kept positions in ascending order;
      * gathered = [(gpu_rows, oracle_rows, source), ...]: rows of requests that are not
        excused equal the oracle's gathered rows; rows of excused requests equal
        source[r, position].
    """
    goff, roff = gpu["offsets"].astype(np.int64), ref["offsets"].astype(np.int64)
    gkept = gpu["keep"].astype(np.int64).sum(axis=1)
    assert np.array_equal(goff, np.concatenate([[0], np.cumsum(gkept)])), "offsets != running total"
    first = min(excused) if excused else B
    assert np.array_equal(goff[: first + 1], roff[: first + 1]), "offsets differ before a near-tie"
    if rule[0] == "fixed":
        assert np.array_equal(goff, roff), "offsets differ"
    lim_g, lim_r = len(gpu["kept_pos"]), len(ref["kept_pos"])
    ex = set(int(r) for r in excused)
    for r in range(B):
        # rows at or past the GPU's capacity are not written: compare what it holds
        gs = gpu["kept_pos"][min(goff[r], lim_g): min(goff[r + 1], lim_g)]
        n = len(gs)
        if r in ex:
            want = np.nonzero(gpu["keep"][r])[0][:n]
        else:
            assert goff[r + 1] - goff[r] == roff[r + 1] - roff[r], f"request {r}: kept count"
            want = ref["kept_pos"][min(roff[r], lim_r): min(roff[r + 1], lim_r)][:n]
        assert np.array_equal(gs, want), f"request {r}: kept positions {gs} != {want}"
        for si, (grows, rrows, src) in enumerate(gathered or ()):
            gr = grows[min(goff[r], lim_g): min(goff[r + 1], lim_g)]
            if r in ex:
                wr = src[r, gs]
            else:
                wr = rrows[min(roff[r], lim_r): min(roff[r + 1], lim_r)][:n]
            assert np.array_equal(gr, wr), f"request {r}: gathered rows of set {si} differ"


def gathered_sets(gpu, st, ref_keep):
    """(gpu rows, oracle rows, source) of the gathered row sets (the hidden states, and the
    attention queries when the step gathers them): the oracle's compaction of the same sources
    under its own kept sets."""
    sets = []
    if "q_rows" in gpu:
        sets.append((gpu["q_rows"], O.compact(ref_keep, st.q_att)[2], st.q_att))
    if "hidden_rows" in gpu:
        sets.append((gpu["hidden_rows"], O.compact(ref_keep, st.hidden)[2], st.hidden))
    return sets


def rows_by_token(offsets, kept_pos, B, lim):
    """{(request, position): row index} for rows below lim."""
    m = {}
    for r in range(B):
        for n in range(int(offsets[r]), min(int(offsets[r + 1]), lim)):
            m[(r, int(kept_pos[n]))] = n
    return m


def compare_attention(gpu, ref, B, excused=()):
    """Compare O / LSE on the (request, position) rows kept by both sides."""
    gmap = rows_by_token(gpu["offsets"], gpu["kept_pos"], B, len(gpu["kept_pos"]))
    rmap = rows_by_token(ref["offsets"], ref["kept_pos"], B, len(ref["kept_pos"]))
    common = sorted(set(gmap) & set(rmap))
    gi = np.array([gmap[k] for k in common], dtype=np.int64)
    ri = np.array([rmap[k] for k in common], dtype=np.int64)
    if len(common) == 0:
        return 0.0, 0.0
    oerr = np.abs(gpu["out"][gi] - ref["out"][ri]).max()
    assert oerr <= OUT_TOL, f"attention max abs error {oerr}"
    lerr = 0.0
    if gpu.get("lse") is not None:
        lerr = np.abs(gpu["lse"][gi] - ref["lse"][ri]).max()
        assert lerr <= LSE_TOL, f"lse max abs error {lerr}"
    return oerr, lerr


def attn_case_inputs(st, keep, device="cuda"):
    """Oracle-compacted queries of a step under a given keep mask, plus device copies."""
    q64 = O.bf16_to_f64(st.q_att)
    offsets, kept_pos, _ = O.compact(keep)
    owner = np.repeat(np.arange(st.B), np.diff(offsets))
    qbits = st.q_att[owner, kept_pos] if len(kept_pos) else \
        np.zeros((0, st.Hq, st.d), dtype=np.uint16)
    return {
        "offsets": offsets, "kept_pos": kept_pos, "q_rows64": q64[owner, kept_pos],
        "q_bits": qbits,
        "d_offsets": torch.from_numpy(offsets).to(device),
        "d_q": bf16_tensor(qbits.reshape(-1, st.Hq, st.d), device),
    }


def oracle_attention(st, q_rows64, offsets, requests=None, cap=None):
    """Oracle attention, optionally restricted to a subset of requests (sampling at full size)."""
    kc, vc = O.bf16_to_f64(st.k_cache), O.bf16_to_f64(st.v_cache)
    kb, vb = O.bf16_to_f64(st.k_blk), O.bf16_to_f64(st.v_blk)
    if requests is None:
        return O.ragged_paged_attn(q_rows64, offsets, kc, vc, st.page_table, st.prefix_len, kb,
                                   vb, st.sm_scale, cap=cap)
    requests = np.asarray(sorted(requests))
    rows = np.concatenate([np.arange(offsets[r], offsets[r + 1]) for r in requests]).astype(int)
    sub_off = np.concatenate([[0], np.cumsum(np.diff(offsets)[requests])]).astype(np.int32)
    out, lse = O.ragged_paged_attn(q_rows64[rows], sub_off, kc, vc, st.page_table[requests],
                                   st.prefix_len[requests], kb[requests], vb[requests],
                                   st.sm_scale)
    return rows, out, lse
