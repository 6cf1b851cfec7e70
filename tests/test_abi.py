"""CPU-only checks of the C ABI: the library loads, exports every function include/focus.h
declares, and rejects invalid arguments on the host (nothing is launched, no device touched)."""
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "focus.h")

F = pytest.importorskip("decodability_aware_token_amd.binding")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(focus_[a-z0-9_]+)\s*\(", src,
                       flags=re.M)
    return sorted(set(names))


def test_header_declares_the_four_calls():
    names = declared_functions()
    for n in ("focus_score_l01", "focus_select_budget", "focus_compact",
              "focus_ragged_paged_attn"):
        assert n in names


def test_library_exports_every_declared_symbol():
    L = F.lib()
    for name in declared_functions():
        assert hasattr(L, name), name
        assert name in F.SIGNATURES, name


def test_status_strings_and_version():
    assert F.status_string(0) == "ok"
    assert "workspace" in F.status_string(-3)
    assert F.lib().focus_version() >= 100


P = 0x10000  # a 16-byte aligned non-null address that is never dereferenced


def _score(**kw):
    a = dict(q0=P, k0=P, q1=P, k1=P, dt=1, B=4, blk=32, Hq=32, Hkv=8, d=128, sc=0.1, delta=P,
             ws=P, wsb=1 << 30)
    a.update(kw)
    return F.lib().focus_score_l01(a["q0"], a["k0"], a["q1"], a["k1"], a["dt"], a["B"], a["blk"],
                                   a["Hq"], a["Hkv"], a["d"], a["sc"], a["delta"], a["ws"],
                                   a["wsb"], None)


def test_score_errors():
    assert _score(q0=None) == F.FOCUS_ERR_INVALID_ARG
    assert _score(delta=None) == F.FOCUS_ERR_INVALID_ARG
    assert _score(B=0) == F.FOCUS_ERR_INVALID_ARG
    assert _score(sc=0.0) == F.FOCUS_ERR_INVALID_ARG
    assert _score(sc=float("nan")) == F.FOCUS_ERR_INVALID_ARG
    assert _score(Hq=30) == F.FOCUS_ERR_INVALID_ARG          # Hq % Hkv != 0
    assert _score(Hq=128, Hkv=8) == F.FOCUS_ERR_UNSUPPORTED  # G = 16
    assert _score(blk=24) == F.FOCUS_ERR_UNSUPPORTED
    assert _score(blk=128) == F.FOCUS_ERR_UNSUPPORTED
    assert _score(d=96) == F.FOCUS_ERR_UNSUPPORTED
    assert _score(dt=7) == F.FOCUS_ERR_UNSUPPORTED
    assert _score(B=5000) == F.FOCUS_ERR_UNSUPPORTED
    assert _score(q1=P + 8) == F.FOCUS_ERR_INVALID_ARG       # misaligned
    assert _score(ws=None) == F.FOCUS_ERR_WORKSPACE
    need = F.lib().focus_score_l01_workspace_size(4, 32, 32, 8, 128)
    assert need == 4 * 8 * 32 * 4   # per-kv-head partial sums
    assert _score(wsb=need - 1) == F.FOCUS_ERR_WORKSPACE


def _score_lse(**kw):
    a = dict(q0=P, k0=P, q1=P, k1=P, l0=P, l1=P, dt=1, B=4, blk=32, Hq=32, Hkv=8, d=128, sc=0.1,
             delta=P, ws=P, wsb=1 << 30)
    a.update(kw)
    return F.lib().focus_score_l01_lse(a["q0"], a["k0"], a["q1"], a["k1"], a["l0"], a["l1"],
                                       a["dt"], a["B"], a["blk"], a["Hq"], a["Hkv"], a["d"],
                                       a["sc"], a["delta"], a["ws"], a["wsb"], None)


def test_score_lse_errors():
    # the full-domain variant validates like focus_score_l01 and needs both row LSE arrays
    assert _score_lse(l0=None) == F.FOCUS_ERR_INVALID_ARG
    assert _score_lse(l1=None) == F.FOCUS_ERR_INVALID_ARG
    assert _score_lse(l0=P + 2) == F.FOCUS_ERR_INVALID_ARG   # misaligned
    assert _score_lse(q0=None) == F.FOCUS_ERR_INVALID_ARG
    assert _score_lse(blk=24) == F.FOCUS_ERR_UNSUPPORTED
    assert _score_lse(ws=None) == F.FOCUS_ERR_WORKSPACE


def _select(**kw):
    a = dict(delta=P, masked=P, budget=P, ad=0, beta=0.5, lo=2, hi=16, B=4, blk=32, keep=P,
             kept=P)
    a.update(kw)
    return F.lib().focus_select_budget(a["delta"], a["masked"], a["budget"], a["ad"], a["beta"],
                                       a["lo"], a["hi"], a["B"], a["blk"], a["keep"], a["kept"],
                                       None)


def test_select_errors():
    assert _select(delta=None) == F.FOCUS_ERR_INVALID_ARG
    assert _select(budget=None) == F.FOCUS_ERR_INVALID_ARG     # fixed rule needs budgets
    assert _select(kept=None) == F.FOCUS_ERR_INVALID_ARG
    assert _select(ad=1, lo=5, hi=2) == F.FOCUS_ERR_INVALID_ARG
    assert _select(ad=1, beta=float("inf")) == F.FOCUS_ERR_INVALID_ARG
    assert _select(B=-1) == F.FOCUS_ERR_INVALID_ARG
    assert _select(blk=48) == F.FOCUS_ERR_UNSUPPORTED
    assert _select(blk=8) == F.FOCUS_ERR_UNSUPPORTED


def _compact(**kw):
    a = dict(keep=P, B=4, blk=32, rows=P, rb=8192, cap=128, off=P, pos=P, gat=P)
    a.update(kw)
    return F.lib().focus_compact(a["keep"], a["B"], a["blk"], a["rows"], a["rb"], a["cap"],
                                 a["off"], a["pos"], a["gat"], None)


def test_compact_errors():
    assert _compact(keep=None) == F.FOCUS_ERR_INVALID_ARG
    assert _compact(off=None) == F.FOCUS_ERR_INVALID_ARG
    assert _compact(gat=None) == F.FOCUS_ERR_INVALID_ARG      # rows without a destination
    assert _compact(rows=None) == F.FOCUS_ERR_INVALID_ARG
    assert _compact(cap=-1) == F.FOCUS_ERR_INVALID_ARG
    assert _compact(rb=0) == F.FOCUS_ERR_INVALID_ARG
    assert _compact(rb=8200) == F.FOCUS_ERR_UNSUPPORTED       # not a multiple of 16
    assert _compact(keep=P + 2) == F.FOCUS_ERR_INVALID_ARG    # keep must be 4-byte aligned
    assert _compact(blk=20) == F.FOCUS_ERR_UNSUPPORTED
    assert _compact(B=4097) == F.FOCUS_ERR_UNSUPPORTED


def _ssc(**kw):
    import ctypes
    a = dict(q0=P, k0=P, q1=P, k1=P, dt=1, B=4, blk=32, Hq=32, Hkv=8, d=128, sc=0.1, msk=P,
             bud=P, delta=P, keep=P, kc=P, n=1, rows=[P], rb=[8192], gat=[P], cap=128, off=P,
             pos=P, mk=4, ws=P, wsb=1 << 30)
    a.update(kw)
    n = max(len(a["rows"]), 1)
    rows = (ctypes.c_void_p * n)(*a["rows"])
    rb = (ctypes.c_int64 * n)(*a["rb"])
    gat = (ctypes.c_void_p * n)(*a["gat"])
    return F.lib().focus_score_select_compact(
        a["q0"], a["k0"], a["q1"], a["k1"], a["dt"], a["B"], a["blk"], a["Hq"], a["Hkv"], a["d"],
        a["sc"], a["msk"], a["bud"], a["delta"], a["keep"], a["kc"], a["n"], rows, rb, gat,
        a["cap"], a["off"], a["pos"], a["mk"], a["ws"], a["wsb"], None)


def test_score_select_compact_errors():
    assert _ssc(bud=None) == F.FOCUS_ERR_INVALID_ARG          # per-request budgets only
    assert _ssc(msk=None) == F.FOCUS_ERR_INVALID_ARG
    assert _ssc(keep=None) == F.FOCUS_ERR_INVALID_ARG
    assert _ssc(q0=None) == F.FOCUS_ERR_INVALID_ARG
    assert _ssc(off=None) == F.FOCUS_ERR_INVALID_ARG
    assert _ssc(msk=P + 2) == F.FOCUS_ERR_INVALID_ARG         # masked must be 4-byte aligned
    assert _ssc(blk=20) == F.FOCUS_ERR_UNSUPPORTED
    assert _ssc(rb=[8200]) == F.FOCUS_ERR_UNSUPPORTED          # not a multiple of 16
    assert _ssc(n=3, rows=[P] * 3, rb=[16] * 3, gat=[P] * 3) == F.FOCUS_ERR_UNSUPPORTED
    assert _ssc(wsb=16) == F.FOCUS_ERR_WORKSPACE
    assert _ssc(cap=-1) == F.FOCUS_ERR_INVALID_ARG
    assert _ssc(mk=0) == F.FOCUS_ERR_INVALID_ARG
    assert _ssc(mk=33) == F.FOCUS_ERR_INVALID_ARG             # max_kept > blk


def _ssc_noalloc(**kw):
    import ctypes
    a = dict(q0=P, k0=P, q1=P, k1=P, dt=1, B=4, blk=32, Hq=32, Hkv=8, d=128, sc=0.1, msk=P,
             bud=P, delta=P, keep=P, kc=P, n=1, rows=[P], rb=[8192], gat=[P], cap=128, off=P,
             pos=P, mk=4)
    a.update(kw)
    n = max(len(a["rows"]), 1)
    rows = (ctypes.c_void_p * n)(*a["rows"])
    rb = (ctypes.c_int64 * n)(*a["rb"])
    gat = (ctypes.c_void_p * n)(*a["gat"])
    return F.lib().focus_score_select_compact_noalloc(
        a["q0"], a["k0"], a["q1"], a["k1"], a["dt"], a["B"], a["blk"], a["Hq"], a["Hkv"], a["d"],
        a["sc"], a["msk"], a["bud"], a["delta"], a["keep"], a["kc"], a["n"], rows, rb, gat,
        a["cap"], a["off"], a["pos"], a["mk"], None)


def test_score_select_compact_noalloc_errors():
    # every check happens before the device is touched (these calls return without a GPU)
    assert F.lib().focus_noalloc_scratch_bytes() == 4 << 20
    # the partials B*Hkv*blk*4 bytes must fit the 4 MiB array: 4096*8*32*4 fits exactly
    assert _ssc_noalloc(B=4096, Hkv=16, Hq=32, q0=None) == F.FOCUS_ERR_UNSUPPORTED
    assert _ssc_noalloc(B=4096, blk=64, Hq=32, Hkv=8) == F.FOCUS_ERR_UNSUPPORTED
    assert _ssc_noalloc(B=4096, q0=None) == F.FOCUS_ERR_INVALID_ARG
    assert _ssc_noalloc(bud=None) == F.FOCUS_ERR_INVALID_ARG
    assert _ssc_noalloc(msk=P + 2) == F.FOCUS_ERR_INVALID_ARG
    assert _ssc_noalloc(blk=20) == F.FOCUS_ERR_UNSUPPORTED
    assert _ssc_noalloc(mk=33) == F.FOCUS_ERR_INVALID_ARG
    assert _ssc_noalloc(B=0) == F.FOCUS_ERR_INVALID_ARG


def _attn(**kw):
    a = dict(q=P, off=P, cap=64, kc=P, vc=P, npages=100, pt=P, maxp=16, pl=P, kb=P, vb=P, B=4,
             blk=32, Hq=32, Hkv=8, d=128, S=64, mk=4, sc=0.088, out=P, lse=P, ws=P,
             wsb=1 << 40)
    a.update(kw)
    return F.lib().focus_ragged_paged_attn(a["q"], a["off"], a["cap"], a["kc"], a["vc"],
                                           a["npages"], a["pt"], a["maxp"], a["pl"], a["kb"],
                                           a["vb"], a["B"], a["blk"], a["Hq"], a["Hkv"], a["d"],
                                           a["S"], a["mk"], a["sc"], a["out"], a["lse"], a["ws"],
                                           a["wsb"], None)


def test_attn_errors():
    assert _attn(q=None) == F.FOCUS_ERR_INVALID_ARG
    assert _attn(kc=None) == F.FOCUS_ERR_INVALID_ARG
    assert _attn(pt=None) == F.FOCUS_ERR_INVALID_ARG
    assert _attn(npages=0) == F.FOCUS_ERR_INVALID_ARG
    assert _attn(mk=0) == F.FOCUS_ERR_INVALID_ARG
    assert _attn(mk=33) == F.FOCUS_ERR_INVALID_ARG            # max_kept > blk
    assert _attn(sc=-1.0) == F.FOCUS_ERR_INVALID_ARG
    assert _attn(Hq=12) == F.FOCUS_ERR_INVALID_ARG
    assert _attn(S=8) == F.FOCUS_ERR_UNSUPPORTED
    assert _attn(S=48) == F.FOCUS_ERR_UNSUPPORTED
    assert _attn(d=256) == F.FOCUS_ERR_UNSUPPORTED
    assert _attn(Hq=64, Hkv=4) == F.FOCUS_ERR_UNSUPPORTED     # G = 16
    assert _attn(out=P + 4) == F.FOCUS_ERR_INVALID_ARG
    assert _attn(maxp=1 << 20) == F.FOCUS_ERR_UNSUPPORTED
    assert _attn(npages=(1 << 31) - 1, Hkv=8, Hq=32) == F.FOCUS_ERR_UNSUPPORTED  # 32-bit blocks
    # long prefixes need a split workspace
    need = F.attn_workspace_bytes(4, 32, 32, 8, 128, 64, 128, 4)
    assert need > 0
    assert _attn(maxp=128, ws=None) == F.FOCUS_ERR_WORKSPACE
    assert _attn(maxp=128, wsb=need - 1) == F.FOCUS_ERR_WORKSPACE
    # log-sum-exp only: no output, no values, but then lse is required
    assert _attn(out=None, lse=None) == F.FOCUS_ERR_INVALID_ARG
    assert _attn(out=None, vc=None, vb=None, maxp=128, ws=None) == F.FOCUS_ERR_WORKSPACE
    assert _attn(vc=None) == F.FOCUS_ERR_INVALID_ARG            # values needed for the output
    # nothing kept: no query or output rows, nothing launched
    assert _attn(cap=0, q=None, out=None) == F.FOCUS_OK
    assert _attn(cap=0, q=None, out=None, S=48) == F.FOCUS_ERR_UNSUPPORTED


def test_attn_pos_errors():
    def ap(**kw):
        a = dict(q=P, pos=P, off=P, cap=64, kc=P, vc=P, npages=100, pt=P, maxp=16, pl=P, kb=P,
                 vb=P, B=4, blk=32, Hq=32, Hkv=8, d=128, S=64, mk=4, sc=0.088, out=P, lse=P,
                 ws=P, wsb=1 << 40)
        a.update(kw)
        return F.lib().focus_ragged_paged_attn_pos(
            a["q"], a["pos"], a["off"], a["cap"], a["kc"], a["vc"], a["npages"], a["pt"],
            a["maxp"], a["pl"], a["kb"], a["vb"], a["B"], a["blk"], a["Hq"], a["Hkv"], a["d"],
            a["S"], a["mk"], a["sc"], a["out"], a["lse"], a["ws"], a["wsb"], None)
    assert ap(pos=None) == F.FOCUS_ERR_INVALID_ARG              # the kept positions are needed
    assert ap(q=None) == F.FOCUS_ERR_INVALID_ARG
    assert ap(q=P + 8) == F.FOCUS_ERR_INVALID_ARG               # misaligned
    assert ap(S=48) == F.FOCUS_ERR_UNSUPPORTED                  # as call 4
    assert ap(ws=None, maxp=128) == F.FOCUS_ERR_WORKSPACE
    assert ap(out=None) == F.FOCUS_ERR_UNSUPPORTED              # log-sum-exp only: call 4
    assert ap(cap=0, q=None, pos=None, out=None) == F.FOCUS_OK  # nothing kept: nothing launched


def test_attn_plan_is_bounded():
    # the workspace grows with batch, heads and maximal prefix, never with the data
    small = F.attn_workspace_bytes(64, 32, 16, 4, 128, 16, 512, 4)
    big = F.attn_workspace_bytes(256, 32, 32, 8, 128, 64, 64, 4)
    assert 0 < small < (256 << 20) and 0 < big < (256 << 20)
    # the workspace holds per-item counters plus partials sized by the grid, not by the prefixes
    assert F.attn_workspace_bytes(256, 32, 32, 8, 128, 64, 8, 4) == \
        F.attn_workspace_bytes(256, 32, 32, 8, 128, 64, 64, 4)


def test_attn_plan_fills_the_chip_at_full_size():
    # Workspace = arrival counters (2 x 256 CUs x 4 waves ints) + partial O (2 slots per wave x
    # rows x d f32) + partial max/sum (2 slots x 2 x rows f32), so it fixes the persistent grid:
    # one 4-wave workgroup per CU with 16-row waves at the 256-request size, two per CU with
    # shared 64-row items (the grid shrinks only for problems with few key tiles).
    cnt = 2 * 256 * 4 * 4
    W = 256 * 4
    assert F.attn_workspace_bytes(256, 32, 32, 8, 128, 64, 64, 4) == \
        cnt + 2 * W * 16 * 128 * 4 + 2 * W * 2 * 16 * 4
    W = 2 * 256 * 4
    assert F.attn_workspace_bytes(128, 64, 32, 8, 128, 64, 32, 16) == \
        cnt + 2 * W * 16 * 128 * 4 + 2 * W * 2 * 16 * 4
    # a tiny problem runs on a smaller grid: whole column groups on every XCD
    assert F.attn_workspace_bytes(2, 16, 4, 4, 64, 16, 4, 4) < \
        F.attn_workspace_bytes(256, 32, 32, 8, 128, 64, 64, 4)


def test_kv_writeback_errors():
    def wb(**kw):
        a = dict(kr=P, vr=P, off=P, pos=P, cap=8, B=4, blk=32, Hkv=8, d=128, kb=P, vb=P)
        a.update(kw)
        return F.lib().focus_kv_writeback(a["kr"], a["vr"], a["off"], a["pos"], a["cap"], a["B"],
                                          a["blk"], a["Hkv"], a["d"], a["kb"], a["vb"], None)
    assert wb(kr=None) == F.FOCUS_ERR_INVALID_ARG
    assert wb(pos=None) == F.FOCUS_ERR_INVALID_ARG
    assert wb(cap=-1) == F.FOCUS_ERR_INVALID_ARG
    assert wb(blk=48) == F.FOCUS_ERR_UNSUPPORTED
    assert wb(d=32) == F.FOCUS_ERR_UNSUPPORTED
    assert wb(kb=P + 4) == F.FOCUS_ERR_INVALID_ARG
    assert wb(cap=0) == F.FOCUS_OK          # nothing to write, nothing launched


def test_block_commit_errors():
    def bc(**kw):
        a = dict(cm=P, kb=P, vb=P, B=4, blk=32, Hkv=8, d=128, S=64, kc=P, vc=P, np=100, pt=P,
                 mp=8, pi=P, po=P + 64, fp=P, fcap=10, fi=P + 128, fo=P + 192, st=P + 256)
        a.update(kw)
        return F.lib().focus_block_commit(a["cm"], a["kb"], a["vb"], a["B"], a["blk"], a["Hkv"],
                                          a["d"], a["S"], a["kc"], a["vc"], a["np"], a["pt"],
                                          a["mp"], a["pi"], a["po"], a["fp"], a["fcap"], a["fi"],
                                          a["fo"], a["st"], None)
    assert bc(cm=None) == F.FOCUS_ERR_INVALID_ARG
    assert bc(st=None) == F.FOCUS_ERR_INVALID_ARG
    assert bc(po=P) == F.FOCUS_ERR_INVALID_ARG       # prefix_len in and out alias
    assert bc(fo=P + 128) == F.FOCUS_ERR_INVALID_ARG # free_count in and out alias
    assert bc(fp=None) == F.FOCUS_ERR_INVALID_ARG    # pages listed but no array
    assert bc(S=48) == F.FOCUS_ERR_UNSUPPORTED
    assert bc(mp=1 << 20) == F.FOCUS_ERR_UNSUPPORTED # max_pages * S > 2^24
    assert bc(kc=P + 8) == F.FOCUS_ERR_INVALID_ARG


def test_kv_pack_errors():
    nb = 4 * 8 * 64 * 128 * 2  # bytes of one matrix at the default sizes
    def kp(**kw):
        a = dict(ks=P, vs=P + nb, lay=0, n=4, Hkv=8, S=64, d=128, ko=P + 2 * nb, vo=P + 3 * nb)
        a.update(kw)
        return F.lib().focus_kv_pack(a["ks"], a["vs"], a["lay"], a["n"], a["Hkv"], a["S"],
                                     a["d"], a["ko"], a["vo"], None)
    assert kp(ks=None) == F.FOCUS_ERR_INVALID_ARG            # a pair with one pointer
    assert kp(vo=None) == F.FOCUS_ERR_INVALID_ARG
    assert kp(ks=None, ko=None, vs=None, vo=None) == F.FOCUS_ERR_INVALID_ARG
    assert kp(n=0) == F.FOCUS_ERR_INVALID_ARG
    assert kp(lay=2) == F.FOCUS_ERR_UNSUPPORTED
    assert kp(S=48) == F.FOCUS_ERR_UNSUPPORTED
    assert kp(S=128) == F.FOCUS_ERR_UNSUPPORTED
    assert kp(d=96) == F.FOCUS_ERR_UNSUPPORTED
    assert kp(Hkv=65) == F.FOCUS_ERR_UNSUPPORTED
    assert kp(n=1 << 30) == F.FOCUS_ERR_UNSUPPORTED          # n_blocks * Hkv >= 2^31
    assert kp(ko=P + 2 * nb + 8) == F.FOCUS_ERR_INVALID_ARG  # misaligned
    assert kp(ko=P + nb // 2) == F.FOCUS_ERR_INVALID_ARG     # output overlaps an input
    assert kp(vo=P + 2 * nb + 16) == F.FOCUS_ERR_INVALID_ARG # the two outputs overlap
