"""The no-allocation front end (focus_score_select_compact_noalloc, scores in the library's own
device array) against the front end with a caller workspace (focus_score_select_compact): two
calls in a row, the second on a smaller batch, every output compared bit for bit, and no device
memory allocated by the no-allocation calls."""
import numpy as np
import pytest
import torch

from decodability_aware_token_amd import binding as F
from workloads import BY_NAME, make_step
from workloads.torch_io import upload

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _outputs(st, dev):
    B, blk = st.B, st.blk
    cap = B * blk
    t = upload(st, dev)
    sets = [t["hidden"], t["q_att"]]
    outs = {
        "delta": torch.full((B, blk), float("nan"), dtype=torch.float32, device=dev),
        "keep": torch.full((B, blk), 7, dtype=torch.uint8, device=dev),
        "kept_count": torch.full((B,), -1, dtype=torch.int32, device=dev),
        "offsets": torch.full((B + 1,), -1, dtype=torch.int32, device=dev),
        "kept_pos": torch.full((cap,), -1, dtype=torch.int32, device=dev),
        "gathered": [torch.zeros((cap,) + tuple(s.shape[2:]), dtype=s.dtype, device=dev)
                     for s in sets],
    }
    return t, sets, cap, outs


def _call(st, noalloc, dev=DEV):
    t, sets, cap, o = _outputs(st, dev)
    torch.cuda.synchronize()
    before = torch.cuda.memory_allocated(dev)
    F.score_select_compact(t["q0"], t["k0"], t["q1"], t["k1"], t["sm_scale"], t["masked"],
                           t["budget"], sets, cap, max_kept=t["max_kept"], delta=o["delta"],
                           keep=o["keep"], kept_count=o["kept_count"], offsets=o["offsets"],
                           kept_pos=o["kept_pos"], gathered=o["gathered"], noalloc=noalloc)
    torch.cuda.synchronize()
    if noalloc:
        assert torch.cuda.memory_allocated(dev) == before, "the no-allocation call allocated"
    T = int(o["offsets"][-1])
    res = {k: o[k].cpu().numpy() for k in ("delta", "keep", "kept_count", "offsets")}
    res["kept_pos"] = o["kept_pos"][:T].cpu().numpy()
    res["gathered"] = [g[:T].view(torch.int16).cpu().numpy() for g in o["gathered"]]
    return res


def test_noalloc_front_end_equals_workspace_front_end():
    rec = BY_NAME["sdar_b256_blk32"]
    steps = [make_step(rec.scaled(B=48)), make_step(rec.scaled(B=20), seed=rec.seed + 7)]
    for i, st in enumerate(steps):
        print(f"\n[case] no-alloc front end call {i}: B={st.B}", flush=True)
        ref = _call(st, noalloc=False)
        got = _call(st, noalloc=True)
        for k in ("delta", "keep", "kept_count", "offsets", "kept_pos"):
            assert np.array_equal(got[k], ref[k]), (i, k)
        for a, b in zip(got["gathered"], ref["gathered"]):
            assert np.array_equal(a, b), i
        assert int(ref["offsets"][-1]) > 0
