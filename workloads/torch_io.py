"""Moves a generated ``Step`` onto a torch device (bf16 bit patterns become bfloat16 tensors)."""
from __future__ import annotations

import numpy as np
import torch


def bf16_tensor(bits: np.ndarray, device) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.bfloat16).to(device)


def score_tensor(x: np.ndarray, dtype: str, device) -> torch.Tensor:
    if dtype == "bf16":
        return bf16_tensor(x, device)
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(device)


def upload(st, device="cuda"):
    """Device tensors of ``st`` as a dict keyed like the step's fields."""
    d = {
        "q0": score_tensor(st.q0, st.score_dtype, device),
        "k0": score_tensor(st.k0, st.score_dtype, device),
        "q1": score_tensor(st.q1, st.score_dtype, device),
        "k1": score_tensor(st.k1, st.score_dtype, device),
        "masked": torch.from_numpy(st.masked).to(device),
        "budget": None if st.budget is None else torch.from_numpy(st.budget).to(device),
        "adaptive": None if st.rule[0] != "adaptive" else tuple(st.rule[1:]),
        "max_kept": int(st.max_kept),
        "q_att": bf16_tensor(st.q_att, device),
        "k_cache": bf16_tensor(st.k_cache, device),
        "v_cache": bf16_tensor(st.v_cache, device),
        "page_table": torch.from_numpy(st.page_table).to(device),
        "prefix_len": torch.from_numpy(st.prefix_len).to(device),
        "k_blk": bf16_tensor(st.k_blk, device),
        "v_blk": bf16_tensor(st.v_blk, device),
        "sm_scale": float(st.sm_scale),
        "hidden": None if st.hidden is None else bf16_tensor(st.hidden, device),
        "k_cache0": None if st.k_cache0 is None else bf16_tensor(st.k_cache0, device),
        "k_blk0": None if st.k_blk0 is None else bf16_tensor(st.k_blk0, device),
    }
    return d
