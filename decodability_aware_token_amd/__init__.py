"""MI355X-native hot path of FOCUS's focused block-diffusion step.

The computation lives in libfocus.so (hand-written HIP kernels for gfx950 behind the C ABI in
include/focus.h); this package only binds it (``binding``) and strings the four calls into a
step (``pipeline``).
"""
from .binding import (  # noqa: F401
    FocusError, compact, lib, ragged_paged_attn, score_l01, select_budget, status_string,
)
from .pipeline import FocusStep, FullBlockStep, FullDomainScore, StepInputs  # noqa: F401

__version__ = "0.1.0"
