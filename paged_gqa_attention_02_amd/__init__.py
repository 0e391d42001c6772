"""Paged GQA attention (split-KV decode, speculative verify and prefix-prefill
extend) for MI355X.

The computation runs in hand-written HIP kernels for gfx950 behind the C ABI
of ``include/paged_attn.h`` (``libpaged_attn.so``); this package is its thin
Python binding plus the seeded synthetic inputs used by tests and the bench.
"""
from .binding import (PA_MODE_DECODE, PA_MODE_EXTEND, PA_MODE_VERIFY,  # noqa: F401
                      NOALLOC_SCRATCH_BYTES, PagedAttnError, Plan, cache_append, check_inputs,
                      decode, decode_merge, decode_noalloc, decode_plan, decode_split, extend,
                      extend_plan, gather, lib, plan, set_input_checks, status_str, verify,
                      verify_plan, workspace_for)

__all__ = ["PA_MODE_DECODE", "PA_MODE_EXTEND", "PA_MODE_VERIFY", "NOALLOC_SCRATCH_BYTES",
           "PagedAttnError", "Plan", "cache_append", "check_inputs", "decode", "decode_merge",
           "decode_noalloc", "decode_plan", "decode_split", "extend", "extend_plan", "gather",
           "lib", "plan", "set_input_checks", "status_str", "verify", "verify_plan",
           "workspace_for"]
