"""The Python binding checks every tensor against the plan before it calls the
library: the kernels take all sizes from the plan, so a tensor smaller than
the plan describes (or of another element type) would be read or written past
its end on the GPU.  These run on the CPU; each case fails in the binding,
before any call into the library that could launch."""
import pytest
import torch

import paged_gqa_attention_02_amd as pa

B, HQ, HKV, D, P, PAGES, WIDTH = 4, 32, 8, 128, 16, 40, 8


def decode_args(**over):
    a = dict(q=torch.zeros(B, HQ, D, dtype=torch.bfloat16),
             k_pool=torch.zeros(PAGES, P, HKV, D, dtype=torch.bfloat16),
             v_pool=torch.zeros(PAGES, P, HKV, D, dtype=torch.bfloat16),
             block_table=torch.zeros(B, WIDTH, dtype=torch.int32),
             seq_lens=torch.full((B,), 100, dtype=torch.int32))
    a.update(over)
    return a


def decode_plan():
    a = decode_args()
    return pa.decode_plan(a["q"], a["k_pool"], a["block_table"], 100)


def call_decode(**over):
    a = decode_args(**over)
    extra = {k: a.pop(k) for k in ("sinks", "alibi_slopes", "out") if k in a}
    pa.decode(decode_plan(), a["q"], a["k_pool"], a["v_pool"], a["block_table"],
              a["seq_lens"], 0.1, **extra)


FP8 = torch.zeros(PAGES, P, HKV, D, dtype=torch.float8_e4m3fn)


@pytest.mark.parametrize("over,exc", [
    (dict(q=torch.zeros(B - 1, HQ, D, dtype=torch.bfloat16)), ValueError),   # fewer sequences
    (dict(q=torch.zeros(B, HQ // 2, D, dtype=torch.bfloat16)), ValueError),  # fewer heads
    (dict(q=torch.zeros(B, HQ, 64, dtype=torch.bfloat16)), ValueError),      # head dim
    (dict(k_pool=FP8, v_pool=FP8), TypeError),                              # fp8 pool, bf16 plan
    (dict(k_pool=torch.zeros(PAGES, P, 4, D, dtype=torch.bfloat16),
          v_pool=torch.zeros(PAGES, P, 4, D, dtype=torch.bfloat16)), ValueError),
    (dict(k_pool=torch.zeros(PAGES, 32, HKV, D, dtype=torch.bfloat16),
          v_pool=torch.zeros(PAGES, 32, HKV, D, dtype=torch.bfloat16)), ValueError),
    (dict(block_table=torch.zeros(B - 1, WIDTH, dtype=torch.int32)), ValueError),
    (dict(block_table=torch.zeros(B, WIDTH - 2, dtype=torch.int32)), ValueError),
    (dict(seq_lens=torch.zeros(B - 1, dtype=torch.int32)), ValueError),
    (dict(seq_lens=torch.zeros(B, dtype=torch.int64)), TypeError),
    (dict(sinks=torch.zeros(HQ - 1)), ValueError),
    (dict(alibi_slopes=torch.zeros(HQ // 2)), ValueError),
    (dict(out=torch.zeros(B, HQ, D, dtype=torch.bfloat16, device="meta")), ValueError),
    (dict(seq_lens=torch.zeros(B, dtype=torch.int32, device="meta")), ValueError),
])
def test_decode_tensor_checks(over, exc):
    with pytest.raises(exc):
        call_decode(**over)


def test_verify_q_len_must_match_plan():
    a = decode_args(q=torch.zeros(B, 3, HQ, D, dtype=torch.bfloat16))
    pl = pa.verify_plan(a["q"], a["k_pool"], a["block_table"], 100)
    q2 = torch.zeros(B, 2, HQ, D, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        pa.verify(pl, q2, a["k_pool"], a["v_pool"], a["block_table"], a["seq_lens"], 0.1)


T = 50


def extend_args(**over):
    a = dict(q=torch.zeros(T, HQ, D, dtype=torch.bfloat16),
             k_new=torch.zeros(T, HKV, D, dtype=torch.bfloat16),
             v_new=torch.zeros(T, HKV, D, dtype=torch.bfloat16),
             cu_seqlens_q=torch.tensor([0, 10, 20, 30, T], dtype=torch.int32),
             ctx_lens=torch.full((B,), 100, dtype=torch.int32),
             k_pool=torch.zeros(PAGES, P, HKV, D, dtype=torch.bfloat16),
             v_pool=torch.zeros(PAGES, P, HKV, D, dtype=torch.bfloat16),
             block_table=torch.zeros(B, WIDTH, dtype=torch.int32))
    a.update(over)
    return a


def call_extend(**over):
    base = extend_args()
    pl = pa.extend_plan(base["q"], base["k_pool"], base["block_table"], B, 100, 20)
    a = extend_args(**over)
    extra = {k: a.pop(k) for k in ("sinks",) if k in a}
    pa.extend(pl, a["q"], a["k_new"], a["v_new"], a["cu_seqlens_q"], a["ctx_lens"],
              a["k_pool"], a["v_pool"], a["block_table"], 0.1, **extra)


@pytest.mark.parametrize("over,exc", [
    (dict(q=torch.zeros(T - 1, HQ, D, dtype=torch.bfloat16)), ValueError),
    (dict(k_new=torch.zeros(T, HKV // 2, D, dtype=torch.bfloat16)), ValueError),
    (dict(v_new=torch.zeros(T - 5, HKV, D, dtype=torch.bfloat16)), ValueError),
    (dict(cu_seqlens_q=torch.tensor([0, 10, 20, 30], dtype=torch.int32)), ValueError),
    (dict(ctx_lens=torch.full((B - 1,), 100, dtype=torch.int32)), ValueError),
    (dict(k_pool=FP8, v_pool=FP8), TypeError),
    (dict(block_table=torch.zeros(B - 2, WIDTH, dtype=torch.int32)), ValueError),
    (dict(sinks=torch.zeros(3)), ValueError),
    (dict(k_new=torch.zeros(T, HKV, D, dtype=torch.bfloat16, device="meta")), ValueError),
])
def test_extend_tensor_checks(over, exc):
    with pytest.raises(exc):
        call_extend(**over)


def test_gather_tensor_checks():
    a = decode_args()
    pl = decode_plan()
    with pytest.raises(ValueError):
        pa.gather(pl, a["k_pool"], a["v_pool"], a["block_table"][:2], a["seq_lens"], 400)
    with pytest.raises(TypeError):
        pa.gather(pl, FP8, FP8, a["block_table"], a["seq_lens"], 400)
