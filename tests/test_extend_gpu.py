"""Extend (prefix-prefill) parity on the GPU: the HIP path through the C ABI
against the fp64 oracle on the same seeded inputs, |err| <= 1e-2 + 1e-2*|ref|
per element."""
import dataclasses
import sys

import numpy as np
import pytest
import torch

import oracle
import paged_gqa_attention_02_amd as pa
from paged_gqa_attention_02_amd import inputs as I
from tests._gpu import DEV, assert_close, run_decode, run_extend, to_f64

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def case_of(ctx, ql, Hq, Hkv, D, P, seed, **kw):
    return I.make_extend(f"x{seed}", ctx, ql, Hq, Hkv, D, P, seed, **kw)


def ctx_tokens(case):
    """Logical context rows [sum C, Hkv, D] of K and V, read back through the
    block table on the host."""
    P, bt = case.kv.page_size, case.kv.block_table
    ks, vs = [], []
    for b, C in enumerate(case.ctx_lens):
        t = np.arange(int(C))
        ks.append(case.kv.k_pool[bt[b, t // P], t % P])
        vs.append(case.kv.v_pool[bt[b, t // P], t % P])
    return np.concatenate(ks), np.concatenate(vs)


def check(case, what="", rows=None, num_splits=0):
    say(f"[extend] {what} B={case.batch} ctx={list(case.ctx_lens)[:8]} "
        f"q={list(case.q_lens)[:8]} Hq={case.num_q_heads} Hkv={case.num_kv_heads} "
        f"D={case.head_dim} P={case.kv.page_size} kv={case.kv_dtype} W={case.window} "
        f"cap={case.softcap} splits={num_splits}")
    out, _ = run_extend(case, num_splits=num_splits)
    got = to_f64(out)
    ref = oracle.extend(case, rows=rows)
    if rows is not None:
        got, ref = got[rows], ref[rows]
    assert_close(got, ref, what)
    return out


def test_extend_workload_all_rows():
    """The full extend workload (3,577 new rows x 32 heads): every output
    element against the oracle."""
    check(I.extend_config(5), "extend workload (all rows)")


def test_extend_workload_sampled_rows():
    """The full extend workload; 192 seeded rows (all heads) checked against
    the oracle, including each sequence's first and last row."""
    case = I.extend_config(5)
    rng = np.random.default_rng(55)
    cu = case.cu_seqlens_q
    edge = np.concatenate([cu[:-1], cu[1:] - 1])
    rows = np.unique(np.concatenate([edge, rng.choice(case.total_q, 176, replace=False)]))
    check(case, "extend workload (sampled rows)", rows=rows)


@pytest.mark.parametrize("ctx,ql,Hq,Hkv,D,P,kw", [
    ([0, 1, 37, 300], [1, 5, 130, 77], 8, 2, 128, 16, {}),            # C = 0, ragged
    ([100, 64, 1000], [33, 64, 200], 32, 8, 128, 16, {}),             # G 4
    ([129, 500], [300, 17], 16, 16, 64, 16, {}),                      # MHA, D 64
    ([70, 257], [40, 9], 32, 2, 128, 32, {}),                         # G 16
    ([333, 50], [100, 250], 8, 8, 128, 1, {}),                        # P 1
    ([1000, 20], [150, 70], 16, 2, 64, 64, dict(window=64)),          # window < q_len
    ([300, 700], [90, 300], 8, 1, 128, 16, dict(window=400, softcap=20.0)),
    ([500, 3], [64, 128], 16, 4, 128, 16, dict(kv_dtype="fp8_e4m3", scale_range=(0.5, 2.0))),
    ([5000, 3], [70, 200], 16, 4, 128, 4096, {}),                    # P 4096
    ([77, 640], [129, 31], 32, 8, 64, 8, dict(kv_dtype="fp8_e4m3", scale_range=(0.5, 2.0),
                                                window=100)),
    ([40, 0, 90], [0, 12, 3], 8, 2, 128, 16, {}),                     # a sequence with no rows
])
def test_extend_shapes(ctx, ql, Hq, Hkv, D, P, kw):
    case = case_of(ctx, ql, Hq, Hkv, D, P, 200 + len(ctx) + sum(ql) % 97, **kw)
    check(case, f"ctx={ctx} q={ql}")


@pytest.mark.parametrize("splits", [1, 3, 8, 61, 700, 20000])
def test_extend_persistent_block_counts(splits):
    """Any number of persistent blocks gives the same rows: one block walking
    every item, few blocks splitting items into parts merged by log-sum-exp,
    more blocks than key tiles (empty blocks)."""
    case = case_of([300, 0, 1500, 77], [200, 64, 33, 129], 32, 8, 128, 16, 600,
                   softcap=25.0)
    check(case, f"{splits} blocks", num_splits=splits)


@pytest.mark.parametrize("splits", [0, 50, 333])
def test_extend_many_short_items(splits):
    """40 sequences with short contexts and few new tokens: every item is
    charged a fixed cost in front of its key tiles, so many block ranges
    begin or end inside that part and some hold no tile."""
    rng = np.random.default_rng(71)
    ctx = [int(x) for x in rng.integers(0, 200, size=40)]
    ql = [int(x) for x in rng.integers(1, 40, size=40)]
    ctx[7], ql[7] = 2500, 300
    case = case_of(ctx, ql, 8, 2, 64, 16, 710)
    check(case, f"40 short, {splits} blocks", num_splits=splits)


@pytest.mark.parametrize("kw", [dict(window=300), dict(kv_dtype="fp8_e4m3",
                                                       scale_range=(0.5, 2.0))])
def test_extend_parts_with_window_and_fp8(kw):
    case = case_of([900, 40], [150, 300], 16, 4, 128, 16, 601, **kw)
    check(case, f"parts {kw}", num_splits=13)


def test_extend_parts_with_sinks():
    case = I.with_extras(case_of([1200, 5], [100, 60], 32, 8, 128, 16, 602), 602,
                         descales=True)
    check(case, "parts with sinks", num_splits=9)


def test_extend_single_row_is_decode():
    """One new token on a context of C tokens is decode over C + 1 tokens whose
    last key/value is the new one: both kernels against the same oracle
    result and each other."""
    ctx, Hq, Hkv, D, P = [200, 31, 1000], 16, 4, 128, 16
    ext = case_of(ctx, [1, 1, 1], Hq, Hkv, D, P, 301)
    kc, vc = ctx_tokens(ext)
    off = np.concatenate([[0], np.cumsum(ctx)])
    k_tok = np.concatenate([np.concatenate([kc[off[b]:off[b + 1]], ext.k_new[b:b + 1]])
                            for b in range(3)])
    v_tok = np.concatenate([np.concatenate([vc[off[b]:off[b + 1]], ext.v_new[b:b + 1]])
                            for b in range(3)])
    dec = I.decode_case_from_tokens("x-as-decode", ext.q, k_tok, v_tok,
                                    [c + 1 for c in ctx], P, 302)
    a = to_f64(run_extend(ext)[0])
    b = to_f64(run_decode(dec)[0])
    ref, _ = oracle.decode(dec)
    assert_close(a, ref, "extend q_len 1")
    assert_close(b, ref, "decode")
    assert_close(a, b, "extend vs decode")


def test_extend_page_permutation_bit_identical():
    """Another physical page permutation of the same context: the same bytes."""
    case = case_of([300, 129], [70, 40], 16, 4, 128, 16, 303)
    a, _ = run_extend(case)
    kc, vc = ctx_tokens(case)
    kv = I.page_tokens(kc, vc, case.ctx_lens, 16, np.random.default_rng(304))
    b, _ = run_extend(dataclasses.replace(case, kv=kv))
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_extend_empty_batch_rows():
    case = case_of([10, 20], [0, 0], 8, 2, 64, 16, 305)
    out, _ = run_extend(case)
    assert out.shape[0] == 0
