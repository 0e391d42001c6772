"""Latent-cache (MLA) decode parity on the GPU: paged_attn_decode with
head_dim_v < head_dim through the C ABI against the fp64 oracle on the same
seeded inputs, |err| <= 1e-2 + 1e-2*|ref| per element.  The value of a token
is the first head_dim_v entries of its row: one pool for both (alias) or a
separate pool of the same layout whose entries past head_dim_v are NaN."""
import sys

import numpy as np
import pytest
import torch

import oracle
from paged_gqa_attention_02_amd import inputs as I
from tests._gpu import DEV, assert_close, run_decode, to_f64

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def mla_case(lens, Hq, Hkv, D, Dv, P, seed, alias=True, **kw):
    rng = np.random.default_rng(seed)
    return I.make_mla_decode(f"m{seed}", lens, Hq, Hkv, D, Dv, P, seed, alias=alias,
                             lens_rng=rng, **kw)


def check(case, num_splits=None, what=""):
    say(f"[mla] {what} B={case.batch} Hq={case.num_q_heads} Hkv={case.num_kv_heads} "
        f"D={case.head_dim} Dv={case.dv} P={case.page_size} alias={case.latent_alias} "
        f"W={case.window} cap={case.softcap} splits={num_splits}")
    out, pl = run_decode(case, num_splits)
    ref, _ = oracle.decode(case)
    assert_close(to_f64(out), ref, f"{what} ({pl.describe()})")
    return out, pl


@pytest.mark.parametrize("lens,Hq,Hkv,D,Dv,P,alias,kw", [
    ([37, 100, 64], 16, 1, 576, 512, 16, True, {}),
    ([1, 2, 31, 32, 33, 500, 1025], 16, 1, 576, 512, 64, True, {}),      # ragged tails
    ([300, 45, 700], 16, 1, 576, 512, 1, True, dict(softcap=20.0)),      # P 1
    ([2000, 33, 700, 5], 32, 2, 576, 512, 16, False, dict(window=100)),  # two waves, own V
    ([129, 511], 128, 1, 576, 512, 64, True, {}),                        # G 128: 8 waves
    ([129, 511, 60], 48, 1, 576, 512, 32, True, {}),                     # G 48: an idle wave
    ([100, 1000], 8, 1, 576, 512, 16, True, dict(window=37)),            # G 8: padded rows
    ([77, 400, 3000], 16, 1, 288, 256, 16, True, {}),
    ([77, 400], 64, 2, 288, 256, 8, False, dict(softcap=10.0, window=50)),
    ([0, 50, 0, 3], 16, 1, 576, 512, 16, True, {}),                      # empty sequences
    ([300, 64, 1000], 100, 1, 576, 512, 16, True, dict(softcap=12.0)),   # two halves of 50 heads
    ([200, 31], 65, 1, 576, 512, 32, True, {}),                          # 65 heads: 8-wave blocks
    ([0, 90, 2100], 128, 1, 288, 256, 64, True, dict(window=500)),       # halves, 288/256
    ([700, 2000, 3], 16, 1, 576, 512, 256, True, {}),                    # P 256
])
def test_mla_decode_matches_oracle(lens, Hq, Hkv, D, Dv, P, alias, kw):
    case = mla_case(lens, Hq, Hkv, D, Dv, P, 100 + Hq + P, alias=alias, **kw)
    out, _ = check(case, what="shape")
    for b, L in enumerate(lens):
        if L == 0:
            assert not out[b].any()


@pytest.mark.parametrize("splits", [1, 3, 7, 64, 1000])
def test_mla_forced_splits(splits):
    """Any cut of the key ranges into pieces (one block each) merges to the
    same result; 1000 blocks leave some with no tile."""
    case = mla_case([700, 33, 1500, 64], 16, 1, 576, 512, 16, 7, softcap=15.0)
    check(case, num_splits=splits, what=f"splits={splits}")


@pytest.mark.parametrize("splits", [0, 37, 500])
def test_mla_many_short_sequences(splits):
    """80 sequences of 1..40 tokens and two long ones: the ranges charge
    every segment a fixed cost in front of its first tile, so many ranges
    begin or end inside that part and some hold no tile."""
    rng = np.random.default_rng(13)
    lens = rng.integers(1, 41, size=82)
    lens[[10, 60]] = [1500, 900]
    lens[[3, 70]] = 0
    case = mla_case(lens, 16, 1, 576, 512, 16, 14)
    out, _ = check(case, num_splits=splits or None, what=f"short splits={splits}")
    for b in np.flatnonzero(lens == 0):
        assert not out[b].any()


def test_mla_extras():
    """Sinks, per-request descales and ALiBi slopes on a latent cache."""
    case = I.with_extras(mla_case([300, 1200, 45], 16, 1, 576, 512, 16, 11), 12,
                         sinks=True, descales=True, alibi=True)
    check(case, what="sinks+descales+alibi")
    check(case, num_splits=5, what="sinks+descales+alibi split")


def test_mla_extras_head_halves():
    """128 heads over one kv head run as two virtual kv heads of 64: sinks,
    ALiBi slopes and descales must still reach their own query heads."""
    case = I.with_extras(mla_case([700, 1500, 3], 128, 1, 576, 512, 16, 15), 16,
                         sinks=True, descales=True, alibi=True)
    check(case, what="128 heads, sinks+descales+alibi")
    check(case, num_splits=9, what="128 heads, sinks+descales+alibi split")


def test_mla_alias_and_copy_agree():
    """v_pool == k_pool reads the values from the staged key rows; a copy of
    the pool takes the separate-value path: the results are bit-identical."""
    case = mla_case([900, 61, 2000], 16, 1, 576, 512, 16, 13)
    t = I.decode_tensors(case, DEV)
    a, _ = run_decode(case, tensors=t)
    t2 = dict(t, v_pool=t["k_pool"].clone())
    b, _ = run_decode(case, tensors=t2)
    assert torch.equal(a, b)


def test_mla_deterministic():
    case = mla_case([3000, 17, 800], 32, 1, 576, 512, 64, 14)
    t = I.decode_tensors(case, DEV)
    a, _ = run_decode(case, tensors=t)
    b, _ = run_decode(case, tensors=t)
    assert torch.equal(a, b)


@pytest.mark.parametrize("heads,batch", [(16, 128), (128, 16)])
def test_mla_workload(heads, batch):
    """The DeepSeek-V3-shaped latent workload (16 query heads, B 128: the
    bench's configuration; 128 heads on a smaller batch), every output row."""
    case = I.mla_config(heads, batch)
    check(case, what=case.name)
