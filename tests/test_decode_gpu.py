"""Decode parity on the GPU: the HIP path through the C ABI against the fp64
oracle on the same seeded inputs, |err| <= 1e-2 + 1e-2*|ref| per element;
gather and one-key results bit-exact."""
import sys

import numpy as np
import pytest
import torch

import oracle
import paged_gqa_attention_02_amd as pa
from paged_gqa_attention_02_amd import inputs as I
from tests._gpu import DEV, assert_close, run_decode, to_f64

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def rand_case(lens, Hq, Hkv, D, P, seed, **kw):
    rng = np.random.default_rng(seed)
    return I.make_decode(f"r{seed}", lens, Hq, Hkv, D, P, seed, lens_rng=rng, **kw)


def check(case, num_splits=None, what=""):
    say(f"[decode] {what or case.name} B={case.batch} Hq={case.num_q_heads} "
        f"Hkv={case.num_kv_heads} D={case.head_dim} P={case.page_size} kv={case.kv_dtype} "
        f"W={case.window} cap={case.softcap} splits={num_splits}")
    out, pl = run_decode(case, num_splits)
    ref, _ = oracle.decode(case)
    assert_close(to_f64(out), ref, f"{what} ({pl.describe()})")
    return out, pl


# ------------------------------------------------------------ the workloads
def test_tiny_workload():
    case = I.decode_config(1)
    out, pl = check(case, what="tiny")
    assert pl.num_splits == 2


@pytest.mark.parametrize("n,P", [(2, None), (3, 64), (3, 1), (4, None)])
def test_workload_full_size(n, P):
    case = I.decode_config(n, page_size=P)
    check(case, what=f"workload {n} P={case.page_size}")


def test_mha_workload_full_size():
    """G = 1 (one query head per kv head) at the Llama-3-8B-shaped sizes:
    B 64, 32/32 heads, D 128, L ~ U{512..4096}."""
    check(I.mha_config(), what="mha G1")


@pytest.mark.parametrize("splits", [8, 32, 20000])
def test_long_context_forced_splits(splits):
    case = I.decode_config(3)
    out, pl = check(case, num_splits=splits, what=f"long-context S<={splits}")
    assert pl.num_splits <= splits


def test_long_context_page_size_1_vs_64():
    """Same logical tokens at page size 64 and 1: both within tolerance of the
    oracle (whose result is identical for both) and of each other."""
    c64 = I.decode_config(3, page_size=64)
    c1 = I.decode_config(3, page_size=1)
    np.testing.assert_array_equal(c64.q, c1.q)
    a, _ = run_decode(c64)
    b, _ = run_decode(c1)
    assert_close(to_f64(b), to_f64(a), "P=1 vs P=64")


# ------------------------------------------------------------ shapes / edges
@pytest.mark.parametrize("lens,Hq,Hkv,D,P,kw", [
    ([1, 2, 31, 32, 33, 63, 64, 65, 100], 8, 2, 128, 16, {}),
    ([1, 17, 300, 1000], 16, 16, 64, 16, {}),                    # MHA, D 64
    ([5, 77, 1025], 32, 2, 128, 32, {}),                          # G 16
    ([40, 129, 511], 16, 8, 64, 8, {}),                            # G 2, P 8
    ([40, 129, 511], 8, 1, 128, 2, {}),                            # P 2
    ([300, 7, 1500], 8, 1, 64, 4, dict(softcap=5.0)),
    ([2000, 33, 700], 32, 8, 128, 64, dict(window=100)),
    ([2000, 33, 700], 32, 8, 128, 1, dict(window=37, softcap=20.0)),
    ([900, 1, 64], 64, 8, 128, 16, dict(kv_dtype="fp8_e4m3", scale_range=(0.5, 2.0))),
    ([900, 1, 64], 64, 8, 64, 16, dict(kv_dtype="fp8_e4m3", scale_range=(0.5, 2.0),
                                       window=50)),
    ([300, 40], 16, 4, 64, 1, dict(kv_dtype="fp8_e4m3", scale_range=(0.5, 2.0))),
    ([0, 5, 0, 70], 8, 2, 128, 16, {}),                            # empty sequences
    ([1500, 9, 2100], 16, 4, 128, 256, dict(kv_dtype="fp8_e4m3", scale_range=(0.5, 2.0))),
    ([5000, 129], 8, 1, 64, 1024, dict(window=1500, softcap=8.0)),  # P 1024
    ([3000, 5, 4097, 700], 32, 8, 128, 4096, {}),                  # P 4096: one or two pages
    ([100, 2000, 37], 12, 3, 128, 16, {}),                         # 3 kv heads: 1023 blocks
    ([700, 50, 1300], 48, 12, 128, 16, {}),                        # 12 kv heads: one stream
])
def test_shapes(lens, Hq, Hkv, D, P, kw):
    case = rand_case(lens, Hq, Hkv, D, P, 100 + len(lens), **kw)
    check(case, what=f"lens={lens}")


@pytest.mark.parametrize("splits", [1, 2, 3, 8, 32, 257, 5000])
def test_split_counts(splits):
    """Any cut of the tile lists into ranges gives the same result (the 8 kv
    heads each cut into splits / 8 ranges, the count rounded up to a multiple
    of 8; 5000 ranges exceed the tiles: empty ranges must write nothing)."""
    case = rand_case([1, 31, 100, 257, 1000, 4000], 32, 8, 128, 16, 7, softcap=10.0,
                     window=900)
    check(case, num_splits=splits, what=f"S={splits}")


@pytest.mark.parametrize("n", [2, 3])
def test_split_then_merge_is_decode(n):
    """The two passes enqueued by separate calls give decode's bytes."""
    case = I.decode_config(n)
    say(f"[decode] split+merge vs decode, workload {n}")
    t = I.decode_tensors(case, DEV)
    pl = pa.decode_plan(t["q"], t["k_pool"], t["block_table"], case.max_kv_len,
                        window=case.window)
    args = (pl, t["q"], t["k_pool"], t["v_pool"], t["block_table"], t["seq_lens"], case.scale)
    kw = dict(softcap=case.softcap, window=case.window, k_scale=case.k_scale,
              v_scale=case.v_scale)
    ws = pa.workspace_for(pl, DEV)
    whole = pa.decode(*args, workspace=ws, **kw)
    out = torch.full_like(whole, float("nan"))
    pa.decode_split(*args, out=out, workspace=ws, **kw)
    pa.decode_merge(*args, out=out, workspace=ws, **kw)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), whole.view(torch.int16))


def test_all_empty():
    case = rand_case([0, 0], 8, 2, 64, 16, 8, pool_pages=4)   # the pools must exist
    out, _ = run_decode(case)
    assert not to_f64(out).any()


# ------------------------------------------------------------ bit-exact checks
def test_gather_bit_exact():
    for case in (I.decode_config(1), rand_case([1, 33, 100], 8, 2, 128, 4, 9),
                 rand_case([70, 3], 16, 8, 128, 16, 10, kv_dtype="fp8_e4m3")):
        t = I.decode_tensors(case, DEV)
        pl = pa.decode_plan(t["q"], t["k_pool"], t["block_table"], case.max_kv_len)
        k, v = pa.gather(pl, t["k_pool"], t["v_pool"], t["block_table"], t["seq_lens"],
                         int(case.seq_lens.sum()))
        torch.cuda.synchronize()
        np.testing.assert_array_equal(k.cpu().view(torch.uint8).numpy(),
                                      case.k_tok.view(np.uint8))
        np.testing.assert_array_equal(v.cpu().view(torch.uint8).numpy(),
                                      case.v_tok.view(np.uint8))


def test_window_one_is_last_value_bit_exact():
    """W = 1: a one-term softmax, so the output is V[L-1] exactly (bf16 bits)."""
    case = rand_case([1, 16, 17, 500, 1023], 16, 4, 128, 16, 11, window=1)
    out, _ = run_decode(case)
    got = out.cpu().view(torch.int16).numpy().view(np.uint16)
    off = np.concatenate([[0], np.cumsum(case.seq_lens)])
    for b, L in enumerate(case.seq_lens):
        last = case.v_tok[off[b] + L - 1]                    # [Hkv, D]
        np.testing.assert_array_equal(got[b], np.repeat(last, 4, axis=0))


def test_gather_probe_every_row():
    """B' = L sequences share one table row with lengths 1..L and W = 1:
    sequence i returns V[i-1] bit-exactly, reconstructing every row."""
    base = rand_case([300], 8, 8, 64, 16, 12)
    L = 300
    q = np.repeat(base.q, L, axis=0)
    case = I.DecodeCase(name="probe", num_q_heads=8, num_kv_heads=8, head_dim=64,
                        kv_dtype="bf16", q=q,
                        kv=I.PagedKV(base.kv.k_pool, base.kv.v_pool,
                                     np.repeat(base.kv.block_table, L, axis=0), 16),
                        seq_lens=np.arange(1, L + 1, dtype=np.int32), scale=base.scale,
                        window=1)
    out, _ = run_decode(case)
    got = out.cpu().view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(got, base.v_tok[:L])


def test_page_permutation_bit_identical():
    case = rand_case([500, 77, 1400], 32, 8, 128, 16, 13, softcap=30.0)
    a, _ = run_decode(case, num_splits=4)
    b, _ = run_decode(I.relayout(case, 16, seed=77, pool_pages=400), num_splits=4)
    np.testing.assert_array_equal(a.cpu().view(torch.int16).numpy(),
                                  b.cpu().view(torch.int16).numpy())


def test_head_major_pool_layout_bit_identical():
    """A [pages, Hkv, P, D] pool passed by strides gives the same bits."""
    case = rand_case([500, 77], 16, 4, 128, 16, 14)
    t = I.decode_tensors(case, DEV)
    a, _ = run_decode(case, tensors=t)
    hnd = {k: (v.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)
               if k in ("k_pool", "v_pool") else v) for k, v in t.items()}
    assert hnd["k_pool"].stride(1) == 128
    b, _ = run_decode(case, tensors=hnd)
    np.testing.assert_array_equal(a.cpu().view(torch.int16).numpy(),
                                  b.cpu().view(torch.int16).numpy())


def test_fp8_table_on_device():
    """All 256 e4m3fn codes through the kernel: one-key sequences return
    dec(code) * v_scale, compared with the oracle's table."""
    D, Hkv = 128, 1
    codes = np.arange(256, dtype=np.uint8)
    codes = codes[(codes & 0x7F) != 0x7F]                     # NaN codes excluded
    n = codes.size
    v_tok = np.repeat(codes[:, None, None], D, axis=2).reshape(n, Hkv, D)
    k_tok = np.zeros_like(v_tok)
    q = I.bf16_bits(np.ones((n, 4, D), np.float32))
    case = I.decode_case_from_tokens("fp8tab", q, k_tok, v_tok, [1] * n, 16, 15,
                                     kv_dtype="fp8_e4m3")
    out, _ = run_decode(case)
    ref = np.array([oracle.decode_e4m3fn(int(c)) for c in codes])
    np.testing.assert_array_equal(to_f64(out)[:, 0, 0], ref)


@pytest.mark.parametrize("kv_dtype", ["fp8_e4m3", "bf16"])
@pytest.mark.parametrize("splits", [0, 1, 7, 500, 3000])
def test_batches_between_64_and_256_with_empty_sequences(kv_dtype, splits):
    """65..256 sequences (the fp8 kernels find their first sequence in one
    round of length reads, four sequences a lane; the bf16 ones scan twice),
    with empty sequences at lane boundaries and some waves holding no tile."""
    rng = np.random.default_rng(77)
    lens = rng.integers(1, 300, size=150)
    lens[[0, 3, 4, 63, 64, 127, 128, 149]] = 0
    case = rand_case(lens, 16, 2, 128, 16, 78, kv_dtype=kv_dtype, window=200,
                     scale_range=(0.5, 2.0) if kv_dtype != "bf16" else None)
    out, _ = check(case, num_splits=splits or None, what=f"B150 {kv_dtype} splits={splits}")
    for b in np.flatnonzero(lens == 0):
        assert not out[b].any()


@pytest.mark.parametrize("kv_dtype", ["fp8_e4m3", "bf16"])
@pytest.mark.parametrize("splits", [0, 16, 600, 4000])
def test_many_short_sequences(kv_dtype, splits):
    """300 sequences, most of 1..70 tokens: the ranges charge every segment
    a fixed cost in front of its first tile, so here many ranges begin or end
    in that part, some hold no tile at all, and with 4000 splits most are
    empty.  8 kv heads (one stream per head) at fp8 and bf16."""
    rng = np.random.default_rng(91)
    lens = rng.integers(1, 71, size=300)
    lens[rng.choice(300, size=12, replace=False)] = rng.integers(500, 3000, size=12)
    lens[[5, 64, 200]] = 0
    case = rand_case(lens, 32, 8, 128, 16, 92, kv_dtype=kv_dtype,
                     scale_range=(0.5, 2.0) if kv_dtype != "bf16" else None)
    out, _ = check(case, num_splits=splits or None, what=f"B300 short {kv_dtype} splits={splits}")
    for b in np.flatnonzero(lens == 0):
        assert not out[b].any()
