"""KV-cache append on the GPU through the C ABI: the pools it writes are
compared byte for byte with the oracle's; a gather after the append returns
the appended rows; decode after the append matches the oracle."""
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


def pools(kv_dtype, num_pages, P, Hkv, D, seed):
    rng = np.random.default_rng(seed)
    pdt = np.uint16 if kv_dtype == "bf16" else np.uint8
    kp = rng.integers(0, np.iinfo(pdt).max, size=(num_pages, P, Hkv, D), dtype=pdt)
    vp = rng.integers(0, np.iinfo(pdt).max, size=(num_pages, P, Hkv, D), dtype=pdt)
    return kp, vp


def run_append(key, value, kp, vp, slots, kv_dtype, ks=1.0, vs=1.0):
    tdt = torch.bfloat16 if kv_dtype == "bf16" else torch.float8_e4m3fn
    dk = torch.from_numpy(kp.copy()).view(tdt).to(DEV)
    dv = torch.from_numpy(vp.copy()).view(tdt).to(DEV)
    kt = torch.from_numpy(key.view(np.int16)).view(torch.bfloat16).to(DEV)
    vt = torch.from_numpy(value.view(np.int16)).view(torch.bfloat16).to(DEV)
    st = torch.from_numpy(np.asarray(slots, dtype=np.int64)).to(DEV)
    pa.cache_append(kt, vt, dk, dv, st, k_scale=ks, v_scale=vs)
    torch.cuda.synchronize()
    ndt = np.uint16 if kv_dtype == "bf16" else np.uint8
    idt = torch.int16 if kv_dtype == "bf16" else torch.uint8
    return (dk.view(idt).cpu().numpy().view(ndt), dv.view(idt).cpu().numpy().view(ndt))


@pytest.mark.parametrize("kv_dtype,ks,vs", [("bf16", 1.0, 1.0), ("fp8_e4m3", 0.8, 1.7)])
@pytest.mark.parametrize("D,P", [(128, 16), (64, 1), (128, 64), (128, 4096)])
def test_append_matches_oracle(kv_dtype, ks, vs, D, P):
    """The new tokens of the extend workload (3,577 rows, 8 kv heads) at seeded
    random distinct slots, every fifth token padding."""
    say(f"[append] kv={kv_dtype} D={D} P={P}")
    ext = I.extend_config(5)
    T, Hkv = ext.total_q, ext.num_kv_heads
    rng = np.random.default_rng(7)
    key = I.bf16_bits(rng.standard_normal((T, Hkv, D), dtype=np.float32) * 4)
    value = I.bf16_bits(rng.standard_normal((T, Hkv, D), dtype=np.float32) * 4)
    num_pages = (2 * T + P - 1) // P
    kp, vp = pools(kv_dtype, num_pages, P, Hkv, D, 8)
    slots = rng.permutation(num_pages * P)[:T].astype(np.int64)
    slots[::5] = -1
    gk, gv = run_append(key, value, kp, vp, slots, kv_dtype, ks, vs)
    rk, rv = oracle.cache_append(key, value, kp, vp, slots, kv_dtype, k_scale=ks, v_scale=vs)
    np.testing.assert_array_equal(gk, rk)
    np.testing.assert_array_equal(gv, rv)


def test_append_fp8_special_values():
    """Zeros of both signs, exact ties, subnormal-range values, values past
    448, infinities and NaN: bit-exact against the oracle."""
    specials = [0.0, -0.0, 1.0625, 1.1875, -1.0625, 2 ** -9, 2 ** -10, 1.5 * 2 ** -9,
                3 * 2 ** -10, 440.0, 448.0, 456.0, 464.0, 1e4, -1e30, float("inf"),
                float("-inf"), float("nan"), 2 ** -6, 2 ** -7 * 1.875, 0.01, -7.25e-3]
    D, Hkv, P = 64, 1, 16
    T = 8
    vals = np.resize(np.array(specials, dtype=np.float32), T * Hkv * D)
    key = I.bf16_bits(vals.reshape(T, Hkv, D))
    value = I.bf16_bits(-vals[::-1].reshape(T, Hkv, D))
    kp, vp = pools("fp8_e4m3", 2, P, Hkv, D, 9)
    slots = np.arange(T, dtype=np.int64) * 3
    for ks in (1.0, 0.5, 3.0):
        gk, gv = run_append(key, value, kp, vp, slots, "fp8_e4m3", ks, ks)
        rk, rv = oracle.cache_append(key, value, kp, vp, slots, "fp8_e4m3", k_scale=ks,
                                     v_scale=ks)
        np.testing.assert_array_equal(gk, rk)
        np.testing.assert_array_equal(gv, rv)


def test_append_then_gather_round_trip():
    """Tokens appended at each sequence's slots through a block table come back
    unchanged from the gather (bf16): gather(append(x)) == x."""
    lens, Hkv, D, P = [37, 100, 1, 64], 4, 128, 16
    rng = np.random.default_rng(12)
    table, num_pages = I.deal_pages(lens, P, rng)
    T = sum(lens)
    key = I.bf16_bits(rng.standard_normal((T, Hkv, D), dtype=np.float32))
    value = I.bf16_bits(rng.standard_normal((T, Hkv, D), dtype=np.float32))
    slots = np.concatenate([table[b, np.arange(L) // P] * P + np.arange(L) % P
                            for b, L in enumerate(lens)]).astype(np.int64)
    kp, vp = pools("bf16", num_pages, P, Hkv, D, 13)
    gk, gv = run_append(key, value, kp, vp, slots, "bf16")
    dk = torch.from_numpy(gk).view(torch.bfloat16).to(DEV)
    dv = torch.from_numpy(gv).view(torch.bfloat16).to(DEV)
    bt = torch.from_numpy(table).to(DEV)
    sl = torch.tensor(lens, dtype=torch.int32, device=DEV)
    q = torch.zeros(len(lens), Hkv, D, dtype=torch.bfloat16, device=DEV)
    pl = pa.decode_plan(q, dk, bt, max(lens))
    ok, ov = pa.gather(pl, dk, dv, bt, sl, T)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(ok.view(torch.int16).cpu().numpy().view(np.uint16), key)
    np.testing.assert_array_equal(ov.view(torch.int16).cpu().numpy().view(np.uint16), value)


def test_decode_after_append():
    """Decode of a step whose newest token was written by the append, fp8 cache:
    matches the oracle on the pools the oracle's append produced."""
    case = I.make_decode("append-decode", [300, 45, 1000], 32, 8, 128, 16, 14,
                         kv_dtype="fp8_e4m3", scale_range=(0.5, 2.0))
    rng = np.random.default_rng(15)
    key = I.bf16_bits(rng.standard_normal((3, 8, 128), dtype=np.float32))
    value = I.bf16_bits(rng.standard_normal((3, 8, 128), dtype=np.float32))
    P, bt = case.kv.page_size, case.kv.block_table
    last = case.seq_lens.astype(np.int64) - 1
    slots = bt[np.arange(3), last // P].astype(np.int64) * P + last % P
    gk, gv = run_append(key, value, case.kv.k_pool, case.kv.v_pool, slots, "fp8_e4m3",
                        case.k_scale, case.v_scale)
    rk, rv = oracle.cache_append(key, value, case.kv.k_pool, case.kv.v_pool, slots,
                                 "fp8_e4m3", k_scale=case.k_scale, v_scale=case.v_scale)
    np.testing.assert_array_equal(gk, rk)
    np.testing.assert_array_equal(gv, rv)
    case.kv.k_pool, case.kv.v_pool = rk, rv
    out, _ = run_decode(case)
    ref, _ = oracle.decode(case)
    assert_close(to_f64(out), ref, "decode after append")
