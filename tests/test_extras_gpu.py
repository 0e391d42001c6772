"""Sinks and per-request descales on the GPU: decode, verify and extend through
the C ABI against the fp64 oracle on the same seeded inputs,
|err| <= 1e-2 + 1e-2*|ref| per element."""
import sys

import numpy as np
import pytest
import torch

import oracle
import paged_gqa_attention_02_amd as pa
from paged_gqa_attention_02_amd import inputs as I
from tests._gpu import DEV, assert_close, run_decode, run_extend, run_verify, to_f64

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def dcase(lens, Hq, Hkv, D, P, seed, sinks=True, descales=False, **kw):
    rng = np.random.default_rng(seed)
    case = I.make_decode(f"x{seed}", lens, Hq, Hkv, D, P, seed, lens_rng=rng, **kw)
    return I.with_extras(case, seed + 7, sinks=sinks, descales=descales)


@pytest.mark.parametrize("lens,Hq,Hkv,D,P,splits,kw", [
    ([1, 2, 33, 100, 1000], 8, 2, 128, 16, None, {}),
    ([1, 2, 33, 100, 1000], 8, 2, 128, 16, 50, {}),                    # split segments
    ([5, 700, 3000], 32, 8, 128, 16, 8, dict(softcap=30.0)),
    ([64, 900, 1500], 16, 16, 64, 8, None, dict(window=300)),
    ([900, 1, 64, 4000], 64, 8, 128, 16, 40,
     dict(kv_dtype="fp8_e4m3", scale_range=(0.5, 2.0), window=1000)),
])
@pytest.mark.parametrize("descales", [False, True])
def test_decode_sinks(lens, Hq, Hkv, D, P, splits, kw, descales):
    case = dcase(lens, Hq, Hkv, D, P, 500 + len(lens), descales=descales, **kw)
    say(f"[extras] decode lens={lens} Hq={Hq} Hkv={Hkv} D={D} P={P} splits={splits} "
        f"descales={descales} {kw}")
    out, pl = run_decode(case, splits)
    ref, _ = oracle.decode(case)
    assert_close(to_f64(out), ref, f"decode sinks ({pl.describe()})")


def test_decode_descales_only_and_broadcast():
    """Per-request descales without sinks; a single-entry descale vector is
    shared by every request (the same as a per-tensor scale)."""
    case = dcase([50, 400, 2000, 7], 32, 8, 128, 16, 510, sinks=False, descales=True,
                 kv_dtype="fp8_e4m3", scale_range=(0.5, 2.0))
    out, _ = run_decode(case)
    assert_close(to_f64(out), oracle.decode(case)[0], "per-request descales")
    t = I.decode_tensors(case, DEV)
    one_k = torch.tensor([1.5], dtype=torch.float32, device=DEV)
    one_v = torch.tensor([0.75], dtype=torch.float32, device=DEV)
    pl = pa.decode_plan(t["q"], t["k_pool"], t["block_table"], case.max_kv_len)
    got = pa.decode(pl, t["q"], t["k_pool"], t["v_pool"], t["block_table"], t["seq_lens"],
                    case.scale, k_scale=case.k_scale, v_scale=case.v_scale,
                    k_descale=one_k, v_descale=one_v)
    torch.cuda.synchronize()
    case.k_descale = case.v_descale = None
    case.k_scale *= 1.5
    case.v_scale *= 0.75
    assert_close(to_f64(got), oracle.decode(case)[0], "broadcast descales")


def test_decode_sinks_minus_inf_is_bit_identical():
    case = dcase([3, 77, 1500], 32, 8, 128, 16, 520, sinks=False, softcap=20.0)
    ref, _ = run_decode(case, 30)
    case.sinks = np.full(32, -np.inf, dtype=np.float32)
    got, _ = run_decode(case, 30)
    assert torch.equal(got.view(torch.int16), ref.view(torch.int16))


def test_decode_large_sinks_take_the_mass():
    """Sinks far above every score leave (almost) nothing for the values."""
    case = dcase([40, 600], 8, 2, 64, 16, 530)
    case.sinks = np.full(8, 60.0, dtype=np.float32)
    out, _ = run_decode(case, 9)
    ref, _ = oracle.decode(case)
    assert_close(to_f64(out), ref, "large sinks")
    assert np.abs(to_f64(out)).max() < 1e-6


@pytest.mark.parametrize("q_len,Hq,kw", [(4, 32, {}), (8, 32, dict(softcap=30.0)),
                                         (3, 64, dict(kv_dtype="fp8_e4m3",
                                                      scale_range=(0.5, 2.0)))])
def test_verify_sinks_descales(q_len, Hq, kw):
    case = dcase([2, 300, 1800], Hq, 8, 128, 16, 540 + q_len, descales=True, **kw)
    q = I.bf16_bits(np.random.default_rng(541).standard_normal(
        (3, q_len, Hq, 128), dtype=np.float32))
    say(f"[extras] verify q_len={q_len} Hq={Hq} {kw}")
    out, pl = run_verify(case, q, 20)
    assert_close(to_f64(out), oracle.verify(case, q), f"verify sinks ({pl.describe()})")


@pytest.mark.parametrize("kw", [{}, dict(softcap=25.0), dict(window=200),
                                dict(kv_dtype="fp8_e4m3", scale_range=(0.5, 2.0))])
def test_extend_sinks_descales(kw):
    case = I.with_extras(I.make_extend("xe", [0, 70, 1000], [3, 130, 260], 32, 8, 128, 16,
                                       550, **kw), 551, descales=True)
    say(f"[extras] extend {kw}")
    out, _ = run_extend(case)
    assert_close(to_f64(out), oracle.extend(case), f"extend sinks {kw}")


# ------------------------------------------------------------------- ALiBi
@pytest.mark.parametrize("lens,Hq,Hkv,D,P,splits,kw", [
    ([1, 2, 33, 100, 1000], 8, 2, 128, 16, None, {}),
    ([5, 700, 3000], 32, 8, 128, 16, 40, dict(softcap=30.0)),
    ([64, 900, 1500], 16, 16, 64, 8, None, dict(window=300)),
    ([900, 1, 64, 4000], 64, 8, 128, 16, 40,
     dict(kv_dtype="fp8_e4m3", scale_range=(0.5, 2.0))),
])
def test_decode_alibi(lens, Hq, Hkv, D, P, splits, kw):
    case = I.with_extras(I.make_decode("al", lens, Hq, Hkv, D, P, 560,
                                       lens_rng=np.random.default_rng(560), **kw),
                         561, sinks=False, alibi=True)
    say(f"[extras] decode alibi lens={lens} Hq={Hq} D={D} splits={splits} {kw}")
    out, pl = run_decode(case, splits)
    assert_close(to_f64(out), oracle.decode(case)[0], f"decode alibi ({pl.describe()})")


def test_verify_alibi_with_sinks():
    case = I.with_extras(I.make_decode("alv", [3, 300, 1800], 32, 8, 128, 16, 562,
                                       lens_rng=np.random.default_rng(562)), 563, alibi=True)
    q = I.bf16_bits(np.random.default_rng(564).standard_normal((3, 6, 32, 128),
                                                               dtype=np.float32))
    out, pl = run_verify(case, q, 25)
    assert_close(to_f64(out), oracle.verify(case, q), f"verify alibi ({pl.describe()})")


@pytest.mark.parametrize("kw,splits", [({}, 0), (dict(softcap=25.0), 11),
                                       (dict(window=200), 0),
                                       (dict(kv_dtype="fp8_e4m3", scale_range=(0.5, 2.0)), 7)])
def test_extend_alibi(kw, splits):
    case = I.with_extras(I.make_extend("xa", [0, 70, 1000], [3, 130, 260], 32, 8, 128, 16,
                                       565, **kw), 566, sinks=False, alibi=True)
    say(f"[extras] extend alibi {kw} splits={splits}")
    out, _ = run_extend(case, num_splits=splits)
    assert_close(to_f64(out), oracle.extend(case), f"extend alibi {kw}")
