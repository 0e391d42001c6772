"""Property tests on the GPU: hypothesis draws small decode, verify and extend
problems -- batch, heads (G = 1..16), head dim, page size in {1, 16, 64},
lengths including 0, 1 and page multiples, window, soft-cap, split count,
cache dtype, sinks, descales and ALiBi -- and each is run through the C ABI
and compared element by element with the fp64 oracle on the same inputs,
|err| <= 1e-2 + 1e-2*|ref|.

Derandomized (the same examples every run), a bounded number of examples,
no shrinking and no example database: the run is fixed and stops at the first
failure."""
import sys

import numpy as np
import pytest
from hypothesis import HealthCheck, Phase, given, settings
from hypothesis import strategies as st

import oracle
from paged_gqa_attention_02_amd import inputs as I
from tests._gpu import assert_close, run_decode, run_extend, run_verify, to_f64

pytestmark = pytest.mark.gpu


def bounded(n):
    return settings(derandomize=True, max_examples=n, deadline=None, database=None,
                    phases=[Phase.explicit, Phase.generate],
                    suppress_health_check=list(HealthCheck))


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@st.composite
def lengths(draw, n, page_size, top):
    """n lengths: 0, 1, a multiple of the page size (16 for P = 1), or any."""
    unit = page_size if page_size > 1 else 16
    one = st.one_of(st.just(0), st.just(1),
                    st.integers(1, max(1, top // unit)).map(lambda k: k * unit),
                    st.integers(0, top))
    return draw(st.lists(one, min_size=n, max_size=n))


@st.composite
def common(draw):
    return dict(P=draw(st.sampled_from([1, 16, 64])),
                D=draw(st.sampled_from([64, 128])),
                G=draw(st.sampled_from([1, 2, 4, 8, 16])),
                Hkv=draw(st.sampled_from([1, 2])),
                kv=draw(st.sampled_from(["bf16", "fp8_e4m3"])),
                window=draw(st.sampled_from([0, 0, 1, 17, 128, 500])),
                cap=draw(st.sampled_from([0.0, 0.0, 20.0])),
                seed=draw(st.integers(0, 1 << 20)),
                sinks=draw(st.booleans()),
                descales=draw(st.booleans()),
                alibi=draw(st.sampled_from([False, False, True])))


def _extras(case, c):
    if c["sinks"] or c["descales"] or c["alibi"]:
        I.with_extras(case, c["seed"] + 1, sinks=c["sinks"], descales=c["descales"],
                      alibi=c["alibi"])
    return case


@st.composite
def decode_problem(draw):
    c = draw(common())
    B = draw(st.integers(1, 6))
    c["lens"] = draw(lengths(B, c["P"], 900))
    c["splits"] = draw(st.sampled_from([0, 0, 1, 3, 64, 500]))
    return c


def make_decode(c, name):
    fp8 = c["kv"] == "fp8_e4m3"
    case = I.make_decode(name, c["lens"], c["G"] * c["Hkv"], c["Hkv"], c["D"], c["P"],
                         c["seed"], kv_dtype=c["kv"], softcap=c["cap"], window=c["window"],
                         num_splits=c["splits"], scale_range=(0.5, 2.0) if fp8 else None)
    return _extras(case, c)


@bounded(60)
@given(decode_problem())
def test_decode_property(c):
    say(f"[prop decode] {c}")
    case = make_decode(c, "prop-decode")
    out, pl = run_decode(case)
    ref, _ = oracle.decode(case)
    assert_close(to_f64(out), ref, pl.describe())


@st.composite
def verify_problem(draw):
    c = draw(decode_problem())
    c["q_len"] = draw(st.integers(1, 4))
    return c


@bounded(40)
@given(verify_problem())
def test_verify_property(c):
    say(f"[prop verify] {c}")
    case = make_decode(c, "prop-verify")
    q = I.bf16_bits(np.random.default_rng(c["seed"] + 2).standard_normal(
        (case.batch, c["q_len"], case.num_q_heads, case.head_dim), dtype=np.float32))
    out, pl = run_verify(case, q)
    ref = oracle.verify(case, q)
    assert_close(to_f64(out), ref, pl.describe())


@st.composite
def extend_problem(draw):
    c = draw(common())
    B = draw(st.integers(1, 3))
    c["G"] = draw(st.sampled_from([1, 2, 4, 8]))
    c["ctx"] = draw(lengths(B, c["P"], 400))
    c["q_lens"] = draw(st.lists(st.one_of(st.just(0), st.just(1), st.integers(1, 100)),
                                min_size=B, max_size=B))
    c["splits"] = draw(st.sampled_from([0, 0, 1, 5, 300]))
    return c


@bounded(40)
@given(extend_problem())
def test_extend_property(c):
    say(f"[prop extend] {c}")
    fp8 = c["kv"] == "fp8_e4m3"
    case = I.make_extend("prop-extend", c["ctx"], c["q_lens"], c["G"] * c["Hkv"], c["Hkv"],
                         c["D"], c["P"], c["seed"], kv_dtype=c["kv"], softcap=c["cap"],
                         window=c["window"], scale_range=(0.5, 2.0) if fp8 else None)
    case = _extras(case, c)
    if case.total_q == 0:
        return
    out, pl = run_extend(case, num_splits=c["splits"])
    ref = oracle.extend(case)
    assert_close(to_f64(out), ref, pl.describe())
