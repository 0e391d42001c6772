"""Each plausible mistake planted in a copy of the oracle (on the CPU) must make
at least one pin in test_oracle.py fail; otherwise the pins would not be
pinning that part of the definition."""
import inspect
import os
import tempfile

import pytest

import oracle
from oracle import build as obuild
from tests import test_oracle as pins
from tests._orc import Oracle

# (name, original text, mutated text) -- every original must occur in the source
MUTANTS = [
    ("gqa-index", "int g = h / G;", "int g = h % pr->Hkv;"),
    ("no-scale", "cap_score(pr->scale * dot, pr->softcap)", "cap_score(dot, pr->softcap)"),
    ("cap-before-scale", "cap_score(pr->scale * dot, pr->softcap)",
     "pr->scale * cap_score(dot, pr->softcap)"),
    ("cap-inner", "c * tanh(s / c)", "c * tanh(s * c)"),
    ("cap-sign", "c * tanh(s / c)", "-c * tanh(s / c)"),
    ("cap-off-when-positive", "return c > 0.0 ?", "return c < 0.0 ?"),
    ("window-off-by-one", "L - pr->window > 0) ? L - pr->window : 0",
     "L - pr->window > 0) ? L - pr->window + 1 : 0"),
    ("window-extend-ctx", "if (pr->window > 0 && pos - j >= pr->window)",
     "if (pr->window > 0 && pos - j > pr->window)"),
    ("causal-diagonal", "for (j = 0; j <= i; ++j) {", "for (j = 0; j < i; ++j) {"),
    ("row-in-page", "int row = (int)(t % pr->P);", "int row = (int)((t + 1) % pr->P);"),
    ("layout-transposed", "int64_t idx = ((page * P + row) * (int64_t)Hkv + g) * D + d;",
     "int64_t idx = ((page * P + row) * (int64_t)D + d) * Hkv + g;"),
    ("no-k-scale", "pr->P, pr->Hkv, pr->D) * ks;", "pr->P, pr->Hkv, pr->D);"),
    ("no-v-scale", "pr->Hkv, pr->D) * vs;", "pr->Hkv, pr->D);"),
    ("merge-sign", "w = exp(lses[sp] - M);", "w = exp(M - lses[sp]);"),
    ("split-drops-token", "int64_t e = a + len < L ? a + len : L;",
     "int64_t e = a + len < L ? a + len - 1 : L;"),
    ("lse-no-max", "*lse = m + log(z);", "*lse = log(z);"),
    ("no-normalise", "out[d] /= z;\n    *lse", "out[d] /= 1.0;\n    *lse"),
    ("e4m3-bias", "expo - 10", "expo - 11"),
    ("e4m3-subnormal", "ldexp((double)mant, -9)", "ldexp((double)mant, -10)"),
    ("e4m3-nan", "if (expo == 0xF && mant == 0x7)", "if (expo == 0xF && mant == 0x6)"),
    ("bf16-shift", "(uint32_t)bits << 16", "(uint32_t)bits << 15"),
    ("new-key-row", "int64_t row = pr->cu_q[b] + j;", "int64_t row = pr->cu_q[b] + j + (j < i);"),
    ("new-key-head", "pr->k_new[(row * pr->Hkv + g) * D + d]", "pr->k_new[(row * pr->Hkv) * D + d]"),
    ("ctx-len-seq", "C = pr->ctx_lens[b];", "C = pr->ctx_lens[pr->B - 1 - b];"),
    ("e4m3-enc-tie-odd", "(c & 1) == 0 && (best & 1) == 1", "(c & 1) == 1 && (best & 1) == 0"),
    ("e4m3-enc-sign", "signbit(x) ? 0x80 : 0x00", "signbit(x) ? 0x00 : 0x80"),
    ("append-row", "(slot % P) * s_tok", "((slot + 1) % P) * s_tok"),
    ("append-scale", "orc_e4m3fn_encode(kf / k_scale)", "orc_e4m3fn_encode(kf * k_scale)"),
    ("append-value-from-key", "uint16_t vb = value[", "uint16_t vb = key["),
    ("verify-causal", "int64_t L = (int64_t)pr->seq_lens[b] - ql + i + 1;",
     "int64_t L = (int64_t)pr->seq_lens[b] - ql + i;"),
    ("verify-row-order", "int b = (int)(bi / ql), i = (int)(bi % ql);",
     "int b = (int)(bi / ql), i = ql - 1 - (int)(bi % ql);"),
    ("sink-scaled", "return pr->sinks ? (double)pr->sinks[h] : -INFINITY;",
     "return pr->sinks ? pr->scale * (double)pr->sinks[h] : -INFINITY;"),
    ("sink-kv-head", "return pr->sinks ? (double)pr->sinks[h] : -INFINITY;",
     "return pr->sinks ? (double)pr->sinks[h % pr->Hkv] : -INFINITY;"),
    ("sink-sign", "        z = exp(sink - m);", "        z = exp(m - sink);"),
    ("sink-in-every-split", "softmax_sum(s, v, e - a, Dv, -INFINITY,",
     "softmax_sum(s, v, e - a, Dv, sink_of(pr, h),"),
    ("sink-missing-from-merge", "            z = exp(sink_of(pr, h) - M);", "            z = 0.0;"),
    ("descale-first-request", "(pr->k_desc ? (double)pr->k_desc[b] : 1.0)",
     "(pr->k_desc ? (double)pr->k_desc[0] : 1.0)"),
    ("v-descale-from-k", "(pr->v_desc ? (double)pr->v_desc[b] : 1.0)",
     "(pr->v_desc ? (double)pr->k_desc[b] : 1.0)"),
    ("alibi-sign", "(double)pr->alibi[h] * (double)(j - pos)",
     "(double)pr->alibi[h] * (double)(pos - j)"),
    ("alibi-kv-head", "(double)pr->alibi[h] * (double)(j - pos)",
     "(double)pr->alibi[h % pr->Hkv] * (double)(j - pos)"),
    ("alibi-decode-pos", "s[t - lo] += alibi_bias(pr, h, t, L - 1);\n        softmax_sum",
     "s[t - lo] += alibi_bias(pr, h, t, L);\n        softmax_sum"),
    ("alibi-new-key-pos", "+ alibi_bias(pr, h, C + j, pos);", "+ alibi_bias(pr, h, j, pos);"),
    ("latent-value-pitch", "cache_elem(pr->v_pool, pr->kv_dtype, page, row, g, d, pr->P,\n"
     "                           pr->Hkv, pr->D) * vs;",
     "cache_elem(pr->v_pool, pr->kv_dtype, page, row, g, d, pr->P,\n"
     "                           pr->Hkv, pr->Dv) * vs;"),
    ("latent-value-suffix", "cache_elem(pr->v_pool, pr->kv_dtype, page, row, g, d, pr->P,",
     "cache_elem(pr->v_pool, pr->kv_dtype, page, row, g, pr->D - pr->Dv + d, pr->P,"),
    ("latent-value-from-key-pool", "cache_elem(pr->v_pool, pr->kv_dtype, page, row, g, d, pr->P,",
     "cache_elem(pr->k_pool, pr->kv_dtype, page, row, g, d, pr->P,"),
]


def _pin_calls():
    """Every (name, callable) of the pins, parametrisations expanded."""
    calls = []
    for name, fn in inspect.getmembers(pins, inspect.isfunction):
        if not name.startswith("test_"):
            continue
        params = [m for m in getattr(fn, "pytestmark", []) if m.name == "parametrize"]
        if not params:
            calls.append((name, fn, {}))
            continue
        argnames, argvalues = params[0].args[0], params[0].args[1]
        names = [a.strip() for a in argnames.split(",")]
        for vals in argvalues:
            vals = vals if len(names) > 1 else (vals,)
            calls.append((name, fn, dict(zip(names, vals))))
    return calls


@pytest.fixture(scope="module")
def source():
    with open(obuild.SRC) as f:
        return f.read()


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(source, name, old, new):
    assert old in source, f"mutation site for {name} not found"
    with tempfile.TemporaryDirectory() as d:
        src = os.path.join(d, "mutant.c")
        with open(src, "w") as f:
            f.write(source.replace(old, new))
        lib = oracle.bind(obuild.build(src=src, out=os.path.join(d, "libmutant.so")))
        orc = Oracle(lib)
        for pname, fn, kw in _pin_calls():
            try:
                fn(orc, **kw)
            except AssertionError:
                return          # caught by this pin
        pytest.fail(f"mutant {name} passed every pin")
