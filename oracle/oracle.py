"""ctypes front end of the fp64 CPU oracle, plus a NumPy brute force.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the bench's
CPU-baseline leg are the only callers.  Nothing here imports or calls the HIP
library; inputs arrive as raw bit arrays from the seeded input module.

``decode`` / ``extend`` call ``pa_oracle.c`` (the definitions are written out
there).  ``brute_decode`` / ``brute_extend`` are a second, independent
formulation: they materialise each sequence's keys and values densely through
the block table and run a full softmax with NumPy matrix products.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np

from . import build as _build

_LIB = None
_KV = {"bf16": 0, "fp8_e4m3": 1}


def bind(path: str):
    """Load a build of pa_oracle.c and declare its C signatures."""
    L = ctypes.CDLL(path)
    p, i, i64, d = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_double
    L.orc_decode.argtypes = [i, i, i, i, i, i, i, p, p, p, i64, p, i64, p,
                             d, d, i, d, d, i, p, p, i, p, p, p, p]
    L.orc_decode.restype = i
    L.orc_extend.argtypes = [i, i, i, i, i, i, p, p, p, p, p, p, p, i64, p,
                             i64, d, d, i, d, d, p, i64, p, i, p, p, p, p]
    L.orc_extend.restype = i
    L.orc_bf16.argtypes = [ctypes.c_uint16]
    L.orc_bf16.restype = d
    L.orc_e4m3fn.argtypes = [ctypes.c_uint8]
    L.orc_e4m3fn.restype = d
    L.orc_verify.argtypes = [i, i, i, i, i, i, i, p, p, p, i64, p, i64, p, d, d, i, d, d, p, i,
                             p, p, p, p]
    L.orc_verify.restype = i
    L.orc_e4m3fn_encode.argtypes = [ctypes.c_float]
    L.orc_e4m3fn_encode.restype = ctypes.c_uint8
    L.orc_cache_append.argtypes = [i64, i, i, i, i, p, p, i64, p, p, i64, i64, i64, i64, p,
                                   ctypes.c_float, ctypes.c_float]
    L.orc_cache_append.restype = i
    return L


def lib():
    """The oracle's C library: the in-tree build, or the build PA_ORACLE_LIB
    names (the sanitized build the CPU tests load)."""
    global _LIB
    if _LIB is None:
        path = os.environ.get("PA_ORACLE_LIB")
        if not path:
            path = _build.LIB
            if not os.path.exists(path):
                _build.build()
        _LIB = bind(path)
    return _LIB


def host_cpus() -> dict:
    """The host's CPU counts: all of them, the ones this process may run on,
    and the share the environment grants a job (OMP_NUM_THREADS, when set)."""
    env = os.environ.get("OMP_NUM_THREADS", "")
    return {"nproc": os.cpu_count() or 1, "affinity": len(os.sched_getaffinity(0)),
            "omp_num_threads": int(env) if env.isdigit() and int(env) > 0 else None}


def default_threads() -> int:
    """Every core this process may use: the affinity set, or the job's share
    of it when the environment fixes one (OMP_NUM_THREADS)."""
    c = host_cpus()
    n = c["affinity"]
    if c["omp_num_threads"]:
        n = min(n, c["omp_num_threads"])
    return max(1, n)


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(a)


def _extras(case):
    """fp32 sinks [Hq], per-request descales [B] and ALiBi slopes [Hq] of a
    case (None = off), kept alive by the caller while the C call runs."""
    def f32(name):
        a = getattr(case, name, None)
        return None if a is None else np.ascontiguousarray(a, dtype=np.float32)
    return f32("sinks"), f32("k_descale"), f32("v_descale"), f32("alibi_slopes")


def decode(case, num_splits: int = 0, threads: Optional[int] = None, clib=None):
    """fp64 decode of a DecodeCase -> (out [B,Hq,Dv] float64, lse [B,Hq]);
    Dv = case.head_dim_v (the value head dim; head_dim unless set)."""
    B, Hq, D = case.batch, case.num_q_heads, case.head_dim
    Dv = getattr(case, "head_dim_v", 0) or D
    out = np.zeros((B, Hq, Dv), dtype=np.float64)
    lse = np.zeros((B, Hq), dtype=np.float64)
    q, kp, vp = _c(case.q), _c(case.kv.k_pool), _c(case.kv.v_pool)
    bt, sl = _c(case.kv.block_table), _c(case.seq_lens)
    sk, kd, vd, al = _extras(case)
    rc = (clib or lib()).orc_decode(B, Hq, case.num_kv_heads, D, Dv, case.page_size,
                          _KV[case.kv_dtype], _ptr(q), _ptr(kp), _ptr(vp),
                          kp.shape[0], _ptr(bt), bt.shape[1], _ptr(sl),
                          case.scale, case.softcap, case.window, case.k_scale,
                          case.v_scale, num_splits, _ptr(out), _ptr(lse),
                          threads or default_threads(), _ptr(sk), _ptr(kd), _ptr(vd), _ptr(al))
    if rc != 0:
        raise RuntimeError(f"orc_decode failed: {rc}")
    return out, lse


def extend(case, rows: Optional[np.ndarray] = None,
           threads: Optional[int] = None, clib=None) -> np.ndarray:
    """fp64 extend of an ExtendCase -> out [total_q,Hq,D] (only `rows` filled
    when a row list is given)."""
    Hq, D = case.num_q_heads, case.head_dim
    out = np.zeros((case.total_q, Hq, D), dtype=np.float64)
    q, kn, vn = _c(case.q), _c(case.k_new), _c(case.v_new)
    cu, ctx = _c(case.cu_seqlens_q), _c(case.ctx_lens)
    kp, vp, bt = _c(case.kv.k_pool), _c(case.kv.v_pool), _c(case.kv.block_table)
    r = None if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    sk, kd, vd, al = _extras(case)
    rc = (clib or lib()).orc_extend(case.batch, Hq, case.num_kv_heads, D, case.kv.page_size,
                          _KV[case.kv_dtype], _ptr(q), _ptr(kn), _ptr(vn),
                          _ptr(cu), _ptr(ctx), _ptr(kp), _ptr(vp), kp.shape[0],
                          _ptr(bt), bt.shape[1], case.scale, case.softcap,
                          case.window, case.k_scale, case.v_scale, _ptr(r),
                          0 if r is None else r.shape[0], _ptr(out),
                          threads or default_threads(), _ptr(sk), _ptr(kd), _ptr(vd), _ptr(al))
    if rc != 0:
        raise RuntimeError(f"orc_extend failed: {rc}")
    return out


def verify(case, q: np.ndarray, threads: Optional[int] = None, clib=None) -> np.ndarray:
    """fp64 verify of the decode case's sequences with query rows q (bf16 bits
    [B, q_len, Hq, D]); the last q_len cached tokens of each sequence are the
    query tokens.  Returns out [B, q_len, Hq, D]."""
    B, ql, Hq, D = q.shape
    out = np.zeros((B, ql, Hq, D), dtype=np.float64)
    qb = _c(q)
    kp, vp, bt = _c(case.kv.k_pool), _c(case.kv.v_pool), _c(case.kv.block_table)
    sl = _c(case.seq_lens)
    sk, kd, vd, al = _extras(case)
    rc = (clib or lib()).orc_verify(B, Hq, case.num_kv_heads, D, case.kv.page_size,
                                    _KV[case.kv_dtype], ql, _ptr(qb), _ptr(kp), _ptr(vp),
                                    kp.shape[0], _ptr(bt), bt.shape[1], _ptr(sl), case.scale,
                                    case.softcap, case.window, case.k_scale, case.v_scale,
                                    _ptr(out), threads or default_threads(), _ptr(sk),
                                    _ptr(kd), _ptr(vd), _ptr(al))
    if rc != 0:
        raise RuntimeError(f"orc_verify failed: {rc}")
    return out


def encode_e4m3fn(x: float, clib=None) -> int:
    """e4m3fn code nearest to the float32 x (ties to even, saturating)."""
    return (clib or lib()).orc_e4m3fn_encode(x)


def cache_append(key: np.ndarray, value: np.ndarray, k_pool: np.ndarray,
                 v_pool: np.ndarray, slot_mapping: np.ndarray, kv_dtype: str,
                 k_scale: float = 1.0, v_scale: float = 1.0, clib=None):
    """Cache append of bf16 key/value bits [T, Hkv, D] into copies of the
    pools [num_pages, P, Hkv, D] (uint16 or uint8 bits) at int64 slots;
    returns the new pools."""
    T, Hkv, D = key.shape
    kp, vp = np.array(k_pool, copy=True), np.array(v_pool, copy=True)
    num_pages, P = kp.shape[0], kp.shape[1]
    kb, vb, sm = _c(key), _c(value), _c(np.asarray(slot_mapping, dtype=np.int64))
    rc = (clib or lib()).orc_cache_append(T, Hkv, D, P, _KV[kv_dtype], _ptr(kb), _ptr(vb),
                                          Hkv * D, _ptr(kp), _ptr(vp), P * Hkv * D, Hkv * D, D,
                                          num_pages, _ptr(sm), k_scale, v_scale)
    if rc != 0:
        raise RuntimeError(f"orc_cache_append failed: {rc}")
    return kp, vp


def decode_bf16(bits: int, clib=None) -> float:
    return (clib or lib()).orc_bf16(bits)


def decode_e4m3fn(bits: int, clib=None) -> float:
    return (clib or lib()).orc_e4m3fn(bits)


# --------------------------------------------------------------------------
# NumPy brute force: dense materialisation + full softmax
# --------------------------------------------------------------------------
def _elem_table(kv_dtype: str) -> np.ndarray:
    if kv_dtype == "bf16":
        codes = np.arange(1 << 16, dtype=np.uint32) << 16
        with np.errstate(invalid="ignore"):
            return codes.view(np.float32).astype(np.float64)
    return np.array([decode_e4m3fn(c) for c in range(256)], dtype=np.float64)


def _dense_seq(case_kv, b: int, L: int, kv_dtype: str, table: np.ndarray):
    P = case_kv.page_size
    t = np.arange(L)
    pages = case_kv.block_table[b, t // P].astype(np.int64)
    rows = t % P
    k = table[case_kv.k_pool[pages, rows].astype(np.int64)]
    v = table[case_kv.v_pool[pages, rows].astype(np.int64)]
    return k, v                                  # [L, Hkv, D] float64


def _softmax_rows(scores: np.ndarray) -> np.ndarray:
    m = scores.max(axis=-1, keepdims=True)
    e = np.exp(scores - m)
    return e / e.sum(axis=-1, keepdims=True)


def _no_extras(case):
    if any(getattr(case, n, None) is not None
           for n in ("sinks", "k_descale", "v_descale", "alibi_slopes")):
        raise ValueError("the brute-force formulation takes no sinks, per-request descales "
                         "or ALiBi")


def brute_decode(case) -> np.ndarray:
    _no_extras(case)
    bf = _elem_table("bf16")
    kt = _elem_table(case.kv_dtype)
    B, Hq, D = case.batch, case.num_q_heads, case.head_dim
    Dv = getattr(case, "head_dim_v", 0) or D
    G = Hq // case.num_kv_heads
    out = np.zeros((B, Hq, Dv))
    for b in range(B):
        L = int(case.seq_lens[b])
        lo = max(0, L - case.window) if case.window > 0 else 0
        if L - lo <= 0:
            continue
        k, v = _dense_seq(case.kv, b, L, case.kv_dtype, kt)
        k = k[lo:] * case.k_scale
        v = v[lo:, :, :Dv] * case.v_scale      # value: the row's first Dv entries
        for h in range(Hq):
            q = bf[case.q[b, h].astype(np.int64)]
            s = case.scale * (k[:, h // G, :] @ q)
            if case.softcap > 0:
                s = case.softcap * np.tanh(s / case.softcap)
            out[b, h] = _softmax_rows(s[None, :])[0] @ v[:, h // G, :]
    return out


def brute_extend(case) -> np.ndarray:
    _no_extras(case)
    bf = _elem_table("bf16")
    kt = _elem_table(case.kv_dtype)
    Hq, D = case.num_q_heads, case.head_dim
    G = Hq // case.num_kv_heads
    out = np.zeros((case.total_q, Hq, D))
    for b in range(case.batch):
        a, e = int(case.cu_seqlens_q[b]), int(case.cu_seqlens_q[b + 1])
        n, C = e - a, int(case.ctx_lens[b])
        if n == 0:
            continue
        kc, vc = _dense_seq(case.kv, b, C, case.kv_dtype, kt)
        k = np.concatenate([kc * case.k_scale, bf[case.k_new[a:e].astype(np.int64)]])
        v = np.concatenate([vc * case.v_scale, bf[case.v_new[a:e].astype(np.int64)]])
        qpos = C + np.arange(n)[:, None]
        kpos = np.arange(C + n)[None, :]
        keep = kpos <= qpos
        if case.window > 0:
            keep &= (qpos - kpos) < case.window
        for h in range(Hq):
            q = bf[case.q[a:e, h].astype(np.int64)]            # [n, D]
            s = case.scale * (q @ k[:, h // G, :].T)           # [n, C+n]
            if case.softcap > 0:
                s = case.softcap * np.tanh(s / case.softcap)
            s = np.where(keep, s, -np.inf)
            out[a:e, h] = _softmax_rows(s) @ v[:, h // G, :]
    return out
