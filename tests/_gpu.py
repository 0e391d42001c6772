"""GPU-side helpers for the parity tests: run the HIP library on a seeded case
(everything through the C ABI) and compare with the oracle."""
import numpy as np
import torch

import paged_gqa_attention_02_amd as pa
from paged_gqa_attention_02_amd import inputs as I

DEV = "cuda:0"
ATOL = RTOL = 1e-2      # |err| <= 1e-2 + 1e-2*|ref| for bf16/fp8-KV outputs


def extras(t: dict) -> dict:
    """The optional sink / descale tensors of a case's device tensors."""
    return {k: t.get(k) for k in ("sinks", "k_descale", "v_descale", "alibi_slopes")}


def run_decode(case, num_splits=None, tensors=None, pool_view=None):
    t = tensors or I.decode_tensors(case, DEV)
    kp, vp = t["k_pool"], t["v_pool"]
    if pool_view is not None:
        kp, vp = pool_view(kp), pool_view(vp)
    ns = case.num_splits if num_splits is None else num_splits
    pl = pa.decode_plan(t["q"], kp, t["block_table"], case.max_kv_len,
                        window=case.window, num_splits=ns,
                        head_dim_v=getattr(case, "head_dim_v", 0))
    out = pa.decode(pl, t["q"], kp, vp, t["block_table"], t["seq_lens"], case.scale,
                    softcap=case.softcap, window=case.window, k_scale=case.k_scale,
                    v_scale=case.v_scale, **extras(t))
    torch.cuda.synchronize()
    return out, pl


def run_verify(case, q_bits, num_splits=None, tensors=None):
    """paged_attn_verify on a decode case's cache with query rows q_bits
    (bf16 bits [B, q_len, Hq, D])."""
    t = tensors or I.decode_tensors(case, DEV)
    q = I._dev(q_bits, DEV, torch.bfloat16)
    ns = case.num_splits if num_splits is None else num_splits
    pl = pa.verify_plan(q, t["k_pool"], t["block_table"], case.max_kv_len,
                        window=case.window, num_splits=ns)
    out = pa.verify(pl, q, t["k_pool"], t["v_pool"], t["block_table"], t["seq_lens"],
                    case.scale, softcap=case.softcap, window=case.window,
                    k_scale=case.k_scale, v_scale=case.v_scale, **extras(t))
    torch.cuda.synchronize()
    return out, pl


def run_extend(case, tensors=None, num_splits=0):
    t = tensors or I.extend_tensors(case, DEV)
    pl = pa.extend_plan(t["q"], t["k_pool"], t["block_table"], case.batch,
                        case.max_kv_len, case.max_q_len, window=case.window,
                        num_splits=num_splits)
    out = pa.extend(pl, t["q"], t["k_new"], t["v_new"], t["cu_seqlens_q"], t["ctx_lens"],
                    t["k_pool"], t["v_pool"], t["block_table"], case.scale,
                    softcap=case.softcap, window=case.window, k_scale=case.k_scale,
                    v_scale=case.v_scale, **extras(t))
    torch.cuda.synchronize()
    return out, pl


def to_f64(out: torch.Tensor) -> np.ndarray:
    return out.float().cpu().numpy().astype(np.float64)


def assert_close(got: np.ndarray, ref: np.ndarray, what: str = ""):
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = np.abs(got - ref)
    bad = err > ATOL + RTOL * np.abs(ref)
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError(f"{what}: {bad.sum()} of {bad.size} elements out of tolerance; "
                             f"max err {err.max():.3e}; first {idx.tolist()} "
                             f"got {got[tuple(idx[0])]:.6f} ref {ref[tuple(idx[0])]:.6f}")
