"""Dense references for pinning the oracle: torch's scaled_dot_product_attention
in float64 on the CPU, fed with keys/values materialised through the block
table by NumPy indexing.  (Test-side code; shares nothing with the oracle.)"""
import numpy as np
import torch
import torch.nn.functional as F

from paged_gqa_attention_02_amd.inputs import bits_to_float


def dense_tokens(kv, b, L, kv_dtype):
    """Keys/values of sequence b, positions [0, L), as float64 [L, Hkv, D]."""
    P = kv.page_size
    t = np.arange(L)
    pages = kv.block_table[b, t // P].astype(np.int64)
    k = bits_to_float(kv.k_pool[pages, t % P], kv_dtype).astype(np.float64)
    v = bits_to_float(kv.v_pool[pages, t % P], kv_dtype).astype(np.float64)
    return k, v


def _sdpa(q, k, v, scale, mask=None, sinks=None, bias=None):
    """q [H, n, D], k/v [H, m, D] float64 -> [H, n, D].  `mask` is a boolean
    keep-mask [n, m]; `bias` [H, n, m] is added to the scaled scores (as
    torch's float attn_mask).  `sinks` [H] adds, per head, one more key whose
    value row is zero and whose score is the sink logit: a zero key (score 0)
    with the sink as an additive mask term."""
    if sinks is not None or bias is not None:
        H, n, D = q.shape
        m = k.shape[1]
        extra = 1 if sinks is not None else 0
        if extra:
            k = np.concatenate([k, np.zeros((H, 1, D))], axis=1)
            v = np.concatenate([v, np.zeros((H, 1, D))], axis=1)
        fm = np.zeros((H, n, m + extra))
        if bias is not None:
            fm[:, :, :m] = bias
        if mask is not None:
            fm[:, :, :m] = np.where(mask.numpy()[None], fm[:, :, :m], -np.inf)
        if extra:
            fm[:, :, m] = np.asarray(sinks, dtype=np.float64)[:, None]
        mask = torch.from_numpy(fm)
    return F.scaled_dot_product_attention(
        torch.from_numpy(q)[None], torch.from_numpy(k)[None],
        torch.from_numpy(v)[None], attn_mask=mask, scale=scale)[0].numpy()


def _alibi(case, qpos, kpos):
    """ALiBi biases slope[h] * (key position - query position), [H, n, m]
    (None without slopes)."""
    if getattr(case, "alibi_slopes", None) is None:
        return None
    sl = np.asarray(case.alibi_slopes, dtype=np.float64)[:, None, None]
    return sl * (kpos - qpos).astype(np.float64)[None]


def _scales(case, b):
    """Cache scales of sequence b: per-tensor times the per-request descale."""
    ks = case.k_scale * (1.0 if case.k_descale is None else float(case.k_descale[b]))
    vs = case.v_scale * (1.0 if case.v_descale is None else float(case.v_descale[b]))
    return ks, vs


def sdpa_decode(case):
    """Decode without soft-cap through the library routine (value head dim
    Dv = case.dv: torch's routine takes a value width other than the key's)."""
    assert case.softcap == 0
    B, Hq, D = case.batch, case.num_q_heads, case.head_dim
    Dv = getattr(case, "dv", D)
    G = Hq // case.num_kv_heads
    out = np.zeros((B, Hq, Dv))
    for b in range(B):
        L = int(case.seq_lens[b])
        lo = max(0, L - case.window) if case.window > 0 else 0
        if L == 0:
            continue
        k, v = dense_tokens(case.kv, b, L, case.kv_dtype)
        v = v[:, :, :Dv]                  # the value: the row's first Dv entries
        ks, vs = _scales(case, b)
        k = np.repeat(k[lo:] * ks, G, axis=1).transpose(1, 0, 2)
        v = np.repeat(v[lo:] * vs, G, axis=1).transpose(1, 0, 2)
        q = bits_to_float(case.q[b], "bf16").astype(np.float64)[:, None, :]
        out[b] = _sdpa(q, np.ascontiguousarray(k), np.ascontiguousarray(v),
                       case.scale, sinks=case.sinks,
                       bias=_alibi(case, np.array([[L - 1]]), np.arange(lo, L)[None, :]))[:, 0, :]
    return out


def sdpa_extend(case):
    """Extend without soft-cap: SDPA with an explicit keep-mask
    (all cached keys, causal among new keys, optional window)."""
    assert case.softcap == 0
    Hq, D = case.num_q_heads, case.head_dim
    G = Hq // case.num_kv_heads
    out = np.zeros((case.total_q, Hq, D))
    for b in range(case.batch):
        a, e = int(case.cu_seqlens_q[b]), int(case.cu_seqlens_q[b + 1])
        n, C = e - a, int(case.ctx_lens[b])
        if n == 0:
            continue
        kc, vc = dense_tokens(case.kv, b, C, case.kv_dtype)
        kn = bits_to_float(case.k_new[a:e], "bf16").astype(np.float64)
        vn = bits_to_float(case.v_new[a:e], "bf16").astype(np.float64)
        ks, vs = _scales(case, b)
        k = np.concatenate([kc * ks, kn])
        v = np.concatenate([vc * vs, vn])
        k = np.ascontiguousarray(np.repeat(k, G, axis=1).transpose(1, 0, 2))
        v = np.ascontiguousarray(np.repeat(v, G, axis=1).transpose(1, 0, 2))
        qpos = C + np.arange(n)[:, None]
        kpos = np.arange(C + n)[None, :]
        keep = kpos <= qpos
        if case.window > 0:
            keep &= (qpos - kpos) < case.window
        q = bits_to_float(case.q[a:e], "bf16").astype(np.float64).transpose(1, 0, 2)
        out[a:e] = _sdpa(np.ascontiguousarray(q), k, v, case.scale,
                         torch.from_numpy(keep), sinks=case.sinks,
                         bias=_alibi(case, qpos, kpos)).transpose(1, 0, 2)
    return out


def sdpa_verify(case, q_bits):
    """Verify without soft-cap: the last q_len cached tokens of every sequence
    are the query tokens; SDPA with a causal (and window) keep-mask."""
    assert case.softcap == 0
    B, ql, Hq, D = q_bits.shape
    G = Hq // case.num_kv_heads
    out = np.zeros((B, ql, Hq, D))
    for b in range(B):
        L = int(case.seq_lens[b])
        k, v = dense_tokens(case.kv, b, L, case.kv_dtype)
        ks, vs = _scales(case, b)
        k = np.ascontiguousarray(np.repeat(k * ks, G, axis=1).transpose(1, 0, 2))
        v = np.ascontiguousarray(np.repeat(v * vs, G, axis=1).transpose(1, 0, 2))
        qpos = L - ql + np.arange(ql)[:, None]
        kpos = np.arange(L)[None, :]
        keep = kpos <= qpos
        if case.window > 0:
            keep &= (qpos - kpos) < case.window
        q = bits_to_float(q_bits[b], "bf16").astype(np.float64).transpose(1, 0, 2)
        out[b] = _sdpa(np.ascontiguousarray(q), k, v, case.scale,
                       torch.from_numpy(keep), sinks=case.sinks,
                       bias=_alibi(case, qpos, kpos)).transpose(1, 0, 2)
    return out
