"""Seeded synthetic inputs for paged GQA attention (decode and extend).

This module draws lengths, page tables and random tensors, encodes them as
bf16 / OCP e4m3fn bits and lays them out in a paged pool.  It holds none of
the attention arithmetic; both the HIP library's tests and the CPU oracle
take their inputs from here.

Conventions
-----------
* K/V pool: ``[num_pages, page_size, num_kv_heads, head_dim]`` (the
  ``[num_blocks, P, Hkv, D]`` view of ``_kv_cache_views`` on the vLLM "b12x"
  backend page).  bf16 pools hold ``uint16`` bits, fp8 pools ``uint8`` bits.
* Token ``t`` of sequence ``b`` sits in page ``block_table[b, t // P]`` at row
  ``t % P``.  Table padding is -1 and every slot that no sequence owns (whole
  spare pages and the tail of a sequence's last page) holds NaN bits, so any
  stray read shows up in the results.
* Random draws use ``numpy.random.default_rng(seed)`` in the order: lengths,
  new-token counts, page permutation, Q, K, V, k/v scales.  Normals are drawn
  in float32 and rounded to bf16 (round-to-nearest-even) by torch on the CPU;
  fp8 values are ``e4m3fn(x / scale)`` rounded the same way.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional, Sequence

import numpy as np
import torch

BF16_NAN_BITS = 0x7FC0
E4M3_NAN_BITS = 0x7F
KV_DTYPES = ("bf16", "fp8_e4m3")


# --------------------------------------------------------------------------
# element encodings
# --------------------------------------------------------------------------
def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 array -> bf16 bit patterns (uint16), round-to-nearest-even."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def e4m3_bits(x: np.ndarray) -> np.ndarray:
    """float32 array -> OCP e4m3fn bit patterns (uint8), round-to-nearest-even."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def bits_to_float(bits: np.ndarray, kv_dtype: str = "bf16") -> np.ndarray:
    """Bit patterns -> float32 (exact for both encodings); used only for tests."""
    t = torch.from_numpy(np.ascontiguousarray(bits))
    if kv_dtype == "bf16":
        return t.view(torch.bfloat16).float().numpy()
    return t.view(torch.float8_e4m3fn).float().numpy()


# --------------------------------------------------------------------------
# paged layout
# --------------------------------------------------------------------------
@dataclasses.dataclass
class PagedKV:
    k_pool: np.ndarray          # [num_pages, P, Hkv, D] uint16|uint8
    v_pool: np.ndarray
    block_table: np.ndarray     # int32 [B, width], padding -1
    page_size: int

    @property
    def num_pages(self) -> int:
        return int(self.k_pool.shape[0])


def deal_pages(lens: Sequence[int], page_size: int, rng: np.random.Generator,
               pool_pages: Optional[int] = None,
               width: Optional[int] = None) -> tuple[np.ndarray, int]:
    """Give each sequence ceil(L/P) distinct physical pages from a seeded
    random permutation of the pool, dealt in sequence order.  The pool has at
    least one page (the C ABI takes no empty pool), also when every length
    is 0."""
    need = [-(-int(L) // page_size) for L in lens]
    total = sum(need)
    num_pages = max(total, 1) if pool_pages is None else int(pool_pages)
    if num_pages < total:
        raise ValueError("pool too small")
    perm = rng.permutation(num_pages).astype(np.int32)
    w = max(need + [1]) if width is None else int(width)
    table = np.full((len(lens), w), -1, dtype=np.int32)
    pos = 0
    for b, n in enumerate(need):
        table[b, :n] = perm[pos:pos + n]
        pos += n
    return table, num_pages


def scatter_tokens(tokens: np.ndarray, lens: Sequence[int], table: np.ndarray,
                   page_size: int, num_pages: int, nan_bits: int) -> np.ndarray:
    """Place logical tokens ``[sum L, Hkv, D]`` into a pool through the table."""
    Hkv, D = tokens.shape[1], tokens.shape[2]
    pool = np.full((num_pages * page_size, Hkv, D), nan_bits, dtype=tokens.dtype)
    off = 0
    for b, L in enumerate(lens):
        L = int(L)
        if L == 0:
            continue
        t = np.arange(L)
        slots = table[b, t // page_size].astype(np.int64) * page_size + t % page_size
        pool[slots] = tokens[off:off + L]
        off += L
    return pool.reshape(num_pages, page_size, Hkv, D)


def page_tokens(k_tok: np.ndarray, v_tok: np.ndarray, lens: Sequence[int],
                page_size: int, rng: np.random.Generator,
                pool_pages: Optional[int] = None) -> PagedKV:
    nan = BF16_NAN_BITS if k_tok.dtype == np.uint16 else E4M3_NAN_BITS
    table, num_pages = deal_pages(lens, page_size, rng, pool_pages)
    k_pool = scatter_tokens(k_tok, lens, table, page_size, num_pages, nan)
    # one array for both when the values are the keys' rows (a latent cache)
    v_pool = (k_pool if v_tok is k_tok else
              scatter_tokens(v_tok, lens, table, page_size, num_pages, nan))
    return PagedKV(k_pool, v_pool, table, page_size)


def _normal(rng: np.random.Generator, shape) -> np.ndarray:
    return rng.standard_normal(size=shape, dtype=np.float32)


def _kv_tokens(rng, n_tok, Hkv, D, kv_dtype):
    """Draw K then V as N(0,1) float32 for n_tok logical tokens."""
    k = _normal(rng, (n_tok, Hkv, D))
    v = _normal(rng, (n_tok, Hkv, D))
    return k, v


def _encode_kv(k, v, kv_dtype, k_scale, v_scale):
    if kv_dtype == "bf16":
        return bf16_bits(k), bf16_bits(v)
    return e4m3_bits(k / np.float32(k_scale)), e4m3_bits(v / np.float32(v_scale))


# --------------------------------------------------------------------------
# decode cases
# --------------------------------------------------------------------------
@dataclasses.dataclass
class DecodeCase:
    name: str
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    kv_dtype: str
    q: np.ndarray               # uint16 [B, Hq, D]
    kv: PagedKV
    seq_lens: np.ndarray        # int32 [B]
    scale: float
    softcap: float = 0.0
    window: int = 0
    k_scale: float = 1.0
    v_scale: float = 1.0
    num_splits: int = 0         # 0 = chosen by the plan
    k_tok: Optional[np.ndarray] = None   # logical tokens [sum L, Hkv, D] (bits)
    v_tok: Optional[np.ndarray] = None
    sinks: Optional[np.ndarray] = None      # float32 [Hq] sink logits (None: off)
    k_descale: Optional[np.ndarray] = None  # float32 [B] per-request descales (None: 1)
    v_descale: Optional[np.ndarray] = None
    alibi_slopes: Optional[np.ndarray] = None   # float32 [Hq] ALiBi slopes (None: off)
    head_dim_v: int = 0         # value head dim (0: head_dim); smaller: the value
                                # is the first head_dim_v entries of the pool row

    @property
    def batch(self) -> int:
        return int(self.seq_lens.shape[0])

    @property
    def page_size(self) -> int:
        return self.kv.page_size

    @property
    def dv(self) -> int:
        return self.head_dim_v or self.head_dim

    @property
    def latent_alias(self) -> bool:
        """One pool holds keys and values (a latent cache)."""
        return self.kv.v_pool is self.kv.k_pool

    @property
    def max_kv_len(self) -> int:
        return int(self.seq_lens.max()) if self.batch else 0

    def attended_tokens(self) -> int:
        L = self.seq_lens.astype(np.int64)
        if self.window > 0:
            L = np.minimum(L, self.window)
        return int(L.sum())

    def kv_bytes(self) -> int:
        """Algorithmic K+V bytes one decode call must read (a latent cache:
        each key row once, its first head_dim_v entries being the value)."""
        elem = 2 if self.kv_dtype == "bf16" else 1
        per_row = self.head_dim + (0 if self.latent_alias else self.dv)
        return self.attended_tokens() * self.num_kv_heads * per_row * elem

    def verify_bytes(self, q_len: int) -> int:
        """Algorithmic bytes of a verify call with q_len query tokens per
        sequence: K/V of keys [max(0, L - q_len + 1 - W), L), Q and out rows,
        table entries, lengths (split partials excluded)."""
        B, Hq, D, P = self.batch, self.num_q_heads, self.head_dim, self.page_size
        L = self.seq_lens.astype(np.int64)
        lo = (np.maximum(L - q_len + 1 - self.window, 0) if self.window > 0
              else np.zeros_like(L))
        elem = 2 if self.kv_dtype == "bf16" else 1
        pages = np.where(L > lo, (L - 1) // P - lo // P + 1, 0)
        kv = int((L - lo).sum()) * self.num_kv_heads * D * 2 * elem
        return int(kv + 2 * B * q_len * Hq * D * 2 + 4 * pages.sum() + 4 * B)

    def algorithmic_bytes(self) -> int:
        """K/V + Q + out + table entries + lengths (split partials excluded)."""
        B, Hq, D, P = self.batch, self.num_q_heads, self.head_dim, self.page_size
        L = self.seq_lens.astype(np.int64)
        lo = np.maximum(L - self.window, 0) if self.window > 0 else np.zeros_like(L)
        pages = np.where(L > lo, (L - 1) // P - lo // P + 1, 0)
        return int(self.kv_bytes() + B * Hq * (D + self.dv) * 2 + 4 * pages.sum() + 4 * B)


def make_decode(name: str, lens: Sequence[int], Hq: int, Hkv: int, D: int,
                page_size: int, seed: int, kv_dtype: str = "bf16",
                softcap: float = 0.0, window: int = 0, num_splits: int = 0,
                pool_pages: Optional[int] = None,
                scale_range: Optional[tuple[float, float]] = None,
                lens_rng: Optional[np.random.Generator] = None) -> DecodeCase:
    """A decode case: lens must already be drawn (from ``lens_rng`` if given)."""
    rng = lens_rng if lens_rng is not None else np.random.default_rng(seed)
    lens = [int(x) for x in lens]
    B = len(lens)
    table, num_pages = deal_pages(lens, page_size, rng, pool_pages)
    q = bf16_bits(_normal(rng, (B, Hq, D)))
    k, v = _kv_tokens(rng, sum(lens), Hkv, D, kv_dtype)
    k_scale = v_scale = 1.0
    if scale_range is not None:
        k_scale = float(rng.uniform(*scale_range))
        v_scale = float(rng.uniform(*scale_range))
    k_tok, v_tok = _encode_kv(k, v, kv_dtype, k_scale, v_scale)
    del k, v
    nan = BF16_NAN_BITS if kv_dtype == "bf16" else E4M3_NAN_BITS
    kv = PagedKV(scatter_tokens(k_tok, lens, table, page_size, num_pages, nan),
                 scatter_tokens(v_tok, lens, table, page_size, num_pages, nan),
                 table, page_size)
    return DecodeCase(name=name, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D,
                      kv_dtype=kv_dtype, q=q, kv=kv,
                      seq_lens=np.asarray(lens, dtype=np.int32),
                      scale=1.0 / math.sqrt(D), softcap=softcap, window=window,
                      k_scale=k_scale, v_scale=v_scale, num_splits=num_splits,
                      k_tok=k_tok, v_tok=v_tok)


def relayout(case: DecodeCase, page_size: int, seed: int,
             pool_pages: Optional[int] = None) -> DecodeCase:
    """The same logical tokens in a new pool: another page size and/or another
    seeded physical permutation."""
    rng = np.random.default_rng(seed)
    kv = page_tokens(case.k_tok, case.v_tok, case.seq_lens, page_size, rng,
                     pool_pages)
    return dataclasses.replace(case, kv=kv, name=f"{case.name}/P{page_size}s{seed}")


def decode_config(n: int, page_size: Optional[int] = None) -> DecodeCase:
    """The decode workloads, numbered as their seeds.

    1  tiny: B 2, 4/1 heads, D 64, P 16, L {37, 100}, 64-page pool, 2 splits
    2  Llama-3-8B-shaped: B 64, 32/8 heads, D 128, P 16, L ~ U{512..4096}
    3  long context: B 4, 32/8, D 128, P 64, L ~ U{32768..131072}, soft-cap 30;
       another page_size re-pages the same logical tokens
    4  fp8 KV: B 256, 64/8, D 128, P 16, e4m3fn K/V with scales ~ U[0.5, 2],
       L lognormal (median 1024, sigma 1, clipped to [16, 8192]), window 4096
    """
    rng = np.random.default_rng(n)
    if n == 1:
        return make_decode("tiny", [37, 100], 4, 1, 64, 16, n, num_splits=2,
                           pool_pages=64, lens_rng=rng)
    if n == 2:
        lens = rng.integers(512, 4096, size=64, endpoint=True)
        return make_decode("llama3-8b", lens, 32, 8, 128, page_size or 16, n,
                           lens_rng=rng)
    if n == 3:
        lens = rng.integers(32768, 131072, size=4, endpoint=True)
        case = make_decode("long-context", lens, 32, 8, 128, 64, n, softcap=30.0,
                           lens_rng=rng)
        if page_size not in (None, 64):
            # the same logical tokens, re-paged (seeded permutation of a new pool)
            case = relayout(case, page_size, seed=100 + n)
        return case
    if n == 4:
        lens = np.clip(np.rint(rng.lognormal(math.log(1024.0), 1.0, size=256)),
                       16, 8192).astype(np.int64)
        return make_decode("fp8-kv", lens, 64, 8, 128, page_size or 16, n,
                           kv_dtype="fp8_e4m3", window=4096,
                           scale_range=(0.5, 2.0), lens_rng=rng)
    raise ValueError(f"no decode workload {n}")


def mha_config(page_size: int = 16) -> DecodeCase:
    """Multi-head decode (G = 1: one query head per kv head) at the
    Llama-3-8B-shaped workload's sizes: B 64, 32/32 heads, D 128, bf16,
    P 16, L ~ U{512..4096}, seed 7."""
    rng = np.random.default_rng(7)
    lens = rng.integers(512, 4096, size=64, endpoint=True)
    return make_decode("mha", lens, 32, 32, 128, page_size, 7, lens_rng=rng)


def make_mla_decode(name: str, lens: Sequence[int], Hq: int, Hkv: int, D: int, Dv: int,
                    page_size: int, seed: int, alias: bool = True, softcap: float = 0.0,
                    window: int = 0, num_splits: int = 0,
                    lens_rng: Optional[np.random.Generator] = None) -> DecodeCase:
    """A decode case over a latent cache: q ``[B, Hq, D]``, key rows of D
    entries whose first Dv entries are the value (alias: one pool for both),
    or (alias False) a separate value pool of the same layout whose entries
    past Dv are NaN bits (never read).  Draw order after the lengths: page
    permutation, Q, latent rows, separate value rows."""
    rng = lens_rng if lens_rng is not None else np.random.default_rng(seed)
    lens = [int(x) for x in lens]
    B = len(lens)
    table, num_pages = deal_pages(lens, page_size, rng)
    q = bf16_bits(_normal(rng, (B, Hq, D)))
    k_tok = bf16_bits(_normal(rng, (sum(lens), Hkv, D)))
    if alias:
        v_tok = k_tok
    else:
        v_tok = bf16_bits(_normal(rng, (sum(lens), Hkv, D)))
        v_tok[:, :, Dv:] = BF16_NAN_BITS
    k_pool = scatter_tokens(k_tok, lens, table, page_size, num_pages, BF16_NAN_BITS)
    v_pool = (k_pool if alias else
              scatter_tokens(v_tok, lens, table, page_size, num_pages, BF16_NAN_BITS))
    return DecodeCase(name=name, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D,
                      kv_dtype="bf16", q=q, kv=PagedKV(k_pool, v_pool, table, page_size),
                      seq_lens=np.asarray(lens, dtype=np.int32),
                      scale=1.0 / math.sqrt(D), softcap=softcap, window=window,
                      num_splits=num_splits, k_tok=k_tok, v_tok=v_tok, head_dim_v=Dv)


def mla_config(num_q_heads: int = 16, batch: int = 128, page_size: int = 64) -> DecodeCase:
    """Latent-cache (MLA) decode shaped like DeepSeek-V3: one kv head of 576
    entries (512 latent + 64 rope), values the first 512, query heads 16 (a
    tensor-parallel shard of 128) or all 128, L ~ U{512..4096}, seed 6."""
    rng = np.random.default_rng(6)
    lens = rng.integers(512, 4096, size=batch, endpoint=True)
    return make_mla_decode(f"mla-h{num_q_heads}", lens, num_q_heads, 1, 576, 512, page_size,
                           6, lens_rng=rng)


# --------------------------------------------------------------------------
# extend cases
# --------------------------------------------------------------------------
@dataclasses.dataclass
class ExtendCase:
    name: str
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    kv_dtype: str
    q: np.ndarray               # uint16 [total_q, Hq, D]
    k_new: np.ndarray           # uint16 [total_q, Hkv, D]
    v_new: np.ndarray
    cu_seqlens_q: np.ndarray    # int32 [B+1]
    ctx_lens: np.ndarray        # int32 [B]
    kv: PagedKV                 # cached context
    scale: float
    softcap: float = 0.0
    window: int = 0
    k_scale: float = 1.0
    v_scale: float = 1.0
    sinks: Optional[np.ndarray] = None      # float32 [Hq] sink logits (None: off)
    k_descale: Optional[np.ndarray] = None  # float32 [B] per-request cache descales
    v_descale: Optional[np.ndarray] = None
    alibi_slopes: Optional[np.ndarray] = None   # float32 [Hq] ALiBi slopes (None: off)

    @property
    def batch(self) -> int:
        return int(self.ctx_lens.shape[0])

    @property
    def total_q(self) -> int:
        return int(self.cu_seqlens_q[-1])

    @property
    def q_lens(self) -> np.ndarray:
        return np.diff(self.cu_seqlens_q)

    @property
    def max_q_len(self) -> int:
        return int(self.q_lens.max()) if self.batch else 0

    @property
    def max_kv_len(self) -> int:
        return int(self.ctx_lens.max()) if self.batch else 0

    def attended_pairs(self) -> int:
        """Unmasked (row token, key) pairs per query head."""
        n = self.q_lens.astype(np.int64)
        C = self.ctx_lens.astype(np.int64)
        if self.window <= 0:
            return int((n * C + n * (n + 1) // 2).sum())
        tot = 0
        for nb, cb in zip(n, C):
            i = np.arange(nb)
            pos = cb + i
            lo = np.maximum(pos - self.window + 1, 0)
            tot += int((pos + 1 - lo).sum())
        return tot

    def flops(self) -> int:
        """Algorithmic flops: 4*D per (row, key, q-head) pair (QK and PV)."""
        return 4 * self.head_dim * self.num_q_heads * self.attended_pairs()


def make_extend(name: str, ctx_lens: Sequence[int], q_lens: Sequence[int],
                Hq: int, Hkv: int, D: int, page_size: int, seed: int,
                kv_dtype: str = "bf16", softcap: float = 0.0, window: int = 0,
                scale_range: Optional[tuple[float, float]] = None,
                rng: Optional[np.random.Generator] = None) -> ExtendCase:
    rng = rng if rng is not None else np.random.default_rng(seed)
    ctx = [int(x) for x in ctx_lens]
    ql = [int(x) for x in q_lens]
    B = len(ctx)
    table, num_pages = deal_pages(ctx, page_size, rng)
    total_q = sum(ql)
    q = bf16_bits(_normal(rng, (total_q, Hq, D)))
    k_ctx, v_ctx = _kv_tokens(rng, sum(ctx), Hkv, D, kv_dtype)
    k_new = bf16_bits(_normal(rng, (total_q, Hkv, D)))
    v_new = bf16_bits(_normal(rng, (total_q, Hkv, D)))
    k_scale = v_scale = 1.0
    if scale_range is not None:
        k_scale = float(rng.uniform(*scale_range))
        v_scale = float(rng.uniform(*scale_range))
    k_tok, v_tok = _encode_kv(k_ctx, v_ctx, kv_dtype, k_scale, v_scale)
    del k_ctx, v_ctx
    nan = BF16_NAN_BITS if kv_dtype == "bf16" else E4M3_NAN_BITS
    kv = PagedKV(scatter_tokens(k_tok, ctx, table, page_size, num_pages, nan),
                 scatter_tokens(v_tok, ctx, table, page_size, num_pages, nan),
                 table, page_size)
    cu = np.zeros(B + 1, dtype=np.int32)
    cu[1:] = np.cumsum(ql)
    return ExtendCase(name=name, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D,
                      kv_dtype=kv_dtype, q=q, k_new=k_new, v_new=v_new,
                      cu_seqlens_q=cu, ctx_lens=np.asarray(ctx, dtype=np.int32),
                      kv=kv, scale=1.0 / math.sqrt(D), softcap=softcap,
                      window=window, k_scale=k_scale, v_scale=v_scale)


def extend_config(n: int = 5) -> ExtendCase:
    """5  prefix-prefill/extend: B 8, 32/8 heads, D 128, bf16, context
    ~ U{1024..8192} paged at P 16, new tokens ~ U{128..1024}, causal."""
    if n != 5:
        raise ValueError(f"no extend workload {n}")
    rng = np.random.default_rng(n)
    ctx = rng.integers(1024, 8192, size=8, endpoint=True)
    ql = rng.integers(128, 1024, size=8, endpoint=True)
    return make_extend("extend", ctx, ql, 32, 8, 128, 16, n, rng=rng)


# --------------------------------------------------------------------------
# device upload (torch is only memory here)
# --------------------------------------------------------------------------
def _dev(a: np.ndarray, device, dtype=None) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.view(dtype)
    return t.to(device)


def kv_torch_dtype(kv_dtype: str) -> torch.dtype:
    return torch.bfloat16 if kv_dtype == "bf16" else torch.float8_e4m3fn


def alibi_slopes(num_heads: int) -> np.ndarray:
    """The ALiBi head slopes: for n heads (n a power of two) the geometric
    sequence 2^(-8/n), 2^(-16/n), ..., 2^(-8); for other n the slopes of the
    next lower power of two m, then every other slope of 2m."""
    def pow2(n):
        return [2.0 ** (-8.0 * (i + 1) / n) for i in range(n)]
    m = 1 << (num_heads.bit_length() - 1)
    s = pow2(m)
    if m < num_heads:
        s += pow2(2 * m)[0::2][: num_heads - m]
    return np.asarray(s, dtype=np.float32)


def with_extras(case, seed: int, sinks: bool = True, descales: bool = False,
                alibi: bool = False, sink_range: tuple[float, float] = (0.0, 8.0),
                descale_range: tuple[float, float] = (0.5, 2.0)):
    """Give a decode or extend case seeded sink logits ~ U(sink_range) per
    query head and/or per-request descales ~ U(descale_range), drawn from
    default_rng(seed) in that order (sinks, k descales, v descales), and/or
    the ALiBi slopes of its query heads."""
    rng = np.random.default_rng(seed)
    if sinks:
        case.sinks = rng.uniform(*sink_range, size=case.num_q_heads).astype(np.float32)
    if descales:
        case.k_descale = rng.uniform(*descale_range, size=case.batch).astype(np.float32)
        case.v_descale = rng.uniform(*descale_range, size=case.batch).astype(np.float32)
    if alibi:
        case.alibi_slopes = alibi_slopes(case.num_q_heads)
    return case


def _extra_tensors(case, device) -> dict:
    out = {}
    for name in ("sinks", "k_descale", "v_descale", "alibi_slopes"):
        a = getattr(case, name, None)
        out[name] = None if a is None else _dev(np.asarray(a, dtype=np.float32), device)
    return out


def decode_tensors(case: DecodeCase, device) -> dict:
    kd = kv_torch_dtype(case.kv_dtype)
    k_pool = _dev(case.kv.k_pool, device, kd)
    return dict(
        q=_dev(case.q, device, torch.bfloat16),
        k_pool=k_pool,
        v_pool=k_pool if case.kv.v_pool is case.kv.k_pool else _dev(case.kv.v_pool, device, kd),
        block_table=_dev(case.kv.block_table, device),
        seq_lens=_dev(case.seq_lens, device),
        **_extra_tensors(case, device),
    )


def extend_tensors(case: ExtendCase, device) -> dict:
    kd = kv_torch_dtype(case.kv_dtype)
    return dict(
        q=_dev(case.q, device, torch.bfloat16),
        k_new=_dev(case.k_new, device, torch.bfloat16),
        v_new=_dev(case.v_new, device, torch.bfloat16),
        cu_seqlens_q=_dev(case.cu_seqlens_q, device),
        ctx_lens=_dev(case.ctx_lens, device),
        k_pool=_dev(case.kv.k_pool, device, kd),
        v_pool=_dev(case.kv.v_pool, device, kd),
        block_table=_dev(case.kv.block_table, device),
        **_extra_tensors(case, device),
    )


def decode_case_from_tokens(name: str, q_bits: np.ndarray, k_tok: np.ndarray,
                            v_tok: np.ndarray, lens: Sequence[int],
                            page_size: int, seed: int, kv_dtype: str = "bf16",
                            pool_pages: Optional[int] = None, **params) -> DecodeCase:
    """A decode case from explicit bits: q ``[B,Hq,D]``, logical tokens
    ``[sum L, Hkv, D]``, paged through a seeded random permutation."""
    rng = np.random.default_rng(seed)
    lens = [int(x) for x in lens]
    kv = page_tokens(k_tok, v_tok, lens, page_size, rng, pool_pages)
    D = q_bits.shape[2]
    params.setdefault("scale", 1.0 / math.sqrt(D))
    return DecodeCase(name=name, num_q_heads=q_bits.shape[1],
                      num_kv_heads=k_tok.shape[1], head_dim=D, kv_dtype=kv_dtype,
                      q=q_bits, kv=kv, seq_lens=np.asarray(lens, dtype=np.int32),
                      k_tok=k_tok, v_tok=v_tok, **params)
