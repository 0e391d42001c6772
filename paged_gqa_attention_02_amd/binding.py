"""Python binding of ``libpaged_attn.so`` (the C ABI in include/paged_attn.h).

Argument marshalling only: tensors become device pointers, element strides and
the current HIP stream; every step of the computation runs in the library's
kernels.  torch provides device memory and streams.  The library must be
built (``python -m paged_gqa_attention_02_amd.build``); nothing here falls back
to another implementation.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import torch

# PAGED_ATTN_LIB names another build of the same sources (the host-sanitized
# build the CPU tests load); by default the in-tree library.
LIB_PATH = os.environ.get("PAGED_ATTN_LIB") or os.path.join(
    os.path.dirname(os.path.abspath(__file__)), "libpaged_attn.so")

PA_MODE_DECODE, PA_MODE_EXTEND, PA_MODE_VERIFY = 0, 1, 2
NOALLOC_SCRATCH_BYTES = 48 << 20   # PAGED_ATTN_NOALLOC_SCRATCH_BYTES
ABI_VERSION = 4          # PAGED_ATTN_ABI_VERSION these structures mirror
PA_KV = {"bf16": 0, "fp8_e4m3": 1}


class PaExtras(ctypes.Structure):
    _fields_ = [("sinks", ctypes.c_void_p), ("k_descale", ctypes.c_void_p),
                ("v_descale", ctypes.c_void_p), ("alibi_slopes", ctypes.c_void_p),
                ("num_descales", ctypes.c_int32), ("reserved", ctypes.c_int32)]


class PaProblem(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "mode", "num_seqs", "num_q_heads", "num_kv_heads", "head_dim", "page_size",
        "kv_dtype", "window", "max_pages_per_seq", "max_kv_len", "total_q",
        "max_q_len", "num_splits", "head_dim_v")]


class PaPlan(ctypes.Structure):
    _fields_ = [("prob", PaProblem), ("num_splits", ctypes.c_int32),
                ("tokens_per_split", ctypes.c_int32), ("waves_per_block", ctypes.c_int32),
                ("num_cus", ctypes.c_int32), ("workspace_bytes", ctypes.c_uint64),
                ("reserved", ctypes.c_int32 * 8)]


class PagedAttnError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn}: {status_str(status)} (status {status})")


_LIB = None


def lib():
    """Load the library once, after torch, so both share one HIP runtime."""
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run "
                           "`python -m paged_gqa_attention_02_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    p, i32, i64, u64, f32 = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64,
                             ctypes.c_uint64, ctypes.c_float)
    PP = ctypes.POINTER(PaPlan)
    L.paged_attn_plan.argtypes = [ctypes.POINTER(PaProblem), ctypes.c_int, PP]
    L.paged_attn_plan.restype = ctypes.c_int
    PX = ctypes.POINTER(PaExtras)
    L.paged_attn_decode.argtypes = [PP, p, i64, p, p, i64, i64, i64, i64, p, i64, p,
                                    i32, f32, f32, i32, f32, f32, p, i64, p, u64, PX, p]
    L.paged_attn_decode.restype = ctypes.c_int
    for fn in ("paged_attn_decode_split", "paged_attn_decode_merge", "paged_attn_verify"):
        getattr(L, fn).argtypes = L.paged_attn_decode.argtypes
        getattr(L, fn).restype = ctypes.c_int
    L.paged_attn_decode_noalloc.argtypes = [PP, p, i64, p, p, i64, i64, i64, i64, p, i64, p,
                                            i32, f32, f32, i32, f32, f32, p, i64, PX, p]
    L.paged_attn_decode_noalloc.restype = ctypes.c_int
    L.paged_attn_extend.argtypes = [PP, p, p, p, p, p, p, p, i64, i64, i64, i64, p, i64,
                                    i32, f32, f32, i32, f32, f32, p, p, u64, PX, p]
    L.paged_attn_extend.restype = ctypes.c_int
    L.paged_attn_gather.argtypes = [PP, p, p, i64, i64, i64, i64, p, i64, p, p, p, p]
    L.paged_attn_cache_append.argtypes = [p, p, i64, i64, ctypes.c_int32, ctypes.c_int32, p, p,
                                          i64, i64, i64, i64, ctypes.c_int32, ctypes.c_int32, p,
                                          ctypes.c_float, ctypes.c_float, p]
    L.paged_attn_cache_append.restype = ctypes.c_int
    L.paged_attn_gather.restype = ctypes.c_int
    L.paged_attn_check_inputs.argtypes = [PP, p, p, i64, i64, p, ctypes.POINTER(i32),
                                          ctypes.POINTER(i64)]
    L.paged_attn_check_inputs.restype = ctypes.c_int
    L.paged_attn_status_str.argtypes = [ctypes.c_int]
    L.paged_attn_status_str.restype = ctypes.c_char_p
    L.paged_attn_plan_describe.argtypes = [PP, ctypes.c_char_p, ctypes.c_int]
    L.paged_attn_plan_describe.restype = ctypes.c_int
    L.paged_attn_abi_version.argtypes = []
    L.paged_attn_abi_version.restype = ctypes.c_int
    L.paged_attn_hip_runtime_path.argtypes = []
    L.paged_attn_hip_runtime_path.restype = ctypes.c_char_p
    if L.paged_attn_abi_version() != ABI_VERSION:
        raise RuntimeError(f"{LIB_PATH} has ABI version {L.paged_attn_abi_version()}, this "
                           f"binding expects {ABI_VERSION}; rebuild the library")
    rt = L.paged_attn_hip_runtime_path().decode()
    torch_rt = os.path.join(os.path.dirname(torch.__file__), "lib", "libamdhip64.so")
    if os.path.exists(torch_rt) and os.path.realpath(rt) != os.path.realpath(torch_rt):
        raise RuntimeError(f"libpaged_attn.so resolved the HIP runtime {rt}, but torch "
                           f"uses {torch_rt}; import torch before this library")
    _LIB = L
    return L


def status_str(status: int) -> str:
    return lib().paged_attn_status_str(status).decode()


def _check(fn: str, status: int):
    if status != 0:
        raise PagedAttnError(fn, status)


@dataclass
class Plan:
    c: PaPlan

    @property
    def num_splits(self) -> int:
        return self.c.num_splits

    @property
    def tokens_per_split(self) -> int:
        return self.c.tokens_per_split

    @property
    def workspace_bytes(self) -> int:
        return self.c.workspace_bytes

    @property
    def problem(self) -> PaProblem:
        return self.c.prob

    def describe(self) -> str:
        buf = ctypes.create_string_buffer(512)
        lib().paged_attn_plan_describe(ctypes.byref(self.c), buf, 512)
        return buf.value.decode()


def plan(mode: int, num_seqs: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
         page_size: int, kv_dtype: str = "bf16", window: int = 0,
         max_pages_per_seq: int = 0, max_kv_len: int = 0, total_q: int = 0,
         max_q_len: int = 0, num_splits: int = 0, device: Optional[int] = None,
         head_dim_v: int = 0) -> Plan:
    """paged_attn_plan.  device=None plans for the current torch device when one
    exists, else for an MI355X without touching a device.  head_dim_v <
    head_dim: a latent cache (values are the first head_dim_v entries)."""
    prob = PaProblem(mode, num_seqs, num_q_heads, num_kv_heads, head_dim, page_size,
                     PA_KV[kv_dtype], window, max_pages_per_seq, max_kv_len, total_q,
                     max_q_len, num_splits, head_dim_v)
    if device is None:
        device = torch.cuda.current_device() if torch.cuda.is_available() else -1
    out = PaPlan()
    _check("paged_attn_plan", lib().paged_attn_plan(ctypes.byref(prob), device, ctypes.byref(out)))
    return Plan(out)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _extras(sinks, k_descale, v_descale, alibi_slopes=None, num_q_heads=0):
    """pa_extras for optional fp32 device tensors (None when all are None):
    sinks [Hq]; k_descale/v_descale with 1 or >= B entries; alibi_slopes [Hq]."""
    if sinks is None and k_descale is None and v_descale is None and alibi_slopes is None:
        return None
    for name, t in (("sinks", sinks), ("k_descale", k_descale), ("v_descale", v_descale),
                    ("alibi_slopes", alibi_slopes)):
        if t is not None and (t.dtype != torch.float32 or t.dim() != 1 or
                              not t.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous fp32 vector")
    for name, t in (("sinks", sinks), ("alibi_slopes", alibi_slopes)):
        if t is not None and t.numel() < num_q_heads:
            raise ValueError(f"{name} must hold one value per query head ({num_q_heads})")
    n = [t.numel() for t in (k_descale, v_descale) if t is not None]
    if len(n) == 2 and n[0] != n[1]:
        raise ValueError("k_descale and v_descale must have the same length")
    ptr = lambda t: None if t is None else t.data_ptr()
    ex = PaExtras(ptr(sinks), ptr(k_descale), ptr(v_descale), ptr(alibi_slopes),
                  n[0] if n else 0, 0)
    return ctypes.byref(ex)


def _stream(stream) -> ctypes.c_void_p:
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _kv_dtype_name(t: torch.Tensor) -> str:
    if t.dtype == torch.bfloat16:
        return "bf16"
    if t.dtype in (torch.float8_e4m3fn, torch.uint8):
        return "fp8_e4m3"
    raise TypeError(f"unsupported K/V cache dtype {t.dtype}")


def _pool_strides(k_pool: torch.Tensor, v_pool: torch.Tensor):
    if k_pool.dim() != 4 or k_pool.shape != v_pool.shape or k_pool.stride() != v_pool.stride():
        raise ValueError("k_pool/v_pool must be 4-D [pages, page_size, kv_heads, head_dim] "
                         "views with equal shapes and strides")
    if k_pool.stride(3) != 1:
        raise ValueError("head_dim must be contiguous")
    return k_pool.stride(0), k_pool.stride(1), k_pool.stride(2)


_KV_NAME = {v: k for k, v in PA_KV.items()}


def _same_device(ref: torch.Tensor, **tensors):
    for name, t in tensors.items():
        if t is not None and t.device != ref.device:
            raise ValueError(f"{name} is on {t.device}, expected {ref.device}")


def _check_cache(pl: Plan, k_pool: torch.Tensor, block_table: torch.Tensor,
                 lens: torch.Tensor, lens_name: str):
    """The pools, block table and per-sequence lengths against the plan: the
    kernels take every size from the plan, so a tensor smaller than it
    describes would be read past its end."""
    pr = pl.problem
    if _kv_dtype_name(k_pool) != _KV_NAME[pr.kv_dtype]:
        raise TypeError(f"k_pool/v_pool hold {k_pool.dtype}, the plan was made for "
                        f"{_KV_NAME[pr.kv_dtype]}")
    if k_pool.dim() != 4 or k_pool.shape[1] != pr.page_size or \
            k_pool.shape[2] != pr.num_kv_heads or k_pool.shape[3] != pr.head_dim:
        raise ValueError(f"k_pool/v_pool must be [pages, {pr.page_size}, {pr.num_kv_heads}, "
                         f"{pr.head_dim}] as planned, got {tuple(k_pool.shape)}")
    if block_table.dim() != 2 or block_table.shape[0] < pr.num_seqs or \
            block_table.shape[1] < pr.max_pages_per_seq:
        raise ValueError(f"block_table must be [>= {pr.num_seqs}, >= {pr.max_pages_per_seq}] "
                         f"as planned, got {tuple(block_table.shape)}")
    if lens.dim() != 1 or lens.numel() < pr.num_seqs or not lens.is_contiguous():
        raise ValueError(f"{lens_name} must be a contiguous int32 vector of >= {pr.num_seqs} "
                         f"entries")


_INPUT_CHECKS = False
_BAD_ARRAY = {1: "lens", 2: "block_table", 3: "cu_seqlens_q"}


def set_input_checks(on: bool) -> bool:
    """Make every compute call check the device-content contract on the host
    first (check_inputs; it copies the metadata to the host and so
    synchronises).  Returns the previous setting."""
    global _INPUT_CHECKS
    prev, _INPUT_CHECKS = _INPUT_CHECKS, bool(on)
    return prev


def check_inputs(pl: Plan, block_table: torch.Tensor, lens: torch.Tensor, num_pages: int,
                 cu_seqlens_q: Optional[torch.Tensor] = None) -> None:
    """paged_attn_check_inputs on host copies: lengths within the plan's
    bound, every page id a call reads in [0, num_pages), and (extend) the
    query offsets cu_seqlens_q.  Raises ValueError naming the bad element."""
    bt = block_table.detach().to("cpu", torch.int32).contiguous()
    ln = lens.detach().to("cpu", torch.int32).contiguous()
    cu = None if cu_seqlens_q is None else cu_seqlens_q.detach().to("cpu", torch.int32).contiguous()
    arr, idx = ctypes.c_int32(0), ctypes.c_int64(-1)
    st = lib().paged_attn_check_inputs(
        ctypes.byref(pl.c), _ptr(ln), _ptr(bt), bt.stride(0) if bt.dim() == 2 else 0,
        int(num_pages), _ptr(cu), ctypes.byref(arr), ctypes.byref(idx))
    if st == 2 and arr.value:
        name = _BAD_ARRAY[arr.value]
        i = idx.value
        if name == "block_table":
            where = f"[{i // bt.stride(0)}, {i % bt.stride(0)}] = {int(bt.view(-1)[i])}"
        else:
            where = f"[{i}] = {int((ln if name == 'lens' else cu)[i])}"
        raise ValueError(f"device-content contract broken: {name}{where} "
                         f"({pl.describe()}, num_pages={num_pages})")
    _check("paged_attn_check_inputs", st)


def workspace_for(pl: Plan, device) -> Optional[torch.Tensor]:
    """Device scratch of plan.workspace_bytes bytes (None when none is needed)."""
    if pl.workspace_bytes == 0:
        return None
    return torch.empty(pl.workspace_bytes, dtype=torch.uint8, device=device)


def _workspace(pl: Plan, workspace, device):
    if pl.workspace_bytes == 0 or workspace is not None:
        return workspace
    return workspace_for(pl, device)


def decode_plan(q: torch.Tensor, k_pool: torch.Tensor, block_table: torch.Tensor,
                max_kv_len: int, window: int = 0, num_splits: int = 0,
                head_dim_v: int = 0) -> Plan:
    """Plan a decode call for tensors shaped like these (head_dim_v: the value
    width of a latent cache, 0 = the key width)."""
    B, Hq, D = q.shape
    return plan(PA_MODE_DECODE, B, Hq, k_pool.shape[2], D, k_pool.shape[1],
                _kv_dtype_name(k_pool), window, block_table.shape[1], max_kv_len,
                num_splits=num_splits, device=q.device.index, head_dim_v=head_dim_v)


def decode(pl: Plan, q: torch.Tensor, k_pool: torch.Tensor, v_pool: torch.Tensor,
           block_table: torch.Tensor, seq_lens: torch.Tensor, scale: float,
           softcap: float = 0.0, window: int = 0, k_scale: float = 1.0,
           v_scale: float = 1.0, out: Optional[torch.Tensor] = None,
           workspace: Optional[torch.Tensor] = None, stream=None, sinks=None,
           k_descale=None, v_descale=None, alibi_slopes=None) -> torch.Tensor:
    """paged_attn_decode: q bf16 [B, Hq, D] -> out bf16 [B, Hq, D] (a plan
    with head_dim_v = Dv < D: out [B, Hq, Dv], values the first Dv entries of
    v_pool's rows; pass v_pool = k_pool for a latent cache).
    A workspace passed in needs plan.workspace_bytes bytes.  sinks: fp32 [Hq]
    sink logits; k_descale/v_descale: fp32 per-request descales (1 or >= B)."""
    return _decode("paged_attn_decode", pl, q, k_pool, v_pool, block_table, seq_lens, scale,
                   softcap, window, k_scale, v_scale, out, workspace, stream,
                   sinks, k_descale, v_descale, alibi_slopes)


def decode_split(pl: Plan, q, k_pool, v_pool, block_table, seq_lens, scale, softcap=0.0,
                 window=0, k_scale=1.0, v_scale=1.0, out=None, workspace=None, stream=None,
                 sinks=None, k_descale=None, v_descale=None, alibi_slopes=None):
    """paged_attn_decode_split: the split pass alone (writes the segments one
    block covers whole to `out`, the others to the workspace)."""
    return _decode("paged_attn_decode_split", pl, q, k_pool, v_pool, block_table, seq_lens,
                   scale, softcap, window, k_scale, v_scale, out, workspace, stream,
                   sinks, k_descale, v_descale, alibi_slopes)


def decode_merge(pl: Plan, q, k_pool, v_pool, block_table, seq_lens, scale, softcap=0.0,
                 window=0, k_scale=1.0, v_scale=1.0, out=None, workspace=None, stream=None,
                 sinks=None, k_descale=None, v_descale=None, alibi_slopes=None):
    """paged_attn_decode_merge: the merge pass alone, over the workspace the
    split pass left."""
    return _decode("paged_attn_decode_merge", pl, q, k_pool, v_pool, block_table, seq_lens,
                   scale, softcap, window, k_scale, v_scale, out, workspace, stream,
                   sinks, k_descale, v_descale, alibi_slopes)


def decode_noalloc(pl: Plan, q, k_pool, v_pool, block_table, seq_lens, scale, softcap=0.0,
                   window=0, k_scale=1.0, v_scale=1.0, out=None, stream=None, sinks=None,
                   k_descale=None, v_descale=None, alibi_slopes=None):
    """paged_attn_decode_noalloc: decode with the library's fixed scratch array
    instead of a workspace (no device allocation in the library; pass `out`
    to allocate nothing here either).  Plans needing more than
    NOALLOC_SCRATCH_BYTES are rejected; calls overlapping on one GPU race."""
    return _decode("paged_attn_decode_noalloc", pl, q, k_pool, v_pool, block_table, seq_lens,
                   scale, softcap, window, k_scale, v_scale, out, None, stream,
                   sinks, k_descale, v_descale, alibi_slopes)


def verify_plan(q: torch.Tensor, k_pool: torch.Tensor, block_table: torch.Tensor,
                max_kv_len: int, window: int = 0, num_splits: int = 0) -> Plan:
    """Plan a verify call for q shaped [B, q_len, Hq, D]."""
    B, q_len, Hq, D = q.shape
    return plan(PA_MODE_VERIFY, B, Hq, k_pool.shape[2], D, k_pool.shape[1],
                _kv_dtype_name(k_pool), window, block_table.shape[1], max_kv_len,
                max_q_len=q_len, num_splits=num_splits, device=q.device.index)


def verify(pl: Plan, q: torch.Tensor, k_pool: torch.Tensor, v_pool: torch.Tensor,
           block_table: torch.Tensor, seq_lens: torch.Tensor, scale: float,
           softcap: float = 0.0, window: int = 0, k_scale: float = 1.0,
           v_scale: float = 1.0, out: Optional[torch.Tensor] = None,
           workspace: Optional[torch.Tensor] = None, stream=None, sinks=None,
           k_descale=None, v_descale=None, alibi_slopes=None) -> torch.Tensor:
    """paged_attn_verify: q bf16 [B, q_len, Hq, D] -> out bf16 [B, q_len, Hq, D];
    seq_lens count the q_len query tokens, which are already in the cache."""
    return _decode("paged_attn_verify", pl, q, k_pool, v_pool, block_table, seq_lens, scale,
                   softcap, window, k_scale, v_scale, out, workspace, stream,
                   sinks, k_descale, v_descale, alibi_slopes)


def _rows_contiguous(t: torch.Tensor) -> bool:
    """All dims after the first are dense (the sequence stride is free)."""
    if t.numel() == 0:
        return True
    step = 1
    for d in range(t.dim() - 1, 0, -1):
        if t.shape[d] > 1 and t.stride(d) != step:
            return False
        step *= t.shape[d]
    return True


def _decode(fn, pl, q, k_pool, v_pool, block_table, seq_lens, scale, softcap, window,
            k_scale, v_scale, out, workspace, stream, sinks=None, k_descale=None,
            v_descale=None, alibi_slopes=None):
    if fn not in ("paged_attn_decode", "paged_attn_verify", "paged_attn_decode_noalloc") and (
            out is None or (workspace is None and pl.workspace_bytes > 0)):
        raise ValueError(f"{fn}: the passes share `out` and the workspace; pass both")
    dims = 4 if fn == "paged_attn_verify" else 3
    shape = "[B, q_len, Hq, D]" if dims == 4 else "[B, Hq, D]"
    if q.dtype != torch.bfloat16 or q.dim() != dims or not _rows_contiguous(q):
        raise ValueError(f"q must be bf16 {shape}, dense after the sequence dimension")
    if block_table.dtype != torch.int32 or seq_lens.dtype != torch.int32:
        raise TypeError("block_table and seq_lens must be int32")
    if block_table.stride(1) != 1:
        raise ValueError("block_table rows must be contiguous")
    pr = pl.problem
    want = (pr.num_seqs,) + ((pr.max_q_len,) if dims == 4 else ()) + (pr.num_q_heads,
                                                                       pr.head_dim)
    if tuple(q.shape) != want:
        raise ValueError(f"q must be {want} as planned, got {tuple(q.shape)}")
    _check_cache(pl, k_pool, block_table, seq_lens, "seq_lens")
    _same_device(q, k_pool=k_pool, v_pool=v_pool, block_table=block_table,
                 seq_lens=seq_lens, out=out, workspace=workspace, sinks=sinks,
                 k_descale=k_descale, v_descale=v_descale, alibi_slopes=alibi_slopes)
    if _INPUT_CHECKS:
        check_inputs(pl, block_table, seq_lens, k_pool.shape[0])
    dv = pr.head_dim_v or q.shape[-1]
    oshape = q.shape[:-1] + (dv,)
    if out is None:
        out = torch.empty(oshape, dtype=torch.bfloat16, device=q.device)
    if out.dtype != torch.bfloat16 or out.shape != oshape or not _rows_contiguous(out):
        raise ValueError(f"out must be bf16 {shape} like q (last dim {dv}), dense after the "
                         "sequence dimension")
    sp, st, sh = _pool_strides(k_pool, v_pool)
    if fn == "paged_attn_decode_noalloc":
        _check(fn, lib().paged_attn_decode_noalloc(
            ctypes.byref(pl.c), _ptr(q), q.stride(0), _ptr(k_pool), _ptr(v_pool), sp, st, sh,
            k_pool.shape[0], _ptr(block_table), block_table.stride(0), _ptr(seq_lens),
            k_pool.shape[1], float(scale), float(softcap), int(window), float(k_scale),
            float(v_scale), _ptr(out), out.stride(0),
            _extras(sinks, k_descale, v_descale, alibi_slopes, pr.num_q_heads),
            _stream(stream)))
        return out
    workspace = _workspace(pl, workspace, q.device)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(fn, getattr(lib(), fn)(
        ctypes.byref(pl.c), _ptr(q), q.stride(0), _ptr(k_pool), _ptr(v_pool), sp, st, sh,
        k_pool.shape[0], _ptr(block_table), block_table.stride(0), _ptr(seq_lens),
        k_pool.shape[1], float(scale), float(softcap), int(window), float(k_scale),
        float(v_scale), _ptr(out), out.stride(0), _ptr(workspace), wbytes,
        _extras(sinks, k_descale, v_descale, alibi_slopes, pr.num_q_heads), _stream(stream)))
    return out


def extend_plan(q: torch.Tensor, k_pool: torch.Tensor, block_table: torch.Tensor,
                num_seqs: int, max_kv_len: int, max_q_len: int, window: int = 0,
                num_splits: int = 0) -> Plan:
    """Plan an extend call; num_splits > 0 forces the persistent block count."""
    T, Hq, D = q.shape
    return plan(PA_MODE_EXTEND, num_seqs, Hq, k_pool.shape[2], D, k_pool.shape[1],
                _kv_dtype_name(k_pool), window, block_table.shape[1], max_kv_len,
                total_q=T, max_q_len=max_q_len, num_splits=num_splits, device=q.device.index)


def extend(pl: Plan, q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor,
           cu_seqlens_q: torch.Tensor, ctx_lens: torch.Tensor, k_pool: torch.Tensor,
           v_pool: torch.Tensor, block_table: torch.Tensor, scale: float,
           softcap: float = 0.0, window: int = 0, k_scale: float = 1.0,
           v_scale: float = 1.0, out: Optional[torch.Tensor] = None,
           workspace: Optional[torch.Tensor] = None, stream=None, sinks=None,
           k_descale=None, v_descale=None, alibi_slopes=None) -> torch.Tensor:
    """paged_attn_extend: q bf16 [total_q, Hq, D] -> out bf16 [total_q, Hq, D].
    sinks / k_descale / v_descale / alibi_slopes as for decode (descales: cached
    context only)."""
    for name, t in (("q", q), ("k_new", k_new), ("v_new", v_new)):
        if t.dtype != torch.bfloat16 or not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous bf16")
    if cu_seqlens_q.dtype != torch.int32 or ctx_lens.dtype != torch.int32 \
            or block_table.dtype != torch.int32:
        raise TypeError("cu_seqlens_q, ctx_lens and block_table must be int32")
    if block_table.stride(1) != 1:
        raise ValueError("block_table rows must be contiguous")
    pr = pl.problem
    if tuple(q.shape) != (pr.total_q, pr.num_q_heads, pr.head_dim):
        raise ValueError(f"q must be ({pr.total_q}, {pr.num_q_heads}, {pr.head_dim}) as "
                         f"planned, got {tuple(q.shape)}")
    for name, t in (("k_new", k_new), ("v_new", v_new)):
        if tuple(t.shape) != (pr.total_q, pr.num_kv_heads, pr.head_dim):
            raise ValueError(f"{name} must be ({pr.total_q}, {pr.num_kv_heads}, "
                             f"{pr.head_dim}) as planned, got {tuple(t.shape)}")
    if cu_seqlens_q.dim() != 1 or cu_seqlens_q.numel() < pr.num_seqs + 1 or \
            not cu_seqlens_q.is_contiguous():
        raise ValueError(f"cu_seqlens_q must be a contiguous vector of >= {pr.num_seqs + 1} "
                         "entries")
    _check_cache(pl, k_pool, block_table, ctx_lens, "ctx_lens")
    _same_device(q, k_new=k_new, v_new=v_new, cu_seqlens_q=cu_seqlens_q, ctx_lens=ctx_lens,
                 k_pool=k_pool, v_pool=v_pool, block_table=block_table, out=out,
                 workspace=workspace, sinks=sinks, k_descale=k_descale, v_descale=v_descale,
                 alibi_slopes=alibi_slopes)
    if _INPUT_CHECKS:
        check_inputs(pl, block_table, ctx_lens, k_pool.shape[0], cu_seqlens_q)
    if out is None:
        out = torch.empty_like(q)
    if out.dtype != torch.bfloat16 or out.shape != q.shape or not out.is_contiguous():
        raise ValueError("out must be contiguous bf16 [total_q, Hq, D] like q")
    sp, st, sh = _pool_strides(k_pool, v_pool)
    workspace = _workspace(pl, workspace, q.device)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("paged_attn_extend", lib().paged_attn_extend(
        ctypes.byref(pl.c), _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(cu_seqlens_q),
        _ptr(ctx_lens), _ptr(k_pool), _ptr(v_pool), sp, st, sh, k_pool.shape[0],
        _ptr(block_table), block_table.stride(0), k_pool.shape[1], float(scale),
        float(softcap), int(window), float(k_scale), float(v_scale), _ptr(out),
        _ptr(workspace), wbytes,
        _extras(sinks, k_descale, v_descale, alibi_slopes, pr.num_q_heads), _stream(stream)))
    return out


def cache_append(key: torch.Tensor, value: torch.Tensor, k_pool: torch.Tensor,
                 v_pool: torch.Tensor, slot_mapping: torch.Tensor, k_scale: float = 1.0,
                 v_scale: float = 1.0, stream=None) -> None:
    """paged_attn_cache_append: key/value bf16 [T, Hkv, D] into the pools at
    int64 slots (slot < 0: skipped)."""
    for name, t in (("key", key), ("value", value)):
        if t.dtype != torch.bfloat16 or t.dim() != 3 or t.stride(2) != 1 \
                or t.stride(1) != t.shape[2]:
            raise ValueError(f"{name} must be bf16 [T, Hkv, D] with contiguous heads")
    if key.shape != value.shape or key.stride() != value.stride():
        raise ValueError("key and value must have the same shape and strides")
    if slot_mapping.dtype != torch.int64 or slot_mapping.shape != (key.shape[0],):
        raise TypeError("slot_mapping must be int64 [T]")
    sp, st, sh = _pool_strides(k_pool, v_pool)
    T, Hkv, D = key.shape
    if _INPUT_CHECKS and T > 0:
        top = int(slot_mapping.max())
        if top >= k_pool.shape[0] * k_pool.shape[1]:
            raise ValueError(f"device-content contract broken: slot_mapping holds {top}, "
                             f"the pools have {k_pool.shape[0] * k_pool.shape[1]} slots")
        live = slot_mapping[slot_mapping >= 0]
        if live.numel() != torch.unique(live).numel():
            raise ValueError("device-content contract broken: slot_mapping repeats a slot")
    _check("paged_attn_cache_append", lib().paged_attn_cache_append(
        _ptr(key), _ptr(value), T, key.stride(0), Hkv, D, _ptr(k_pool), _ptr(v_pool), sp, st,
        sh, k_pool.shape[0], k_pool.shape[1], PA_KV[_kv_dtype_name(k_pool)],
        _ptr(slot_mapping), float(k_scale), float(v_scale), _stream(stream)))


def gather(pl: Plan, k_pool: torch.Tensor, v_pool: torch.Tensor, block_table: torch.Tensor,
           seq_lens: torch.Tensor, total_tokens: int, stream=None):
    """paged_attn_gather: every cached row, dense [sum L, Hkv, D] (test aid)."""
    if block_table.dtype != torch.int32 or seq_lens.dtype != torch.int32:
        raise TypeError("block_table and seq_lens must be int32")
    if block_table.stride(1) != 1:
        raise ValueError("block_table rows must be contiguous")
    _check_cache(pl, k_pool, block_table, seq_lens, "seq_lens")
    _same_device(k_pool, v_pool=v_pool, block_table=block_table, seq_lens=seq_lens)
    if _INPUT_CHECKS:
        check_inputs(pl, block_table, seq_lens, k_pool.shape[0])
        need = int(seq_lens[:pl.problem.num_seqs].to("cpu", torch.int64).sum())
        if total_tokens < need:
            raise ValueError(f"total_tokens {total_tokens} < sum(seq_lens) = {need}")
    sp, st, sh = _pool_strides(k_pool, v_pool)
    shape = (total_tokens, k_pool.shape[2], k_pool.shape[3])
    k_out = torch.empty(shape, dtype=k_pool.dtype, device=k_pool.device)
    v_out = torch.empty(shape, dtype=k_pool.dtype, device=k_pool.device)
    _check("paged_attn_gather", lib().paged_attn_gather(
        ctypes.byref(pl.c), _ptr(k_pool), _ptr(v_pool), sp, st, sh, k_pool.shape[0],
        _ptr(block_table), block_table.stride(0), _ptr(seq_lens), _ptr(k_out), _ptr(v_out),
        _stream(stream)))
    return k_out, v_out
