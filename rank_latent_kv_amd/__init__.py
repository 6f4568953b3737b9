"""MI355X-native decode attention for Multi-Head Low-Rank Attention (MLRA) and
single-latent MLA.

All compute runs in the HIP library ``libmlra.so`` (built in-tree by
``rank_latent_kv_amd.build``); this module only marshals torch tensors into the
C ABI declared in ``include/mlra.h``. PyTorch provides device memory and the
stream. There is no fallback: if the library is missing, every call raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmlra.so")

MLRA_OK = 0
MLRA_ERR_INVALID_ARG = 1
MLRA_ERR_UNSUPPORTED = 2
MLRA_ERR_WORKSPACE = 3
MLRA_ERR_NO_PAGES = 4
MLRA_ERR_HIP = 5
MLRA_BF16 = 0
MLRA_F32 = 1
FLAG_SEQ_LEN_CLAMPED = 1
FLAG_BAD_PAGE = 2

EXPORTED_SYMBOLS = (
    "mlra_last_error", "mlra_version", "mlra_decode_workspace_size", "mlra_decode_validate", "mlra_decode",
    "mla_decode", "mlra_paged_append", "mlra_paged_gather", "mlra_page_table_check", "mlra_page_pool_create",
    "mlra_page_pool_alloc", "mlra_page_pool_free", "mlra_page_pool_num_free", "mlra_page_pool_destroy",
    "mlra_decode_prepare", "mlra_read_probe_words", "mlra_read_probe", "mlra_decode_plan",
    "mlra_decode_noalloc",
)
MLRA_KERNEL_MFMA = 0
MLRA_KERNEL_GENERIC = 1
PLAN_GENERIC_DTYPE = 1
PLAN_GENERIC_SHAPE = 2
PLAN_GENERIC_ALIGNMENT = 4
PLAN_GENERIC_PAGE_SIZE = 8
NOALLOC_SCRATCH_BYTES = 16 << 20   # MLRA_NOALLOC_SCRATCH_BYTES: the allocation-free entry point's device array


class MlraError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"mlra status {status}: {message}")
        self.status = status


class DecodeArgs(ctypes.Structure):
    """Mirror of ``mlra_decode_args`` (include/mlra.h)."""
    _fields_ = [
        ("batch", ctypes.c_int32), ("num_heads", ctypes.c_int32), ("num_branches", ctypes.c_int32),
        ("branch_dim", ctypes.c_int32), ("rope_dim", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("dtype", ctypes.c_int32), ("out_dtype", ctypes.c_int32),
        ("sm_scale", ctypes.c_float), ("alpha", ctypes.c_float),
        ("q_lat", ctypes.c_void_p), ("q_rope", ctypes.c_void_p), ("kv_lat", ctypes.c_void_p),
        ("kv_rope", ctypes.c_void_p),
        ("row_stride", ctypes.c_int64), ("seq_stride", ctypes.c_int64),
        ("seq_lens", ctypes.c_void_p), ("seq_lens_host", ctypes.c_void_p), ("max_seq_len", ctypes.c_int32),
        ("page_size", ctypes.c_int32), ("page_table", ctypes.c_void_p), ("max_pages", ctypes.c_int32),
        ("num_pages", ctypes.c_int32), ("num_splits", ctypes.c_int32),
        ("w_v", ctypes.c_void_p), ("out", ctypes.c_void_p), ("workspace", ctypes.c_void_p),
        ("workspace_bytes", ctypes.c_size_t), ("error_flags", ctypes.c_void_p),
        ("event_attn_begin", ctypes.c_void_p), ("event_attn_end", ctypes.c_void_p),
    ]


class PlanInfo(ctypes.Structure):
    """Mirror of ``mlra_plan_info`` (include/mlra.h)."""
    _fields_ = [
        ("kernel", ctypes.c_int32), ("generic_reason", ctypes.c_int32), ("num_splits", ctypes.c_int32),
        ("split_tokens", ctypes.c_int32), ("work_groups", ctypes.c_int32), ("cu_count", ctypes.c_int32),
        ("workspace_bytes", ctypes.c_size_t),
    ]


class PrepareArgs(ctypes.Structure):
    """Mirror of ``mlra_prepare_args`` (include/mlra.h)."""
    _fields_ = [
        ("batch", ctypes.c_int32), ("num_heads", ctypes.c_int32), ("num_branches", ctypes.c_int32),
        ("branch_dim", ctypes.c_int32), ("rope_dim", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("dtype", ctypes.c_int32), ("rope_base", ctypes.c_float),
        ("q_nope", ctypes.c_void_p), ("q_pe", ctypes.c_void_p), ("w_uk", ctypes.c_void_p),
        ("c_new", ctypes.c_void_p), ("k_pe_new", ctypes.c_void_p),
        ("positions", ctypes.c_void_p), ("positions_host", ctypes.c_void_p),
        ("q_lat", ctypes.c_void_p), ("q_rope", ctypes.c_void_p),
        ("kv_lat", ctypes.c_void_p), ("kv_rope", ctypes.c_void_p),
        ("row_stride", ctypes.c_int64), ("seq_stride", ctypes.c_int64), ("max_seq_len", ctypes.c_int32),
        ("page_size", ctypes.c_int32), ("page_table", ctypes.c_void_p), ("max_pages", ctypes.c_int32),
        ("num_pages", ctypes.c_int32), ("error_flags", ctypes.c_void_p),
    ]


_lib = None


def lib() -> ctypes.CDLL:
    """Load libmlra.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m rank_latent_kv_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
        P = ctypes.POINTER
        L.mlra_last_error.restype = ctypes.c_char_p
        L.mlra_version.restype = ctypes.c_char_p
        L.mlra_decode_workspace_size.argtypes = [P(DecodeArgs)]
        L.mlra_decode_workspace_size.restype = ctypes.c_size_t
        L.mlra_decode_validate.argtypes = [P(DecodeArgs)]
        L.mlra_decode.argtypes = [P(DecodeArgs), vp]
        L.mla_decode.argtypes = [P(DecodeArgs), vp]
        L.mlra_decode_noalloc.argtypes = [P(DecodeArgs), vp]
        L.mlra_decode_prepare.argtypes = [P(PrepareArgs), vp]
        L.mlra_paged_append.argtypes = [vp, i64, i32, i32, i32, vp, i32, vp, vp, i32, i32, vp, vp]
        L.mlra_paged_gather.argtypes = [vp, i64, i32, i32, i32, vp, i32, vp, i32, i32, i32, vp, vp, vp]
        L.mlra_page_table_check.argtypes = [vp, i32, i32, vp, i32, i32]
        L.mlra_page_pool_create.argtypes = [i32, P(vp)]
        L.mlra_page_pool_alloc.argtypes = [vp, i32, vp]
        L.mlra_page_pool_free.argtypes = [vp, i32, vp]
        L.mlra_page_pool_num_free.argtypes = [vp]
        L.mlra_page_pool_num_free.restype = i32
        L.mlra_page_pool_destroy.argtypes = [vp]
        L.mlra_page_pool_destroy.restype = None
        L.mlra_read_probe_words.argtypes = []
        L.mlra_read_probe_words.restype = i32
        L.mlra_read_probe.argtypes = [vp, ctypes.c_size_t, vp, i32, vp]
        L.mlra_decode_plan.argtypes = [P(DecodeArgs), i32, P(PlanInfo)]
        for name in ("mlra_decode_validate", "mlra_decode", "mla_decode", "mlra_decode_noalloc", "mlra_decode_prepare", "mlra_paged_append",
                     "mlra_paged_gather", "mlra_page_table_check", "mlra_page_pool_create",
                     "mlra_page_pool_alloc", "mlra_page_pool_free", "mlra_read_probe", "mlra_decode_plan"):
            getattr(L, name).restype = i32
        _lib = L
    return _lib


def last_error() -> str:
    return lib().mlra_last_error().decode()


def _check(status: int):
    if status != MLRA_OK:
        raise MlraError(status, last_error())


def _dtype_code(t: torch.dtype) -> int:
    if t == torch.bfloat16:
        return MLRA_BF16
    if t == torch.float32:
        return MLRA_F32
    raise TypeError(f"unsupported dtype {t}")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _need(t: Optional[torch.Tensor], name: str, *, device: torch.device, dtype=None, contiguous: bool = True,
          rows_contiguous: bool = False, numel_at_least: Optional[int] = None) -> None:
    """Refuse a tensor whose raw pointer the library would misread: wrong dtype (an int64 length
    array read as int32 halves, say), another device, or a layout the C side does not assume.
    Raises TypeError or ValueError; None passes (optional arguments)."""
    if t is None:
        return
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor (got {type(t).__name__})")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, the other operands on {device}")
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if contiguous and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if rows_contiguous and t.dim() > 0 and t.stride(-1) != 1:
        raise ValueError(f"{name} must have unit stride in its last dimension (got {t.stride(-1)})")
    if numel_at_least is not None and t.numel() < numel_at_least:
        raise ValueError(f"{name} holds {t.numel()} elements, needs at least {numel_at_least}")


def _need_host_int32(t: Optional[torch.Tensor], name: str, n: int) -> None:
    if t is None:
        return
    if not isinstance(t, torch.Tensor) or t.device.type != "cpu" or t.dtype != torch.int32 or not t.is_contiguous():
        raise TypeError(f"{name} must be a contiguous int32 CPU tensor")
    if t.numel() < n:
        raise ValueError(f"{name} holds {t.numel()} entries, needs {n}")


def _stream_handle(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def make_args(q_lat, q_rope, kv_lat, kv_rope, seq_lens, w_v, *, sm_scale: float, alpha: float,
              row_stride: Optional[int] = None, seq_stride: Optional[int] = None,
              max_seq_len: Optional[int] = None, seq_lens_host: Optional[torch.Tensor] = None,
              page_table: Optional[torch.Tensor] = None, page_size: int = 64, num_pages: int = 0,
              out: Optional[torch.Tensor] = None, out_dtype: Optional[torch.dtype] = None,
              workspace: Optional[torch.Tensor] = None, num_splits: int = 0,
              error_flags: Optional[torch.Tensor] = None, events=None) -> DecodeArgs:
    """Fill ``mlra_decode_args`` from tensors (shapes as in include/mlra.h).

    ``kv_lat`` / ``kv_rope`` may be views into one combined [.., rows, d_c + d_R]
    tensor; ``row_stride`` / ``seq_stride`` default to that tensor's strides. The struct
    holds raw pointers, so it keeps a reference to every tensor it points into: the
    memory stays valid for as long as the struct is alive."""
    if q_lat.dim() != 4:
        raise ValueError(f"q_lat must be [B, h, n_b, d_b] (got shape {tuple(q_lat.shape)})")
    B, H, NB, DB = q_lat.shape
    DR = q_rope.shape[-1]
    dev, dt = q_lat.device, q_lat.dtype
    _dtype_code(dt)
    _need(q_lat, "q_lat", device=dev)
    _need(q_rope, "q_rope", device=dev, dtype=dt)
    if tuple(q_rope.shape) != (B, H, DR):
        raise ValueError(f"q_rope must be [B, h, d_R] = {(B, H, DR)} (got {tuple(q_rope.shape)})")
    _need(kv_lat, "kv_lat", device=dev, dtype=dt, contiguous=False, rows_contiguous=True)
    _need(kv_rope, "kv_rope", device=dev, dtype=dt, contiguous=False, rows_contiguous=True)
    _need(seq_lens, "seq_lens", device=dev, dtype=torch.int32, numel_at_least=B)
    _need_host_int32(seq_lens_host, "seq_lens_host", B)
    _need(page_table, "page_table", device=dev, dtype=torch.int32)
    if page_table is not None and (page_table.dim() != 2 or page_table.shape[0] < B):
        raise ValueError(f"page_table must be [B, max_pages] with B >= {B} (got {tuple(page_table.shape)})")
    # the merge reads W^V in the inputs' dtype
    _need(w_v, "w_v", device=dev, dtype=dt)
    if w_v.dim() != 3 or w_v.shape[0] != H or w_v.shape[2] != NB * DB:
        raise ValueError(f"w_v must be [h, d_h, n_b*d_b] = [{H}, d_h, {NB * DB}] (got {tuple(w_v.shape)})")
    _need(out, "out", device=dev, dtype=(torch.bfloat16, torch.float32))
    if out is not None and tuple(out.shape) != (B, H, w_v.shape[1]):
        raise ValueError(f"out must be [B, h, d_h] = {(B, H, w_v.shape[1])} (got {tuple(out.shape)})")
    _need(workspace, "workspace", device=dev)
    _need(error_flags, "error_flags", device=dev, dtype=torch.int32, numel_at_least=1)
    a = DecodeArgs()
    a.batch, a.num_heads, a.num_branches, a.branch_dim, a.rope_dim = B, H, NB, DB, DR
    a.head_dim = w_v.shape[1]
    a.dtype = _dtype_code(q_lat.dtype)
    a.out_dtype = _dtype_code(out.dtype if out is not None else (out_dtype or q_lat.dtype))
    a.sm_scale, a.alpha = float(sm_scale), float(alpha)
    a.q_lat, a.q_rope, a.kv_lat, a.kv_rope = _ptr(q_lat), _ptr(q_rope), _ptr(kv_lat), _ptr(kv_rope)
    a.row_stride = int(row_stride if row_stride is not None else kv_lat.stride(-2))
    if page_table is None:
        a.seq_stride = int(seq_stride if seq_stride is not None else kv_lat.stride(0))
        a.max_seq_len = int(max_seq_len if max_seq_len is not None else kv_lat.shape[-2])
    else:
        a.seq_stride = 0
        a.max_seq_len = int(max_seq_len if max_seq_len is not None else page_table.shape[1] * page_size)
        a.page_table = _ptr(page_table)
        a.max_pages = page_table.shape[1]
        a.page_size = page_size
        a.num_pages = num_pages
    a.seq_lens = _ptr(seq_lens)
    if seq_lens_host is not None:
        a.seq_lens_host = seq_lens_host.data_ptr()
    a.num_splits = num_splits
    a.w_v, a.out = _ptr(w_v), _ptr(out)
    if workspace is not None:
        a.workspace = workspace.data_ptr()
        a.workspace_bytes = workspace.numel() * workspace.element_size()
    a.error_flags = _ptr(error_flags)
    if events is not None:
        a.event_attn_begin, a.event_attn_end = events
    a._keep = (q_lat, q_rope, kv_lat, kv_rope, seq_lens, seq_lens_host, page_table, w_v, out, workspace, error_flags)
    return a


def workspace_size(args: DecodeArgs) -> int:
    n = lib().mlra_decode_workspace_size(ctypes.byref(args))
    if n == 0:
        raise MlraError(MLRA_ERR_INVALID_ARG, last_error())
    return n


def alloc_workspace(args: DecodeArgs, device) -> torch.Tensor:
    n = workspace_size(args)
    return torch.empty(n, dtype=torch.uint8, device=device)


def plan(args: DecodeArgs, cu_count: int = 0) -> dict:
    """How a decode call with ``args`` would run: which attention kernel ("mfma" or "generic",
    with the reasons for the generic one), splits, work-groups and workspace bytes, planned for
    ``cu_count`` compute units (0 = the current device). Raises MlraError on invalid args."""
    info = PlanInfo()
    _check(lib().mlra_decode_plan(ctypes.byref(args), int(cu_count), ctypes.byref(info)))
    reasons = [n for bit, n in ((PLAN_GENERIC_DTYPE, "dtype"), (PLAN_GENERIC_SHAPE, "shape"),
                                (PLAN_GENERIC_ALIGNMENT, "alignment"), (PLAN_GENERIC_PAGE_SIZE, "page_size"))
               if info.generic_reason & bit]
    return {"kernel": "mfma" if info.kernel == MLRA_KERNEL_MFMA else "generic", "generic_reasons": reasons,
            "num_splits": info.num_splits, "split_tokens": info.split_tokens, "work_groups": info.work_groups,
            "cu_count": info.cu_count, "workspace_bytes": info.workspace_bytes}


def validate(args: DecodeArgs) -> int:
    """Host-only argument check; returns the status code (0 = OK)."""
    return lib().mlra_decode_validate(ctypes.byref(args))


def _run(fn_name: str, q_lat, q_rope, kv_lat, kv_rope, seq_lens, w_v, *, sm_scale, alpha, out=None,
         out_dtype=None, workspace=None, stream=None, **kw):
    if not q_lat.is_cuda:
        raise ValueError("the decode runs on the GPU: pass device tensors (q_lat is on the CPU)")
    B, H, NB, DB = q_lat.shape
    if out is None:
        out = torch.empty((B, H, w_v.shape[1]), dtype=out_dtype or q_lat.dtype, device=q_lat.device)
    args = make_args(q_lat, q_rope, kv_lat, kv_rope, seq_lens, w_v, sm_scale=sm_scale, alpha=alpha, out=out,
                     workspace=workspace, **kw)
    if workspace is None:
        workspace = alloc_workspace(args, q_lat.device)
        args.workspace = workspace.data_ptr()
        args.workspace_bytes = workspace.numel()
        args._keep = args._keep + (workspace,)
        if stream is not None and isinstance(stream, torch.cuda.Stream):
            # the workspace comes from the current stream's pool but is used on `stream`:
            # keep the allocator from handing it out again before that stream's work ends
            workspace.record_stream(stream)
    _check(getattr(lib(), fn_name)(ctypes.byref(args), _stream_handle(stream)))
    return out


def decode(q_lat, q_rope, kv_lat, kv_rope, seq_lens, w_v, *, sm_scale: float, alpha: float, **kw) -> torch.Tensor:
    """MLRA decode (any number of branches). Returns y [B, h, d_h]."""
    return _run("mlra_decode", q_lat, q_rope, kv_lat, kv_rope, seq_lens, w_v, sm_scale=sm_scale, alpha=alpha, **kw)


def decode_noalloc(q_lat, q_rope, kv_lat, kv_rope, seq_lens, w_v, *, sm_scale: float, alpha: float, out: torch.Tensor,
                   stream=None, **kw) -> torch.Tensor:
    """``mlra_decode_noalloc``: the decode with the library's own device scratch (no workspace,
    no device allocation in the call; ``out`` must be given). Calls that overlap on one GPU race."""
    if not q_lat.is_cuda:
        raise ValueError("the decode runs on the GPU: pass device tensors (q_lat is on the CPU)")
    args = make_args(q_lat, q_rope, kv_lat, kv_rope, seq_lens, w_v, sm_scale=sm_scale, alpha=alpha, out=out, **kw)
    _check(lib().mlra_decode_noalloc(ctypes.byref(args), _stream_handle(stream)))
    return out


def mla_decode(q_lat, q_rope, kv_lat, kv_rope, seq_lens, w_v, *, sm_scale: float, alpha: float = 1.0,
               **kw) -> torch.Tensor:
    """Single-latent MLA decode; q_lat is [B, h, d_c] or [B, h, 1, d_c]."""
    if q_lat.dim() == 3:
        q_lat = q_lat.unsqueeze(2)
    return _run("mla_decode", q_lat, q_rope, kv_lat, kv_rope, seq_lens, w_v, sm_scale=sm_scale, alpha=alpha, **kw)


def make_prepare_args(q_nope, q_pe, w_uk_t, c_new, k_pe_new, positions, kv_lat, kv_rope, *, num_branches: int,
                      q_lat: torch.Tensor, q_rope: torch.Tensor, rope_base: float = 10000.0,
                      positions_host: Optional[torch.Tensor] = None, row_stride: Optional[int] = None,
                      seq_stride: Optional[int] = None, max_seq_len: Optional[int] = None,
                      page_table: Optional[torch.Tensor] = None, page_size: int = 64, num_pages: int = 0,
                      error_flags: Optional[torch.Tensor] = None) -> PrepareArgs:
    """Fill ``mlra_prepare_args`` (shapes as in include/mlra.h; w_uk_t is [h, d_c, d_h]). The struct
    keeps a reference to every tensor it points into."""
    B, H, DH = q_nope.shape
    DC = w_uk_t.shape[1]
    dev, dt = q_nope.device, q_nope.dtype
    _dtype_code(dt)
    _need(q_nope, "q_nope", device=dev)
    for name, t in (("q_pe", q_pe), ("w_uk_t", w_uk_t), ("c_new", c_new), ("k_pe_new", k_pe_new), ("q_lat", q_lat),
                    ("q_rope", q_rope)):
        _need(t, name, device=dev, dtype=dt)
    _need(kv_lat, "kv_lat", device=dev, dtype=dt, contiguous=False, rows_contiguous=True)
    _need(kv_rope, "kv_rope", device=dev, dtype=dt, contiguous=False, rows_contiguous=True)
    _need(positions, "positions", device=dev, dtype=torch.int32, numel_at_least=B)
    _need_host_int32(positions_host, "positions_host", B)
    _need(page_table, "page_table", device=dev, dtype=torch.int32)
    _need(error_flags, "error_flags", device=dev, dtype=torch.int32, numel_at_least=1)
    a = PrepareArgs()
    a.batch, a.num_heads, a.num_branches = B, H, num_branches
    a.branch_dim, a.rope_dim, a.head_dim = DC // num_branches, q_pe.shape[-1], DH
    a.dtype = _dtype_code(q_nope.dtype)
    a.rope_base = float(rope_base)
    a.q_nope, a.q_pe, a.w_uk = _ptr(q_nope), _ptr(q_pe), _ptr(w_uk_t)
    a.c_new, a.k_pe_new, a.positions = _ptr(c_new), _ptr(k_pe_new), _ptr(positions)
    if positions_host is not None:
        a.positions_host = positions_host.data_ptr()
    a.q_lat, a.q_rope = _ptr(q_lat), _ptr(q_rope)
    a.kv_lat, a.kv_rope = _ptr(kv_lat), _ptr(kv_rope)
    a.row_stride = int(row_stride if row_stride is not None else kv_lat.stride(-2))
    if page_table is None:
        a.seq_stride = int(seq_stride if seq_stride is not None else kv_lat.stride(0))
        a.max_seq_len = int(max_seq_len if max_seq_len is not None else kv_lat.shape[-2])
    else:
        a.page_table, a.max_pages, a.page_size, a.num_pages = _ptr(page_table), page_table.shape[1], page_size, num_pages
    a.error_flags = _ptr(error_flags)
    # the struct holds raw pointers: keep the tensors behind them alive with it
    a._keep = (q_nope, q_pe, w_uk_t, c_new, k_pe_new, positions, positions_host, kv_lat, kv_rope, q_lat, q_rope,
               page_table, error_flags)
    return a


def prepare(q_nope, q_pe, w_uk_t, c_new, k_pe_new, positions, kv_lat, kv_rope, *, num_branches: int,
            q_lat: Optional[torch.Tensor] = None, q_rope: Optional[torch.Tensor] = None, stream=None, **kw):
    """The step before a decode call: absorbed query, rotated RoPE query, new cache row.
    Returns (q_lat [B, h, n_b, d_b], q_rope [B, h, d_R])."""
    if not q_nope.is_cuda:
        raise ValueError("the prepare step runs on the GPU: pass device tensors (q_nope is on the CPU)")
    B, H, _ = q_nope.shape
    DC = w_uk_t.shape[1]
    if q_lat is None:
        q_lat = torch.empty((B, H, num_branches, DC // num_branches), dtype=q_nope.dtype, device=q_nope.device)
    if q_rope is None:
        q_rope = torch.empty_like(q_pe)
    args = make_prepare_args(q_nope, q_pe, w_uk_t, c_new, k_pe_new, positions, kv_lat, kv_rope,
                             num_branches=num_branches, q_lat=q_lat, q_rope=q_rope, **kw)
    _check(lib().mlra_decode_prepare(ctypes.byref(args), _stream_handle(stream)))
    return q_lat, q_rope


def split_rows(kv: torch.Tensor, latent_dim: int):
    """Latent and RoPE views of a combined cache [.., rows, d_c + d_R]."""
    return kv[..., :latent_dim], kv[..., latent_dim:]


# ---- paged cache -------------------------------------------------------------------------

def _check_paged_copy(pool, page_table, lens_or_pos, name, error_flags, rows=None, out=None) -> None:
    if not pool.is_cuda:
        raise ValueError("paged copies run on the GPU: pass device tensors (pool is on the CPU)")
    dev = pool.device
    _dtype_code(pool.dtype)
    _need(pool, "pool", device=dev, contiguous=False, rows_contiguous=True)
    _need(page_table, "page_table", device=dev, dtype=torch.int32)
    if page_table.dim() != 2:
        raise ValueError(f"page_table must be [B, max_pages] (got {tuple(page_table.shape)})")
    _need(lens_or_pos, name, device=dev, dtype=torch.int32, numel_at_least=page_table.shape[0])
    _need(error_flags, "error_flags", device=dev, dtype=torch.int32, numel_at_least=1)
    if rows is not None:
        _need(rows, "rows", device=dev, dtype=pool.dtype, contiguous=False, rows_contiguous=True)
        if rows.dim() != 2 or rows.shape[-1] > pool.shape[-1]:
            raise ValueError(f"rows must be [B, R] with R <= the pool row ({pool.shape[-1]})")
    if out is not None:
        _need(out, "out", device=dev, dtype=pool.dtype)


def paged_append(pool: torch.Tensor, page_table: torch.Tensor, positions: torch.Tensor, rows: torch.Tensor, *,
                 page_size: int, error_flags: Optional[torch.Tensor] = None, stream=None):
    """pool [P, page_size, R] (or any [P*page_size, R] view), rows [B, R]."""
    _check_paged_copy(pool, page_table, positions, "positions", error_flags, rows=rows)
    R = rows.shape[-1]
    num_pages = pool.numel() // (page_size * pool.shape[-1])
    _check(lib().mlra_paged_append(pool.data_ptr(), pool.stride(-2), R, page_size, num_pages, page_table.data_ptr(),
                                   page_table.shape[1], positions.data_ptr(), rows.data_ptr(), rows.shape[0],
                                   _dtype_code(pool.dtype), _ptr(error_flags), _stream_handle(stream)))


def paged_gather(pool: torch.Tensor, page_table: torch.Tensor, seq_lens: torch.Tensor, max_seq_len: int, *,
                 page_size: int, out: Optional[torch.Tensor] = None, error_flags: Optional[torch.Tensor] = None,
                 stream=None) -> torch.Tensor:
    _check_paged_copy(pool, page_table, seq_lens, "seq_lens", error_flags, out=out)
    R = pool.shape[-1]
    B = page_table.shape[0]
    if out is None:
        out = torch.zeros((B, max_seq_len, R), dtype=pool.dtype, device=pool.device)
    num_pages = pool.numel() // (page_size * R)
    _check(lib().mlra_paged_gather(pool.data_ptr(), pool.stride(-2), R, page_size, num_pages, page_table.data_ptr(),
                                   page_table.shape[1], seq_lens.data_ptr(), max_seq_len, B, _dtype_code(pool.dtype),
                                   out.data_ptr(), _ptr(error_flags), _stream_handle(stream)))
    return out


def page_table_check(page_table, seq_lens, page_size: int, num_pages: int) -> None:
    """Host check of a page table (torch int32 CPU tensors). Raises MlraError."""
    pt = page_table.to(torch.int32).contiguous().cpu()
    sl = seq_lens.to(torch.int32).contiguous().cpu()
    _check(lib().mlra_page_table_check(pt.data_ptr(), pt.shape[0], pt.shape[1], sl.data_ptr(), page_size, num_pages))


class PagePool:
    """Deterministic host page allocator (LIFO free list) from libmlra."""

    def __init__(self, num_pages: int):
        self._h = ctypes.c_void_p()
        _check(lib().mlra_page_pool_create(num_pages, ctypes.byref(self._h)))

    def alloc(self, n: int) -> list:
        buf = (ctypes.c_int32 * max(n, 1))()
        _check(lib().mlra_page_pool_alloc(self._h, n, buf))
        return list(buf[:n])

    def free(self, ids: Sequence[int]) -> None:
        buf = (ctypes.c_int32 * max(len(ids), 1))(*ids)
        _check(lib().mlra_page_pool_free(self._h, len(ids), buf))

    @property
    def num_free(self) -> int:
        return lib().mlra_page_pool_num_free(self._h)

    def close(self):
        if self._h:
            lib().mlra_page_pool_destroy(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def read_probe(buf: torch.Tensor, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Read every byte of the device tensor `buf` once (streaming-read probe) and return the
    per-work-group XOR words (int32 [mlra_read_probe_words()]) on the current stream."""
    n = int(lib().mlra_read_probe_words())
    if out is None:
        out = torch.empty(n, dtype=torch.int32, device=buf.device)
    _check(lib().mlra_read_probe(ctypes.c_void_p(buf.data_ptr()), buf.numel() * buf.element_size(),
                                 ctypes.c_void_p(out.data_ptr()), out.numel(),
                                 ctypes.c_void_p(torch.cuda.current_stream(buf.device).cuda_stream)))
    return out
