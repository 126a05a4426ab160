"""Thin ctypes binding of libmla_decode.so (see include/mla_decode.h).

Functions carry the C names and only marshal arguments: torch tensors become
device pointers, the current torch stream becomes the hipStream_t.  Every step
of the decode runs in the library's HIP kernels; there is no fallback, and
importing this module raises if the library has not been built.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np
import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmla_decode.so")

MLA_KV_BF16, MLA_KV_FP8_E4M3, MLA_KV_MXFP4 = 0, 1, 2
KV_DTYPES = {"bf16": MLA_KV_BF16, "fp8": MLA_KV_FP8_E4M3, "mxfp4": MLA_KV_MXFP4}
STATUS = {0: "MLA_OK", 1: "MLA_ERR_INVALID_ARG", 2: "MLA_ERR_UNSUPPORTED",
          3: "MLA_ERR_NOT_PLANNED", 4: "MLA_ERR_WORKSPACE_TOO_SMALL", 5: "MLA_ERR_HIP"}

NUM_HEADS, QK_DIM, V_DIM = 16, 576, 512
MLA_SCRATCH_BYTES = 16 << 20  # the allocation-free run's device array (MLA_SCRATCH_BYTES)
MLA_QUERY_EXACT, MLA_QUERY_E4M3 = 0, 1
QUERY_FORMATS = {"exact": MLA_QUERY_EXACT, "e4m3": MLA_QUERY_E4M3}

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with `python -m latent_attention_decode_amd.build`"
                      " (there is no fallback implementation)")

_lib = ctypes.CDLL(LIB_PATH)
_P = ctypes.c_void_p
_I32P = ctypes.POINTER(ctypes.c_int32)
_H = ctypes.c_void_p

_lib.mla_decode_version.restype = ctypes.c_int
_lib.mla_status_string.argtypes = [ctypes.c_int]
_lib.mla_status_string.restype = ctypes.c_char_p
_lib.mla_decode_create.argtypes = [ctypes.POINTER(_H), ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                   ctypes.c_int, ctypes.c_float, ctypes.c_int, ctypes.c_int]
_lib.mla_decode_plan.argtypes = [_H, ctypes.c_int, _P, _P, ctypes.c_int,
                                 ctypes.POINTER(ctypes.c_size_t)]
_lib.mla_decode_plan_preview.argtypes = [ctypes.c_int, _P, _P, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                         ctypes.c_int, ctypes.c_int, _P, ctypes.c_int,
                                         ctypes.POINTER(ctypes.c_int), ctypes.POINTER(ctypes.c_int),
                                         ctypes.POINTER(ctypes.c_size_t)]
_lib.mla_decode_plan_multi.argtypes = [_H, ctypes.c_int, _P, _P, _P, ctypes.c_int,
                                       ctypes.POINTER(ctypes.c_size_t)]
_lib.mla_decode_plan_preview_multi.argtypes = [ctypes.c_int, _P, _P, _P, ctypes.c_int, ctypes.c_int,
                                               ctypes.c_int, ctypes.c_int, ctypes.c_int, _P, ctypes.c_int,
                                               ctypes.POINTER(ctypes.c_int), ctypes.POINTER(ctypes.c_int),
                                               ctypes.POINTER(ctypes.c_size_t)]
_lib.mla_decode_plan_info.argtypes = [_H, ctypes.POINTER(ctypes.c_int), ctypes.POINTER(ctypes.c_int),
                                      ctypes.POINTER(ctypes.c_int)]
_lib.mla_decode_run.argtypes = [_H, _P, _P, _P, ctypes.c_int64, _P, _P, _P, _P, _P,
                                ctypes.c_size_t, _P]
_lib.mla_decode_run_noalloc.argtypes = [_H, _P, _P, _P, ctypes.c_int64, _P, _P, _P, _P, _P]
_lib.mla_decode_set_profiling.argtypes = [_H, ctypes.c_int]
_lib.mla_decode_set_query_format.argtypes = [_H, ctypes.c_int]
_lib.mla_decode_kernel_time_ms.argtypes = [_H, ctypes.c_int, ctypes.POINTER(ctypes.c_float)]
_lib.mla_decode_kernel_resources.argtypes = [_H, ctypes.c_int, ctypes.POINTER(ctypes.c_int),
                                             ctypes.POINTER(ctypes.c_int), ctypes.POINTER(ctypes.c_int)]
_lib.mla_decode_destroy.argtypes = [_H]
_lib.mla_decode_last_error.argtypes = [_H]
_lib.mla_decode_last_error.restype = ctypes.c_char_p
for _name in ("mla_decode_create", "mla_decode_plan", "mla_decode_plan_preview", "mla_decode_plan_multi",
              "mla_decode_plan_preview_multi",
              "mla_decode_plan_info", "mla_decode_run", "mla_decode_run_noalloc", "mla_decode_set_profiling",
              "mla_decode_set_query_format", "mla_decode_kernel_time_ms", "mla_decode_kernel_resources",
              "mla_decode_destroy"):
    getattr(_lib, _name).restype = ctypes.c_int

EXPORTED = ("mla_decode_version", "mla_status_string", "mla_decode_create", "mla_decode_plan",
            "mla_decode_plan_preview", "mla_decode_plan_multi", "mla_decode_plan_preview_multi",
            "mla_decode_plan_info", "mla_decode_run", "mla_decode_run_noalloc",
            "mla_decode_set_profiling", "mla_decode_set_query_format", "mla_decode_kernel_time_ms",
            "mla_decode_kernel_resources", "mla_decode_destroy", "mla_decode_last_error")


class MlaError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str = ""):
        self.status = status
        super().__init__(f"{where}: {STATUS.get(status, status)}" + (f" ({detail})" if detail else ""))


def _check(st: int, where: str, h=None):
    if st != 0:
        detail = _lib.mla_decode_last_error(h).decode() if h else ""
        raise MlaError(st, where, detail)


def _host_i32(a) -> np.ndarray:
    if isinstance(a, torch.Tensor):
        a = a.detach().cpu().numpy()
    return np.ascontiguousarray(a, dtype=np.int32)


def _dptr(t: Optional[torch.Tensor]) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("mla_decode_run takes device tensors")
    if not t.is_contiguous():
        raise ValueError("mla_decode_run takes contiguous tensors")
    return t.data_ptr()


_BF16, _I32 = torch.bfloat16, torch.int32


def _check_run_tensors(q, out, *int32_arrays) -> None:
    qs, os_ = q.shape, out.shape
    if q.dtype is not _BF16 or len(qs) < 2 or qs[-1] != QK_DIM or qs[-2] != NUM_HEADS:
        raise ValueError(f"q must be bf16 [rows, {NUM_HEADS}, {QK_DIM}] (got {q.dtype} {tuple(qs)})")
    if out.dtype is not _BF16 or len(os_) < 2 or os_[-1] != V_DIM or os_[-2] != NUM_HEADS:
        raise ValueError(f"out must be bf16 [rows, {NUM_HEADS}, {V_DIM}] (got {out.dtype} {tuple(os_)})")
    if q.numel() * V_DIM != out.numel() * QK_DIM:
        raise ValueError(f"q {tuple(qs)} and out {tuple(os_)} hold different numbers of rows")
    for a in int32_arrays:
        if a is not None and a.dtype is not _I32:
            raise ValueError(f"kv_indptr and the page table arrays must be int32 (got {a.dtype})")


ROW_BYTES = {"bf16": 2 * QK_DIM, "fp8": QK_DIM, "mxfp4": QK_DIM // 2}
_KV_DTYPES = {"bf16": (torch.bfloat16, torch.uint8), "fp8": (torch.uint8, torch.float8_e4m3fn, torch.int8),
              "mxfp4": (torch.uint8,)}


def check_cache_tensors(kv_dtype: str, page_size: int, batch: int, indptr_end: int, total_tokens: int, kv,
                        kv_scales, kv_indptr, kv_page_indices=None, kv_last_page_len=None) -> None:
    """The cache tensors of a run against the handle's format and its plan.

    A plan of `batch` sequences whose host kv_indptr ends at `indptr_end`
    (tokens, or pages when page_size > 1) and covers `total_tokens` tokens
    reads cache rows up to kv_indptr[-1] (contiguous), or page-table entries
    up to kv_indptr[-1] (paged), and per MXFP4 row 18 scale bytes.  The
    library takes bare pointers, so a tensor of the wrong element type or too
    few rows is refused here.  (With pages, the page ids themselves sit in
    device memory and are not checked: each must name a page inside kv.)"""
    rb = ROW_BYTES[kv_dtype]
    if total_tokens == 0 and kv is None:
        return
    if kv is None:
        raise ValueError("kv is None for a plan that reads the cache")
    if kv.dtype not in _KV_DTYPES[kv_dtype]:
        raise ValueError(f"a {kv_dtype} cache cannot be a {kv.dtype} tensor")
    if kv.dim() < 2 or kv.shape[-1] * kv.element_size() != rb:
        raise ValueError(f"{kv_dtype} cache rows are {rb} bytes (got {kv.dtype} {tuple(kv.shape)})")
    rows = kv.numel() * kv.element_size() // rb
    if page_size == 1 and rows < indptr_end:
        raise ValueError(f"the plan reads cache rows up to {indptr_end}; kv holds {rows}")
    if page_size > 1:
        if rows < page_size:
            raise ValueError(f"kv holds {rows} rows, less than one page of {page_size}")
        if kv_page_indices is None or kv_page_indices.numel() < indptr_end:
            raise ValueError(f"the plan reads {indptr_end} page-table entries; kv_page_indices holds "
                             f"{0 if kv_page_indices is None else kv_page_indices.numel()}")
        if kv_last_page_len is None or kv_last_page_len.numel() < batch:
            raise ValueError(f"kv_last_page_len needs {batch} entries")
    if kv_indptr.numel() < batch + 1:
        raise ValueError(f"kv_indptr needs {batch + 1} entries (got {kv_indptr.numel()})")
    if kv_dtype == "fp8":
        if kv_scales is None or kv_scales.dtype is not torch.float32 or kv_scales.numel() < 1:
            raise ValueError("an fp8 cache takes kv_scales: one float32 per-tensor scale")
    elif kv_dtype == "mxfp4":
        if (kv_scales is None or kv_scales.dtype is not torch.uint8 or kv_scales.dim() != 2
                or kv_scales.shape[1] < 18):
            raise ValueError("an MXFP4 cache takes kv_scales: uint8 [rows, stride >= 18] e8m0 scales")
        if kv_scales.shape[0] < rows:
            raise ValueError(f"kv_scales holds {kv_scales.shape[0]} rows of scales for {rows} cache rows")


def mla_decode_version() -> int:
    return _lib.mla_decode_version()


def mla_status_string(status: int) -> str:
    return _lib.mla_status_string(int(status)).decode()


def mla_decode_create(device: int, kv_dtype: str, page_size: int = 1, num_heads: int = NUM_HEADS,
                      qk_dim: int = QK_DIM, v_dim: int = V_DIM, sm_scale: Optional[float] = None):
    """Returns an opaque handle (int)."""
    if sm_scale is None:
        sm_scale = 1.0 / float(np.sqrt(qk_dim))
    h = _H()
    st = _lib.mla_decode_create(ctypes.byref(h), int(device), int(num_heads), int(qk_dim), int(v_dim),
                                float(sm_scale), KV_DTYPES[kv_dtype] if isinstance(kv_dtype, str)
                                else int(kv_dtype), int(page_size))
    _check(st, "mla_decode_create")
    return h.value


def mla_decode_plan(h, kv_indptr_host, kv_last_page_len_host=None, split_override: int = 0) -> int:
    """Plans the batch; returns the workspace size in bytes."""
    ip = _host_i32(kv_indptr_host)
    lp = None if kv_last_page_len_host is None else _host_i32(kv_last_page_len_host)
    ws = ctypes.c_size_t()
    st = _lib.mla_decode_plan(h, ip.size - 1, ip.ctypes.data, None if lp is None else lp.ctypes.data,
                              int(split_override), ctypes.byref(ws))
    _check(st, "mla_decode_plan", h)
    return ws.value


def mla_decode_plan_multi(h, qo_indptr_host, kv_indptr_host, kv_last_page_len_host=None,
                          split_override: int = 0) -> int:
    """Plans a multi-token batch (query tokens per sequence from qo_indptr); returns the
    workspace size in bytes."""
    qo = _host_i32(qo_indptr_host)
    ip = _host_i32(kv_indptr_host)
    lp = None if kv_last_page_len_host is None else _host_i32(kv_last_page_len_host)
    if qo.size != ip.size:
        raise ValueError("qo_indptr and kv_indptr must have the same length")
    ws = ctypes.c_size_t()
    st = _lib.mla_decode_plan_multi(h, ip.size - 1, qo.ctypes.data, ip.ctypes.data,
                                    None if lp is None else lp.ctypes.data, int(split_override), ctypes.byref(ws))
    _check(st, "mla_decode_plan_multi", h)
    return ws.value


def mla_decode_plan_preview(kv_indptr_host, kv_last_page_len_host=None, page_size: int = 1,
                            split_override: int = 0, num_cus: int = 256, blocks_per_cu: int = 2,
                            kv_dtype: str = "fp8", qo_indptr_host=None):
    """Host-only planner.  Returns (items int32 [n, 5], num_slots, workspace_bytes); an item
    row is (query row, first token, end token, slot, workgroup).  With qo_indptr_host, the
    multi-token planner (query rows per sequence from qo_indptr)."""
    ip = _host_i32(kv_indptr_host)
    lp = None if kv_last_page_len_host is None else _host_i32(kv_last_page_len_host)
    qo = None if qo_indptr_host is None else _host_i32(qo_indptr_host)
    n = ctypes.c_int()
    slots = ctypes.c_int()
    ws = ctypes.c_size_t()
    rest = (None if lp is None else lp.ctypes.data, int(page_size), KV_DTYPES[kv_dtype], int(split_override),
            int(num_cus), int(blocks_per_cu))

    def call(items_ptr, cap):
        if qo is None:
            return _lib.mla_decode_plan_preview(ip.size - 1, ip.ctypes.data, *rest, items_ptr, cap, ctypes.byref(n),
                                                ctypes.byref(slots), ctypes.byref(ws))
        return _lib.mla_decode_plan_preview_multi(ip.size - 1, qo.ctypes.data, ip.ctypes.data, *rest, items_ptr,
                                                  cap, ctypes.byref(n), ctypes.byref(slots), ctypes.byref(ws))

    st = call(None, 0)
    if st != 0 and n.value == 0:
        _check(st, "mla_decode_plan_preview")
    items = np.zeros((max(n.value, 1), 5), dtype=np.int32)
    st = call(items.ctypes.data, n.value)
    _check(st, "mla_decode_plan_preview")
    return items[:n.value], slots.value, ws.value


def mla_decode_plan_info(h):
    """Returns (num_items, max_splits, num_partials)."""
    n, ms, npart = ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
    _check(_lib.mla_decode_plan_info(h, ctypes.byref(n), ctypes.byref(ms), ctypes.byref(npart)),
           "mla_decode_plan_info", h)
    return n.value, ms.value, npart.value


def mla_decode_run(h, q: torch.Tensor, kv: torch.Tensor, kv_scales: Optional[torch.Tensor],
                   kv_indptr: torch.Tensor, out: torch.Tensor,
                   workspace: Optional[torch.Tensor] = None,
                   kv_page_indices: Optional[torch.Tensor] = None,
                   kv_last_page_len: Optional[torch.Tensor] = None,
                   stream: Optional[torch.cuda.Stream] = None) -> None:
    """Launches the planned decode on `stream` (default: torch's current stream).

    The library takes bare pointers, so the tensors' element types and row
    shapes are checked here: a wrong one would otherwise be read or written
    out of bounds on the device."""
    _check_run_tensors(q, out, kv_indptr, kv_page_indices, kv_last_page_len)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    stride = int(kv_scales.shape[-1]) if (kv_scales is not None and kv_scales.dtype == torch.uint8) else 0
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = _lib.mla_decode_run(h, _dptr(q), _dptr(kv), _dptr(kv_scales), stride, _dptr(kv_indptr),
                             _dptr(kv_page_indices), _dptr(kv_last_page_len), _dptr(out),
                             _dptr(workspace), ws_bytes, stream.cuda_stream)
    _check(st, "mla_decode_run", h)


def mla_decode_run_noalloc(h, q: torch.Tensor, kv: torch.Tensor, kv_scales: Optional[torch.Tensor],
                           kv_indptr: torch.Tensor, out: torch.Tensor,
                           kv_page_indices: Optional[torch.Tensor] = None,
                           kv_last_page_len: Optional[torch.Tensor] = None,
                           stream: Optional[torch.cuda.Stream] = None) -> None:
    """mla_decode_run with the library's own device scratch array in place of a
    workspace (no allocation anywhere; calls on one GPU must not overlap)."""
    _check_run_tensors(q, out, kv_indptr, kv_page_indices, kv_last_page_len)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    stride = int(kv_scales.shape[-1]) if (kv_scales is not None and kv_scales.dtype == torch.uint8) else 0
    st = _lib.mla_decode_run_noalloc(h, _dptr(q), _dptr(kv), _dptr(kv_scales), stride, _dptr(kv_indptr),
                                     _dptr(kv_page_indices), _dptr(kv_last_page_len), _dptr(out),
                                     stream.cuda_stream)
    _check(st, "mla_decode_run_noalloc", h)


class PreparedRun:
    """mla_decode_run with its arguments marshalled once (the same checks as
    mla_decode_run).  Each call launches the planned decode on the same
    tensors and stream, at the cost of one foreign call.  The tensors must stay
    alive and in place (the object holds references), and the handle must not
    be planned again while the object is used."""

    def __init__(self, h, q, kv, kv_scales, kv_indptr, out, workspace=None, kv_page_indices=None,
                 kv_last_page_len=None, stream=None):
        _check_run_tensors(q, out, kv_indptr, kv_page_indices, kv_last_page_len)
        if stream is None:
            stream = torch.cuda.current_stream(q.device)
        stride = int(kv_scales.shape[-1]) if (kv_scales is not None and kv_scales.dtype == torch.uint8) else 0
        ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
        self._keep = (q, kv, kv_scales, kv_indptr, out, workspace, kv_page_indices, kv_last_page_len, stream)
        self._h = h
        self._args = (h, _dptr(q), _dptr(kv), _dptr(kv_scales), stride, _dptr(kv_indptr), _dptr(kv_page_indices),
                      _dptr(kv_last_page_len), _dptr(out), _dptr(workspace), ws_bytes, stream.cuda_stream)

    def __call__(self) -> None:
        st = _lib.mla_decode_run(*self._args)
        if st != 0:
            _check(st, "mla_decode_run", self._h)


def mla_decode_set_query_format(h, query_format: str) -> None:
    """'exact' (default: the query as e4m3 hi + lo) or 'e4m3' (one e4m3 code per element)."""
    if query_format not in QUERY_FORMATS:
        raise ValueError(f"query_format must be one of {sorted(QUERY_FORMATS)}")
    _check(_lib.mla_decode_set_query_format(h, QUERY_FORMATS[query_format]), "mla_decode_set_query_format", h)


def mla_decode_set_profiling(h, enable: bool) -> None:
    _check(_lib.mla_decode_set_profiling(h, int(bool(enable))), "mla_decode_set_profiling", h)


def mla_decode_kernel_time_ms(h, which: int = 0) -> float:
    """Elapsed ms of kernel `which` (0 split stage, 1 merge) in the last timed run."""
    ms = ctypes.c_float()
    _check(_lib.mla_decode_kernel_time_ms(h, int(which), ctypes.byref(ms)),
           "mla_decode_kernel_time_ms", h)
    return ms.value


def mla_decode_kernel_resources(h, which: int = 0):
    v, l, s = ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
    _check(_lib.mla_decode_kernel_resources(h, int(which), ctypes.byref(v), ctypes.byref(l),
                                            ctypes.byref(s)), "mla_decode_kernel_resources", h)
    return {"vgprs": v.value, "lds_bytes": l.value, "scratch_bytes": s.value}


def mla_decode_destroy(h) -> None:
    _check(_lib.mla_decode_destroy(h), "mla_decode_destroy")


def mla_decode_last_error(h) -> str:
    return _lib.mla_decode_last_error(h).decode()


class MlaDecode:
    """Convenience owner of one handle plus its workspace (torch-allocated)."""

    def __init__(self, kv_dtype: str, page_size: int = 1, device: Optional[int] = None,
                 sm_scale: Optional[float] = None):
        self.device = torch.cuda.current_device() if device is None else int(device)
        self.kv_dtype = kv_dtype
        self.page_size = page_size
        self.h = mla_decode_create(self.device, kv_dtype, page_size, sm_scale=sm_scale)
        self.workspace: Optional[torch.Tensor] = None
        self.rows: Optional[int] = None

    def plan(self, kv_indptr_host, kv_last_page_len_host=None, split_override: int = 0,
             qo_indptr_host=None) -> int:
        self.rows = None
        if qo_indptr_host is None:
            nbytes = mla_decode_plan(self.h, kv_indptr_host, kv_last_page_len_host, split_override)
            rows = len(_host_i32(kv_indptr_host)) - 1
        else:
            nbytes = mla_decode_plan_multi(self.h, qo_indptr_host, kv_indptr_host, kv_last_page_len_host,
                                           split_override)
            rows = int(_host_i32(qo_indptr_host)[-1])
        self.rows = rows  # query / output rows the plan covers
        ip = _host_i32(kv_indptr_host)
        self._batch = len(ip) - 1
        self._indptr_end = int(ip[-1])
        if self.page_size == 1:
            self._total_tokens = int(ip[-1] - ip[0])
        else:
            lp = _host_i32(kv_last_page_len_host)
            n = np.diff(ip.astype(np.int64))
            self._total_tokens = int(np.where(n > 0, (n - 1) * self.page_size + lp[:len(n)], 0).sum())
        if nbytes and (self.workspace is None or self.workspace.numel() * 4 < nbytes):
            self.workspace = torch.empty((nbytes + 3) // 4, dtype=torch.float32,
                                         device=f"cuda:{self.device}")
        return nbytes

    def run(self, q, kv, kv_scales, kv_indptr, out, kv_page_indices=None, kv_last_page_len=None,
            stream=None) -> torch.Tensor:
        self._check_rows(q, out)
        self._check_cache(kv, kv_scales, kv_indptr, kv_page_indices, kv_last_page_len)
        mla_decode_run(self.h, q, kv, kv_scales, kv_indptr, out, self.workspace, kv_page_indices,
                       kv_last_page_len, stream)
        return out

    def prepare(self, q, kv, kv_scales, kv_indptr, out, kv_page_indices=None, kv_last_page_len=None,
                stream=None) -> PreparedRun:
        """A PreparedRun of this handle's current plan and workspace."""
        self._check_rows(q, out)
        self._check_cache(kv, kv_scales, kv_indptr, kv_page_indices, kv_last_page_len)
        return PreparedRun(self.h, q, kv, kv_scales, kv_indptr, out, self.workspace, kv_page_indices,
                           kv_last_page_len, stream)

    def _check_cache(self, kv, kv_scales, kv_indptr, kv_page_indices, kv_last_page_len) -> None:
        if self.rows is None:
            raise ValueError("run before a successful plan")
        check_cache_tensors(self.kv_dtype, self.page_size, self._batch, self._indptr_end, self._total_tokens, kv,
                            kv_scales, kv_indptr, kv_page_indices, kv_last_page_len)

    def _check_rows(self, q, out) -> None:
        if self.rows is not None and (q.numel() // (NUM_HEADS * QK_DIM) < self.rows
                                      or out.numel() // (NUM_HEADS * V_DIM) < self.rows):
            raise ValueError(f"the plan covers {self.rows} query rows; q {tuple(q.shape)} / out "
                             f"{tuple(out.shape)} hold fewer")

    def set_query_format(self, query_format: str) -> None:
        mla_decode_set_query_format(self.h, query_format)

    def close(self) -> None:
        if self.h:
            mla_decode_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def case_to_device(case, device="cuda") -> dict:
    """Device tensors for a synthetic case (see synth.DecodeCase)."""
    t = {
        "q": torch.from_numpy(case.q_bits.view(np.int16)).view(torch.bfloat16).to(device),
        "kv": torch.from_numpy(case.kv).to(device),
        "kv_indptr": torch.from_numpy(case.kv_indptr.astype(np.int32)).to(device),
        "kv_page_indices": None,
        "kv_last_page_len": None,
    }
    if case.kv_dtype == "fp8":
        t["kv_scales"] = torch.tensor([case.kv_scale], dtype=torch.float32, device=device)
    elif case.kv_dtype == "mxfp4":
        t["kv_scales"] = torch.from_numpy(case.kv_scales).to(device)
    else:
        t["kv_scales"] = None
    if case.page_size > 1:
        t["kv_page_indices"] = torch.from_numpy(case.kv_page_indices.astype(np.int32)).to(device)
        t["kv_last_page_len"] = torch.from_numpy(case.kv_last_page_len.astype(np.int32)).to(device)
    return t
