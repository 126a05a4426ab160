"""fp64 CPU oracle for MLA decode (single- and multi-token) -- TEST INFRASTRUCTURE ONLY.

Only the tests, the package smoke check and the benchmark's CPU-baseline leg
may import this package.  The product path (``latent_attention_decode_amd``)
never imports it, and this package imports nothing from the product: inputs
are plain numpy arrays (or any object with the same attribute names as the
synthetic-input generator's case record).

The arithmetic lives in ``mla_oracle.c`` (plain C, double precision); this
module only marshals arrays through ctypes.  ``build.py`` compiles it.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np

from . import build as _build

_FMT = {"bf16": 0, "fp8": 1, "mxfp4": 2}


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else ctypes.c_void_p(a.ctypes.data)


class OracleLib:
    """ctypes view of one build of ``mla_oracle.c`` (the default build, or a
    variant compiled by a test)."""

    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        P = ctypes.c_void_p
        lib.oracle_bf16_to_f64.argtypes = [ctypes.c_uint16]
        lib.oracle_bf16_to_f64.restype = ctypes.c_double
        for name in ("oracle_e4m3_to_f64", "oracle_e8m0_to_f64", "oracle_e2m1_to_f64"):
            getattr(lib, name).argtypes = [ctypes.c_uint8]
            getattr(lib, name).restype = ctypes.c_double
        lib.oracle_dequant_rows.argtypes = [ctypes.c_int, ctypes.c_int, P, P, ctypes.c_int64,
                                            ctypes.c_double, P, ctypes.c_int64, P]
        lib.oracle_dequant_rows.restype = ctypes.c_int
        lib.oracle_mla_decode.argtypes = [P, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                          ctypes.c_double, ctypes.c_int, P, ctypes.c_double, P,
                                          ctypes.c_int64, P, P, P, ctypes.c_int, P, P, P,
                                          ctypes.c_int, ctypes.c_int, P, P]
        lib.oracle_mla_decode.restype = ctypes.c_int
        lib.oracle_mla_decode_multi.argtypes = [P, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                                ctypes.c_double, ctypes.c_int, P, ctypes.c_double, P,
                                                ctypes.c_int64, P, P, P, ctypes.c_int, P, P,
                                                ctypes.c_int, ctypes.c_int, P, P]
        lib.oracle_mla_decode_multi.restype = ctypes.c_int
        lib.oracle_round_query_e4m3.argtypes = [P, ctypes.c_int64, ctypes.c_int, ctypes.c_int, P]
        lib.oracle_round_query_e4m3.restype = ctypes.c_int
        self.lib = lib
        self.path = path

    def bf16_to_f64(self, bits: int) -> float:
        return self.lib.oracle_bf16_to_f64(int(bits))

    def e4m3_to_f64(self, code: int) -> float:
        return self.lib.oracle_e4m3_to_f64(int(code))

    def e8m0_to_f64(self, code: int) -> float:
        return self.lib.oracle_e8m0_to_f64(int(code))

    def e2m1_to_f64(self, nibble: int) -> float:
        return self.lib.oracle_e2m1_to_f64(int(nibble))

    def round_query_e4m3(self, q_bits: np.ndarray) -> np.ndarray:
        """The query rounded to one e4m3 code per element under the power-of-two
        scale of each (row, head), as bf16 bit patterns of the same shape."""
        q_bits = np.ascontiguousarray(q_bits, dtype=np.uint16)
        rows, nh, qk_dim = q_bits.shape
        out = np.empty_like(q_bits)
        rc = self.lib.oracle_round_query_e4m3(_ptr(q_bits), rows, nh, qk_dim, _ptr(out))
        if rc:
            raise ValueError(f"oracle_round_query_e4m3 failed (code {rc})")
        return out

    def dequant_rows(self, kv_dtype: str, kv: np.ndarray, rows: Sequence[int], *,
                     kv_scale: float = 1.0, kv_scales: Optional[np.ndarray] = None,
                     qk_dim: int = 576) -> np.ndarray:
        """Dequantised fp64 rows [len(rows), qk_dim] of a stored cache."""
        kv = np.ascontiguousarray(kv, dtype=np.uint8)
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        sc = None if kv_scales is None else np.ascontiguousarray(kv_scales, dtype=np.uint8)
        stride = 0 if sc is None else sc.shape[1]
        out = np.empty((rows.size, qk_dim), dtype=np.float64)
        rc = self.lib.oracle_dequant_rows(_FMT[kv_dtype], qk_dim, _ptr(kv), _ptr(sc), stride,
                                          float(kv_scale), _ptr(rows), rows.size, _ptr(out))
        if rc:
            raise ValueError("oracle_dequant_rows rejected its arguments")
        return out

    def mla_decode(self, q_bits: np.ndarray, kv_dtype: str, kv: np.ndarray, kv_indptr: np.ndarray,
                   *, kv_scale: float = 1.0, kv_scales: Optional[np.ndarray] = None,
                   page_size: int = 1, kv_page_indices: Optional[np.ndarray] = None,
                   kv_last_page_len: Optional[np.ndarray] = None, v_dim: int = 512,
                   sm_scale: Optional[float] = None,
                   splits: Optional[Sequence[Sequence[int]]] = None,
                   batches: Optional[Sequence[int]] = None, nthreads: Optional[int] = None,
                   qo_indptr: Optional[np.ndarray] = None):
        """Exact decode.  Returns (out [rows, nh, v_dim] fp64, lse [rows, nh] fp64).

        q_bits: uint16 bf16 patterns [rows, nh, qk_dim]; one row per sequence,
        or with ``qo_indptr`` (multi-token decode, int32 [bs + 1]) rows
        qo_indptr[b] .. qo_indptr[b + 1] - 1 for the query tokens of sequence
        b.  ``splits[b]`` (split mode, single-token only) lists the exclusive
        end token of each range of sequence b, in order, the last one being
        the sequence length.  ``batches`` restricts the work to those
        sequences (the other rows are NaN).
        """
        q_bits = np.ascontiguousarray(q_bits, dtype=np.uint16)
        rows, nh, qk_dim = q_bits.shape
        bs = rows if qo_indptr is None else len(qo_indptr) - 1
        qo = None if qo_indptr is None else np.ascontiguousarray(qo_indptr, dtype=np.int32)
        if qo is not None and (qo[-1] != rows or splits is not None):
            raise ValueError("qo_indptr must end at the number of query rows, without split mode")
        if sm_scale is None:
            sm_scale = 1.0 / np.sqrt(float(qk_dim))
        kv = np.ascontiguousarray(kv, dtype=np.uint8)
        indptr = np.ascontiguousarray(kv_indptr, dtype=np.int32)
        pages = None if kv_page_indices is None else np.ascontiguousarray(kv_page_indices, dtype=np.int32)
        last = None if kv_last_page_len is None else np.ascontiguousarray(kv_last_page_len, dtype=np.int32)
        sc = None if kv_scales is None else np.ascontiguousarray(kv_scales, dtype=np.uint8)
        stride = 0 if sc is None else sc.shape[1]
        split_indptr = split_bounds = None
        if splits is not None:
            counts = [len(s) for s in splits]
            split_indptr = np.zeros(bs + 1, dtype=np.int32)
            split_indptr[1:] = np.cumsum(counts)
            split_bounds = np.ascontiguousarray(
                np.concatenate([np.asarray(s, dtype=np.int32) for s in splits]) if sum(counts)
                else np.zeros(1, dtype=np.int32), dtype=np.int32)
        sel = None if batches is None else np.ascontiguousarray(batches, dtype=np.int32)
        n_sel = 0 if sel is None else sel.size
        out = np.full((rows, nh, v_dim), np.nan, dtype=np.float64)
        lse = np.full((rows, nh), np.nan, dtype=np.float64)
        if nthreads is None:
            nthreads = max(1, len(os.sched_getaffinity(0)))
        if qo is None:
            rc = self.lib.oracle_mla_decode(_ptr(q_bits), bs, nh, qk_dim, v_dim, float(sm_scale),
                                            _FMT[kv_dtype], _ptr(kv), float(kv_scale), _ptr(sc), stride,
                                            _ptr(indptr), _ptr(pages), _ptr(last), int(page_size),
                                            _ptr(split_indptr), _ptr(split_bounds), _ptr(sel), n_sel,
                                            int(nthreads), _ptr(out), _ptr(lse))
        else:
            rc = self.lib.oracle_mla_decode_multi(_ptr(q_bits), bs, nh, qk_dim, v_dim, float(sm_scale),
                                                  _FMT[kv_dtype], _ptr(kv), float(kv_scale), _ptr(sc), stride,
                                                  _ptr(indptr), _ptr(pages), _ptr(last), int(page_size),
                                                  _ptr(qo), _ptr(sel), n_sel, int(nthreads), _ptr(out),
                                                  _ptr(lse))
        if rc:
            raise ValueError(f"oracle_mla_decode failed (code {rc})")
        return out, lse

    def decode_case(self, case, **kw):
        """Oracle decode of a synthetic case record (duck-typed attributes)."""
        return self.mla_decode(case.q_bits, case.kv_dtype, case.kv, case.kv_indptr,
                               kv_scale=case.kv_scale, kv_scales=case.kv_scales,
                               page_size=case.page_size, kv_page_indices=case.kv_page_indices,
                               kv_last_page_len=case.kv_last_page_len,
                               qo_indptr=getattr(case, "qo_indptr", None), **kw)


_default: Optional[OracleLib] = None


def default() -> OracleLib:
    global _default
    if _default is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        _default = OracleLib(_build.LIB)
    return _default


def bf16_to_f64(bits):
    return default().bf16_to_f64(bits)


def e4m3_to_f64(code):
    return default().e4m3_to_f64(code)


def e8m0_to_f64(code):
    return default().e8m0_to_f64(code)


def e2m1_to_f64(nibble):
    return default().e2m1_to_f64(nibble)


def round_query_e4m3(*a, **kw):
    return default().round_query_e4m3(*a, **kw)


def dequant_rows(*a, **kw):
    return default().dequant_rows(*a, **kw)


def mla_decode(*a, **kw):
    return default().mla_decode(*a, **kw)


def decode_case(case, **kw):
    return default().decode_case(case, **kw)
