"""Seeded synthetic inputs for single-token MLA decode.

This module only *makes* inputs: standard-normal query and latent-cache values,
stored in the three cache formats (bf16, fp8-e4m3 with one fp32 scale per
tensor, MXFP4 with one e8m0 scale per 32 elements), laid out contiguously or
through a (shuffled) page table.  It holds none of the attention arithmetic and
imports nothing else from this package, so both the HIP path and the fp64
oracle can take their inputs from it.

Shapes follow the amd-mixed-mla submissions (16 query heads, one shared latent
KV head of width 576 = 512 latent + 64 rope, V = the first 512 columns of the
same row) -- see submission 599694 ("overhead elimination"), module constants,
and submission 727205 ("v25: LEAN"), module constants.

Every array returned is a host numpy array; callers move them to the device.
"""

from __future__ import annotations

import dataclasses
from typing import Optional, Sequence

import numpy as np
import torch

NUM_HEADS = 16
QK_DIM = 576
V_DIM = 512
MX_BLOCK = 32
MX_BLOCKS = QK_DIM // MX_BLOCK  # 18 e8m0 scales per row

FORMATS = ("bf16", "fp8", "mxfp4")
ROW_BYTES = {"bf16": 2 * QK_DIM, "fp8": QK_DIM, "mxfp4": QK_DIM // 2}

FP8_MAX = 448.0  # largest finite e4m3fn value
E2M1_GRID = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)  # codes 0..7 (OCP MX v1.0)


@dataclasses.dataclass
class DecodeCase:
    """One decode call's worth of inputs (host arrays).

    q_bits            uint16 [rows, 16, 576]: bf16 bit patterns of the query (rows =
                      batch, or the query tokens of all sequences with qo_indptr).
    kv                uint8  [rows, row_bytes]: the cache rows as stored.
    kv_scale          fp32 per-tensor dequant scale (fp8); 1.0 otherwise.
    kv_scales         uint8  [rows, scale_stride] e8m0 block scales (mxfp4) or None.
    kv_indptr         int32  [batch+1]: token offsets (page_size 1) or page offsets.
    kv_page_indices   int32  [num_pages_used] physical page ids, or None (page_size 1).
    kv_last_page_len  int32  [batch] valid tokens in each last page, or None.
    lens              int64  [batch] tokens per sequence.
    qo_indptr         int32  [batch+1] query rows per sequence (multi-token decode), or None.
    """

    kv_dtype: str
    batch: int
    page_size: int
    lens: np.ndarray
    q_bits: np.ndarray
    kv: np.ndarray
    kv_scale: float
    kv_scales: Optional[np.ndarray]
    kv_indptr: np.ndarray
    kv_page_indices: Optional[np.ndarray]
    kv_last_page_len: Optional[np.ndarray]
    qo_indptr: Optional[np.ndarray] = None

    @property
    def rows(self) -> int:
        """Query (and output) rows."""
        return int(self.q_bits.shape[0])

    @property
    def scale_stride(self) -> int:
        return 0 if self.kv_scales is None else int(self.kv_scales.shape[1])

    @property
    def total_tokens(self) -> int:
        return int(self.lens.sum())

    def token_rows(self, b: int) -> np.ndarray:
        """Physical row of each logical token of sequence ``b`` (layout only)."""
        n = int(self.lens[b])
        j = np.arange(n, dtype=np.int64)
        if self.page_size == 1:
            return int(self.kv_indptr[b]) + j
        pages = self.kv_page_indices[int(self.kv_indptr[b]) + j // self.page_size]
        return pages.astype(np.int64) * self.page_size + j % self.page_size

    def kv_algorithmic_bytes(self) -> int:
        per_row = ROW_BYTES[self.kv_dtype] + (MX_BLOCKS if self.kv_dtype == "mxfp4" else 0)
        return self.total_tokens * per_row


# ----------------------------------------------------------------------------
# encoders (input preparation only)
# ----------------------------------------------------------------------------

def to_bf16_bits(x: torch.Tensor) -> np.ndarray:
    """fp32 -> bf16 (round to nearest even, torch's cast) -> uint16 bit patterns."""
    return x.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def encode_fp8_per_tensor(x: torch.Tensor) -> tuple[np.ndarray, float]:
    """Per-tensor fp8-e4m3fn: scale = amax/448 (fp32); codes = e4m3(clamp(x/scale))."""
    amax = float(x.abs().max()) if x.numel() else 1.0
    scale = np.float32(amax / FP8_MAX) if amax > 0 else np.float32(1.0)
    y = (x / torch.tensor(scale, dtype=torch.float32)).clamp(-FP8_MAX, FP8_MAX)
    codes = y.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return codes, float(scale)


def _e2m1_codes(y: torch.Tensor) -> torch.Tensor:
    """Nearest e2m1 code (ties to the even code), saturating at +-6."""
    grid = torch.tensor(E2M1_GRID, dtype=torch.float32)
    a = y.abs().clamp(max=6.0)
    hi = torch.searchsorted(grid, a.contiguous(), right=False).clamp(max=7)
    lo = (hi - 1).clamp(min=0)
    d_lo = a - grid[lo]
    d_hi = grid[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = torch.where(pick_hi, hi, lo)
    sign = (y < 0).to(torch.int64) << 3
    return (code | sign).to(torch.uint8)


def encode_mxfp4(x: torch.Tensor, scale_stride: int = MX_BLOCKS) -> tuple[np.ndarray, np.ndarray]:
    """MXFP4 rows: 32-element blocks share one e8m0 exponent.

    The block exponent follows the query quantiser of submission 727205
    ("v25: LEAN", device helper ``qquant32``): take the block amax, round it up
    to the next power of two when its two leading mantissa bits are both set,
    and use that exponent minus 2, so amax/scale stays below 8 and the largest
    e2m1 magnitude (6) saturates.  Element 2i is the low nibble of byte i.
    Returns (packed [rows, 288] u8, scales [rows, scale_stride] u8); unused
    scale columns hold 127 (= 1.0).
    """
    rows = x.shape[0]
    blk = x.reshape(rows, MX_BLOCKS, MX_BLOCK).to(torch.float32)
    amax = blk.abs().amax(dim=2)
    bits = amax.contiguous().view(torch.int32).to(torch.int64)
    rounded = (bits + 0x200000) & 0x7F800000
    exp_field = rounded >> 23
    su = torch.where(amax > 0, exp_field - 129, torch.full_like(exp_field, -127))
    su = su.clamp(-127, 127)
    e8 = (su + 127).to(torch.int64)
    if rows and (int(e8.min()) <= 0 or int(e8.max()) >= 255):
        raise ValueError("block scale outside the e8m0 range this generator emits (1..254)")
    scale = torch.pow(torch.tensor(2.0, dtype=torch.float64), (e8 - 127).to(torch.float64))
    y = (blk.to(torch.float64) / scale.unsqueeze(2)).to(torch.float32)
    codes = _e2m1_codes(y).reshape(rows, QK_DIM).to(torch.int64)
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).to(torch.uint8).numpy()
    scales = np.full((rows, scale_stride), 127, dtype=np.uint8)
    scales[:, :MX_BLOCKS] = e8.to(torch.uint8).numpy()
    return packed, scales


# ----------------------------------------------------------------------------
# case builder
# ----------------------------------------------------------------------------

def _poison_rows(kv_dtype: str, kv: np.ndarray, scales: Optional[np.ndarray], rows: np.ndarray) -> None:
    """Fill cache rows that no sequence references with NaN-producing bytes."""
    if rows.size == 0:
        return
    if kv_dtype == "fp8":
        kv[rows] = 0x7F  # e4m3fn NaN
    elif kv_dtype == "bf16":
        kv[rows] = np.frombuffer(np.array([0x7FC0], dtype="<u2").tobytes() * QK_DIM, dtype=np.uint8)
    else:
        kv[rows] = 0x77  # e2m1 code 7 (=6.0) everywhere
        scales[rows] = 0xFF  # e8m0 NaN


def make_case(kv_dtype: str,
              lens: Sequence[int],
              *,
              seed: int,
              page_size: int = 1,
              shuffle_pages: bool = False,
              scale_stride: int = MX_BLOCKS,
              guard_rows: int = 0,
              q_values: Optional[np.ndarray] = None,
              kv_values: Optional[np.ndarray] = None,
              q_lens: Optional[Sequence[int]] = None) -> DecodeCase:
    """Build a seeded decode case.

    Values: q ~ N(0,1) [batch,16,576] and one N(0,1) latent row per token, in
    logical token order (sequence 0 first), both drawn from one
    ``torch.Generator`` seeded with ``seed`` (q first, then the cache, then the
    page permutation).  ``q_values`` / ``kv_values`` (fp32, same shapes)
    replace the draws for structured tests.  ``q_lens`` (multi-token decode)
    gives each sequence that many query rows: q is then [sum(q_lens), 16, 576]
    and the case carries qo_indptr.  Unreferenced rows -- the slack of
    each last page and ``guard_rows`` extra rows at the end -- are filled with
    NaN-producing bytes so that reading them shows up in the output.
    """
    if kv_dtype not in FORMATS:
        raise ValueError(f"kv_dtype must be one of {FORMATS}")
    if page_size < 1 or (page_size & (page_size - 1)):
        raise ValueError("page_size must be a power of two")
    lens_np = np.asarray(lens, dtype=np.int64)
    batch = int(lens_np.size)
    total = int(lens_np.sum())
    g = torch.Generator().manual_seed(int(seed))

    qo_indptr = None
    rows = batch
    if q_lens is not None:
        ql = np.asarray(q_lens, dtype=np.int64)
        if ql.size != batch or np.any(ql < 0) or np.any(ql > lens_np):
            raise ValueError("q_lens: one count per sequence, 0 <= q_len <= its length")
        qo_indptr = np.zeros(batch + 1, dtype=np.int32)
        qo_indptr[1:] = np.cumsum(ql)
        rows = int(qo_indptr[-1])
    if q_values is None:
        q = torch.randn((rows, NUM_HEADS, QK_DIM), generator=g, dtype=torch.float32)
    else:
        q = torch.as_tensor(np.asarray(q_values, dtype=np.float32)).reshape(rows, NUM_HEADS, QK_DIM)
    if kv_values is None:
        x = torch.randn((total, QK_DIM), generator=g, dtype=torch.float32)
    else:
        x = torch.as_tensor(np.asarray(kv_values, dtype=np.float32)).reshape(total, QK_DIM)

    q_bits = to_bf16_bits(q)

    # logical -> physical rows
    if page_size == 1:
        indptr = np.zeros(batch + 1, dtype=np.int32)
        indptr[1:] = np.cumsum(lens_np)
        phys = np.arange(total, dtype=np.int64)
        n_rows = total + guard_rows
        page_indices = None
        last_len = None
    else:
        pages = (lens_np + page_size - 1) // page_size
        pool = int(pages.sum())
        perm = (torch.randperm(pool, generator=g).numpy().astype(np.int64)
                if shuffle_pages else np.arange(pool, dtype=np.int64))
        indptr = np.zeros(batch + 1, dtype=np.int32)
        indptr[1:] = np.cumsum(pages)
        page_indices = perm.astype(np.int32)
        last_len = np.where(pages > 0, lens_np - page_size * (pages - 1), 0).astype(np.int32)
        phys_parts = []
        for b in range(batch):
            j = np.arange(int(lens_np[b]), dtype=np.int64)
            pg = perm[int(indptr[b]) + j // page_size]
            phys_parts.append(pg * page_size + j % page_size)
        phys = np.concatenate(phys_parts) if phys_parts else np.zeros(0, dtype=np.int64)
        n_rows = pool * page_size + guard_rows

    row_bytes = ROW_BYTES[kv_dtype]
    kv = np.zeros((n_rows, row_bytes), dtype=np.uint8)
    scales = None
    kv_scale = 1.0
    if kv_dtype == "bf16":
        kv[phys] = to_bf16_bits(x).view(np.uint8).reshape(total, row_bytes)
    elif kv_dtype == "fp8":
        codes, kv_scale = encode_fp8_per_tensor(x)
        kv[phys] = codes
    else:
        packed, sc = encode_mxfp4(x, scale_stride)
        kv[phys] = packed
        scales = np.full((n_rows, scale_stride), 127, dtype=np.uint8)
        scales[phys] = sc

    used = np.zeros(n_rows, dtype=bool)
    used[phys] = True
    _poison_rows(kv_dtype, kv, scales, np.nonzero(~used)[0])

    return DecodeCase(kv_dtype=kv_dtype, batch=batch, page_size=page_size, lens=lens_np,
                      q_bits=q_bits, kv=kv, kv_scale=float(kv_scale), kv_scales=scales,
                      kv_indptr=indptr, kv_page_indices=page_indices, kv_last_page_len=last_len,
                      qo_indptr=qo_indptr)


def ragged_lens(batch: int, lo: int, hi: int, seed: int) -> np.ndarray:
    """Sequence lengths drawn uniformly from [lo, hi] (inclusive), seeded."""
    g = torch.Generator().manual_seed(int(seed))
    return torch.randint(lo, hi + 1, (batch,), generator=g).numpy().astype(np.int64)


# The benchmark workloads: (kv_dtype, batch, kv_len or (lo, hi), page_size, shuffled, seed).
CONFIGS = {
    "bs4_kv1024_bf16": ("bf16", 4, 1024, 1, False, 1000),
    "bs64_kv1024_fp8": ("fp8", 64, 1024, 1, False, 1001),
    "bs4_kv8192_fp8": ("fp8", 4, 8192, 1, False, 1002),
    "bs64_kv8192_mxfp4": ("mxfp4", 64, 8192, 1, False, 1003),
    "bs256_ragged1024-8192_fp8_paged2": ("fp8", 256, (1024, 8192), 2, True, 1004),
    "bs32_kv8192_fp8": ("fp8", 32, 8192, 1, False, 1005),
    "bs64_kv8192_fp8": ("fp8", 64, 8192, 1, False, 1006),
    # the largest shape of the leaderboard set (256 x 8192), in MXFP4 (the shape
    # submission 727205 reports its split kernel's time for) and in fp8
    "bs256_kv8192_mxfp4": ("mxfp4", 256, 8192, 1, False, 1009),
    "bs256_kv8192_fp8": ("fp8", 256, 8192, 1, False, 1010),
    # a bf16 cache at a serving size (the listed bf16 case is 4 x 1024)
    "bs64_kv8192_bf16": ("bf16", 64, 8192, 1, False, 1011),
    # multi-token decode: every sequence has q query tokens (its last q positions)
    "bs64_kv8192_q2_fp8": ("fp8", 64, 8192, 1, False, 1007, 2),
    "bs16_kv8192_q4_fp8": ("fp8", 16, 8192, 1, False, 1008, 4),
}


def config_lens(name: str) -> np.ndarray:
    kv_dtype, batch, kv_len, _ps, _sh, seed = CONFIGS[name][:6]
    if isinstance(kv_len, tuple):
        return ragged_lens(batch, kv_len[0], kv_len[1], seed + 7919)
    return np.full(batch, kv_len, dtype=np.int64)


def config_case(name: str) -> DecodeCase:
    kv_dtype, batch, _kv_len, ps, shuffled, seed = CONFIGS[name][:6]
    q = CONFIGS[name][6] if len(CONFIGS[name]) > 6 else 1
    return make_case(kv_dtype, config_lens(name), seed=seed, page_size=ps, shuffle_pages=shuffled,
                     q_lens=None if q == 1 else np.full(batch, q))
