"""C-ABI library: exported symbols, host-side validation and the planner (CPU only)."""

import ctypes
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mla_decode.h")


@pytest.fixture(scope="module")
def B():
    from latent_attention_decode_amd import binding
    return binding


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mla_[a-z_0-9]+)\s*\(", text)))


def test_header_symbols_are_exported(B):
    names = _declared_functions()
    assert "mla_decode_run" in names and "mla_decode_plan" in names
    lib = ctypes.CDLL(B.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(B.EXPORTED) == names


def test_scratch_size_matches_the_header(B):
    m = re.search(r"#define\s+MLA_SCRATCH_BYTES\s+\((\d+)u\s*<<\s*(\d+)\)", open(HEADER).read())
    assert m and int(m.group(1)) << int(m.group(2)) == B.MLA_SCRATCH_BYTES


def test_version_and_status_strings(B):
    assert B.mla_decode_version() >= 10000
    for code, name in B.STATUS.items():
        assert B.mla_status_string(code) == name


def test_create_validates_arguments(B):
    with pytest.raises(B.MlaError) as e:
        B.mla_decode_create(0, "fp8", num_heads=8)
    assert e.value.status == 2
    with pytest.raises(B.MlaError) as e:
        B.mla_decode_create(0, "fp8", page_size=3)
    assert e.value.status == 2
    with pytest.raises(B.MlaError) as e:
        B.mla_decode_create(0, "fp8", sm_scale=-1.0)
    assert e.value.status == 1
    with pytest.raises(B.MlaError) as e:
        B.mla_decode_create(-1, "fp8")
    assert e.value.status == 1
    with pytest.raises(B.MlaError):
        B.mla_decode_create(0, 7)
    h = B.mla_decode_create(0, "fp8")  # touches no GPU
    B.mla_decode_destroy(h)
    B.mla_decode_destroy(None)


def test_query_format_setting(B):
    """The query format: exact by default, one e4m3 code on request for fp8
    and MXFP4 caches; refused for bf16 caches and for unknown values (no GPU)."""
    for fmt in ("fp8", "mxfp4"):
        h = B.mla_decode_create(0, fmt)
        try:
            B.mla_decode_set_query_format(h, "e4m3")
            B.mla_decode_set_query_format(h, "exact")
            for bad in (2, -1, 7):
                assert B._lib.mla_decode_set_query_format(h, bad) == 1
                assert b"query_format" in B._lib.mla_decode_last_error(h)
        finally:
            B.mla_decode_destroy(h)
    h = B.mla_decode_create(0, "bf16")
    try:
        B.mla_decode_set_query_format(h, "exact")
        with pytest.raises(B.MlaError) as e:
            B.mla_decode_set_query_format(h, "e4m3")
        assert e.value.status == 2
    finally:
        B.mla_decode_destroy(h)
    assert B._lib.mla_decode_set_query_format(None, 0) == 1
    with pytest.raises(ValueError):
        B.mla_decode_set_query_format(None, "fp4")


def test_plan_and_run_validate_before_any_gpu_call(B):
    h = B.mla_decode_create(0, "fp8", page_size=2)
    try:
        with pytest.raises(B.MlaError) as e:  # decreasing indptr
            B.mla_decode_plan(h, [0, 5, 3], [1, 1])
        assert e.value.status == 1 and "non-decreasing" in str(e.value)
        with pytest.raises(B.MlaError) as e:  # last page length outside [1, page_size]
            B.mla_decode_plan(h, [0, 2, 3], [3, 1])
        assert e.value.status == 1
        with pytest.raises(B.MlaError) as e:  # missing last_page_len for a paged cache
            B.mla_decode_plan(h, [0, 2, 3], None)
        assert e.value.status == 1
        with pytest.raises(B.MlaError) as e:
            B.mla_decode_plan(h, [0], [])  # batch 0
        assert e.value.status == 1
        # run before a successful plan: raw call with dummy pointers
        st = B._lib.mla_decode_run(h, 16, 16, 16, 0, 16, 16, 16, 16, None, 0, None)
        assert st == 3
        st = B._lib.mla_decode_run_noalloc(h, 16, 16, 16, 0, 16, 16, 16, 16, None)
        assert st == 3 and "before a successful plan" in B.mla_decode_last_error(h)
        assert B._lib.mla_decode_run_noalloc(None, 16, 16, 16, 0, 16, 16, 16, 16, None) == 1
        with pytest.raises(B.MlaError) as e:
            B.mla_decode_plan_info(h)
        assert e.value.status == 3
    finally:
        B.mla_decode_destroy(h)


def test_run_rejects_wrong_tensor_types_and_shapes(B):
    """The binding checks element types and row shapes before any pointer reaches the
    library (which takes bare pointers and could not tell)."""
    import torch
    q = torch.zeros((2, 16, 576), dtype=torch.bfloat16)
    out = torch.zeros((2, 16, 512), dtype=torch.bfloat16)
    ip = torch.tensor([0, 4, 8], dtype=torch.int32)
    bad = [
        (q.float(), out, ip, "q must be bf16"),
        (q[:, :, :512], out, ip, "q must be bf16"),
        (q, out.view(2, 16, 16, 32), ip, "out must be bf16"),
        (q, out[:1], ip, "different numbers of rows"),
        (q, out, ip.long(), "must be int32"),
    ]
    for qq, oo, ii, msg in bad:
        with pytest.raises(ValueError, match=msg):
            B.mla_decode_run(None, qq, None, None, ii, oo)
        with pytest.raises(ValueError, match=msg):  # a prepared run checks the same, once
            B.PreparedRun(None, qq, None, None, ii, oo)


def test_cache_tensors_are_checked_against_the_plan(B):
    """The handle's format and plan fix the cache's element type, row bytes and
    row count, the page table's length and the scales; each mismatch is refused
    before a pointer reaches the library."""
    import torch
    u8 = torch.uint8
    ip = torch.tensor([0, 4, 8], dtype=torch.int32)
    fp8_scale = torch.ones(1, dtype=torch.float32)
    ok = dict(kv_dtype="fp8", page_size=1, batch=2, indptr_end=8, total_tokens=8,
              kv=torch.zeros((8, 576), dtype=u8), kv_scales=fp8_scale, kv_indptr=ip)
    B.check_cache_tensors(**ok)
    bad = [
        (dict(kv=torch.zeros((8, 576), dtype=torch.bfloat16)), "cannot be a"),          # bf16 tensor, fp8 handle
        (dict(kv=torch.zeros((8, 288), dtype=u8)), "rows are 576 bytes"),
        (dict(kv=torch.zeros((7, 576), dtype=u8)), "up to 8"),                          # too few rows
        (dict(kv=None), "kv is None"),
        (dict(kv_scales=None), "per-tensor scale"),
        (dict(kv_scales=torch.ones(1, dtype=torch.float64)), "per-tensor scale"),
        (dict(kv_indptr=ip[:2]), "kv_indptr needs 3"),
        (dict(kv_dtype="bf16", kv=torch.zeros((8, 576), dtype=u8)), "rows are 1152 bytes"),
        (dict(kv_dtype="mxfp4", kv=torch.zeros((8, 288), dtype=u8), kv_scales=torch.zeros((8, 17), dtype=u8)),
         "stride >= 18"),
        (dict(kv_dtype="mxfp4", kv=torch.zeros((8, 288), dtype=u8), kv_scales=torch.zeros((7, 18), dtype=u8)),
         "7 rows of scales"),
        (dict(kv_dtype="mxfp4", kv=torch.zeros((8, 288), dtype=u8), kv_scales=fp8_scale), "e8m0"),
        (dict(page_size=4, indptr_end=3, kv=torch.zeros((12, 576), dtype=u8),
              kv_page_indices=torch.zeros(2, dtype=torch.int32), kv_last_page_len=torch.ones(2, dtype=torch.int32)),
         "3 page-table entries"),
        (dict(page_size=4, indptr_end=3, kv=torch.zeros((12, 576), dtype=u8),
              kv_page_indices=torch.zeros(3, dtype=torch.int32), kv_last_page_len=None), "kv_last_page_len"),
        (dict(page_size=4, indptr_end=3, kv=torch.zeros((3, 576), dtype=u8),
              kv_page_indices=torch.zeros(3, dtype=torch.int32), kv_last_page_len=torch.ones(2, dtype=torch.int32)),
         "less than one page"),
    ]
    for change, msg in bad:
        with pytest.raises(ValueError, match=msg):
            B.check_cache_tensors(**{**ok, **change})
    # accepted: the bf16 cache as bf16 elements or bytes, an empty plan without a cache
    B.check_cache_tensors(**{**ok, "kv_dtype": "bf16", "kv": torch.zeros((8, 576), dtype=torch.bfloat16)})
    B.check_cache_tensors(**{**ok, "kv_dtype": "bf16", "kv": torch.zeros((8, 1152), dtype=u8)})
    B.check_cache_tensors(**{**ok, "total_tokens": 0, "indptr_end": 0, "kv": None})


def _check_cover(items, lens, slots):
    """Every token of every sequence is in exactly one item; slots are a partition;
    items are listed workgroup by workgroup."""
    wg = [it[4] for it in items]
    assert wg == sorted(wg) and (not wg or (wg[0] == 0 and set(wg) == set(range(wg[-1] + 1))))
    items = [it[:4] for it in items]
    seen = {b: np.zeros(n, dtype=np.int32) for b, n in enumerate(lens)}
    used_slots = []
    empty = [b for b, t0, t1, s in items if s == -2]
    assert sorted(empty) == [b for b, n in enumerate(lens) if n == 0]  # one zero-writer each
    items = [it for it in items if it[3] != -2]
    for b, t0, t1, s in items:
        assert 0 <= t0 < t1 <= lens[b]
        seen[b][t0:t1] += 1
        if s >= 0:
            used_slots.append(s)
    for b, n in enumerate(lens):
        assert np.all(seen[b] == 1), b
    assert sorted(used_slots) == list(range(slots))
    # a sequence with a single item writes its output directly
    per_seq = {}
    for b, t0, t1, s in items:
        per_seq.setdefault(b, []).append(s)
    for b, ss in per_seq.items():
        assert (ss == [-1]) if len(ss) == 1 else all(x >= 0 for x in ss)
        if len(ss) > 1:  # a sequence's slots are consecutive
            assert sorted(ss) == list(range(min(ss), min(ss) + len(ss)))


@pytest.mark.parametrize("lens", [
    [1024] * 4, [1024] * 64, [8192] * 4, [8192] * 32, [8192] * 64, [1] * 3, [0, 5, 0, 700],
    [63, 64, 65, 127, 128, 129], list(range(1, 300, 7)),
])
def test_planner_covers_every_token_once(B, lens):
    indptr = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    items, slots, ws = B.mla_decode_plan_preview(indptr, num_cus=256, blocks_per_cu=2)
    _check_cover(items.tolist(), lens, slots)
    assert ws == slots * 16 * 513 * 4
    # one item per workgroup (these batches are too small for bins), longest first
    assert np.all(items[:, 4] == np.arange(len(items)))
    sizes = items[:, 2] - items[:, 1]
    assert np.all(np.diff(sizes) <= 0)


def test_planner_paged_lengths(B):
    ps = 4
    lens = [9, 4, 1, 0, 16]
    pages = [(n + ps - 1) // ps for n in lens]
    indptr = np.concatenate([[0], np.cumsum(pages)]).astype(np.int32)
    last = [n - ps * (p - 1) if p else 0 for n, p in zip(lens, pages)]
    items, slots, _ = B.mla_decode_plan_preview(indptr, last, page_size=ps)
    _check_cover(items.tolist(), lens, slots)


def test_planner_fills_the_gpu_for_uniform_batches(B):
    # 256 CUs x 2 resident workgroups: uniform batches become one wave of equal items
    for bs, n in [(32, 8192), (64, 8192), (64, 1024), (4, 8192)]:
        indptr = np.arange(bs + 1, dtype=np.int32) * n
        items, slots, _ = B.mla_decode_plan_preview(indptr, num_cus=256, blocks_per_cu=2)
        sizes = items[:, 2] - items[:, 1]
        assert len(items) <= 512 and len(set(sizes.tolist())) == 1, (bs, n)
        assert len(items) >= min(512, bs * n // 128, bs * 32) // 2
        assert np.bincount(items[:, 0]).max() <= 32


def test_planner_tiles_follow_the_format(B):
    """Items are whole tiles of the format's split kernel (64 tokens for bf16,
    128 for fp8 / MXFP4); a small batch goes down to one 64-token tile (bf16)
    or two 128-token tiles per item, while large uniform batches keep one
    wave of longer items."""
    indptr = np.arange(5, dtype=np.int32) * 1024  # 4 x 1024
    items, _, _ = B.mla_decode_plan_preview(indptr, num_cus=256, blocks_per_cu=2, kv_dtype="bf16")
    assert np.all(items[:, 2] - items[:, 1] == 64) and len(items) == 64
    items, _, _ = B.mla_decode_plan_preview(indptr, num_cus=256, blocks_per_cu=1, kv_dtype="fp8")
    assert np.all(items[:, 2] - items[:, 1] == 256) and len(items) == 16
    for bs, n, per_item in [(64, 1024, 256), (64, 8192, 2048), (32, 8192, 1024)]:
        indptr = np.arange(bs + 1, dtype=np.int32) * n
        for fmt in ("fp8", "mxfp4"):
            items, _, _ = B.mla_decode_plan_preview(indptr, num_cus=256, blocks_per_cu=1, kv_dtype=fmt)
            assert len(items) == 256 and np.all(items[:, 2] - items[:, 1] == per_item), (bs, n, fmt)


@pytest.mark.parametrize("fmt", ["fp8", "mxfp4"])
def test_planner_small_batch_long_context_fills_the_gpu(B, fmt):
    """One or two long sequences are split across every compute unit (up to
    256 items per sequence, merged by a merge spread over 32 workgroups per
    sequence), instead of stopping at 32 splits."""
    for lens, per in (([131072], 512), ([32768, 32768], 256), ([8192] * 4, 256)):
        indptr = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
        items, slots, _ = B.mla_decode_plan_preview(indptr, num_cus=256, blocks_per_cu=1, kv_dtype=fmt)
        assert np.all(items[:, 2] - items[:, 1] == per), lens
        assert len(items) == sum(lens) // per and len(items) <= 256 and slots == len(items)


def test_planner_paged_items_fit_the_staged_pages(B):
    """A paged item's page ids are staged in LDS by the split kernel (2560 for
    fp8, 1024 for MXFP4, 2048 for bf16, an item's first and last page possibly
    partial), so the planner caps paged items at (pages - 2) * page_size
    tokens, in whole tiles (128 tokens, 64 for bf16); uniform batches plan the
    same items as a contiguous cache."""
    ps = 2
    for fmt, pages in (("fp8", 2560), ("mxfp4", 1024), ("bf16", 2048)):
        tile = 64 if fmt == "bf16" else 128
        lens = [100000, 5]
        npg = [(n + ps - 1) // ps for n in lens]
        indptr = np.concatenate([[0], np.cumsum(npg)]).astype(np.int32)
        last = [n - ps * (p - 1) for n, p in zip(lens, npg)]
        items, slots, _ = B.mla_decode_plan_preview(indptr, last, page_size=ps, split_override=1,
                                                    kv_dtype=fmt)
        sizes = items[:, 2] - items[:, 1]
        assert sizes.max() <= (pages - 2) * ps // tile * tile, fmt
        assert sizes.max() > (pages - 2) * ps // 2, fmt
        _check_cover(items.tolist(), lens, slots)
    indptr = np.arange(65, dtype=np.int32) * 4096  # 64 x 8192 tokens in 2-token pages
    last = np.full(64, 2, dtype=np.int32)
    items, _, _ = B.mla_decode_plan_preview(indptr, last, page_size=2, num_cus=256, blocks_per_cu=1)
    assert len(items) == 256 and np.all(items[:, 2] - items[:, 1] == 2048)


def test_planner_split_override(B):
    indptr = np.array([0, 1000, 1033, 1034], dtype=np.int32)
    items, slots, _ = B.mla_decode_plan_preview(indptr, split_override=4)
    counts = np.bincount(items[:, 0], minlength=3)
    assert counts.tolist() == [4, 2, 1]  # at most one split per 32 tokens
    _check_cover(items.tolist(), [1000, 33, 1], slots)


# The planner's cost of an item's start and finish, in tokens, per format.
ITEM_COST = {"fp8": 192, "mxfp4": 288}


def _bin_costs(items, fmt):
    """Tokens plus the item cost per item, of each workgroup's bin."""
    cost = np.zeros(items[:, 4].max() + 1, dtype=np.int64)
    np.add.at(cost, items[:, 4], (items[:, 2] - items[:, 1]) + ITEM_COST[fmt])
    return cost


@pytest.mark.parametrize("fmt", ["fp8", "mxfp4"])
@pytest.mark.parametrize("page_size", [1, 2, 16])
def test_planner_ragged_batch_gets_even_bins(B, fmt, page_size):
    """fp8 / MXFP4 and a ragged batch (lengths spread over 1024..8192): the
    sequences are cut into at most one bin per resident workgroup, whose
    costs (tokens + the format's item cost) are within one short item of each other,
    instead of one item per workgroup that leaves the short ones idle."""
    from latent_attention_decode_amd import synth
    lens = synth.config_lens("bs256_ragged1024-8192_fp8_paged2")
    pages = (lens + page_size - 1) // page_size
    indptr = np.concatenate([[0], np.cumsum(pages)]).astype(np.int32)
    last = (lens - page_size * (pages - 1)).astype(np.int32)
    items, slots, _ = B.mla_decode_plan_preview(indptr, last if page_size > 1 else None, page_size=page_size,
                                                num_cus=256, blocks_per_cu=1, kv_dtype=fmt)
    _check_cover(items.tolist(), lens.tolist(), slots)
    cost = _bin_costs(items, fmt)
    assert len(cost) <= 256
    mean = (lens.sum() + ITEM_COST[fmt] * len(items)) / 256
    assert cost.max() <= mean + 256 + ITEM_COST[fmt], (cost.max(), mean)
    assert cost.max() < 1.1 * mean
    sizes = items[:, 2] - items[:, 1]
    whole = items[:, 3] == -1
    assert np.all(sizes[~whole] >= 256)            # no piece shorter than 256 tokens
    assert np.all(items[~whole, 1] % 128 == 0)     # pieces start on a tile
    assert np.bincount(items[:, 0]).max() <= 12    # the kernels merge these themselves
    if page_size > 1:
        cap = 2560 if fmt == "fp8" else 1024
        first = items[:, 1] // page_size
        lastp = (items[:, 2] - 1) // page_size
        assert np.all(lastp - first + 1 <= cap)


def test_planner_bins_respect_the_page_cap_and_split_limit(B):
    """Bins never give a paged item more pages than the kernel stages (1024
    for MXFP4: at most 1022 whole 2-token pages, 1920 tokens in whole tiles),
    and no sequence more than 32 items; where the page cap alone would need
    more, the batch falls back to one item per workgroup."""
    ps = 2
    for lens in ([60000, 3000, 1200] + [900] * 300, [2000, 120000, 700] + [1000] * 200):
        lens = np.array(lens)
        pages = (lens + ps - 1) // ps
        indptr = np.concatenate([[0], np.cumsum(pages)]).astype(np.int32)
        last = (lens - ps * (pages - 1)).astype(np.int32)
        items, slots, _ = B.mla_decode_plan_preview(indptr, last, page_size=ps, num_cus=256,
                                                    blocks_per_cu=1, kv_dtype="mxfp4")
        _check_cover(items.tolist(), lens.tolist(), slots)
        sizes = items[:, 2] - items[:, 1]
        assert sizes.max() <= 1920
        binned = len(items) > 0 and items[-1, 4] < len(items) - 1
        assert binned == (lens.max() <= 32 * 1920), lens.max()
        if binned:
            assert np.bincount(items[:, 0]).max() <= 32


@pytest.mark.parametrize("fmt", ["fp8", "mxfp4", "bf16"])
def test_planner_bins_hold_empty_sequences(B, fmt):
    """Empty sequences of a binned batch get their zero-output item in some
    bin, for every cache format (every split kernel runs bins)."""
    lens = np.array([0, 5000, 0, 300] + [4000, 1500] * 100 + [0])
    indptr = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    items, slots, _ = B.mla_decode_plan_preview(indptr, num_cus=64, blocks_per_cu=1, kv_dtype=fmt)
    _check_cover(items.tolist(), lens.tolist(), slots)
    assert items[:, 4].max() + 1 <= 64 and len(items) > 64


def _check_cover_multi(items, lens, qls, slots):
    """Row r = qo[b] + j covers tokens [0, n_b - q_b + j] exactly once; slots are a
    partition; items are listed workgroup by workgroup."""
    qo = np.concatenate([[0], np.cumsum(qls)])
    rows = int(qo[-1])
    ends = np.zeros(rows, dtype=np.int64)
    for b, (n, q) in enumerate(zip(lens, qls)):
        for j in range(q):
            ends[qo[b] + j] = n - q + j + 1
    wg = items[:, 4].tolist()
    assert wg == sorted(wg)
    seen = [np.zeros(int(e), dtype=np.int32) for e in ends]
    used = []
    for r, t0, t1, s, _ in items.tolist():
        assert s != -2 and 0 <= t0 < t1 <= ends[r]
        seen[r][t0:t1] += 1
        if s >= 0:
            used.append(s)
    assert all(np.all(x == 1) for x in seen)
    assert sorted(used) == list(range(slots))


@pytest.mark.parametrize("fmt", ["fp8", "bf16"])
@pytest.mark.parametrize("lens,qls,ps", [
    ([8192] * 64, [2] * 64, 1),
    ([1000, 37, 5000, 4], [4, 0, 1, 4], 1),
    ([3000] * 8 + [700] * 8, [3] * 8 + [1] * 8, 2),
    (list(range(1500, 1500 + 300 * 40, 300)), [2, 3] * 20, 4),
])
def test_planner_multi_token_rows(B, fmt, lens, qls, ps):
    """Multi-token plans: every query row covers exactly its causal range; the
    copies of an item for a sequence's query tokens go to workgroups launched
    together on one XCD (bins 8 apart)."""
    lens, qls = np.array(lens), np.array(qls)
    pages = (lens + ps - 1) // ps
    indptr = np.concatenate([[0], np.cumsum(pages)]).astype(np.int32)
    last = (lens - ps * (pages - 1)).astype(np.int32)
    qo = np.concatenate([[0], np.cumsum(qls)]).astype(np.int32)
    items, slots, ws = B.mla_decode_plan_preview(indptr, last if ps > 1 else None, page_size=ps, num_cus=256,
                                                blocks_per_cu=1, kv_dtype=fmt, qo_indptr_host=qo)
    _check_cover_multi(items, lens.tolist(), qls.tolist(), slots)
    assert ws == slots * 16 * 513 * 4
    # rows of one sequence: same start tokens, listed next to each other
    row_seq = np.repeat(np.arange(len(lens)), qls)
    starts = {}
    for r, t0, t1, s, wg in items.tolist():
        starts.setdefault((row_seq[r], t0), []).append((r, wg))
    for (b, t0), lst in starts.items():
        rs = sorted(r for r, _ in lst)
        assert rs == list(range(qo[b] + qls[b] - len(rs), qo[b] + qls[b])), (b, t0, rs)
        wgs = sorted(w for _, w in lst)
        assert len({w % 8 for w in wgs}) == 1 and wgs[-1] - wgs[0] <= 8 * (qls.max() - 1), (b, t0, wgs)


def test_planner_multi_token_single_is_the_plain_plan(B):
    lens = [8192] * 32 + [100] * 3
    indptr = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    qo = np.arange(len(lens) + 1, dtype=np.int32)
    a = B.mla_decode_plan_preview(indptr, num_cus=256, blocks_per_cu=1)
    b = B.mla_decode_plan_preview(indptr, num_cus=256, blocks_per_cu=1, qo_indptr_host=qo)
    assert np.array_equal(a[0], b[0]) and a[1:] == b[1:]


@pytest.mark.parametrize("qo,why", [
    ([0, 2, 1], "decreasing"),
    ([1, 2, 3], "not starting at 0"),
    ([0, 0, 0], "no query tokens"),
    ([0, 11, 12], "more query tokens than cache tokens"),
])
def test_planner_multi_token_rejects_bad_qo_indptr(B, qo, why):
    indptr = np.array([0, 10, 20], dtype=np.int32)
    with pytest.raises(B.MlaError) as e:
        B.mla_decode_plan_preview(indptr, qo_indptr_host=np.array(qo, dtype=np.int32))
    assert e.value.status == 1, why


# ---------------------------------------------------------------------------
# planner properties over random batches
# ---------------------------------------------------------------------------

from hypothesis import given, settings, strategies as st  # noqa: E402

PAGE_CAP = {"fp8": 2560, "mxfp4": 1024, "bf16": 2048}


@settings(max_examples=150, deadline=None)
@given(lens=st.lists(st.integers(0, 20000), min_size=1, max_size=48),
       fmt=st.sampled_from(["fp8", "mxfp4", "bf16"]),
       ps=st.sampled_from([1, 2, 16, 1024]),
       split=st.sampled_from([0, 0, 0, 1, 3, 40]),
       cus=st.sampled_from([8, 64, 256]),
       bpc=st.sampled_from([1, 2]),
       data=st.data())
def test_planner_properties(B, lens, fmt, ps, split, cus, bpc, data):
    """Any batch, format, page size, split override and device size: every
    query row's causal range is covered exactly once, slots partition the
    workspace, items are listed workgroup by workgroup, paged items fit the
    page ids the kernel stages, and bins (if any) number at most the
    resident workgroups times the query tokens of the widest sequence."""
    lens = np.array(lens)
    multi = data.draw(st.booleans())
    qls = None
    if multi:
        qls = np.array([data.draw(st.integers(0, min(4, int(n)))) for n in lens])
        if qls.sum() == 0:
            qls[int(np.argmax(lens))] = 1 if lens.max() > 0 else 0
        if qls.sum() == 0:
            return  # every sequence empty: no query row can exist
    pages = (lens + ps - 1) // ps
    indptr = np.concatenate([[0], np.cumsum(pages)]).astype(np.int32)
    last = np.where(pages > 0, lens - ps * (pages - 1), 0).astype(np.int32)
    qo = None if qls is None else np.concatenate([[0], np.cumsum(qls)]).astype(np.int32)
    items, slots, ws = B.mla_decode_plan_preview(indptr, last if ps > 1 else None, page_size=ps,
                                                split_override=split, num_cus=cus, blocks_per_cu=bpc,
                                                kv_dtype=fmt, qo_indptr_host=qo)
    assert ws == slots * 16 * 513 * 4
    if qls is None:
        _check_cover(items.tolist(), lens.tolist(), slots)
    else:
        _check_cover_multi(items, lens.tolist(), qls.tolist(), slots)
    if ps > 1 and fmt in PAGE_CAP:
        nonempty = items[:, 2] > items[:, 1]
        first, lastp = items[nonempty, 1] // ps, (items[nonempty, 2] - 1) // ps
        assert np.all(lastp - first + 1 <= PAGE_CAP[fmt])
    groups = items[:, 4].max() + 1
    if not np.array_equal(items[:, 4], np.arange(len(items))):  # bins (possibly empty ones)
        if qls is None:
            assert groups <= cus * bpc
        else:  # one group per parent item (or parent bin) and query token, 8 groups to a block
            row_seq = np.repeat(np.arange(len(lens)), qls)
            parents = len({(row_seq[r], t0) for r, t0 in items[:, :2].tolist()})
            qmax = int(qls.max())
            assert groups <= 8 * qmax * -(-parents // 8)
    else:
        assert groups == len(items)
