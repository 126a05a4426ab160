"""GPU parity: the HIP path against the fp64 oracle, through the C ABI.

Tolerances (fixed here, from the task): bf16 cache -> max |gpu - oracle| <= 1e-2;
fp8 / MXFP4 cache -> |gpu - oracle| <= 0.1 + 0.1 |oracle| for every element.
"""

import dataclasses
import sys

import numpy as np
import pytest
import torch

from latent_attention_decode_amd import synth
from conftest import gpu_available

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

TOL = {"bf16": (1e-2, 0.0), "fp8": (0.1, 0.1), "mxfp4": (0.1, 0.1)}


@pytest.fixture(scope="module")
def B():
    from latent_attention_decode_amd import binding
    return binding


def note(msg):
    print(msg, file=sys.stderr, flush=True)


def run_gpu(B, case, split_override=0, repeats=1, query_format=None):
    t = B.case_to_device(case)
    dec = B.MlaDecode(case.kv_dtype, case.page_size)
    try:
        if query_format is not None:
            dec.set_query_format(query_format)
        dec.plan(case.kv_indptr, case.kv_last_page_len, split_override, case.qo_indptr)
        outs = []
        for _ in range(repeats):
            out = torch.full((case.rows, 16, 512), float("nan"), dtype=torch.bfloat16, device="cuda")
            dec.run(t["q"], t["kv"], t["kv_scales"], t["kv_indptr"], out, t["kv_page_indices"],
                    t["kv_last_page_len"])
            torch.cuda.synchronize()
            outs.append(out.float().cpu().numpy().astype(np.float64))
        return outs if repeats > 1 else outs[0]
    finally:
        dec.close()


def check_close(got, ref, fmt, what=""):
    atol, rtol = TOL[fmt]
    err = np.abs(got - ref)
    bound = atol + rtol * np.abs(ref)
    bad = ~(err <= bound)  # NaN counts as bad
    stats = (f"{what} max|err|={np.nanmax(err):.3e} p99={np.nanpercentile(err, 99):.3e} "
             f"mean={np.nanmean(err):.3e}")
    note(stats)
    assert not bad.any(), f"{bad.sum()} elements outside tolerance; {stats}"


def oracle_out(oracle_mod, case, batches=None):
    out, _ = oracle_mod.decode_case(case, batches=batches)
    return out


SMALL = [
    # fmt, lens, page_size, shuffled
    ("fp8", [1, 63, 64, 65, 200, 1000], 1, False),
    ("bf16", [1, 63, 64, 65, 200, 1000], 1, False),
    ("mxfp4", [1, 63, 64, 65, 200, 1000], 1, False),
    ("fp8", [5, 130, 777, 2], 2, True),
    ("bf16", [33, 300, 64], 4, True),
    ("mxfp4", [31, 129, 500], 2, True),
    ("fp8", [3000, 17], 8, True),
]


@pytest.mark.parametrize("split", [0, 1, 3])
@pytest.mark.parametrize("fmt,lens,ps,shuffled", SMALL)
def test_small_parity(B, oracle_mod, fmt, lens, ps, shuffled, split):
    note(f"case fmt={fmt} lens={lens} ps={ps} split={split}")
    case = synth.make_case(fmt, lens, seed=100 + sum(lens) + ps, page_size=ps,
                           shuffle_pages=shuffled, guard_rows=2)
    got = run_gpu(B, case, split)
    ref = oracle_out(oracle_mod, case)
    check_close(got, ref, fmt, f"{fmt} {lens} ps{ps} split{split}")


@pytest.mark.parametrize("fmt", synth.FORMATS)
def test_single_token_cache_returns_value_row(B, oracle_mod, fmt):
    case = synth.make_case(fmt, [1, 1, 1, 1], seed=21)
    got = run_gpu(B, case)
    rows = oracle_mod.dequant_rows(fmt, case.kv, np.arange(4), kv_scale=case.kv_scale,
                                   kv_scales=case.kv_scales)
    ref = np.broadcast_to(rows[:, None, :512], (4, 16, 512))
    if fmt == "bf16":
        assert np.array_equal(got, ref)  # weight exactly 1: bit-exact
    else:
        check_close(got, ref, fmt, "one token")


@pytest.mark.parametrize("fmt", synth.FORMATS)
def test_zero_query_gives_mean(B, oracle_mod, fmt):
    lens = [300, 65]
    case = synth.make_case(fmt, lens, seed=22, q_values=np.zeros((2, 16, 576), np.float32))
    got = run_gpu(B, case)
    check_close(got, oracle_out(oracle_mod, case), fmt, "q=0")


@pytest.mark.parametrize("fmt", synth.FORMATS)
def test_constant_values(B, oracle_mod, fmt):
    lens = [500, 70]
    rng = np.random.default_rng(23)
    kv = rng.standard_normal((sum(lens), 576)).astype(np.float32)
    kv[:, :512] = 1.0
    case = synth.make_case(fmt, lens, seed=23, kv_values=kv)
    got = run_gpu(B, case)
    ref = oracle_out(oracle_mod, case)
    check_close(got, ref, fmt, "V=1")
    assert np.abs(got - ref).max() <= 1e-2


def test_mxfp4_wide_block_scales(B, oracle_mod):
    """Rows scaled by 2^r, r uniform in -10..10 per token, so the 32 tokens of
    a P.V block have e8m0 scales up to 20 binades apart: each row's V is
    converted to e4m3 relative to its own largest scale, and the row's scale
    joins its softmax weight."""
    lens = [700, 129, 64]
    rng = np.random.default_rng(41)
    kv = rng.standard_normal((sum(lens), 576)).astype(np.float32)
    kv *= np.exp2(rng.integers(-10, 11, size=(sum(lens), 1))).astype(np.float32)
    case = synth.make_case("mxfp4", lens, seed=41, kv_values=kv)
    for split in (0, 3):
        check_close(run_gpu(B, case, split), oracle_out(oracle_mod, case), "mxfp4", f"wide scales split {split}")


def sink_values(lens, deltas, seed, mean_v=0.7):
    """Query and cache values for the sink regime: every query head of a
    sequence is one N(0,1) vector q; background rows are N(0,1) with mean_v
    added to the 512 V columns (a shift common to every logit); sink rows are
    a q + mean_v on the V columns, with a chosen so that the sink's logit
    stands delta nats above the background's mean.  With thousands of
    background tokens their total weight is comparable to the sinks', while
    each one weighs e^-delta of a sink or less."""
    rng = np.random.default_rng(seed)
    total = int(sum(lens))
    q = np.zeros((len(lens), 16, 576), np.float32)
    kv = rng.standard_normal((total, 576)).astype(np.float32)
    kv[:, :512] += mean_v
    base = 0
    for b, n in enumerate(lens):
        qb = rng.standard_normal(576).astype(np.float32)
        q[b] = qb
        pos = rng.choice(n, size=len(deltas), replace=False)
        for p, d in zip(pos, deltas):
            a = d * 24.0 / float(qb @ qb)
            kv[base + p] = a * qb
            kv[base + p, :512] += mean_v
        base += n
    return q, kv


def test_mxfp4_row_scale_spread(B, oracle_mod):
    """Each 32-column block of a row scaled by its own 2^r, r uniform in
    -3..3: a row's V scales then lie up to 6 (with the quantiser's rounding,
    up to 8) binades apart, which the e4m3 V rows hold exactly relative to
    the row's largest scale (rounding conversions beyond 5 binades)."""
    lens = [3000, 129, 64]
    rng = np.random.default_rng(42)
    kv = rng.standard_normal((sum(lens), 576)).astype(np.float32)
    kv *= np.repeat(np.exp2(rng.integers(-3, 4, size=(sum(lens), 18))), 32, axis=1).astype(np.float32)
    case = synth.make_case("mxfp4", lens, seed=42, kv_values=kv)
    for split in (0, 1):
        check_close(run_gpu(B, case, split), oracle_out(oracle_mod, case), "mxfp4", f"row spread split {split}")


@pytest.mark.parametrize("delta", [6.0, 9.0, 12.0])
@pytest.mark.parametrize("split", [1, 0])
@pytest.mark.parametrize("fmt", ["fp8", "mxfp4", "bf16"])
def test_sink_logits(B, oracle_mod, fmt, split, delta):
    """A sink token delta nats above 8191 background tokens whose V has a
    non-zero mean: the background's weights are each below e^-delta of the
    sink's but together carry a large share of the output, so every one of
    them must reach P.V.  Single-item plans (the sink sets the maximum of the
    item that holds all the background) and the planner's splits; every
    element against the oracle.  bf16 is the control."""
    lens = [8192, 8192]
    q, kv = sink_values(lens, [delta], seed=300 + int(delta))
    case = synth.make_case(fmt, lens, seed=300, q_values=q, kv_values=kv)
    check_close(run_gpu(B, case, split), oracle_out(oracle_mod, case), fmt,
                f"sink {fmt} split {split} delta {delta}")


@pytest.mark.parametrize("fmt", ["fp8", "mxfp4", "bf16"])
def test_few_sinks_paged(B, oracle_mod, fmt):
    """Three sinks (12, 10 and 8 nats above the background) per sequence, in
    2-token shuffled pages, with ragged lengths and a plan with bins."""
    lens = [8192, 5000, 3001, 8192, 700]
    q, kv = sink_values(lens, [12.0, 10.0, 8.0], seed=310)
    case = synth.make_case(fmt, lens, seed=310, page_size=2, shuffle_pages=True, q_values=q, kv_values=kv)
    for split in (0, 1):
        check_close(run_gpu(B, case, split), oracle_out(oracle_mod, case), fmt,
                    f"few sinks paged {fmt} split {split}")


@pytest.mark.parametrize("split", [1, 0])
@pytest.mark.parametrize("fmt", ["mxfp4", "fp8", "bf16"])
def test_outlier_rows_with_negligible_weight(B, oracle_mod, fmt, split):
    """In every block of 32 tokens one row is 2^10 times larger than the
    others and points away from the query (a logit of about -24000 nats, so
    its weight is zero), while the ordinary rows, with V of mean 0.7, carry
    all the weight.  In MXFP4 the outlier's block scales are 10 binades above
    its neighbours' in the same 32-token block; the values of the rows that
    carry the weight must still reach P.V exactly."""
    lens = [8192, 4099]
    rng = np.random.default_rng(320)
    total = sum(lens)
    q = np.repeat(rng.standard_normal((len(lens), 1, 576)).astype(np.float32), 16, axis=1)
    kv = rng.standard_normal((total, 576)).astype(np.float32)
    kv[:, :512] += 0.7
    base = 0
    for b, n in enumerate(lens):
        qb = q[b, 0]
        for blk in range(0, n, 32):
            p = blk + (blk // 32 * 7) % min(32, n - blk)
            kv[base + p] = -1024.0 * qb / np.sqrt(float(qb @ qb) / 576.0)
        base += n
    case = synth.make_case(fmt, lens, seed=320, q_values=q, kv_values=kv)
    check_close(run_gpu(B, case, split), oracle_out(oracle_mod, case), fmt, f"outliers {fmt} split {split}")


@pytest.mark.parametrize("stride", [18, 19, 20])
def test_mxfp4_scale_strides(B, oracle_mod, stride):
    """Scale rows at any stride >= 18; an odd stride (scales not 2-byte
    aligned) runs the bf16-decoding kernel instead of the MX one."""
    case = synth.make_case("mxfp4", [1000, 300, 5], seed=42, scale_stride=stride)
    check_close(run_gpu(B, case), oracle_out(oracle_mod, case), "mxfp4", f"stride {stride}")


@pytest.mark.parametrize("fmt", ["fp8", "mxfp4", "bf16"])
def test_paged_items_at_the_page_cap(B, oracle_mod, fmt):
    """One split per sequence forces paged items up to the number of page ids
    the split kernel stages in LDS (2560 fp8, 1024 MXFP4, 2048 bf16; 2-token
    pages)."""
    case = synth.make_case(fmt, [11000, 300, 7], seed=43, page_size=2, shuffle_pages=True, guard_rows=3)
    check_close(run_gpu(B, case, 1), oracle_out(oracle_mod, case), fmt, f"{fmt} page cap")


def _binned_lens(kind):
    rng = np.random.default_rng(77 if kind == "mixed" else 78)
    if kind == "mixed":  # short and long sequences, empty and 1-token ones: bins of up to 7 items
        lens = np.concatenate([rng.integers(1, 600, 60), rng.integers(600, 4000, 100), [0, 0, 1, 1, 9000, 7000]])
    else:  # one sequence across more than 12 bins: the merge kernel combines its partials
        lens = np.concatenate([[90000], rng.integers(500, 1100, 250)])
    rng.shuffle(lens)
    return lens.tolist()


@pytest.mark.parametrize("kind", ["mixed", "one_long"])
@pytest.mark.parametrize("fmt,ps,shuffled,stride", [
    ("fp8", 1, False, 18), ("fp8", 2, True, 18), ("mxfp4", 1, False, 18), ("mxfp4", 16, True, 18),
    ("mxfp4", 1, False, 19), ("bf16", 1, False, 18), ("bf16", 4, True, 18),
])
def test_binned_ragged_batch(B, oracle_mod, kind, fmt, ps, shuffled, stride):
    """A ragged batch large enough for bins (one bin of about equal work per
    resident workgroup, whose items one workgroup runs in turn, a sequence
    possibly spanning bins): every output against the oracle, and a repeat
    bit for bit.  With odd MXFP4 scale strides the bf16-decoding kernel runs
    the same items one per workgroup."""
    lens = _binned_lens(kind)
    case = synth.make_case(fmt, lens, seed=44, page_size=ps, shuffle_pages=shuffled, scale_stride=stride)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    items, _, _ = B.mla_decode_plan_preview(case.kv_indptr, case.kv_last_page_len if ps > 1 else None,
                                            page_size=ps, num_cus=cus, blocks_per_cu=1, kv_dtype=fmt)
    per_bin = np.bincount(items[:, 4])
    splits = np.bincount(items[:, 0]).max()
    note(f"{kind} {fmt} ps {ps}: {len(items)} items in {len(per_bin)} bins, up to {per_bin.max()} per bin, "
         f"{splits} per sequence")
    assert per_bin.max() > 1 and (splits > 12) == (kind == "one_long")
    a, b = run_gpu(B, case, repeats=2)
    check_close(a, oracle_out(oracle_mod, case), fmt, f"binned {kind} {fmt} ps {ps}")
    assert np.array_equal(a, b)


@pytest.mark.parametrize("fmt,pairs,merge_kernel", [
    ("fp8", False, True), ("mxfp4", False, True), ("bf16", False, False), ("fp8", True, True),
])
def test_where_the_merge_runs(B, oracle_mod, fmt, pairs, merge_kernel):
    """Which kernel combines a ragged plan's partials (at most 12 per
    sequence): the merge kernel for fp8 and MXFP4 caches (bf16 partials),
    paired query rows included, the split kernel itself (the item that
    finishes last, fp32 partials) for a bf16 cache.  The merge kernel's time
    from the kernel-attached events is 0 exactly when it was not launched;
    every output against the oracle."""
    if pairs:  # at most 2 query tokens per sequence: the fp8 kernel runs rows in pairs
        case = synth.make_case(fmt, [1500, 1100, 129, 1200, 900], seed=96, q_lens=[2, 2, 1, 2, 2])
    else:
        case = synth.make_case(fmt, _binned_lens("mixed"), seed=96)
    t = B.case_to_device(case)
    dec = B.MlaDecode(fmt)
    try:
        dec.plan(case.kv_indptr, None, 0, case.qo_indptr)
        _, splits, _ = B.mla_decode_plan_info(dec.h)
        assert 2 <= splits <= 12
        B.mla_decode_set_profiling(dec.h, True)
        out = torch.full((case.rows, 16, 512), float("nan"), dtype=torch.bfloat16, device="cuda")
        dec.run(t["q"], t["kv"], t["kv_scales"], t["kv_indptr"], out)
        torch.cuda.synchronize()
        assert B.mla_decode_kernel_time_ms(dec.h, 0) > 0
        assert (B.mla_decode_kernel_time_ms(dec.h, 1) > 0) == merge_kernel
    finally:
        dec.close()
    check_close(out.float().cpu().numpy().astype(np.float64), oracle_out(oracle_mod, case), fmt,
                f"merge placement {fmt} pairs {pairs}")


MULTI = [
    # fmt, lens, q_lens, page_size, shuffled
    ("fp8", [1, 63, 200, 1000, 5], [1, 2, 4, 3, 5], 1, False),
    ("bf16", [130, 700, 9], [2, 1, 4], 4, True),
    ("mxfp4", [31, 2, 900], [3, 2, 2], 2, True),
    ("fp8", [3000, 17, 800], [4, 0, 2], 8, True),
    ("mxfp4", [3000, 17, 800], [4, 0, 2], 1, False),
]


@pytest.mark.parametrize("split", [0, 3])
@pytest.mark.parametrize("fmt,lens,qls,ps,shuffled", MULTI)
def test_multi_token_parity(B, oracle_mod, fmt, lens, qls, ps, shuffled, split):
    """Multi-token decode (query token j of a sequence of n tokens with q query
    tokens attends to tokens 0 .. n - q + j): every row against the oracle's
    causal definition, including one-token rows, sequences without query
    tokens and rows whose range ends inside a tile."""
    note(f"multi {fmt} lens {lens} q {qls} ps {ps} split {split}")
    case = synth.make_case(fmt, lens, seed=50, page_size=ps, shuffle_pages=shuffled, q_lens=qls, guard_rows=2)
    check_close(run_gpu(B, case, split), oracle_out(oracle_mod, case), fmt, f"multi {fmt} ps {ps} split {split}")


def test_multi_token_mxfp4_odd_scale_stride(B, oracle_mod):
    """Multi-token rows on an MXFP4 cache whose scale rows have an odd stride:
    the bf16-decoding kernel runs the plan's items one per workgroup."""
    case = synth.make_case("mxfp4", [3000, 17, 800], seed=52, q_lens=[4, 0, 2], scale_stride=19)
    check_close(run_gpu(B, case), oracle_out(oracle_mod, case), "mxfp4", "multi mxfp4 stride 19")


@pytest.mark.parametrize("split", [0, 2, 7])
@pytest.mark.parametrize("ps", [1, 2, 16])
def test_multi_token_pairs_fp8(B, oracle_mod, ps, split):
    """fp8 with at most 2 query tokens per sequence: the kernel runs the two
    rows of a sequence over each token range together (one tile read for
    both, each row masked at its own causal end); sequences with one query
    token run alone in the same kernel.  Every row against the oracle."""
    lens, qls = [1, 63, 200, 1000, 5, 3000, 129], [1, 2, 2, 1, 2, 2, 2]
    case = synth.make_case("fp8", lens, seed=53, page_size=ps, shuffle_pages=ps > 1, q_lens=qls, guard_rows=2)
    check_close(run_gpu(B, case, split), oracle_out(oracle_mod, case), "fp8", f"pairs ps {ps} split {split}")


def test_multi_token_pairs_binned(B, oracle_mod):
    """A ragged fp8 batch large enough for bins, 1 or 2 query tokens per
    sequence: bins of several parent items, each listing its row pair; all
    rows against the oracle, and a repeat bit for bit."""
    rng = np.random.default_rng(54)
    lens = rng.integers(600, 4000, 120).tolist()
    qls = rng.integers(1, 3, 120).tolist()
    case = synth.make_case("fp8", lens, seed=54, page_size=2, shuffle_pages=True, q_lens=qls)
    a, b = run_gpu(B, case, repeats=2)
    check_close(a, oracle_out(oracle_mod, case), "fp8", "pairs binned")
    assert np.array_equal(a, b)


@pytest.mark.parametrize("fmt", ["fp8", "bf16"])
def test_multi_token_binned_ragged_batch(B, oracle_mod, fmt):
    """A ragged batch large enough for bins, with 1..4 query tokens per
    sequence: the copies of each bin for the query tokens run side by side;
    sampled sequences against the oracle, and a repeat bit for bit."""
    rng = np.random.default_rng(51)
    lens = rng.integers(600, 4000, 96).tolist()
    qls = rng.integers(1, 5, 96).tolist()
    case = synth.make_case(fmt, lens, seed=51, page_size=2, shuffle_pages=True, q_lens=qls)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    items, _, _ = B.mla_decode_plan_preview(case.kv_indptr, case.kv_last_page_len, page_size=2, num_cus=cus,
                                            blocks_per_cu=1, kv_dtype=fmt, qo_indptr_host=case.qo_indptr)
    note(f"multi binned: {len(items)} items, {items[:, 4].max() + 1} workgroups")
    assert items[-1, 4] < len(items) - 1  # bins
    a, b = run_gpu(B, case, repeats=2)
    sample = [0, 17, 50, 95]
    ref = oracle_out(oracle_mod, case, batches=sample)
    rows = [r for s in sample for r in range(case.qo_indptr[s], case.qo_indptr[s + 1])]
    check_close(a[rows], ref[rows], fmt, f"multi binned {fmt}")
    assert np.all(np.isfinite(a)) and np.array_equal(a, b)


EXTREMES = [
    # what, fmt, lens, page_size
    ("one 131072-token sequence in 256 items, merge in 32 parts", "fp8", [131072], 1),
    ("one 32768-token MXFP4 sequence", "mxfp4", [32768], 1),
    ("one 65536-token bf16 sequence and a short one", "bf16", [65536, 3], 1),
    ("8 x 4096, merge in 16 parts", "fp8", [4096] * 8, 1),
    ("16 x 2048 MXFP4, merge in 8 parts", "mxfp4", [2048] * 16, 1),
    ("2048 sequences of 0..64 tokens", "fp8", np.random.default_rng(60).integers(0, 65, 2048).tolist(), 1),
    ("1024-token pages", "mxfp4", [5000, 1024, 1, 2047], 1024),
    ("1024-token pages, bf16", "bf16", [5000, 1024, 1, 2047, 0], 1024),
    ("a 9000-token bf16 sequence in 2-token pages, split over many CUs", "bf16", [9000, 3], 2),
]


@pytest.mark.parametrize("what,fmt,lens,ps", EXTREMES, ids=[e[0] for e in EXTREMES])
def test_extreme_shapes(B, oracle_mod, what, fmt, lens, ps):
    """Sizes at the ends of the range: the longest single sequences (split over
    every compute unit), the widest merges, thousands of tiny or empty
    sequences, the largest page size.  Every output against the oracle."""
    note(f"extreme: {what}")
    case = synth.make_case(fmt, lens, seed=61, page_size=ps, shuffle_pages=ps > 1, guard_rows=2)
    check_close(run_gpu(B, case), oracle_out(oracle_mod, case), fmt, what)


def random_cases(n=240, seed=2024):
    """Seeded mixed cases: format, ragged and empty lengths, page size and shuffling,
    MXFP4 scale stride, split override and sometimes several query tokens per
    sequence."""
    rng = np.random.default_rng(seed)
    cases = []
    for k in range(n):
        fmt = synth.FORMATS[k % 3]
        batch = int(rng.integers(1, 13))
        lens = rng.integers(0, 3000, size=batch)
        lens[rng.random(batch) < 0.15] = 0
        if lens.sum() == 0:
            lens[0] = int(rng.integers(1, 600))
        ps = int(rng.choice([1, 1, 2, 4, 16, 64]))
        stride = int(rng.choice([18, 18, 20, 19])) if fmt == "mxfp4" else 18
        split = int(rng.choice([0, 0, 0, 1, 2, 5]))
        q_lens = None
        if rng.random() < 0.3:
            q_lens = [int(min(n_b, rng.integers(0, 4))) for n_b in lens]
            if sum(q_lens) == 0:
                q_lens = None
        cases.append((k, fmt, [int(x) for x in lens], ps, stride, split, q_lens))
    return cases


@pytest.mark.parametrize("k,fmt,lens,ps,stride,split,q_lens", random_cases(), ids=lambda v: None)
def test_random_mixed_cases(B, oracle_mod, k, fmt, lens, ps, stride, split, q_lens):
    """Every third fp8 / MXFP4 case (even scale addresses) takes the
    single-code query, against the decode of the rounded query."""
    e4m3 = fmt != "bf16" and k % 3 == 0 and stride % 2 == 0
    note(f"random case {k}: {fmt} lens={lens} ps={ps} stride={stride} split={split} q_lens={q_lens} "
         f"query {'e4m3' if e4m3 else 'exact'}")
    case = synth.make_case(fmt, lens, seed=5000 + k, page_size=ps, shuffle_pages=ps > 1, scale_stride=stride,
                           q_lens=q_lens, guard_rows=3)
    got = run_gpu(B, case, split, query_format="e4m3" if e4m3 else None)
    ref = dataclasses.replace(case, q_bits=oracle_mod.round_query_e4m3(case.q_bits)) if e4m3 else case
    check_close(got, oracle_out(oracle_mod, ref), fmt, f"random case {k}")


def test_empty_sequences_give_zero(B, oracle_mod):
    case = synth.make_case("fp8", [0, 100, 0, 1], seed=24)
    got = run_gpu(B, case)
    assert np.all(got[0] == 0) and np.all(got[2] == 0)
    check_close(got, oracle_out(oracle_mod, case), "fp8", "empty")
    case = synth.make_case("bf16", [0, 0], seed=25)
    assert np.all(run_gpu(B, case) == 0)


@pytest.mark.parametrize("fmt", synth.FORMATS)
def test_deterministic(B, fmt):
    case = synth.make_case(fmt, [2000, 64, 5], seed=26)
    a, b = run_gpu(B, case, repeats=2)
    assert np.array_equal(a, b)


def test_page_table_permutation_and_size_invariance(B):
    lens = [700, 129, 64, 3]
    base = run_gpu(B, synth.make_case("fp8", lens, seed=27))
    for ps in (2, 8):
        got = run_gpu(B, synth.make_case("fp8", lens, seed=27, page_size=ps, shuffle_pages=True,
                                         guard_rows=5))
        assert np.array_equal(got, base), ps


def test_split_count_changes_only_rounding(B, oracle_mod):
    case = synth.make_case("fp8", [4096, 1500], seed=28)
    ref = oracle_out(oracle_mod, case)
    outs = [run_gpu(B, case, s) for s in (1, 2, 7, 40)]
    for o in outs:
        check_close(o, ref, "fp8", "splits")
        assert np.abs(o - outs[0]).max() < 2e-2


@pytest.mark.parametrize("fmt", ["fp8", "mxfp4", "bf16"])
@pytest.mark.parametrize("split", [2, 5, 12, 13])
def test_merge_repeated_calls(B, oracle_mod, fmt, split):
    """With a bf16 cache, a plan whose items differ in length and at most 12
    splits per sequence, the split kernel merges the partials itself:
    per-sequence completion counters, reset by the item that finishes last,
    pick the merging item; with 13, and for fp8 and MXFP4 caches, the merge
    kernel runs on bf16 partials.  Calls on one plan with new data each time
    must each match the oracle (a partial left from the call before would
    not), and a repeat of the first must agree with it bit for bit (the merge
    order does not depend on which item finished last)."""
    lens = [3000, 1700, 129, 2500, 1]
    cases = [synth.make_case(fmt, lens, seed=31 + r) for r in range(3)]
    dec = B.MlaDecode(fmt, 1)
    try:
        dec.plan(cases[0].kv_indptr, None, split)
        outs = []
        for case in cases + cases[:1]:
            t = B.case_to_device(case)
            out = torch.full((case.batch, 16, 512), float("nan"), dtype=torch.bfloat16, device="cuda")
            dec.run(t["q"], t["kv"], t["kv_scales"], t["kv_indptr"], out)
            torch.cuda.synchronize()
            outs.append(out.float().cpu().numpy().astype(np.float64))
    finally:
        dec.close()
    for r, case in enumerate(cases):
        check_close(outs[r], oracle_out(oracle_mod, case), fmt, f"{fmt} split {split} call {r}")
    assert np.array_equal(outs[0], outs[3])


@pytest.mark.parametrize("fmt,lens,ps", [("fp8", [3000, 40, 700], 2), ("mxfp4", [1500, 9], 1), ("bf16", [600], 1)])
def test_prepared_run_matches_run(B, fmt, lens, ps):
    """A PreparedRun (arguments marshalled once) launches exactly what run() does."""
    case = synth.make_case(fmt, lens, seed=77, page_size=ps, shuffle_pages=ps > 1)
    t = B.case_to_device(case)
    dec = B.MlaDecode(fmt, ps)
    try:
        dec.plan(case.kv_indptr, case.kv_last_page_len)
        ref = torch.full((case.rows, 16, 512), float("nan"), dtype=torch.bfloat16, device="cuda")
        dec.run(t["q"], t["kv"], t["kv_scales"], t["kv_indptr"], ref, t["kv_page_indices"], t["kv_last_page_len"])
        out = torch.full_like(ref, float("nan"))
        call = dec.prepare(t["q"], t["kv"], t["kv_scales"], t["kv_indptr"], out, t["kv_page_indices"],
                           t["kv_last_page_len"])
        for _ in range(3):
            out.fill_(float("nan"))
            call()
            torch.cuda.synchronize()
            assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
    finally:
        dec.close()


@pytest.mark.parametrize("fmt,lens,ps,split,stride", [
    ("fp8", [4096] * 8, 1, 0, 18),                 # uniform plan: the merge kernel
    ("fp8", [3000, 1700, 129, 2500, 1], 2, 5, 18),  # uneven items, then the merge kernel
    ("bf16", [3000, 1700, 129, 2500, 1], 1, 5, 18),  # the merge inside the split kernel
    ("fp8", [3000, 1700, 129, 2500, 1], 1, 13, 18),  # too many splits for it: the merge kernel
    ("mxfp4", [3000, 1700, 129], 1, 0, 18),
    ("mxfp4", [2000, 300, 77], 1, 3, 19),          # odd scale stride: the bf16-decoding kernel
    ("bf16", [3000, 700, 5], 2, 0, 18),
])
def test_workspace_poisoned_with_nan(B, oracle_mod, fmt, lens, ps, split, stride):
    """The workspace is filled with NaN before every run, so any read of a
    partial (output or log-sum-exp) that the run itself did not write first
    shows up as NaN in the output."""
    case = synth.make_case(fmt, lens, seed=95, page_size=ps, shuffle_pages=ps > 1, scale_stride=stride)
    t = B.case_to_device(case)
    dec = B.MlaDecode(fmt, ps)
    try:
        ws = dec.plan(case.kv_indptr, case.kv_last_page_len, split)
        assert ws > 0
        ref = oracle_out(oracle_mod, case)
        for k in range(3):
            dec.workspace.fill_(float("nan"))
            out = torch.full((case.rows, 16, 512), float("nan"), dtype=torch.bfloat16, device="cuda")
            dec.run(t["q"], t["kv"], t["kv_scales"], t["kv_indptr"], out, t["kv_page_indices"],
                    t["kv_last_page_len"])
            torch.cuda.synchronize()
            check_close(out.float().cpu().numpy().astype(np.float64), ref, fmt, f"nan workspace {fmt} call {k}")
    finally:
        dec.close()


def test_workspace_too_small_is_rejected(B):
    case = synth.make_case("fp8", [4096], seed=29)
    t = B.case_to_device(case)
    dec = B.MlaDecode("fp8")
    try:
        ws = dec.plan(case.kv_indptr, None, 4)
        assert ws > 0
        small = torch.empty(ws // 4 - 1, dtype=torch.float32, device="cuda")
        out = torch.empty((1, 16, 512), dtype=torch.bfloat16, device="cuda")
        with pytest.raises(B.MlaError) as e:
            B.mla_decode_run(dec.h, t["q"], t["kv"], t["kv_scales"], t["kv_indptr"], out, small)
        assert e.value.status == 4
        # an output 8 bytes off a 16-byte boundary is refused before any launch
        big = torch.empty(16 * 512 + 8, dtype=torch.bfloat16, device="cuda")
        out8 = big[4:4 + 16 * 512].view(1, 16, 512)
        assert out8.data_ptr() % 16 == 8
        with pytest.raises(B.MlaError) as e:
            B.mla_decode_run(dec.h, t["q"], t["kv"], t["kv_scales"], t["kv_indptr"], out8, dec.workspace)
        assert e.value.status == 1 and "16-byte" in str(e.value)
    finally:
        dec.close()


def test_two_handles_on_two_streams(B, oracle_mod):
    """Handles share no state: two plans (one with a fused merge, one with the merge kernel)
    run interleaved on two streams, several times, and both match the oracle every time."""
    case_a = synth.make_case("bf16", [3000, 700, 4100, 90], seed=91, page_size=2, shuffle_pages=True)
    case_b = synth.make_case("fp8", [2048] * 8, seed=92)
    ref_a, ref_b = oracle_out(oracle_mod, case_a), oracle_out(oracle_mod, case_b)
    ta, tb = B.case_to_device(case_a), B.case_to_device(case_b)
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    da, db = B.MlaDecode("bf16", 2), B.MlaDecode("fp8")
    try:
        da.plan(case_a.kv_indptr, case_a.kv_last_page_len, 5)  # uneven items, at most 12 each: fused
        db.plan(case_b.kv_indptr)
        outs_a = [torch.full((4, 16, 512), float("nan"), dtype=torch.bfloat16, device="cuda") for _ in range(3)]
        outs_b = [torch.full((8, 16, 512), float("nan"), dtype=torch.bfloat16, device="cuda") for _ in range(3)]
        torch.cuda.synchronize()
        for oa, ob in zip(outs_a, outs_b):
            da.run(ta["q"], ta["kv"], ta["kv_scales"], ta["kv_indptr"], oa, ta["kv_page_indices"],
                   ta["kv_last_page_len"], stream=sa)
            db.run(tb["q"], tb["kv"], tb["kv_scales"], tb["kv_indptr"], ob, stream=sb)
        torch.cuda.synchronize()
        for k in range(3):
            check_close(outs_a[k].float().cpu().numpy().astype(np.float64), ref_a, "bf16", f"handle a call {k}")
            check_close(outs_b[k].float().cpu().numpy().astype(np.float64), ref_b, "fp8", f"handle b call {k}")
    finally:
        da.close()
        db.close()


@pytest.mark.parametrize("fmt", synth.FORMATS)
def test_replanning_one_handle(B, oracle_mod, fmt):
    """One handle planned again and again for batches of other shapes (uniform with the
    merge kernel, ragged with bins and the in-kernel merge (bf16), a single item, empty
    sequences, more query rows): every run matches the oracle, so no state of an earlier
    plan (work list, completion counters, bins) leaks into a later one."""
    shapes = [([2048] * 8, None), (list(range(300, 300 + 150 * 60, 150)) + [0, 0], None), ([77], None),
              ([0, 5, 1200], None), ([900, 2500, 40], [2, 1, 3]), ([2048] * 8, None)]
    dec = B.MlaDecode(fmt)
    try:
        for k, (lens, qls) in enumerate(shapes):
            case = synth.make_case(fmt, lens, seed=200 + k, q_lens=qls)
            t = B.case_to_device(case)
            dec.plan(case.kv_indptr, None, 0, case.qo_indptr)
            out = torch.full((case.rows, 16, 512), float("nan"), dtype=torch.bfloat16, device="cuda")
            dec.run(t["q"], t["kv"], t["kv_scales"], t["kv_indptr"], out)
            torch.cuda.synchronize()
            check_close(out.float().cpu().numpy().astype(np.float64), oracle_out(oracle_mod, case), fmt,
                        f"replan {fmt} shape {k}")
    finally:
        dec.close()


@pytest.mark.parametrize("fmt,ps", [("fp8", 1), ("fp8", 2), ("mxfp4", 1), ("bf16", 2)])
def test_replan_while_runs_are_in_flight(B, oracle_mod, fmt, ps):
    """A decode loop: every step appends one token to each sequence, re-plans
    the handle and runs, with no host synchronisation between steps (the
    plan's upload goes to the other of two plan buffers and each run waits for
    its own upload on the device); two plans in a row without a run, and a
    plan that needs a larger buffer, included.  Every step's output against
    the oracle."""
    steps = [[3000, 700, 129, 2500], [3001, 701, 130, 2501], None, [3002, 702, 131, 2502],
             [3003, 703, 132, 2503] + [4000] * 40, [3004, 704, 133, 2504]]
    dec = B.MlaDecode(fmt, ps)
    try:
        runs = []
        for k, lens in enumerate(steps):
            if lens is None:  # a plan no run uses
                dec.plan(*_plan_args(synth.make_case(fmt, [5000, 9], seed=599, page_size=ps)))
                continue
            case = synth.make_case(fmt, lens, seed=600 + k, page_size=ps, shuffle_pages=ps > 1)
            t = B.case_to_device(case)
            out = torch.full((case.rows, 16, 512), float("nan"), dtype=torch.bfloat16, device="cuda")
            dec.plan(*_plan_args(case))
            dec.run(t["q"], t["kv"], t["kv_scales"], t["kv_indptr"], out, t["kv_page_indices"],
                    t["kv_last_page_len"])
            runs.append((case, t, out))
        torch.cuda.synchronize()
        for k, (case, _t, out) in enumerate(runs):
            check_close(out.float().cpu().numpy().astype(np.float64), oracle_out(oracle_mod, case), fmt,
                        f"in-flight re-plan {fmt} ps {ps} step {k}")
    finally:
        dec.close()


def _plan_args(case):
    return case.kv_indptr, case.kv_last_page_len, 0, case.qo_indptr


def test_run_validates_arguments(B):
    """Every malformed run is refused with a status and a message before anything is
    launched; the handle still runs correctly afterwards."""
    def status(fn):
        with pytest.raises(B.MlaError) as e:
            fn()
        return e.value.status, str(e.value)

    case = synth.make_case("mxfp4", [700, 300], seed=81)
    t = B.case_to_device(case)
    dec = B.MlaDecode("mxfp4")
    try:
        dec.plan(case.kv_indptr)
        out = torch.empty((2, 16, 512), dtype=torch.bfloat16, device="cuda")
        run = lambda **kw: B.mla_decode_run(dec.h, **{**dict(q=t["q"], kv=t["kv"], kv_scales=t["kv_scales"],
                                                             kv_indptr=t["kv_indptr"], out=out,
                                                             workspace=dec.workspace), **kw})
        st, msg = status(lambda: run(kv_scales=t["kv_scales"][:, :17].contiguous()))
        assert st == 1 and ">= 18" in msg
        st, msg = status(lambda: run(kv_scales=None))
        assert st == 1 and "kv_scales" in msg
        flat = torch.empty(t["q"].numel() + 8, dtype=torch.bfloat16, device="cuda")
        q8 = flat[4:4 + t["q"].numel()].view_as(t["q"])
        st, msg = status(lambda: run(q=q8))
        assert st == 1 and "16-byte" in msg
        st, msg = status(lambda: run(workspace=None))
        assert st == 4
        got = run_gpu(B, case)  # a fresh handle still agrees with the oracle
        assert np.all(np.isfinite(got))
    finally:
        dec.close()

    paged = synth.make_case("fp8", [50, 9], seed=82, page_size=4, shuffle_pages=True)
    tp = B.case_to_device(paged)
    dec = B.MlaDecode("fp8", 4)
    try:
        dec.plan(paged.kv_indptr, paged.kv_last_page_len)
        out = torch.empty((2, 16, 512), dtype=torch.bfloat16, device="cuda")
        st, msg = status(lambda: B.mla_decode_run(dec.h, tp["q"], tp["kv"], tp["kv_scales"], tp["kv_indptr"], out,
                                                  dec.workspace, None, tp["kv_last_page_len"]))
        assert st == 1 and "page table" in msg
        dec.run(tp["q"], tp["kv"], tp["kv_scales"], tp["kv_indptr"], out, tp["kv_page_indices"],
                tp["kv_last_page_len"])
        torch.cuda.synchronize()
        assert torch.isfinite(out.float()).all()
    finally:
        dec.close()


# Full-size workloads: every output against the oracle.
FULL = list(synth.CONFIGS)


@pytest.mark.parametrize("name", FULL)
def test_full_size_configs(B, oracle_mod, name):
    note(f"config {name}")
    case = synth.config_case(name)
    got = run_gpu(B, case)
    ref = oracle_out(oracle_mod, case)
    check_close(got, ref, case.kv_dtype, name)


@pytest.mark.parametrize("fmt,lens,ps,split,q_lens", [
    ("fp8", [8192, 3000, 129, 0], 1, 0, None),
    ("fp8", [5000, 700, 1], 2, 1, None),
    ("fp8", [3000, 17, 800], 1, 0, [2, 1, 2]),     # paired query rows
    ("fp8", [2000, 900], 4, 0, [3, 4]),            # single rows of a multi-token plan
    ("mxfp4", [8192, 3000, 129, 0], 1, 0, None),
    ("mxfp4", [2000, 300, 33], 16, 1, None),
    ("mxfp4", [3000, 17, 800], 2, 0, [2, 1, 2]),
])
def test_query_e4m3(B, oracle_mod, fmt, lens, ps, split, q_lens):
    """MLA_QUERY_E4M3: the decode of the query rounded to one e4m3 code per
    element (oracle_round_query_e4m3), to the usual tolerance; the distance to
    the exact decode is printed."""
    case = synth.make_case(fmt, lens, seed=97, page_size=ps, shuffle_pages=ps > 1, q_lens=q_lens)
    rounded = dataclasses.replace(case, q_bits=oracle_mod.round_query_e4m3(case.q_bits))
    got = run_gpu(B, case, split, query_format="e4m3")
    check_close(got, oracle_out(oracle_mod, rounded), fmt, f"query e4m3 {fmt} split {split}")
    exact = oracle_out(oracle_mod, case)
    note(f"query e4m3 {fmt}: max|gpu - exact decode| = {np.nanmax(np.abs(got - exact)):.3e}")


def test_query_e4m3_refused_for_odd_scale_addresses(B, oracle_mod):
    """The bf16-decoding MXFP4 kernel (odd scale stride) has no single-code
    query: such a run is refused before any launch, and the exact query still
    runs."""
    case = synth.make_case("mxfp4", [300, 20], seed=98, scale_stride=19)
    with pytest.raises(B.MlaError) as e:
        run_gpu(B, case, query_format="e4m3")
    assert e.value.status == 2
    check_close(run_gpu(B, case, query_format="exact"), oracle_out(oracle_mod, case), "mxfp4", "stride 19 exact")


@pytest.mark.parametrize("fmt,ps,qf", [
    ("fp8", 1, "exact"), ("fp8", 2, "exact"), ("fp8", 1, "e4m3"),
    ("mxfp4", 1, "exact"), ("mxfp4", 2, "exact"), ("mxfp4", 1, "e4m3"), ("mxfp4", 2, "e4m3"),
    ("bf16", 1, "exact"), ("bf16", 2, "exact"),
])
def test_split_kernels_keep_registers_out_of_scratch(B, fmt, ps, qf):
    """The one-row split kernels run without register spills (scratch memory
    per lane 0): a spill of values live across the tile loop costs a round
    trip to memory on every item (the MXFP4 kernel once lost 10 % of its time
    to 20 such registers).  The MXFP4 kernel keeps its two waves per SIMD (at
    most 256 registers each)."""
    case = synth.make_case(fmt, [700, 300], seed=99, page_size=ps, shuffle_pages=ps > 1)
    dec = B.MlaDecode(fmt, ps)
    try:
        if qf != "exact":
            dec.set_query_format(qf)
        dec.plan(case.kv_indptr, case.kv_last_page_len, 0)
        res = B.mla_decode_kernel_resources(dec.h, 0)
    finally:
        dec.close()
    note(f"{fmt} page {ps} query {qf}: {res}")
    assert res["scratch_bytes"] == 0, res
    if fmt == "mxfp4":
        assert res["vgprs"] <= 256, res
