"""Pins for the fp64 oracle (CPU only).

Each test ties the oracle to something other than itself: library decoders
(torch's float8_e4m3fn / float8_e8m0fnu / bfloat16 casts), the OCP e2m1 table
under tests/golden/, closed forms (one-token cache, equal logits, constant V),
the split/merge identity, and a brute-force softmax(q k^T * scale) v written
here with torch in float64 over an independently decoded cache.
"""

import os

import numpy as np
import pytest
import torch

from latent_attention_decode_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _e2m1_table():
    vals = {}
    with open(os.path.join(GOLDEN, "e2m1_values.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            c, v = line.split()
            vals[int(c)] = float(v)
    assert sorted(vals) == list(range(16))
    return np.array([vals[i] for i in range(16)])


# ---------------------------------------------------------------------------
# element decoders
# ---------------------------------------------------------------------------

def test_e4m3_all_codes_match_torch(oracle_mod):
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = np.array([oracle_mod.e4m3_to_f64(c) for c in range(256)])
    nan = np.isnan(ref)
    assert nan.sum() == 2  # S.1111.111 only
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert got[0x7E] == 448.0 and got[1] == 2.0 ** -9


def test_e8m0_all_codes_match_torch(oracle_mod):
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    got = np.array([oracle_mod.e8m0_to_f64(c) for c in range(256)])
    assert np.isnan(got[255]) and np.isnan(ref[255])
    assert np.array_equal(got[:255], ref[:255])
    assert got[127] == 1.0


def test_e2m1_all_codes_match_ocp_table(oracle_mod):
    table = _e2m1_table()
    got = np.array([oracle_mod.e2m1_to_f64(c) for c in range(16)])
    assert np.array_equal(got, table)
    assert np.array_equal(np.signbit(got), np.signbit(table))  # code 8 is -0
    # invariants: odd symmetry, strictly increasing magnitudes, max 6
    assert np.array_equal(got[8:], -got[:8])
    assert np.all(np.diff(got[:8]) > 0) and got[7] == 6.0


def test_bf16_all_patterns_match_torch(oracle_mod):
    bits = np.arange(65536, dtype=np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    sample = np.concatenate([np.arange(0, 65536, 97), [0x7F80, 0xFF80, 0x0001, 0x8001, 0x7F7F]])
    for b in sample:
        g = oracle_mod.bf16_to_f64(int(b))
        r = ref[b]
        assert (np.isnan(g) and np.isnan(r)) or g == r, hex(int(b))


# ---------------------------------------------------------------------------
# independent dequantisation used by the brute-force pins
# ---------------------------------------------------------------------------

def _dequant_independent(case) -> list:
    """Per sequence: fp64 [len, 576] decoded without the oracle's decoders."""
    out = []
    table = _e2m1_table()
    for b in range(case.batch):
        rows = case.token_rows(b)
        raw = case.kv[rows]
        if case.kv_dtype == "bf16":
            v = torch.from_numpy(raw.copy().view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
        elif case.kv_dtype == "fp8":
            v = torch.from_numpy(raw.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
            v = v * np.float64(case.kv_scale)
        else:
            lo = table[raw & 0xF]
            hi = table[raw >> 4]
            codes = np.empty((raw.shape[0], 576))
            codes[:, 0::2] = lo
            codes[:, 1::2] = hi
            e8 = case.kv_scales[rows][:, :18]
            sc = torch.from_numpy(e8.copy()).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
            v = codes * np.repeat(sc, 32, axis=1)
        out.append(v.reshape(rows.size, 576))
    return out


def _brute_force(case):
    """softmax(q k^T / sqrt(576)) v in torch float64 (the bmm formula)."""
    q = torch.from_numpy(case.q_bits.view(np.int16)).view(torch.bfloat16).to(torch.float64)
    seqs = _dequant_independent(case)
    outs, lses = [], []
    for b, c in enumerate(seqs):
        kv = torch.from_numpy(c)
        if kv.shape[0] == 0:
            outs.append(torch.zeros(16, 512, dtype=torch.float64))
            lses.append(torch.full((16,), -np.inf, dtype=torch.float64))
            continue
        z = (q[b] @ kv.T) / np.sqrt(576.0)
        outs.append(torch.softmax(z, dim=-1) @ kv[:, :512])
        lses.append(torch.logsumexp(z, dim=-1))
    return torch.stack(outs).numpy(), torch.stack(lses).numpy()


def _brute_force_multi(case):
    """Multi-token decode: softmax(q k^T / sqrt(576) + mask) v in torch float64,
    with the bottom-right aligned causal mask (query token j of a sequence of n
    tokens with q query tokens is position n - q + j): entries above diagonal
    n - q + 1 of the [q, n] score matrix are masked."""
    q_all = torch.from_numpy(case.q_bits.view(np.int16)).view(torch.bfloat16).to(torch.float64)
    seqs = _dequant_independent(case)
    outs, lses = [], []
    for b, c in enumerate(seqs):
        r0, r1 = int(case.qo_indptr[b]), int(case.qo_indptr[b + 1])
        kv = torch.from_numpy(c)
        n, nq = kv.shape[0], r1 - r0
        z = torch.einsum("jhd,td->jht", q_all[r0:r1], kv) / np.sqrt(576.0)
        masked = torch.ones(nq, n, dtype=torch.bool).triu(n - nq + 1)
        z = z.masked_fill(masked[:, None, :], -np.inf)
        outs.append(torch.softmax(z, dim=-1) @ kv[:, :512])
        lses.append(torch.logsumexp(z, dim=-1))
    return torch.cat(outs).numpy(), torch.cat(lses).numpy()


TINY_MULTI = [
    # fmt, lens, q_lens, page_size, shuffle
    ("bf16", [1, 4, 9], [1, 4, 3], 1, False),
    ("fp8", [17, 6, 2], [2, 0, 2], 2, True),
    ("mxfp4", [33, 5, 40], [5, 1, 7], 4, True),
]


TINY = [
    ("bf16", [1, 2, 3], 1, False),
    ("fp8", [15, 16, 17], 1, False),
    ("mxfp4", [33, 1, 2], 1, False),
    ("fp8", [5, 33, 16], 2, True),
    ("bf16", [7, 0, 9], 4, True),
    ("mxfp4", [17, 3, 8], 8, True),
]


@pytest.mark.parametrize("fmt,lens,ps,shuffle", TINY)
def test_oracle_matches_brute_force(oracle_mod, fmt, lens, ps, shuffle):
    case = synth.make_case(fmt, lens, seed=7 + len(lens) + ps, page_size=ps, shuffle_pages=shuffle,
                           guard_rows=3)
    out, lse = oracle_mod.decode_case(case)
    ref, ref_lse = _brute_force(case)
    assert np.all(np.isfinite(out))
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-12)
    fin = np.isfinite(ref_lse)
    np.testing.assert_allclose(lse[fin], ref_lse[fin], rtol=1e-12, atol=1e-12)
    assert np.all(np.isneginf(lse[~fin]))


@pytest.mark.parametrize("fmt,lens,qls,ps,shuffle", TINY_MULTI)
def test_multi_token_matches_brute_force(oracle_mod, fmt, lens, qls, ps, shuffle):
    case = synth.make_case(fmt, lens, seed=9 + ps, page_size=ps, shuffle_pages=shuffle, guard_rows=2,
                           q_lens=qls)
    out, lse = oracle_mod.decode_case(case)
    ref, ref_lse = _brute_force_multi(case)
    assert out.shape[0] == sum(qls) and np.all(np.isfinite(out))
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse, ref_lse, rtol=1e-12, atol=1e-12)


def test_multi_token_closed_forms(oracle_mod):
    """A sequence whose cache holds only its query tokens: the first returns V
    row 0 exactly; with a zero query, token j returns the mean of V rows
    0..n - q + j."""
    lens, qls = [3, 6], [3, 4]
    case = synth.make_case("fp8", lens, seed=12, q_lens=qls)
    out, _ = oracle_mod.decode_case(case)
    v0 = oracle_mod.dequant_rows("fp8", case.kv, [0], kv_scale=case.kv_scale)[0, :512]
    np.testing.assert_array_equal(out[0], np.broadcast_to(v0, (16, 512)))
    zq = synth.make_case("fp8", lens, seed=12, q_lens=qls, q_values=np.zeros((sum(qls), 16, 576), np.float32))
    out, _ = oracle_mod.decode_case(zq)
    for b in range(2):
        v = oracle_mod.dequant_rows("fp8", zq.kv, zq.token_rows(b), kv_scale=zq.kv_scale)[:, :512]
        for j in range(qls[b]):
            pos = lens[b] - qls[b] + j
            np.testing.assert_allclose(out[zq.qo_indptr[b] + j], np.broadcast_to(v[:pos + 1].mean(0), (16, 512)),
                                       rtol=1e-13, atol=1e-15)


def test_multi_token_reduces_to_single_token(oracle_mod):
    """One query token per sequence is single-token decode, bit for bit; the
    last query token of a sequence sees the whole sequence, and the first the
    sequence without the other query tokens' rows."""
    lens = [40, 7, 19]
    one = synth.make_case("mxfp4", lens, seed=13, q_lens=[1, 1, 1])
    single = synth.make_case("mxfp4", lens, seed=13)
    assert np.array_equal(one.q_bits, single.q_bits)
    np.testing.assert_array_equal(oracle_mod.decode_case(one)[0], oracle_mod.decode_case(single)[0])
    qls = [3, 2, 5]
    case = synth.make_case("bf16", lens, seed=14, q_lens=qls)
    out, _ = oracle_mod.decode_case(case)
    for b in range(3):
        for j, n in ((qls[b] - 1, lens[b]), (0, lens[b] - qls[b] + 1)):
            r = int(case.qo_indptr[b]) + j
            ip = np.array([0, n], dtype=np.int32)
            ref, _ = oracle_mod.mla_decode(case.q_bits[r:r + 1], "bf16", case.kv[case.kv_indptr[b]:], ip)
            np.testing.assert_allclose(out[r], ref[0], rtol=1e-13, atol=1e-15)


def test_dequant_rows_matches_independent_decode(oracle_mod):
    for fmt in synth.FORMATS:
        case = synth.make_case(fmt, [40, 9], seed=3, scale_stride=20 if fmt == "mxfp4" else 18)
        rows = np.concatenate([case.token_rows(b) for b in range(case.batch)])
        got = oracle_mod.dequant_rows(fmt, case.kv, rows, kv_scale=case.kv_scale, kv_scales=case.kv_scales)
        ref = np.concatenate(_dequant_independent(case))
        assert np.array_equal(got, ref), fmt


# ---------------------------------------------------------------------------
# closed forms
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("fmt", synth.FORMATS)
def test_single_token_returns_that_value_row(oracle_mod, fmt):
    case = synth.make_case(fmt, [1, 1, 1], seed=11)
    out, lse = oracle_mod.decode_case(case)
    v = _dequant_independent(case)
    for b in range(3):
        assert np.array_equal(out[b], np.broadcast_to(v[b][0, :512], (16, 512)))


@pytest.mark.parametrize("fmt", synth.FORMATS)
def test_zero_query_gives_mean_of_values(oracle_mod, fmt):
    lens = [37, 5]
    q = np.zeros((2, 16, 576), dtype=np.float32)
    case = synth.make_case(fmt, lens, seed=12, q_values=q)
    out, lse = oracle_mod.decode_case(case)
    v = _dequant_independent(case)
    for b, n in enumerate(lens):
        np.testing.assert_allclose(out[b], np.broadcast_to(v[b][:, :512].mean(0), (16, 512)),
                                   rtol=1e-13, atol=1e-15)
        np.testing.assert_allclose(lse[b], np.log(n), rtol=1e-14)


@pytest.mark.parametrize("fmt", synth.FORMATS)
def test_constant_values_give_that_constant(oracle_mod, fmt):
    """V columns all one (rope columns random, so the weights still vary)."""
    lens = [50, 19]
    rng = np.random.default_rng(5)
    kv = rng.standard_normal((sum(lens), 576)).astype(np.float32)
    kv[:, :512] = 1.0
    case = synth.make_case(fmt, lens, seed=13, kv_values=kv)
    out, _ = oracle_mod.decode_case(case)
    const = _dequant_independent(case)[0][0, 0]
    assert np.all(_dequant_independent(case)[1][:, :512] == const)
    np.testing.assert_allclose(out, const, rtol=1e-13)


def test_empty_sequence_gives_zero(oracle_mod):
    case = synth.make_case("fp8", [0, 4, 0], seed=14)
    out, lse = oracle_mod.decode_case(case)
    assert np.all(out[0] == 0) and np.all(out[2] == 0)
    assert np.all(np.isneginf(lse[0])) and np.all(np.isfinite(lse[1]))


@pytest.mark.parametrize("fmt", synth.FORMATS)
def test_split_merge_equals_unsplit(oracle_mod, fmt):
    lens = [100, 64, 3]
    case = synth.make_case(fmt, lens, seed=15, page_size=2, shuffle_pages=True)
    full, full_lse = oracle_mod.decode_case(case)
    partitions = [
        [[100], [64], [3]],
        [[10, 50, 100], [32, 64], [1, 2, 3]],
        [[0, 33, 33, 99, 100], [64, 64], [3]],  # empty ranges contribute nothing
    ]
    for splits in partitions:
        got, got_lse = oracle_mod.decode_case(case, splits=splits)
        np.testing.assert_allclose(got, full, rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(got_lse, full_lse, rtol=1e-12)


def test_page_shuffle_and_page_size_do_not_change_result(oracle_mod):
    lens = [21, 8, 13]
    base = synth.make_case("fp8", lens, seed=16)
    ref, _ = oracle_mod.decode_case(base)
    for ps, sh in [(2, True), (4, False), (8, True)]:
        case = synth.make_case("fp8", lens, seed=16, page_size=ps, shuffle_pages=sh)
        assert np.array_equal(case.q_bits, base.q_bits)
        got, _ = oracle_mod.decode_case(case)
        assert np.array_equal(got, ref)


def test_batch_subset_matches_full(oracle_mod):
    case = synth.make_case("bf16", [9, 4, 30, 2], seed=17)
    full, _ = oracle_mod.decode_case(case)
    part, _ = oracle_mod.decode_case(case, batches=[2, 0])
    assert np.array_equal(part[[0, 2]], full[[0, 2]])
    assert np.all(np.isnan(part[[1, 3]]))


MUTANTS = {
    # element decoders
    "nibble order swapped": ("(d % 2 == 0) ? (byte & 0xF) : (byte >> 4)",
                             "(d % 2 == 1) ? (byte & 0xF) : (byte >> 4)"),
    "e4m3 bias 8": ("v = ldexp(1.0 + (double)m / 8.0, e - 7);", "v = ldexp(1.0 + (double)m / 8.0, e - 8);"),
    "e2m1 subnormal wrong": ("v = ldexp((double)m / 2.0, 1 - 1);", "v = ldexp((double)m / 2.0, 0 - 1);"),
    "mx block of 64": ("oracle_e8m0_to_f64(sc[d / 32])", "oracle_e8m0_to_f64(sc[d / 64])"),
    "fp8 scale dropped": ("out[d] = oracle_e4m3_to_f64(r[d]) * c->kv_scale;", "out[d] = oracle_e4m3_to_f64(r[d]);"),
    # score and softmax
    "rope term dropped": ("for (d = 0; d < p->qk_dim; ++d) s += oracle_bf16_to_f64(qh[d]) * ct[d];",
                          "for (d = 0; d < p->v_dim; ++d) s += oracle_bf16_to_f64(qh[d]) * ct[d];"),
    "scale not applied": ("z[t] = p->sm_scale * s;", "z[t] = s;"),
    "normaliser off": ("for (d = 0; d < p->v_dim; ++d) o[d] /= Z;", "for (d = 0; d < p->v_dim; ++d) o[d] /= (Z + 1.0);"),
    # multi-token causal mask
    "causal mask off by one": ("t <= pos", "t < pos"),
    "causal mask from the start": ("int64_t pos = n - q + j;", "int64_t pos = j;"),
    "query rows reversed": ("int64_t row = (int64_t)p->qo_indptr[b] + j;",
                            "int64_t row = (int64_t)p->qo_indptr[b] + (q - 1 - j);"),
    "V from the rope end": ("o[d] += w * ct[d];", "o[d] += w * ct[d + (p->qk_dim - p->v_dim)];"),
    # layout
    "page index wrong": ("p->page_indices[(int64_t)p->kv_indptr[b] + j / p->page_size]",
                         "p->page_indices[(int64_t)p->kv_indptr[b] + j % p->page_size]"),
    "last page len ignored": ("return (n - 1) * p->page_size + p->last_page_len[b];",
                              "return n * p->page_size;"),
    # split merge
    "merge weight sign": ("double w = (l == -INFINITY) ? 0.0 : exp(l - M);",
                          "double w = (l == -INFINITY) ? 0.0 : exp(M - l);"),
}


def _pins_pass(lib) -> bool:
    """The brute-force, closed-form and split pins against one oracle build."""
    try:
        for fmt, lens, ps, shuffle in TINY:
            case = synth.make_case(fmt, lens, seed=7 + len(lens) + ps, page_size=ps,
                                   shuffle_pages=shuffle, guard_rows=3)
            out, _ = lib.decode_case(case)
            ref, _ = _brute_force(case)
            np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-12)
        for fmt, lens, qls, ps, shuffle in TINY_MULTI:
            case = synth.make_case(fmt, lens, seed=9 + ps, page_size=ps, shuffle_pages=shuffle, guard_rows=2,
                                   q_lens=qls)
            out, _ = lib.decode_case(case)
            ref, _ = _brute_force_multi(case)
            np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-12)
        case = synth.make_case("fp8", [100, 64, 3], seed=15, page_size=2, shuffle_pages=True)
        full, _ = lib.decode_case(case)
        got, _ = lib.decode_case(case, splits=[[10, 50, 100], [32, 64], [1, 2, 3]])
        np.testing.assert_allclose(got, full, rtol=1e-12, atol=1e-14)
        return True
    except AssertionError:
        return False


def test_planted_mistakes_are_caught(oracle_mod, tmp_path):
    """Each plausible mistake, compiled into a copy of the oracle, fails a pin."""
    from oracle import build as obuild
    src = open(obuild.SRC).read()
    assert _pins_pass(oracle_mod.default())
    for name, (old, new) in MUTANTS.items():
        assert src.count(old) >= 1, name
        mutant = tmp_path / (name.replace(" ", "_") + ".c")
        mutant.write_text(src.replace(old, new))
        lib = oracle_mod.OracleLib(obuild.build(src=str(mutant), lib=str(mutant) + ".so"))
        assert not _pins_pass(lib), f"planted mistake not caught: {name}"


# ---------------------------------------------------------------------------
# the low-precision query (one e4m3 code per element)
# ---------------------------------------------------------------------------

def _bits_to_f64(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).double()


def _torch_round_query_e4m3(q_bits):
    """Written here independently: torch's float8_e4m3fn cast (nearest, ties
    to even) of q * 2^s, s = 8 - frexp exponent of each (row, head) maximum."""
    q = _bits_to_f64(q_bits)
    amax = q.abs().amax(dim=-1, keepdim=True)
    _, ex = torch.frexp(amax)
    s = torch.where(amax > 0, 8 - ex, torch.zeros_like(ex))
    x = torch.ldexp(q, s.double())
    assert float(x.abs().max()) < 256.0
    y = torch.ldexp(x.to(torch.float8_e4m3fn).double(), -s.double())
    return y.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _query_cases():
    """bf16 queries whose heads span 2^-20 .. 2^20, with elements down in
    e4m3's subnormal range after scaling, and exact ties."""
    rng = np.random.default_rng(21)
    q = rng.standard_normal((5, 16, 576)) * np.exp2(rng.integers(-20, 21, size=(5, 16, 1)))
    q[:, :, 100:140] *= np.exp2(-np.arange(40, dtype=np.float64) / 2.0)  # 2^-1 .. 2^-20 of the head's scale
    q[1, 3] = 0.0  # a zero head
    # ties: a head with max 128 (scale 2^0) and elements halfway between e4m3 values
    q[2, 5] = 0.0
    q[2, 5, 0] = 128.0
    q[2, 5, 1:7] = [1.0625, 1.1875, -1.0625, -1.1875, 3.0 / 1024.0, 5.0 / 1024.0]
    t = torch.from_numpy(q).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def test_query_rounding_matches_torch_cast(oracle_mod):
    q = _query_cases()
    got = oracle_mod.round_query_e4m3(q)
    assert np.array_equal(got, _torch_round_query_e4m3(q))


def test_query_rounding_closed_forms(oracle_mod):
    q = _query_cases()
    got = _bits_to_f64(oracle_mod.round_query_e4m3(q)).numpy()
    # ties to the even code: 1.0625 -> 1.0, 1.1875 -> 1.25; below 2^-6 the step is 2^-9
    assert list(got[2, 5, :7]) == [128.0, 1.0, 1.25, -1.0, -1.25, 2.0 / 512.0, 2.0 / 512.0]
    assert np.all(got[1, 3] == 0.0)  # a zero head stays zero
    # values already on the e4m3 grid of their head stay (rounding twice is rounding once)
    qf = _bits_to_f64(q).numpy()
    again = _bits_to_f64(oracle_mod.round_query_e4m3(oracle_mod.round_query_e4m3(q))).numpy()
    assert np.array_equal(again, got)
    # each nonzero head's largest |q| lands in [128, 256) under its scale, its rounding in [128, 256]
    amax_q = np.abs(qf).max(axis=-1)
    live = amax_q > 0
    s = 8 - np.frexp(amax_q[live])[1]
    assert np.all((np.ldexp(amax_q[live], s) >= 128) & (np.ldexp(amax_q[live], s) < 256))
    top = np.ldexp(np.abs(got).max(axis=-1)[live], s)
    assert np.all((top >= 128) & (top <= 256))
    # at most 2^-4 relative error above the subnormal range, 2^-10 of the head's maximum below
    amax = np.abs(qf).max(axis=-1, keepdims=True)
    err = np.abs(got - qf)
    assert np.all(err <= np.maximum(np.abs(qf) / 16.0, amax * 2.0 ** -17) + 0.0)
    # scaling a head by 2^k scales the result by 2^k
    q2 = torch.from_numpy(qf * 2.0 ** 7).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got2 = _bits_to_f64(oracle_mod.round_query_e4m3(q2)).numpy()
    assert np.array_equal(got2, got * 2.0 ** 7)


QUERY_MUTANTS = {
    "ties away from zero": ("r = nearbyint(ldexp(a, 3 - e));", "r = round(ldexp(a, 3 - e));"),
    "truncated": ("r = nearbyint(ldexp(a, 3 - e));", "r = trunc(ldexp(a, 3 - e));"),
    "scale off by one": ("s = 8 - e;", "s = 7 - e;"),
    "no subnormal steps": ("if (e < -6) e = -6;", "if (e < -60) e = -60;"),
    "one scale per row": ("for (d = 0; d < qk_dim; ++d) {\n                double v = fabs(oracle_bf16_to_f64(qh[d]));",
                          "for (d = 0; d < qk_dim * nh; ++d) {\n                double v = fabs(oracle_bf16_to_f64(q[r * nh * qk_dim + d]));"),
}


def _query_pins_pass(lib) -> bool:
    q = _query_cases()
    try:
        got = lib.round_query_e4m3(q)
    except ValueError:
        return False
    if not np.array_equal(got, _torch_round_query_e4m3(q)):
        return False
    f = _bits_to_f64(got).numpy()
    return list(f[2, 5, :7]) == [128.0, 1.0, 1.25, -1.0, -1.25, 2.0 / 512.0, 2.0 / 512.0]


def test_query_rounding_planted_mistakes_are_caught(oracle_mod, tmp_path):
    from oracle import build as obuild
    src = open(obuild.SRC).read()
    assert _query_pins_pass(oracle_mod.default())
    for name, (old, new) in QUERY_MUTANTS.items():
        assert src.count(old) == 1, name
        mutant = tmp_path / (name.replace(" ", "_") + ".c")
        mutant.write_text(src.replace(old, new))
        lib = oracle_mod.OracleLib(obuild.build(src=str(mutant), lib=str(mutant) + ".so"))
        assert not _query_pins_pass(lib), f"planted mistake not caught: {name}"
