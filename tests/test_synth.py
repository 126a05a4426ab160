"""Properties of the seeded input generator (CPU only)."""

import numpy as np
import torch

from latent_attention_decode_amd import synth


def test_seeded_and_deterministic():
    a = synth.make_case("fp8", [10, 3], seed=1)
    b = synth.make_case("fp8", [10, 3], seed=1)
    c = synth.make_case("fp8", [10, 3], seed=2)
    assert np.array_equal(a.kv, b.kv) and np.array_equal(a.q_bits, b.q_bits)
    assert not np.array_equal(a.kv, c.kv)


def test_fp8_encoder_is_per_tensor_amax_over_448():
    x = torch.randn(300, 576, generator=torch.Generator().manual_seed(0))
    codes, scale = synth.encode_fp8_per_tensor(x)
    assert np.float32(scale) == np.float32(float(x.abs().max()) / 448.0)
    dec = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.abs(dec).max() <= 448.0 and not np.isnan(dec).any()
    # round to nearest: error at most half a step of e4m3 (relative 2^-4), plus subnormal step
    y = x.double().numpy() / scale
    assert np.all(np.abs(dec - y) <= np.maximum(np.abs(y) * 2.0 ** -4, 2.0 ** -10) + 1e-9)


def test_mxfp4_encoder_picks_nearest_grid_value():
    x = torch.randn(64, 576, generator=torch.Generator().manual_seed(1))
    packed, scales = synth.encode_mxfp4(x, scale_stride=20)
    assert packed.shape == (64, 288) and scales.shape == (64, 20)
    assert np.all(scales[:, 18:] == 127)
    e8 = scales[:, :18].astype(np.int64)
    assert e8.min() >= 1 and e8.max() <= 254
    grid = np.array(synth.E2M1_GRID)
    codes = np.empty((64, 576), dtype=np.int64)
    codes[:, 0::2] = packed & 0xF
    codes[:, 1::2] = packed >> 4
    mag = grid[codes & 7]
    sign = np.where(codes & 8, -1.0, 1.0)
    scale = np.repeat(2.0 ** (e8 - 127), 32, axis=1)
    y = x.double().numpy() / scale
    dec = sign * mag
    # nearest representable (saturating at 6): no grid point is strictly closer
    dist = np.abs(dec - y)
    best = np.min(np.abs(np.abs(y)[..., None] - grid[None, None, :]), axis=-1)
    assert np.all(dist <= best + 1e-12)
    # the block amax lands in [4, 8) after scaling (so nothing overflows by more than 2)
    amax = np.abs(y).reshape(64, 18, 32).max(-1)
    assert np.all(amax < 8.0) and np.all(amax >= 3.5)


def test_paged_layout_and_poison():
    lens = [5, 0, 4]
    case = synth.make_case("fp8", lens, seed=3, page_size=2, shuffle_pages=True, guard_rows=2)
    assert list(case.kv_indptr) == [0, 3, 3, 5]
    assert list(case.kv_last_page_len) == [1, 0, 2]
    assert sorted(case.kv_page_indices.tolist()) == list(range(5))
    used = np.concatenate([case.token_rows(b) for b in range(3)])
    assert len(set(used.tolist())) == 9
    unused = sorted(set(range(case.kv.shape[0])) - set(used.tolist()))
    assert len(unused) == 1 + 2  # slack of sequence 0's last page + guard rows
    assert np.all(case.kv[unused] == 0x7F)
    flat = synth.make_case("fp8", lens, seed=3)
    # same values, different placement
    for b in range(3):
        assert np.array_equal(case.kv[case.token_rows(b)], flat.kv[flat.token_rows(b)])


def test_named_configs_shapes():
    lens = synth.config_lens("bs256_ragged1024-8192_fp8_paged2")
    assert lens.size == 256 and lens.min() >= 1024 and lens.max() <= 8192
    assert abs(lens.mean() - 4608) < 300
    assert synth.config_lens("bs64_kv8192_fp8").sum() == 64 * 8192
