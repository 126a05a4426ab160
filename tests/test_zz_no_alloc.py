"""The allocation-free run entry point (mla_decode_run_noalloc) against the
workspace entry point (mla_decode_run), through the C ABI."""

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


def check_close(got, ref, fmt, what):
    atol, rtol = TOL[fmt]
    err = np.abs(got - ref)
    print(f"{what}: max|err|={np.nanmax(err):.3e}", file=sys.stderr, flush=True)
    assert np.all(err <= atol + rtol * np.abs(ref)), what


def both_entry_points(B, dec, case, t):
    """One run through each entry point on the current plan; host copies."""
    a = torch.full((case.rows, 16, 512), float("nan"), dtype=torch.bfloat16, device="cuda")
    b = torch.full_like(a, float("nan"))
    dec.run(t["q"], t["kv"], t["kv_scales"], t["kv_indptr"], a, t["kv_page_indices"], t["kv_last_page_len"])
    B.mla_decode_run_noalloc(dec.h, t["q"], t["kv"], t["kv_scales"], t["kv_indptr"], b, t["kv_page_indices"],
                             t["kv_last_page_len"])
    torch.cuda.synchronize()
    return a, b


@pytest.mark.parametrize("fmt,ps", [("fp8", 1), ("fp8", 2), ("mxfp4", 1), ("bf16", 1)])
def test_noalloc_matches_the_workspace_run(B, oracle_mod, fmt, ps):
    """Two calls in a row on one handle, the second planned for a smaller
    input: each matches the workspace entry point bit for bit and the oracle
    within the tolerance (the second call finds the first one's partials in
    the array)."""
    shapes = [[8192, 6000, 3001, 129, 4096], [2048] * 3]
    dec = B.MlaDecode(fmt, ps)
    try:
        sizes = []
        for k, lens in enumerate(shapes):
            case = synth.make_case(fmt, lens, seed=700 + k, page_size=ps, shuffle_pages=ps > 1)
            t = B.case_to_device(case)
            sizes.append(dec.plan(case.kv_indptr, case.kv_last_page_len))
            a, b = both_entry_points(B, dec, case, t)
            assert torch.equal(a.view(torch.int16), b.view(torch.int16)), f"call {k}"
            ref, _ = oracle_mod.decode_case(case)
            check_close(b.float().cpu().numpy().astype(np.float64), ref, fmt, f"noalloc {fmt} ps {ps} call {k}")
        assert 0 < sizes[1] < sizes[0] <= B.MLA_SCRATCH_BYTES
    finally:
        dec.close()


def test_noalloc_refuses_plans_beyond_its_array(B):
    """A plan with more partials than the array holds is refused before any
    launch, and the handle then runs a smaller plan correctly."""
    case = synth.make_case("fp8", [8192] * 3, seed=710)
    t = B.case_to_device(case)
    dec = B.MlaDecode("fp8")
    try:
        ws = dec.plan(case.kv_indptr, None, 256)  # one 32-token item each: 768 partials
        assert ws > B.MLA_SCRATCH_BYTES
        out = torch.full((3, 16, 512), float("nan"), dtype=torch.bfloat16, device="cuda")
        with pytest.raises(B.MlaError) as e:
            B.mla_decode_run_noalloc(dec.h, t["q"], t["kv"], t["kv_scales"], t["kv_indptr"], out)
        assert e.value.status == 2 and "at most" in str(e.value)
        torch.cuda.synchronize()
        assert torch.isnan(out.float()).all()  # nothing ran
        dec.plan(case.kv_indptr, None, 8)
        a, b = both_entry_points(B, dec, case, t)
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    finally:
        dec.close()
