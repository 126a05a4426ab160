"""Host-side checks of bench.py: the one-GPU contract and the traffic records."""

import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_traffic_records_match_their_workloads():
    """Each committed record names its workload and kernel, holds read + written bytes,
    and is used only while its source hash matches the kernel sources."""
    import bench
    from latent_attention_decode_amd import synth
    pdir = os.path.join(ROOT, "profiles")
    names = [f for f in os.listdir(pdir) if f.endswith("_traffic.json")]
    assert names
    for f in names:
        with open(os.path.join(pdir, f)) as fh:
            rec = json.load(fh)
        w = rec["workload"]
        assert f == f"stage1_{w}_traffic.json" and w in synth.CONFIGS
        fmt = synth.CONFIGS[w][0]
        assert rec["hbm_bytes_per_launch"] == rec["hbm_read_bytes_per_launch"] + rec["hbm_write_bytes_per_launch"]
        # HBM bytes cover at least the cache once, and the calibration factors are sane
        assert rec["hbm_read_bytes_per_launch"] >= rec["algorithmic_kv_bytes_per_launch"]
        assert 0.5 < rec["copy_calibration"]["factor_FETCH_SIZE"] < 4
        got = bench.traffic_record(w, fmt)
        if rec["kernel_sha256_16"] == bench.kernel_hash(fmt):
            assert got == rec["hbm_bytes_per_launch"]
        else:
            assert got is None


def test_page_time_is_only_for_its_workload():
    import bench
    from latent_attention_decode_amd import synth
    assert set(bench.PAGE_US) <= set(synth.CONFIGS)
    assert bench.PAGE_US == {"bs256_kv8192_mxfp4": pytest.approx(236.6)}


def test_headline_and_target_workloads():
    """The headline is the largest listed workload (256 ragged sequences in 2-token
    pages); the target shapes (32 and 64 sequences of 8192 tokens, fp8) ride in
    the same line."""
    import bench
    from latent_attention_decode_amd import synth
    assert bench.DEFAULT_WORKLOAD == "bs256_ragged1024-8192_fp8_paged2"
    for t in bench.TARGETS:
        fmt, batch, kv_len = synth.CONFIGS[t][:3]
        assert fmt == "fp8" and batch >= 32 and kv_len == 8192
