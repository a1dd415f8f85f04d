"""Host-side logic of bench.py (CPU only): the one-GPU guard, the roofline
object of a whole call, and the committed HBM byte counts keyed to the
kernel sources."""
import hashlib
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


@pytest.mark.parametrize("gbs,tfs,bound", [(4000.0, 100.0, "hbm"), (100.0, 1500.0, "mfma")])
def test_roofline_of_call_reports_the_binding_fraction(gbs, tfs, bound):
    r = bench.roofline_of_call(gbs, tfs, 123, 456)
    for key in ("bound", "achieved", "peak", "unit", "frac", "traffic"):
        assert key in r
    assert r["bound"] == bound
    hbm, mfma = gbs / bench.HBM_PEAK_GBS, tfs / bench.BF16_PEAK_TFLOPS
    assert r["frac"] == round(max(hbm, mfma), 4)
    assert r["achieved"] / r["peak"] == pytest.approx(max(hbm, mfma), rel=1e-3)
    assert r["unit"] == ("GB/s" if bound == "hbm" else "TFLOP/s")
    assert r["traffic"] is None
    json.dumps(r)


def _source_digest(kernel):
    h = hashlib.sha256()
    for name in bench.KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, "token_level_head_mhla_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def test_measured_traffic_is_tied_to_the_kernel_sources():
    summary = os.path.join(ROOT, "profiles", "k_fused_deit_t_hbm_bytes.md")
    text = open(summary).read()
    value = bench.measured_traffic("k_fused", "deit_t")
    if "source_sha256_16: %s" % _source_digest("k_fused") in text:
        # the committed count applies: it is the FETCH + WRITE bytes of the summary
        assert value is not None and value > 0
        assert "traffic_bytes_per_launch: %d" % value in text
    else:
        assert value is None
    assert bench.measured_traffic("k_fused", "no_such_workload") is None
    assert bench.measured_traffic("no_such_kernel", "deit_t") is None
