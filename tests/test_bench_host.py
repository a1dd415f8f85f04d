"""Host-side logic of bench.py (CPU only): the one-GPU guard, the roofline
objects, the per-kernel work table and the committed HBM byte counts keyed
to the kernel sources."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402
from mhla_inputs import WORKLOADS  # noqa: E402


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


@pytest.mark.parametrize("nbytes,flops,bound", [(8e9, 1e9, "hbm"), (1e6, 2.5e12, "mfma")])
def test_roofline_entry(nbytes, flops, bound):
    r = bench.roofline_entry(nbytes, flops, 1.0)   # 1 ms
    assert r["bound"] == bound
    assert r["frac"] == max(r["hbm_frac"], r["flop_frac"])
    assert r["achieved"] / r["peak"] == pytest.approx(r["frac"], rel=1e-3)
    f = bench.roofline_entry(1.0, 157.3e9, 1.0, fp32=True)
    assert f["bound"] == "alu" and f["frac"] == pytest.approx(1.0)


def test_kernel_work_adds_up_to_the_algorithmic_flops():
    """The step kernels' flops sum to the method's flops of a call; the
    single-kernel paths move exactly the algorithmic bytes; the blocked path's
    kernels move the summary tables on top of them."""
    wl = WORKLOADS["video"]
    names = ["k_summary_mfma", "k_mix_prep", "k_mix_big", "k_readout_mfma"]
    work = [bench.kernel_work(n, wl, "blocked") for n in names]
    z_mix = 2 * wl.M ** 2 * wl.d * wl.B * wl.H        # the z~ = W z product
    assert sum(f for _, f in work) == wl.algorithmic_flops() + z_mix
    assert sum(b for b, _ in work) > wl.algorithmic_bytes()
    assert work[2][1] == 2 * wl.M ** 2 * wl.d ** 2 * wl.B * wl.H
    wl = WORKLOADS["deit_t"]
    assert bench.kernel_work("k_fused", wl, "fused") == (wl.algorithmic_bytes(),
                                                         wl.algorithmic_flops())
    assert bench.kernel_work("unknown", wl, "fused") == (0, 0)


def test_measured_traffic_is_tied_to_the_kernel_sources():
    for fn in os.listdir(os.path.join(ROOT, "profiles")):
        if not fn.endswith("_hbm_bytes.md"):
            continue
        path_name, rest = fn.split("_", 1)
        workload = rest[:-len("_hbm_bytes.md")]
        assert path_name in bench.PATH_SOURCES, fn
        text = open(os.path.join(ROOT, "profiles", fn)).read()
        value = bench.measured_traffic(path_name, workload, None)
        if "source_sha256_16: %s" % bench.sources_digest(path_name) in text:
            # the committed count applies: it is the FETCH + WRITE bytes of the summary
            assert value is not None and value > 0
            assert "traffic_bytes_per_call: %d" % value in text
        else:
            assert value is None
    assert bench.measured_traffic("fused", "no_such_workload", None) is None
    assert bench.measured_traffic("no_such_path", "deit_t", "k_fused") is None
