"""bench.py's host side: the CPU oracle baseline it reports beside the GPU figure."""
import os
import sys

import ttt_inputs as ti

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import bench  # noqa: E402


def test_cpu_baseline_fields():
    cfg = ti.CONFIGS["tiny"].with_(B=2, H=2)
    r = bench.cpu_baseline(cfg, ti.generate(cfg), sample_chains=4)
    assert r["kind"] == "oracle" and r["unit"] == "tokens/s"
    assert r["value"] > 0 and r["cores"] >= 1
    assert isinstance(r["cpu_model"], str) and r["cpu_model"]
    one = r["one_thread"]
    assert one["value"] > 0 and one["unit"] == "tokens/s" and "1 thread" in one["sample"]
    # a 1-thread run must not lower the thread count later calls report
    again = bench.cpu_baseline(cfg, ti.generate(cfg), sample_chains=4)
    assert again["cores"] == r["cores"]


def test_cpu_baseline_layer_norm_forms():
    for name in ("tiny", "mlp"):
        cfg = ti.CONFIGS[name].with_(B=1, H=2, T=32)
        r = bench.cpu_baseline(cfg, ti.generate(cfg), sample_chains=2, ln=True)
        assert r["value"] > 0 and r["one_thread"]["value"] > 0
