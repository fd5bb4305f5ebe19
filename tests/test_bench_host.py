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


def test_cpu_baseline_backward_forms():
    for name, ln in (("tiny", False), ("tiny", True), ("mlp", False), ("mlp", True)):
        cfg = ti.CONFIGS[name].with_(B=1, H=2, T=32)
        r = bench.cpu_baseline_bwd(cfg, ti.generate(cfg), sample_chains=2, ln=ln)
        assert r["value"] > 0 and r["kind"] == "oracle" and "reverse pass" in r["sample"]


def test_mlp_backward_work_counts():
    """Twenty d x dh multiply-adds per token-head, plus the mini-batch corrections."""
    cfg = ti.CONFIGS["mlp"].with_(B=2, H=3, T=64)
    by, fl = bench.algorithmic_mlp_bwd(cfg, (0, 0, 0))
    th = 2 * 3 * 64
    assert fl == th * (40 * 64 * 256 + 3 * (64 + 256) * 17)
    st = 2 * 64 * 256 * 4
    assert by == th * 64 * (3 * 2 + 4 + 12) + 4 + 4 * th + 3 * st + 2 * 6 * st
    by_ln, fl_ln = bench.algorithmic_mlp_bwd(cfg, (0, 0, 0), ln=True)
    assert fl_ln == fl and by_ln == by + 3 * 2 * 64 * 4 + 6 * 2 * 64 * 4   # gamma, beta in; dgamma, dbeta out


def test_mlp_modes_rejected_on_the_host():
    import subprocess

    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    for extra in (["--save"], ["--train", "--ln"], ["--train", "--primal"]):
        r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--config", "mlp", *extra],
                           capture_output=True, text=True, timeout=120)
        assert r.returncode == 2 and "TTT-MLP" in r.stderr, (extra, r.stderr[-300:])
