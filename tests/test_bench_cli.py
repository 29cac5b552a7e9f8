"""bench.py's command-line contract on a host without a GPU: one GPU only (any other --gpus exits
with a message and status 2), and the long-context options are checked before anything runs."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True,
                          text=True, timeout=300)


def test_more_than_one_gpu_is_refused():
    r = _run("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_help_lists_the_workload_options():
    r = _run("--help")
    assert r.returncode == 0
    for opt in ("--config", "--r", "--seq", "--tokens", "--loss-side", "--no-loss-side", "--steps", "--warmup"):
        assert opt in r.stdout


def test_algorithmic_work_counts():
    """The work counts behind the roofline figures, recomputed from the layer shapes by hand."""
    sys.path.insert(0, ROOT)
    import bench
    import synth
    cfg = synth.get_config("tinyllama")
    Mk, H, I, d, nq, nkv = 4916, 2048, 5632, 64, 32, 4
    counts = [1229, 1229, 1229, 1229]
    w = bench.algorithmic_work(cfg, Mk, counts)
    # weights: qkv [2560 x 2048], o [2048 x 2048], gate/up [11264 x 2048], down [2048 x 5632]
    proj = 2560 * 2048 + 2048 * 2048 + 11264 * 2048 + 2048 * 5632
    assert w["gemm_flops"] == 4.0 * Mk * proj                     # dX and dW, 2 M' K N each
    assert abs(w["gemm_flops"] - 8.66e11) / 8.66e11 < 2e-3       # the layer's 866 GFLOP
    pairs = 4 * 1229 * 1230 // 2
    assert w["pairs"] == pairs
    assert w["attn_flops"] == 10.0 * d * nq * pairs
    assert w["attn_dt_flops"] == 2.0 * d * nq * pairs             # the extra P K product
    # gathered per kept token: dY's row (2H B), read and written; the rest is read through idx
    assert w["gather_bytes"] == 2.0 * Mk * 2 * H
    # scatter: +0.0 written to each filtered row of dx
    assert w["scatter_bytes"] == 2.0 * (4 * 2048 - Mk) * H
    assert w["gemm_launches"] == 8
