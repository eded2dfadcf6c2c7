"""bench.py's command line on the CPU: it measures one GPU and says so."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_help_lists_the_options():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--help"], capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 0
    for opt in ("--gpus", "--steps", "--warmup", "--configs", "--pmc"):
        assert opt in r.stdout


def test_a_trial_times_at_least_200_launches_over_whole_pool_passes():
    sys.path.insert(0, ROOT)
    import bench

    assert bench.launches_per_trial(20, 29) == 203  # the driver's --steps 20 over a 29-buffer pool
    assert bench.launches_per_trial(200, 1) == 200
    assert bench.launches_per_trial(500, 29) == 522
    for steps, pool in ((1, 1), (20, 29), (199, 7), (1000, 3)):
        n = bench.launches_per_trial(steps, pool)
        assert n >= max(200, steps) and n % pool == 0 and n - pool < max(200, steps)
