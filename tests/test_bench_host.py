"""bench.py's host-side contract (no GPU needed): it measures one GPU only and
says so for any request of more, before it touches a device; the HBM traffic it
reports comes from the committed counter summary only while that summary's
recorded kernel-source hash matches the current sources."""
import importlib.util
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BENCH = os.path.join(ROOT, "bench.py")


def _bench_module():
    spec = importlib.util.spec_from_file_location("bench_under_test", BENCH)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _run(args, env_extra=None):
    env = dict(os.environ)
    env.update(env_extra or {})
    return subprocess.run([sys.executable, BENCH] + args, capture_output=True, text=True, env=env, timeout=120)


def test_more_than_one_gpu_is_refused_with_a_message():
    r = _run(["--gpus", "2", "--steps", "1", "--warmup", "0"])
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_multi_rank_launch_is_refused_with_a_message():
    r = _run(["--steps", "1", "--warmup", "0"], {"WORLD_SIZE": "4", "RANK": "0"})
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_traffic_follows_the_kernel_source_hash(tmp_path):
    b = _bench_module()
    h = b.kernel_source_hash()
    assert len(h) == 64
    summary = tmp_path / "traffic.md"
    summary.write_text("traffic_bytes_per_launch: 4.25e+09\nkernel_source_sha256: %s\n" % h)
    b.TRAFFIC_FILE = str(summary)
    value, note = b.committed_traffic()
    assert value == 4.25e9 and "FETCH_SIZE" in note
    summary.write_text("traffic_bytes_per_launch: 4.25e+09\nkernel_source_sha256: %s\n" % ("0" * 64))
    value, note = b.committed_traffic()
    assert value is None and "changed" in note
    b.TRAFFIC_FILE = str(tmp_path / "missing.md")
    assert b.committed_traffic()[0] is None


def test_timed_steps_split_into_repetitions():
    """The timed region is exactly K steps, split into at most 5 repetitions whose
    median is reported; fewer steps than repetitions give one step each."""
    bench = _bench_module()
    assert bench.split_reps(20) == [4, 4, 4, 4, 4]
    assert bench.split_reps(7) == [2, 2, 1, 1, 1] and sum(bench.split_reps(7)) == 7
    assert bench.split_reps(3) == [1, 1, 1]
    assert bench.split_reps(1) == [1]
    assert bench.median([3.0, 1.0, 2.0]) == 2.0
    assert bench.median([4.0, 1.0, 2.0, 3.0]) == 2.5
