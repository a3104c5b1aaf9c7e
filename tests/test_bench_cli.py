"""bench.py's command line on the host: the one-GPU contract (any other GPU
count exits with status 2 and says why, before touching a device) and the
help text listing every documented option."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench(*args, env=None):
    e = dict(os.environ)
    e.update(env or {})
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          cwd=ROOT, env=e, timeout=120)


def test_more_than_one_gpu_is_refused_with_a_message():
    r = _bench("--gpus", "2", "--steps", "1", "--warmup", "0")
    assert r.returncode == 2
    assert "one GPU" in r.stderr and "--gpus 2" in r.stderr
    assert r.stdout == ""


def test_a_multi_rank_launch_is_refused_too():
    r = _bench("--steps", "1", env={"WORLD_SIZE": "4"})
    assert r.returncode == 2 and "WORLD_SIZE=4" in r.stderr


def test_help_lists_the_options():
    r = _bench("--help")
    assert r.returncode == 0
    for opt in ("--gpus", "--steps", "--warmup", "--workload", "--path", "--backward", "--fp8", "--headline-only",
                "--cpu-single-thread", "--cpu-sample-qblocks", "--no-cpu-baseline", "--calibrate-copy-mib",
                "--dense-vs-sdpa"):
        assert opt in r.stdout, opt


def test_counter_traffic_follows_the_kernel_code_not_its_comments(tmp_path):
    """The committed fabric-byte counters are reported only for the attention code they were taken on: the source
    hash ignores comments and blank lines, and changes with any code token."""
    sys.path.insert(0, ROOT)
    import bench

    src = tmp_path / "k.hip"
    src.write_text("// header\nint f(int x) {  /* body */\n  return x + 1;  // done\n}\n")
    h0 = bench.sources_hash([str(src)])
    src.write_text("// a longer header\n\nint f(int x) {  /* other words */\n  return x + 1;\n}\n")
    assert bench.sources_hash([str(src)]) == h0
    src.write_text("// header\nint f(int x) {\n  return x + 2;\n}\n")
    assert bench.sources_hash([str(src)]) != h0
