"""bench.py's command line on the CPU: the one-GPU contract and the offline
profile-command listing (no GPU, no library call)."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True,
                          text=True, timeout=120, cwd=ROOT)


def test_more_than_one_gpu_exits_with_a_message():
    r = _run("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_profile_commands_name_committed_files_only():
    r = _run("--print-profile-commands", "prof_out/x")
    assert r.returncode == 0, r.stderr
    lines = [l.split("\t") for l in r.stdout.strip().splitlines()]
    assert [k for k, _ in lines] == ["stats", "fetch", "write", "mfma", "waves", "l2"]
    for _, cmd in lines:
        assert cmd.startswith("rocprofv3 ") and " -- python -u bench.py " in cmd
        assert "_work" not in cmd
    # counter passes never mix with tracing, and stay within one block's limits
    for k, cmd in lines:
        if k != "stats":
            assert "--pmc" in cmd and "--kernel-trace" not in cmd and "--sys-trace" not in cmd
            counters = cmd.split("--pmc ")[1].split(" --")[0].split()
            assert sum(c.startswith("SQ_") for c in counters) <= 8
            assert sum(c.startswith("TCC_") for c in counters) <= 4
            assert sum(c.startswith("GRBM_") for c in counters) <= 2
