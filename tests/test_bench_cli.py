"""Host-side contract of bench.py and of the committed profile summaries (no GPU needed)."""
import glob
import json
import os
import re
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BENCH = os.path.join(ROOT, "bench.py")


def run_bench(*args):
    env = dict(os.environ)
    env.pop("WORLD_SIZE", None)
    return subprocess.run([sys.executable, BENCH, *args], capture_output=True, text=True, timeout=120, env=env,
                          cwd=ROOT)


def test_more_than_one_gpu_is_refused_with_a_message():
    p = run_bench("--gpus", "2", "--steps", "1", "--warmup", "0")
    assert p.returncode == 2
    assert "one GPU" in p.stderr
    assert p.stdout.strip() == ""


def test_help_lists_the_single_leg_options():
    p = run_bench("--help")
    assert p.returncode == 0
    for opt in ("--gpus", "--steps", "--warmup", "--main-only", "--prompt-decode-only", "--no-graphs",
                "--no-cpu-baseline", "--batch-paths"):
        assert opt in p.stdout, opt


def test_every_profile_summary_names_its_command():
    files = sorted(glob.glob(os.path.join(ROOT, "profiles", "*.md")))
    assert files
    for f in files:
        text = open(f).read()
        assert "rocprofv3" in text, f
        assert re.search(r"rocprofv3 [^\n]*--", text), f


def test_counter_summaries_carry_source_hash_and_bytes():
    for f in sorted(glob.glob(os.path.join(ROOT, "profiles", "*_traffic.md"))):
        m = re.search(r"```json\n(.*?)\n```", open(f).read(), re.S)
        assert m, f
        d = json.loads(m.group(1))
        assert os.path.exists(os.path.join(ROOT, d["source"])), f
        assert re.fullmatch(r"[0-9a-f]{64}", d["source_sha256"]), f
