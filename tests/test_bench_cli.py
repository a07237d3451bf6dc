"""CPU tests of bench.py's host side: the one-GPU guard, the oracle baseline
record it prints, and the profiling build's stamp layout it reads."""

import os
import re
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from synthetic import CONFIGS  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_cpu_baseline_record():
    res = bench.cpu_baseline(CONFIGS["tiny-d64-l512"], repeats=1)
    assert res["kind"] == "oracle" and res["unit"] == "GB/s"
    assert res["value"] > 0 and res["cores"] >= 1
    assert res["sample"] and res["cpu_model"]
    wp = res["write_path"]
    assert wp["token_heads_per_s"] > 0 and "W1-W7" in wp["sample"]
    if "single_thread" in res:
        assert res["single_thread"]["cores"] == 1 and res["single_thread"]["value"] > 0


def test_stamp_layout_matches_the_library():
    text = open(os.path.join(ROOT, "long_context_decode_oscar_amd", "csrc", "kernels.h")).read()
    vals = {k: int(v) for k, v in re.findall(r"constexpr int (kStamp\w+) = (\d+);", text)}
    assert vals == {"kStampSlots": bench.STAMP_SLOTS, "kStampWgs": bench.STAMP_WGS, "kStampWaves": bench.STAMP_WAVES}
    # every named phase point fits the per-wave slots
    assert len(bench.PHASES) <= bench.STAMP_SLOTS
