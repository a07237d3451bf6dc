"""CPU tests of bench.py's host side: the one-GPU guard, the oracle baseline
record it prints, the profiling build's stamp layout it reads and the
per-workgroup phase figures it derives from the stamps."""

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


def test_workgroup_phases_on_own_clocks():
    # two INT2 workgroups starting 30 us apart and one BF16 workgroup (no
    # score MFMA stamp): medians are taken on each workgroup's own clock
    import numpy as np
    wgs, waves, slots = 4, bench.STAMP_WAVES, bench.STAMP_SLOTS
    st = np.zeros((wgs, waves, slots))
    for w, t0 in ((0, 100.0), (1, 3100.0)):  # 100 MHz ticks
        st[w, :, 0] = t0 + np.arange(waves)   # wave starts
        st[w, :, 1] = t0 + 200                # first request at +2 us
        st[w, :, 4] = t0 + 500                # first score MFMA at +5 us
        st[w, :, 5] = t0 + 2000 + np.arange(waves) * 10  # loop end, latest at +20.7 us
        st[w, :, 8] = t0 + 2300               # ticket at +23 us
    st[2, :, 0], st[2, :, 5], st[2, :, 8] = 150, 700, 800  # a BF16 unit
    used = st[:, :, 0] > 0
    rel = (st - st[:, :, 0][used].min()) * 1e-2
    r = bench.int2_workgroup_phases(st, rel, used.any(axis=1))
    assert r["workgroups"] == 2
    assert (r["first_request"], r["first_score_mfma"], r["loop_end"], r["ticket"]) == (2.0, 5.0, 20.7, 23.0)
    assert r["fixed_share"] == round((5.0 + 23.0 - 20.7) / 23.0, 3)
