"""Host checks of bench.py's bookkeeping (no GPU): the code hash that keys the
recorded HBM byte counters ignores comments and white space but not code, and
a counter record taken for other code is not reported; the power-cap bound's
arithmetic, and no power fields without a power sensor."""
import json
import os
import shutil

import bench

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


def _tree(tmp_path):
    """A copy of the HIP sources and the C header under tmp_path."""
    shutil.copytree(os.path.join(ROOT, "sync_protocols_amd", "csrc"), tmp_path / "sync_protocols_amd" / "csrc")
    os.makedirs(tmp_path / "include")
    shutil.copy(os.path.join(ROOT, "include", "fg.h"), tmp_path / "include" / "fg.h")
    os.makedirs(tmp_path / "profiles")
    return tmp_path


def _edit(path, old, new):
    with open(path) as f:
        text = f.read()
    assert old in text
    with open(path, "w") as f:
        f.write(text.replace(old, new, 1))


def test_hash_ignores_comments_not_code(tmp_path, monkeypatch):
    root = _tree(tmp_path)
    monkeypatch.setattr(bench, "ROOT", str(root))
    h0 = bench.kernel_source_hash()
    assert h0 == bench.kernel_source_hash()
    hdr = root / "include" / "fg.h"
    _edit(hdr, "/* Per-call flags of fg_gather_gemm. */", "/* Per-call   flags, reworded. */\n\n")
    assert bench.kernel_source_hash() == h0, "a comment or white-space edit changed the hash"
    src = root / "sync_protocols_amd" / "csrc" / "fg_plan.hpp"
    _edit(src, "return (per_list + n_tn - 1) / n_tn;", "return (per_list + n_tn) / n_tn;")
    assert bench.kernel_source_hash() != h0, "a code edit left the hash unchanged"


def test_traffic_record_only_for_the_same_code(tmp_path, monkeypatch):
    root = _tree(tmp_path)
    monkeypatch.setattr(bench, "ROOT", str(root))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(root / "profiles" / "traffic.json"))
    assert bench.recorded_traffic("large") is None          # no record at all
    rec = {"source_sha256": bench.kernel_source_hash(),
           "workloads": {"large": {"hbm_bytes_per_launch": 123456789}}}
    with open(root / "profiles" / "traffic.json", "w") as f:
        json.dump(rec, f)
    assert bench.recorded_traffic("large") == 123456789
    assert bench.recorded_traffic("tp") is None             # no entry for this workload
    rec["source_sha256"] = "0" * 64
    with open(root / "profiles" / "traffic.json", "w") as f:
        json.dump(rec, f)
    assert bench.recorded_traffic("large") is None          # taken for other code


def test_committed_traffic_record_matches_the_sources():
    """The committed counter record is keyed to the committed kernel code, so
    the bench line reports it (re-collected whenever the kernel changes)."""
    with open(os.path.join(ROOT, "profiles", "traffic.json")) as f:
        rec = json.load(f)
    assert rec["source_sha256"] == bench.kernel_source_hash()
    for w in ("large", "tp"):
        assert rec["workloads"][w]["hbm_bytes_per_launch"] > 0


def test_more_than_one_gpu_is_refused():
    """`bench.py --gpus N` with N > 1 (or a multi-rank launch) exits with a
    message before it touches a GPU: the path runs on one GPU."""
    import subprocess
    import sys
    for argv, env in ((["--gpus", "2"], {}), ([], {"WORLD_SIZE": "8"})):
        r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *argv], capture_output=True, text=True,
                           env={**os.environ, **env}, timeout=120)
        assert r.returncode == 2, (argv, env, r.returncode, r.stderr)
        assert "one GPU" in r.stderr and r.stdout == ""


def test_power_sensor_absent_gives_no_power_fields(monkeypatch):
    """Without the board's hwmon node (as on a host with no GPU) the power
    fields are left out rather than invented."""
    monkeypatch.setattr("glob.glob", lambda pattern: [])
    assert bench._power_files() is None


def test_power_bound_arithmetic():
    """The bound under a power cap: with the board at its cap, the fused step
    takes at least T_comp + P_copy * T_comm / P_cap (the copy's whole energy),
    so efficiency (T_comp + T_comm - T_total) / T_comm is at most 1 - P_copy /
    P_cap; counted from the idle board, 1 - (P_copy - P_idle) / P_cap. A fused
    step exactly at the energy floor reaches the whole-energy bound."""
    res = {"cap_W": 1400.0, "idle_W": 300.0,
           "gemm_only": {"W": 1400.0, "us_per_step": 3000.0},
           "comm_only": {"W": 700.0, "us_per_step": 200.0},
           "fused": {"W": 1400.0, "us_per_step": 3100.0}}
    b = bench.power_bounds(res)
    assert b["overlap_bound_whole"] == 0.5
    assert abs(b["overlap_bound_incremental"] - (1 - 400 / 1400)) < 1e-4
    assert b["T_total_energy_floor_us"] == 3100.0
    assert b["overlap_efficiency_back_to_back"] == 0.5
