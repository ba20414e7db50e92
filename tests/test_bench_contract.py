"""Host-side checks of bench.py's contract (no GPU): the one-GPU refusal and
the rule that a committed counter record supplies roofline.traffic only
while it was taken on the current kernel sources."""
import glob
import importlib.util
import json
import os
import re
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2", "--steps", "1"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""  # no JSON line


def test_counter_records():
    paths = sorted(glob.glob(os.path.join(ROOT, "profiles", "*_counters.json")))
    names = {os.path.basename(p) for p in paths}
    assert {"split_decode_hybrid128k_counters.json", "split_decode_exact32k_counters.json",
            "split_decode_ragged_counters.json", "chunk512_counters.json"} <= names
    for p in paths:
        rec = json.load(open(p))
        assert re.fullmatch(r"[0-9a-f]{16}", rec["kernel_source_hash"]), p
        assert rec["fetch_scale"] > 0 and rec["write_scale"] > 0, p
        parts = [rec[k]["hbm_bytes"] for k in ("split_kernel", "merge_kernel")]
        assert all(b > 0 for b in parts), p
        assert abs(sum(parts) - rec["hbm_bytes_per_launch"]) <= 1e-6 * rec["hbm_bytes_per_launch"], p
        assert rec["commands"] and all("rocprofv3 --pmc" in c for c in rec["commands"]), p


def test_traffic_only_with_a_matching_source_hash():
    b = _bench()
    for name in ("split_decode_hybrid128k_counters.json", "chunk512_counters.json"):
        rec = json.load(open(os.path.join(ROOT, "profiles", name)))
        assert b.traffic_from_profile(name, rec["kernel_source_hash"]) == rec["hbm_bytes_per_launch"]
        assert b.traffic_from_profile(name, "0" * 16) is None
    assert b.traffic_from_profile("no_such_record.json", "0" * 16) is None
    # the hash covers the named sources' bytes
    assert b.source_hash(b.KERNEL_SOURCES) != b.source_hash(b.CHUNK_SOURCES)
