"""The benchmark's use of stored HBM counter records: a record counts only
for a run with the partition size and (decode) upload placement it was
taken with, and is rescaled for other step counts; a record of other kernel
sources is never loaded."""
import importlib.util
import json
import os

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
_spec = importlib.util.spec_from_file_location("bench_module", os.path.join(ROOT, "bench.py"))
bench = importlib.util.module_from_spec(_spec)
_spec.loader.exec_module(bench)

REC = {"partition_size": 0, "upload": "within the previous step's decode launch", "steps": 50,
       "warmup": 5, "traffic_bytes_per_launch": 2_000_000, "traffic_over_algorithmic": 0.9,
       "algorithmic_bytes_per_launch": 2_222_222}


def test_record_applies_to_the_same_launch_configuration_only():
    up = REC["upload"]
    assert bench.traffic_for(REC, 0, up, False, 50, 5, 123) == (2_000_000, None)
    assert bench.traffic_for(REC, 512, up, False, 50, 5, 123) == (None, None)
    assert bench.traffic_for(REC, 0, "own launch on a side stream", False, 50, 5, 123) == (None, None)
    assert bench.traffic_for(None, 0, up, False, 50, 5, 123) == (None, None)
    # the prefill step has no upload placement of its own
    pre = dict(REC, upload=None)
    assert bench.traffic_for(pre, 0, "own launch on a side stream", True, 50, 5, 1) == (2_000_000, None)


def test_other_step_counts_rescale_by_traffic_per_algorithmic_byte():
    t, note = bench.traffic_for(REC, 0, REC["upload"], False, 20, 3, 1_000_000)
    assert t == 900_000 and "50-step counter run" in note


def test_committed_records_load_only_for_their_kernel_sources():
    """Every committed record names the sources it was measured on; the
    loader returns it while those sources are unchanged and refuses it
    otherwise."""
    prof = os.path.join(ROOT, "profiles")
    names = [n for n in os.listdir(prof) if n.startswith("traffic_") and n.endswith(".json")]
    assert names
    for n in names:
        rec = json.load(open(os.path.join(prof, n)))
        kind = "prefill" if rec["workload"].startswith("prefill") else "decode"
        for key in ("partition_size", "upload", "kernel_source_sha256", "traffic_bytes_per_launch"):
            assert key in rec, (n, key)
        loaded = bench.load_traffic(rec["workload"], rec["decode_path"], kind)
        if rec["kernel_source_sha256"] == bench.kernel_source_hash(kind):
            assert loaded == rec, n
        else:
            assert loaded is None, n
