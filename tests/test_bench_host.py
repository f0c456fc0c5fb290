"""Host-side checks of the benchmark (CPU only): the one-GPU refusal, and
the committed HBM counter records against the library as built."""
import glob
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


RECORDS = sorted(glob.glob(os.path.join(ROOT, "profiles", "traffic_*.json")))


@pytest.mark.parametrize("path", RECORDS, ids=[os.path.basename(p) for p in RECORDS])
def test_traffic_record_matches_the_built_library(path):
    """Each record names its workload and the library code it was counted
    on; while the built library has that code the bench reports the
    record's traffic, which stays within 1 % of the algorithmic bytes."""
    import bench
    rec = json.load(open(path))
    assert os.path.basename(path) == "traffic_%s.json" % rec["workload"]
    if rec["library_code_sha256_16"] != bench.kernel_hash():
        pytest.skip("counted on library code %s; this build is %s"
                    % (rec["library_code_sha256_16"], bench.kernel_hash()))
    assert bench.measured_traffic(rec["workload"]) == rec["roofline_traffic"]
    assert abs(rec["roofline_traffic"] / algorithmic_bytes(rec) - 1.0) < 0.01


def algorithmic_bytes(rec):
    """The bytes the roofline kernel must move per unit the record counts,
    derived here from the workloads' sizes (not taken from the record)."""
    import zero_sharded_optimizer_step_amd as Z
    from zero_sharded_optimizer_step_amd import workloads as W
    w = W.SHARD_13B_OF_8
    part = Z.zero_partition(w.numel, w.world_size, w.alignment)
    s = Z.zero_partition_valid_numel(part, 0)
    if rec["workload"] in ("shard13b", "shard13b_tiled", "shard13b_pingpong",
                           "shard13b_tiled_pingpong"):    # AdamW + cast: 16 B read, 14 B written
        return 30 * s
    if rec["workload"] == "shard13b_accum":  # adding pass: 8 bf16 replicas and the fp32 sum
        # plus one 16-byte partial per reduce block: 1024 elements a block,
        # the grid rounded up to a multiple of 2048 blocks
        blocks = -(-(-(-s // 1024)) // 2048) * 2048
        return (2 * w.world_size + 8) * s + 16 * blocks
    if rec["workload"] == "shard13b_local":  # adding window pass over the rank's full gradient
        return 10 * part.padded_numel
    if rec["workload"] == "zero3":           # every parameter read and written once
        return 4 * w.numel
    if rec["workload"] == "repartition":     # 3 fp32 arrays: read once, new padded written
        P = W.RAGGED_2000.numel
        return 3 * (4 * P + 4 * Z.zero_partition(P, 3, 128).padded_numel)
    if rec["workload"] == "ragged":          # 8 replicas: each real element read, padded written
        P = W.RAGGED_2000.numel
        return 8 * (2 * P + 2 * Z.zero_partition(P, 8, 128).padded_numel)
    raise AssertionError("no algorithmic figure for " + rec["workload"])


def test_one_host_core_pins_and_restores_the_thread():
    """The oracle's timing runs on one CPU of the thread's set; the set is
    restored afterwards, also when the timed block raises."""
    import threading
    import bench
    tid = threading.get_native_id()
    before = os.sched_getaffinity(tid)
    with bench.one_host_core():
        inside = os.sched_getaffinity(tid)
        rec = bench.cpu_record(10, 1.0, "sample", 100)
    assert inside == {min(before)} and "pinned to CPU %d" % min(before) in rec["sample"]
    assert "%d CPUs available" % len(before) in rec["sample"] and rec["cores"] == 1
    assert os.sched_getaffinity(tid) == before
    try:
        with bench.one_host_core():
            raise RuntimeError("inside")
    except RuntimeError:
        pass
    assert os.sched_getaffinity(tid) == before
