"""Host-side accounting of bench.py, on the CPU: the HBM traffic written from
two rocprofv3 counter runs (scaled by the bench's own device copy, summed
per call), its invalidation when the kernel sources change, the MFMA-busy
summary, and the refusal of more than one GPU.  The counter files are
synthetic, in the column layout rocprofv3 writes."""
import csv
import json
import os
import subprocess
import sys

import pytest

import bench

FIELDS = ["Dispatch_Id", "Kernel_Name", "Grid_Size", "Workgroup_Size", "Counter_Name", "Counter_Value"]
PREP = "void kda::(anonymous namespace)::chunk_prep_kernel<false, false>(kda::ChunkArgs, ...)"
SCAN = "void kda::(anonymous namespace)::chunk_scan_kernel<unsigned short, false, false, true, true>(...)"
DECODE = "void kda::(anonymous namespace)::decode_step_kernel<128, 128, unsigned short, unsigned short>(...)"
COPY = "__amd_rocclr_copyBuffer"
# the staged headline call: pass-1 workgroups of its four stages (96 heads x 657, 236, 85, 46 chunks)
STAGE_WGS = [63072, 22656, 8160, 4416]


def _write_counters(d, counter, rows):
    os.makedirs(os.path.join(d, "host"), exist_ok=True)
    with open(os.path.join(d, "host", "p_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=FIELDS)
        w.writeheader()
        for i, (name, wgs, kib) in enumerate(rows):
            w.writerow({"Dispatch_Id": i, "Kernel_Name": name, "Grid_Size": wgs * 256, "Workgroup_Size": 256,
                        "Counter_Name": counter, "Counter_Value": kib})


def _run(calls, prep_kib, scan_kib, dec_kib, copy_kib, small_copy_kib):
    rows = [(COPY, 4096, small_copy_kib), (COPY, 4096, copy_kib)]
    for _ in range(calls):
        rows += [(PREP, wgs, prep_kib) for wgs in STAGE_WGS]
        rows += [(SCAN, 192, scan_kib) for _ in STAGE_WGS]
    rows += [(DECODE, 24576, dec_kib)] * 3
    return rows


@pytest.fixture
def traffic(tmp_path):
    fetch, write = str(tmp_path / "fetch"), str(tmp_path / "write")
    # FETCH_SIZE reports half the 1 GiB the copy reads; WRITE_SIZE all of it.
    # A smaller copy in the same run must not set the scale.
    _write_counters(fetch, "FETCH_SIZE", _run(2, 1000, 500, 800, 524288, 1000))
    _write_counters(write, "WRITE_SIZE", _run(2, 2000, 300, 700, 1048576, 2000))
    out = str(tmp_path / "traffic.json")
    rec = bench.write_traffic(fetch, write, path=out)
    return rec, out


def test_traffic_is_scaled_by_the_copy_and_summed_per_call(traffic):
    rec, _ = traffic
    c = rec["chunk_fwd"]
    assert c["fetch_scale"] == pytest.approx(2.0)
    assert c["write_scale"] == pytest.approx(1.0)
    # two calls of four stages each: per call, the four dispatches of each pass
    assert c["read_bytes"] == pytest.approx(4 * (1000 + 500) * 1024 * 2.0)
    assert c["write_bytes"] == pytest.approx(4 * (2000 + 300) * 1024 * 1.0)
    assert c["hbm_bytes_per_launch"] == pytest.approx(c["read_bytes"] + c["write_bytes"])
    d = rec["decode"]   # one dispatch per step
    assert d["read_bytes"] == pytest.approx(800 * 1024 * 2.0)
    assert d["write_bytes"] == pytest.approx(700 * 1024)


def test_traffic_is_used_only_for_the_sources_it_was_taken_on(traffic, tmp_path):
    rec, path = traffic
    assert bench.load_traffic("chunk_fwd", path) == pytest.approx(rec["chunk_fwd"]["hbm_bytes_per_launch"])
    assert rec["chunk_fwd"]["source_hash"] == bench.kernel_source_hash("chunk_fwd")
    with open(path) as f:
        stale = json.load(f)
    stale["chunk_fwd"]["source_hash"] = "0" * 16
    stale_path = str(tmp_path / "stale.json")
    with open(stale_path, "w") as f:
        json.dump(stale, f)
    assert bench.load_traffic("chunk_fwd", stale_path) is None
    assert bench.load_traffic("decode", stale_path) == pytest.approx(rec["decode"]["hbm_bytes_per_launch"])
    assert bench.load_traffic("chunk_fwd", str(tmp_path / "missing.json")) is None


def test_committed_traffic_matches_the_committed_sources():
    """profiles/traffic.json was taken on the kernels as they are: the bench
    line's roofline.traffic is filled, not null."""
    assert bench.load_traffic("chunk_fwd") is not None
    assert bench.load_traffic("decode") is not None


def test_mfma_summary(tmp_path, capsys):
    d = str(tmp_path / "pmc")
    os.makedirs(d)
    with open(os.path.join(d, "p_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=FIELDS)
        w.writeheader()
        for disp in range(2):
            for ctr, val in (("SQ_VALU_MFMA_BUSY_CYCLES", 1024.0e6), ("GRBM_GUI_ACTIVE", 8.0e6),
                             ("SQ_BUSY_CYCLES", 5.0)):
                w.writerow({"Dispatch_Id": disp, "Kernel_Name": SCAN, "Grid_Size": 192 * 256, "Workgroup_Size": 256,
                            "Counter_Name": ctr, "Counter_Value": val})
    bench.mfma_summary(d)
    out = json.loads(capsys.readouterr().out)
    (name, rec), = out.items()
    assert name == "kda::chunk_scan_kernel<unsigned short, false, false, true, true>"
    assert rec["dispatches"] == 2
    # 2 x 1.024e9 busy SIMD-cycles over 2 x 1e6 cycles per XCD x 1024 SIMDs
    assert rec["mfma_busy_frac"] == pytest.approx(1.0)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(bench.ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""
