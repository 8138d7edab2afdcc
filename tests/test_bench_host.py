"""Host-side logic of bench.py, on the CPU: the one-GPU guard, the gate that
keeps a counter-derived traffic figure only while the kernel sources match
the ones it was taken on, the scaling of FETCH_SIZE / WRITE_SIZE counters
by the plain-copy reference, and the launch-time spread."""
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

COPY = "__amd_rocclr_copyBuffer"
QUANT = "kvq::quantize_kernel<128, 32, true, 4, false, false>"


def test_bytes_per_vector():
    # fp16 vector + nibble codes + fp16 group scales
    assert bench.bytes_per_vector(128, 32) == 256 + 64 + 8
    assert bench.bytes_per_vector(256, 64) == 512 + 128 + 8
    assert bench.bytes_per_vector(64, 8) == 128 + 32 + 16


def test_launch_time_spread():
    # median of an odd and an even count, with the extremes
    assert bench.spread([3.0, 1.0, 2.0]) == {"median_ms": 2.0, "min_ms": 1.0, "max_ms": 3.0}
    assert bench.spread([4.0, 1.0, 3.0, 2.0]) == {"median_ms": 2.5, "min_ms": 1.0, "max_ms": 4.0}
    assert bench.spread([0.12345]) == {"median_ms": 0.1235, "min_ms": 0.1235, "max_ms": 0.1235}


@pytest.mark.parametrize("argv,env", [(["--gpus", "2"], {}), ([], {"WORLD_SIZE": "2"})])
def test_more_than_one_gpu_is_refused(argv, env):
    e = dict(os.environ, **env)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *argv], capture_output=True,
                       text=True, env=e, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_traffic_is_used_only_for_the_sources_it_was_taken_on(tmp_path, monkeypatch):
    path = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(path))
    assert bench.load_traffic(1) is None                       # no file
    path.write_text(json.dumps({"source_hash": "0" * 16, "traffic_bytes_per_launch": 123}))
    assert bench.load_traffic(1) is None                       # other sources
    path.write_text(json.dumps({"source_hash": bench.kernel_source_hash(), "traffic_bytes_per_launch": 123}))
    assert bench.load_traffic(1) == 123
    path.write_text("not json")
    assert bench.load_traffic(1) is None


def _counter_csv(path, counter, rows):
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        for i, (name, v) in enumerate(rows):
            w.writerow([i, name, counter, v])


def test_ingest_scales_by_the_copy_reference(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "traffic.json"))
    copy_bytes = 1 << 30
    kib = copy_bytes // 1024
    # the reference copy reads and writes copy_bytes; FETCH_SIZE reports half
    # of it (full-line reads), WRITE_SIZE all of it
    fetch = [(COPY + "(void*)", kib / 2), (COPY + "(void*)", 3.0),          # a small unrelated copy
             ("void " + QUANT + "(kvq::Int4Args)", 1000.0), ("void " + QUANT + "(kvq::Int4Args)", 1002.0)]
    write = [(COPY + "(void*)", kib), (COPY + "(void*)", 3.0),
             ("void " + QUANT + "(kvq::Int4Args)", 500.0), ("void " + QUANT + "(kvq::Int4Args)", 500.0)]
    fp, wp = tmp_path / "f.csv", tmp_path / "w.csv"
    _counter_csv(fp, "FETCH_SIZE", fetch)
    _counter_csv(wp, "WRITE_SIZE", write)
    out = bench.ingest_counters(str(fp), str(wp), copy_bytes)
    assert out["fetch_scale"] == pytest.approx(2.0)
    assert out["write_scale"] == pytest.approx(1.0)
    q = out["quantize"]
    assert q["dispatches"] == 2
    assert q["traffic_bytes_per_launch"] == int(1001.0 * 1024 * 2.0 + 500.0 * 1024 * 1.0)
    alg = 36 * 262144 * 8 * bench.bytes_per_vector(128, 32)
    assert q["algorithmic_bytes_per_launch"] == alg
    assert q["traffic_over_algorithmic"] == round(q["traffic_bytes_per_launch"] / alg, 5)
    assert out["traffic_bytes_per_launch"] == q["traffic_bytes_per_launch"]
    assert out["source_hash"] == bench.kernel_source_hash()
    with open(bench.TRAFFIC_FILE) as f:
        assert json.load(f) == out
    # without the reference copy there is nothing to scale by
    _counter_csv(wp, "WRITE_SIZE", write[2:])
    with pytest.raises(SystemExit):
        bench.ingest_counters(str(fp), str(wp), copy_bytes)


def test_ingest_mfma_derives_busy_fractions(tmp_path, monkeypatch):
    """MFMA and VALU busy fractions from summed counters: per-XCD cycles are
    GRBM_GUI_ACTIVE / 8, MFMA busy is over 1024 SIMDs, VALU busy over 256 CUs;
    the summary is used only for the sources it was taken on."""
    path = tmp_path / "mfma.json"
    monkeypatch.setattr(bench, "MFMA_FILE", str(path))
    enc = "void kvq::vq_encode_kernel<128, false>(kvq::VqArgs)"
    cyc = 1_000_000                      # per XCD
    counters = {"GRBM_GUI_ACTIVE": 8 * cyc, "SQ_VALU_MFMA_BUSY_CYCLES": 0.4 * cyc * 1024,
                "SQ_ACTIVE_INST_VALU": 0.65 * cyc * 256, "SQ_INSTS_VALU": 123.0, "SQ_INSTS_MFMA": 45.0,
                "SQ_INSTS_VALU_MFMA_MOPS_F16": 1000.0, "SQ_BUSY_CYCLES": 1.0}
    p = tmp_path / "pmc.csv"
    with open(p, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value", "Start_Timestamp",
                    "End_Timestamp"])
        for d in range(2):
            for k, v in counters.items():
                w.writerow([d, enc, k, v, 1000, 1000 + 500_000])            # 0.5 ms per dispatch
            w.writerow([d, "__amd_rocclr_copyBuffer", "GRBM_GUI_ACTIVE", 5, 0, 1])
    out = bench.ingest_mfma(str(p))
    k = out["kernels"]["kvq::vq_encode_kernel<128, false>"]
    assert k["dispatches"] == 2
    assert k["mfma_busy"] == pytest.approx(0.4) and k["valu_busy"] == pytest.approx(0.65)
    assert k["clock_GHz"] == pytest.approx(2.0)
    assert k["executed_fp16_mfma_flop"] == 512000.0
    assert list(out["kernels"]) == ["kvq::vq_encode_kernel<128, false>"]
    assert bench.load_mfma()["kernels"] == out["kernels"]
    path.write_text(json.dumps(dict(out, source_hash="0" * 16)))
    assert bench.load_mfma() is None
