"""Host logic of bench.py on the CPU: the counter summary, the HBM traffic record and its source
check, the algorithmic byte count, and the refusal of more than one GPU."""
import csv
import importlib.util
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


FIELDS = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]


def write_counters(d, rows):
    """rows: (dispatch id, kernel name, counter, value) as rocprofv3 writes them (csv)."""
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=FIELDS)
        w.writeheader()
        for i, k, c, v in rows:
            w.writerow({"Dispatch_Id": i, "Kernel_Name": k, "Counter_Name": c, "Counter_Value": v})


def test_summarize_counters(bench, tmp_path):
    # two dispatches of one kernel: GRBM_GUI_ACTIVE counts once per XCD (8 x the GPU cycles),
    # MFMA busy cycles sum over the 1024 SIMDs
    cyc = 1000.0
    rows = []
    for i in (1, 2):
        rows += [(i, "dk_kernel<128>", "GRBM_GUI_ACTIVE", 8 * cyc),
                 (i, "dk_kernel<128>", "SQ_VALU_MFMA_BUSY_CYCLES", 0.25 * cyc * 1024),
                 (i, "dk_kernel<128>", "SQ_VALU_MFMA_COEXEC_CYCLES", 0.05 * cyc * 1024),
                 (i, "dk_kernel<128>", "SQ_INSTS_MFMA", 24.0),
                 (i, "dk_kernel<128>", "SQ_WAVE_CYCLES", 400.0),
                 (i, "dk_kernel<128>", "SQ_ACTIVE_INST_ANY", 148.0),
                 (i, "dk_kernel<128>", "SQ_WAIT_INST_ANY", 120.0),
                 (i, "dk_kernel<128>", "SQ_WAIT_ANY", 132.0),
                 (i, "dk_kernel<128>", "SQ_ACTIVE_INST_VALU", 96.0),
                 (i, "dk_kernel<128>", "SQ_ACTIVE_INST_LDS", 12.0),
                 (i, "other_kernel", "SQ_INSTS_MFMA", 5.0)]
    write_counters(str(tmp_path / "a"), rows)
    out = bench.summarize_counters([str(tmp_path / "a")])
    lines = [ln for ln in out.splitlines() if ln.startswith("| dk_kernel")]
    assert len(lines) == 2 and "other_kernel" not in out
    cells = [c.strip() for c in lines[0].strip("|").split("|")]
    assert cells[1] == "1000" and cells[2] == "25.0 %" and cells[3] == "20.0 %" and cells[4] == "24"
    states = [c.strip() for c in lines[1].strip("|").split("|")]
    assert states[1:] == ["37.0 %", "30.0 %", "33.0 %", "24.0 %", "3.0 %"]


def test_traffic_record_and_source_check(bench, tmp_path, monkeypatch):
    kib = 1024.0
    fetch = [(1, "__amd_rocclr_copyBuffer", "FETCH_SIZE", (1 << 30) / 2 / kib)]
    write = [(1, "__amd_rocclr_copyBuffer", "WRITE_SIZE", (1 << 30) / kib)]
    for i in (2, 3):
        fetch.append((i, "_ZN12_GLOBAL__N_19dk_kernelILi128ELi1ELb1ELb0EEEvPKt", "FETCH_SIZE", 1000.0))
        write.append((i, "_ZN12_GLOBAL__N_19dk_kernelILi128ELi1ELb1ELb0EEEvPKt", "WRITE_SIZE", 500.0))
    fetch.append((4, "fwd_kernel", "FETCH_SIZE", 300.0))
    write_counters(str(tmp_path / "f"), fetch)
    write_counters(str(tmp_path / "w"), write)
    rec = tmp_path / "hbm_traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(rec))
    out = bench.write_traffic(str(tmp_path / "f"), str(tmp_path / "w"), "causal_64k_d128")
    # FETCH_SIZE read half of the copy's bytes: fetch counts scale by 2, write counts by 1
    assert out["copy_reference"]["fetch_scale"] == pytest.approx(2.0)
    assert out["copy_reference"]["write_scale"] == pytest.approx(1.0)
    dk = out["kernels"]["dk_kernel_s1"]
    assert dk["fetch_bytes"] == pytest.approx(2 * 1000 * kib)
    assert dk["write_bytes"] == pytest.approx(500 * kib)
    assert out["kernels"]["fwd_kernel"]["write_bytes"] == 0.0
    assert bench.traffic_for("dk_kernel_s1", "causal_64k_d128") == pytest.approx(2500 * kib)
    assert bench.traffic_for("dk_kernel_s1", "nc_4k_d128") is None
    # a record taken from another kernel source is not reported
    r = json.loads(rec.read_text())
    r["source_sha256"] = "0" * 64
    rec.write_text(json.dumps(r))
    assert bench.traffic_for("dk_kernel_s1", "causal_64k_d128") is None


def test_algorithmic_bytes_of_the_headline_step(bench):
    from workloads import WORKLOADS
    w = WORKLOADS["causal_64k_d128"]
    tensor = 32 * 65536 * 128 * 2  # one [1, 32, 64K, 128] bf16 tensor: 512 MiB
    row = 32 * 65536 * 4           # one fp32 value per query row: 8 MiB
    fwd = 4 * tensor + 3 * row     # Q1, K1, Q2, K2 in; KL, LSE1, LSE2 out
    bwd = 4 * tensor + 3 * row + 2 * tensor  # inputs, LSE1, LSE2, g in; dQ2, dK2 out
    assert bench.algorithmic_bytes(w) == fwd + bwd


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2 and "one GPU" in (r.stdout + r.stderr)
