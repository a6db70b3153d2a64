"""Host-side checks of bench.py's profile summaries (no GPU): the rocprofv3
counter-run summary that gives the roofline's `traffic`, and the per-pass
kernel-trace summary, on small synthetic CSV files in rocprofv3's layout."""
import csv
import os

import bench
from flare_inputs import WORKLOADS

COUNTER_COLS = ["Correlation_Id", "Dispatch_Id", "Agent_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]


def write_counters(path, counter, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=COUNTER_COLS)
        w.writeheader()
        for i, (name, value) in enumerate(rows):
            # one dispatch may report its counter in several rows (summed)
            for part in (0.25, 0.75):
                w.writerow({"Correlation_Id": i, "Dispatch_Id": i, "Agent_Id": 1, "Kernel_Name": name,
                            "Counter_Name": counter, "Counter_Value": value * part})


def test_pmc_summary_scales_by_the_copy_kernel(tmp_path):
    w = WORKLOADS[2]
    alg = 2 * w.B * w.H * w.N * w.D * 2
    copy_mib = 512
    enc = "void flare::(anonymous namespace)::encode_partial_bf16<32, 2, 2, 2>(flare::EncodeArgs)"
    dec = "void flare::(anonymous namespace)::decode_bf16<32, 1, float, false>(flare::DecodeArgs)"
    cpy = "flare::(anonymous namespace)::copy_kernel(unsigned int const*, unsigned int*, unsigned long)"
    # FETCH_SIZE reads half the copy's bytes (scale 2), WRITE_SIZE all of them
    fetch_rows = [(cpy, (copy_mib << 20) / 2 / 1024), (enc, alg / 2 / 1024), (dec, alg / 4 / 1024),
                  (enc, alg / 2 / 1024 * 1.02), (dec, alg / 4 / 1024)]
    write_rows = [(cpy, (copy_mib << 20) / 1024), (enc, 1000.0), (dec, alg / 2 / 1024), (enc, 1000.0),
                  (dec, alg / 2 / 1024)]
    fp, wp = str(tmp_path / "f.csv"), str(tmp_path / "w.csv")
    write_counters(fp, "FETCH_SIZE", fetch_rows)
    write_counters(wp, "WRITE_SIZE", write_rows)
    recs = {r["kernel"]: r for r in bench.pmc_summary(fp, wp, w, "bhnd", "flare", copy_mib, None)}
    assert set(recs) == {"encode_partial", "decode"}
    e, d = recs["encode_partial"], recs["decode"]
    assert e["calibration"]["fetch_scale"] == 2.0 and e["calibration"]["write_scale"] == 1.0
    assert abs(e["hbm_read_bytes_per_launch"] - alg * 1.01) <= 2
    assert e["hbm_write_bytes_per_launch"] == 1024000
    assert abs(d["hbm_bytes_per_launch"] - alg) <= 2 and d["alg_bytes_per_launch"] == alg
    assert e["launches"] == 2 and e["kernel_symbol"] == "encode_partial_bf16<32, 2, 2, 2>"
    assert e["source_hash"] == bench.source_hash("encode_partial")
    assert e["workload"] == "pde-mesh-65k"


def test_trace_summary_splits_passes(tmp_path):
    # 3 kernels x (2 warmup + 3 timed + 3 kernel-pass) steps; durations 1, 2, 3 us by pass
    path = tmp_path / "kt.csv"
    t = 0
    with open(path, "w", newline="") as f:
        wr = csv.DictWriter(f, fieldnames=["Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        wr.writeheader()
        for step in range(8):
            us = 1 if step < 2 else (2 if step < 5 else 3)
            for name in ("void a()", "void b()", "void c()"):
                wr.writerow({"Kernel_Name": name, "Start_Timestamp": t, "End_Timestamp": t + us * 1000})
                t += 10000
    out = bench.trace_summary(str(path), 3, False)
    rows = [r for r in out.splitlines() if r.startswith("| a ")]
    assert rows == ["| a | 8 | 2.12 | 2.00 | 3.00 |"]  # all: 17 us / 8


def test_fp32_kernels_hash_their_own_source():
    # the fp32 encode and decode are defined with the combine, not with the
    # bf16 kernels: counters taken on one must not validate the other
    assert bench.kernel_sources("encode_partial", "f32") == bench.kernel_sources("combine")
    assert bench.source_hash("decode", "f32") != bench.source_hash("decode", "bf16")
    assert bench.source_hash("encode_partial", "f32") == bench.source_hash("combine")


def test_sq_summary_per_block_counts_clock_and_busy(tmp_path):
    # one decode dispatch per pass, 50 us long; 2.0 GHz means GRBM_GUI_ACTIVE
    # = 8 XCDs x 2.0e9 x 50e-6; MFMA busy 30% of the SIMD cycles
    w = WORKLOADS[2]
    blocks = w.B * w.H * w.N * w.M / 1024
    dec = "void flare::(anonymous namespace)::decode_bf16<32, 1, float, false>(flare::DecodeArgs)"
    gui = 8 * 2.0e9 * 50e-6
    counts = {"SQ_INSTS_MFMA": 6 * blocks, "SQ_INSTS_VALU": 61 * blocks, "SQ_INSTS_VALU_TRANS_F32": 16 * blocks,
              "SQ_INSTS_VALU_FMA_F32": 16 * blocks, "SQ_INSTS_VALU_CVT": 10 * blocks, "SQ_INSTS_LDS": 4.5 * blocks,
              "SQ_LDS_BANK_CONFLICT": 1.5 * blocks, "SQ_WAIT_INST_ANY": 45.0, "SQ_WAVE_CYCLES": 100.0,
              "SQ_VALU_MFMA_BUSY_CYCLES": 0.3 * 1024 * gui / 8, "GRBM_GUI_ACTIVE": gui}
    paths = []
    for i, names in enumerate(s.split() for s in bench.SQ_SETS):
        path = str(tmp_path / f"p{i + 1}.csv")
        with open(path, "w", newline="") as f:
            wr = csv.DictWriter(f, fieldnames=COUNTER_COLS + ["Start_Timestamp", "End_Timestamp"])
            wr.writeheader()
            for cn in names:
                wr.writerow({"Correlation_Id": 0, "Dispatch_Id": 0, "Agent_Id": 1, "Kernel_Name": dec,
                             "Counter_Name": cn, "Counter_Value": counts.get(cn, 1.0),
                             "Start_Timestamp": 1000, "End_Timestamp": 51000})
        paths.append(path)
    table = bench.sq_summary(paths, w).splitlines()
    assert len(table) == 3
    cells = [c.strip() for c in table[2].strip("|").split("|")]
    assert cells == ["decode_bf16<32, 1, float, false>", "50.0", "2.00", "30%", "6.00", "61.0", "16.0, 16.0, 10.0",
                     "4.50", "1.50", "0.45"]
