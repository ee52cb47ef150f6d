"""The rocprofv3 CSV summarizer on small synthetic files in rocprofv3's column layout."""
import csv

import numpy as np

from weight_quantized_linear_qlinear_amd import profile_summary as ps

TRACE_COLS = ["Kind", "Agent_Id", "Queue_Id", "Stream_Id", "Thread_Id", "Dispatch_Id", "Kernel_Id", "Kernel_Name",
              "Correlation_Id", "Start_Timestamp", "End_Timestamp", "LDS_Block_Size", "Scratch_Size", "VGPR_Count",
              "Accum_VGPR_Count", "SGPR_Count", "Workgroup_Size_X", "Workgroup_Size_Y", "Workgroup_Size_Z",
              "Grid_Size_X", "Grid_Size_Y", "Grid_Size_Z"]
PMC_COLS = ["Correlation_Id", "Dispatch_Id", "Agent_Id", "Queue_Id", "Process_Id", "Thread_Id", "Grid_Size",
            "Kernel_Id", "Kernel_Name", "Workgroup_Size", "LDS_Block_Size", "Scratch_Size", "VGPR_Count",
            "Accum_VGPR_Count", "SGPR_Count", "Counter_Name", "Counter_Value", "Start_Timestamp", "End_Timestamp"]
K = "void qlq::(anonymous namespace)::gemm_mfma_kernel<0, 0, 256, 256, 128, 64, 1, 3, false>(qlq::GemmArgs, int)"


def _write(path, cols, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=cols)
        w.writeheader()
        for r in rows:
            w.writerow({c: r.get(c, 0) for c in cols})


def test_kernel_percentiles(tmp_path, capsys):
    durs = [10.0, 20.0, 30.0, 40.0, 50.0]
    rows = [{"Kernel_Name": K, "Start_Timestamp": 1000 * i, "End_Timestamp": 1000 * i + int(d * 1000),
             "Workgroup_Size_X": 512, "Grid_Size_X": 512 * 172} for i, d in enumerate(durs)]
    p = tmp_path / "t.csv"
    _write(p, TRACE_COLS, rows)
    ps.kernels(str(p), 10)
    line = [l for l in capsys.readouterr().out.splitlines() if l.startswith("gemm_mfma_kernel")][0]
    f = [x.strip() for x in line.split("|")]
    assert f[0] == "gemm_mfma_kernel<0, 0, 256, 256, 128, 64, 1, 3, false>" and f[1] == "172 x 512"
    assert int(f[2]) == 5 and float(f[3]) == 30.0
    assert float(f[4]) == np.percentile(durs, 10) and float(f[6]) == np.percentile(durs, 90)


def test_mfma_utilisation_and_traffic_calibration(tmp_path, capsys):
    agent = tmp_path / "agent.csv"
    _write(agent, ["Agent_Type", "Simd_Count", "Num_Xcc"], [{"Agent_Type": "GPU", "Simd_Count": 1024, "Num_Xcc": 8}])
    # 25 % busy: busy cycles = 0.25 * 1024 SIMDs * (GRBM / 8 XCDs)
    grbm = 8 * 100000
    pmc = [{"Dispatch_Id": 1, "Kernel_Name": K, "Grid_Size": 512 * 172, "Workgroup_Size": 512,
            "Counter_Name": n, "Counter_Value": v, "Start_Timestamp": 0, "End_Timestamp": 50000}
           for n, v in (("GRBM_GUI_ACTIVE", grbm), ("SQ_VALU_MFMA_BUSY_CYCLES", 0.25 * 1024 * 100000),
                        ("SQ_INSTS_VALU_MFMA_MOPS_BF16", 1e9 / 512))]
    p = tmp_path / "m.csv"
    _write(p, PMC_COLS, pmc)
    ps.mfma(str(p), str(agent), "gemm_mfma")
    line = [l for l in capsys.readouterr().out.splitlines() if l.startswith("gemm_mfma_kernel")][0]
    f = [x.strip() for x in line.split("|")]
    assert float(f[3]) == 25.0 and float(f[6]) == 1.0
    # copy of 256 MiB: FETCH_SIZE reads half its bytes, WRITE_SIZE all; a kernel reading 64 KiB-units
    copy = "__amd_rocclr_copyBuffer"
    fetch = [{"Dispatch_Id": 1, "Kernel_Name": K, "Grid_Size": 512, "Workgroup_Size": 512, "Counter_Name": "FETCH_SIZE",
              "Counter_Value": 1000.0},
             {"Dispatch_Id": 2, "Kernel_Name": copy, "Grid_Size": 64, "Workgroup_Size": 64, "Counter_Name": "FETCH_SIZE",
              "Counter_Value": 131072.0}]
    write = [{"Dispatch_Id": 1, "Kernel_Name": K, "Grid_Size": 512, "Workgroup_Size": 512, "Counter_Name": "WRITE_SIZE",
              "Counter_Value": 500.0},
             {"Dispatch_Id": 2, "Kernel_Name": copy, "Grid_Size": 64, "Workgroup_Size": 64, "Counter_Name": "WRITE_SIZE",
              "Counter_Value": 262144.0}]
    pf, pw = tmp_path / "f.csv", tmp_path / "w.csv"
    _write(pf, PMC_COLS, fetch)
    _write(pw, PMC_COLS, write)
    ps.traffic(str(pf), str(pw), "gemm_mfma")
    out = capsys.readouterr().out
    assert "factors 2.000 (fetch), 1.000 (write)" in out
    assert f"fabric_bytes_per_launch: {2 * 1000 * 1024 + 500 * 1024}" in out


def test_family_statistics(tmp_path, capsys):
    rows = [{"Kernel_Name": K, "Start_Timestamp": 0, "End_Timestamp": 1000 * d, "Workgroup_Size_X": 512,
             "Grid_Size_X": 512} for d in (10, 20, 30)]
    rows.append({"Kernel_Name": "other", "Start_Timestamp": 0, "End_Timestamp": 999000, "Workgroup_Size_X": 64,
                 "Grid_Size_X": 64})
    p = tmp_path / "t.csv"
    _write(p, TRACE_COLS, rows)
    ps.family(str(p), r"gemm_mfma_kernel<0, 0")
    assert "family_mean_us: 20.000" in capsys.readouterr().out


def test_counter_ratios_over_passes(tmp_path, capsys):
    """Ratios of counters collected in separate passes of the same program: latencies as
    level / requests, hit rate, and reads in flight per wave by Little's law."""
    def pas(name, counters):
        rows = [{"Dispatch_Id": 1, "Kernel_Name": K, "Grid_Size": 512 * 172, "Workgroup_Size": 512,
                 "Counter_Name": n, "Counter_Value": v, "Start_Timestamp": 0, "End_Timestamp": 10000}
                for n, v in counters]
        p = tmp_path / name
        _write(p, PMC_COLS, rows)
        return str(p)
    # 1376 waves, 137600 reads (100 per wave) of 480 cycles each over 10 us = 24000 cycles: 2.0 in flight
    a = pas("a.csv", (("VmemLatency", 480.0), ("SQ_INSTS_VMEM_RD", 137600.0), ("SQ_WAVES", 1376.0)))
    b = pas("b.csv", (("TCP_TCC_READ_REQ_LATENCY_sum", 3000.0), ("TCP_TCC_READ_REQ_sum", 10.0),
                      ("TCC_HIT_sum", 3.0), ("TCC_MISS_sum", 1.0), ("TCC_EA0_RDREQ_LEVEL_sum", 800.0),
                      ("TCC_EA0_RDREQ_sum", 2.0)))
    ps.counters([a, b], "gemm_mfma", brief=True)
    line = [l for l in capsys.readouterr().out.splitlines() if l.startswith("gemm_mfma_kernel")][0]
    f = [x.strip() for x in line.split("|")]
    assert f[1] == "172 x 512" and int(f[2]) == 2 and float(f[3]) == 10.0
    r = dict(x.rsplit(" ", 1) for x in f[4].split("; "))
    assert float(r["vmem latency (cycles)"]) == 480.0
    assert float(r["L1->L2 read latency (cycles)"]) == 300.0
    assert float(r["L2 hit %"]) == 75.0
    assert float(r["L2->fabric read latency (cycles)"]) == 400.0
    assert float(r["vmem reads in flight per wave"]) == 2.0
    assert "TCC_HIT_sum" not in f[5] and "SQ_WAVES 1376" in f[5]
