"""The rocprofv3 summariser on small hand-made CSV files (no GPU)."""
import os

from gated_linear_recurrence_history_amd import rocprof_summary as rs

HDR = ('"Correlation_Id","Dispatch_Id","Agent_Id","Queue_Id","Process_Id","Thread_Id",'
       '"Grid_Size","Kernel_Id","Kernel_Name","Workgroup_Size","LDS_Block_Size","Scratch_Size",'
       '"VGPR_Count","Accum_VGPR_Count","SGPR_Count","Counter_Name","Counter_Value",'
       '"Start_Timestamp","End_Timestamp"')


def _counters(path, counter, rows):
    os.makedirs(path, exist_ok=True)
    with open(os.path.join(path, "run_counter_collection.csv"), "w") as f:
        f.write(HDR + "\n")
        for disp, name, val in rows:
            f.write(f'{disp},{disp},"Agent 1",1,1,1,64,1,"{name}",256,0,0,8,0,16,'
                    f'"{counter}",{val},0,1\n')


def test_traffic_sums_rows_per_dispatch_and_scales(tmp_path):
    k = "void gscan::(anonymous namespace)::gscan_bwd_kernel<float, 8, true>(float const*)"
    copy = "__amd_rocclr_copyBuffer"
    # two rows per dispatch (per-XCD style): each dispatch sums them
    _counters(tmp_path / "f", "FETCH_SIZE", [(1, copy, 999.0), (2, k, 300.0), (2, k, 100.0),
                                            (3, k, 200.0), (3, k, 200.0), (4, copy, 512.0),
                                            (5, copy, 512.0)])
    _counters(tmp_path / "w", "WRITE_SIZE", [(1, copy, 5.0), (2, k, 50.0), (3, k, 50.0),
                                            (4, copy, 1024.0), (5, copy, 1024.0)])
    rec = rs.write_traffic(str(tmp_path / "f"), str(tmp_path / "w"), str(tmp_path / "t.txt"),
                           "gscan_bwd_kernel<float, 8, true>", "w", 1 << 20, 2, "cmd")
    assert rec["fetch_kib_per_dispatch"] == 400.0 and rec["write_kib_per_dispatch"] == 50.0
    assert rec["fetch_scale"] == 2.0 and rec["write_scale"] == 1.0
    assert rec["traffic_bytes"] == 400 * 1024 * 2 + 50 * 1024
    assert rs.read_traffic(str(tmp_path / "t.txt")) == rec
    assert rs.read_traffic(str(tmp_path / "missing.txt")) is None


def test_stats(tmp_path):
    d = tmp_path / "s"
    d.mkdir()
    (d / "run_kernel_stats.csv").write_text(
        '"Name","Calls","TotalDurationNs","AverageNs","Percentage","MinNs","MaxNs","StdDev"\n'
        '"void gscan::(anonymous namespace)::gscan_fwd_kernel<float, 8>(float const*)",2,'
        '40000,20000.0,100.0,19000,21000,10.0\n')
    rs.write_stats(str(d), str(tmp_path / "o.txt"), "cmd")
    text = (tmp_path / "o.txt").read_text()
    assert "gscan_fwd_kernel<float, 8>" in text and "20.000" in text and "command: cmd" in text


def test_counters_mean_per_dispatch(tmp_path):
    k = "void gscan::(anonymous namespace)::gscan_fwd_kernel<float, 8>(float const*)"
    other = "void gscan::(anonymous namespace)::gscan_reduce_kernel(float const*)"
    _counters(tmp_path / "a", "SQ_INSTS_MFMA", [(1, k, 10.0), (1, k, 30.0), (2, other, 7.0),
                                               (3, k, 60.0)])
    _counters(tmp_path / "b", "MfmaUtil", [(4, k, 12.5), (5, k, 13.5), (6, other, 1.0)])
    t = rs.write_counters([str(tmp_path / "a"), str(tmp_path / "b")], str(tmp_path / "c.txt"),
                          ["gscan_fwd_kernel<float, 8>"], "cmd")
    assert t == {"gscan_fwd_kernel<float, 8>": {"SQ_INSTS_MFMA": 50.0, "MfmaUtil": 13.0}}
    text = (tmp_path / "c.txt").read_text()
    assert "SQ_INSTS_MFMA" in text and "commands: cmd" in text
