"""bench.py's host-side logic, without a GPU: the source hash that ties the
stored counters to the decode code, the counter summary (calibration by the
reference copy, only the C2 step's decode dispatches), and the refusal of
more than one GPU."""
import csv
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_src_hash_tracks_code_not_comments(tmp_path):
    a, b, c = tmp_path / "a.hip", tmp_path / "b.hip", tmp_path / "c.hip"
    a.write_text("int x;  // first\n/* block\n comment */\nint y;\n")
    b.write_text("int x;    // other words\n\n\nint y;   \n")
    c.write_text("int x;\nint z;\n")
    assert bench.src_hash([a]) == bench.src_hash([b])
    assert bench.src_hash([a]) != bench.src_hash([c])


def _counter_csv(path, counter, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name",
                                          "Counter_Value"])
        w.writeheader()
        for i, (name, value) in enumerate(rows):
            w.writerow({"Dispatch_Id": i + 1, "Kernel_Name": name, "Counter_Name": counter,
                        "Counter_Value": value})


def test_summarize_counters_calibrates_and_keeps_c2_dispatches(tmp_path):
    fill = "vectorized_elementwise_kernel<8, at::native::FillFunctor<c10::BFloat16>>"
    copy = "__amd_rocclr_copyBuffer"
    split = "void kvsel::decode_split_kernel<kvsel::bf16_t, 128, 4>(...)"
    comb = "void kvsel::decode_combine_head_kernel<4, 128>(...)"
    gib_kib = (1 << 30) / 1024
    # the reference copy reads 1 GiB as half as many KiB (factor 2) and writes it as is
    fetch = [(fill, 1.0), (copy, gib_kib / 2), (split, 100.0), (comb, 10.0), (split, 300.0),
             (comb, 30.0), ("lmba_row_kernel<64>", 9e9), (split, 9e9), (comb, 9e9)]
    write = [(fill, 1.0), (copy, gib_kib), (split, 5.0), (comb, 1.0), (split, 7.0), (comb, 3.0),
             ("lmba_row_kernel<64>", 9e9), (split, 9e9)]
    fp, wp = tmp_path / "fetch.csv", tmp_path / "write.csv"
    _counter_csv(fp, "FETCH_SIZE", fetch)
    _counter_csv(wp, "WRITE_SIZE", write)
    res = bench.summarize_counters(str(fp), str(wp))
    assert res["FETCH_SIZE"]["scale_factor"] == pytest.approx(2.0)
    assert res["WRITE_SIZE"]["scale_factor"] == pytest.approx(1.0)
    assert res["FETCH_SIZE"]["kernels"]["decode_split_kernel"]["dispatches"] == 2
    # per launch: mean split + mean combine, KiB -> bytes, times the factor
    want = (200.0 + 20.0) * 1024 * 2.0 + (6.0 + 2.0) * 1024 * 1.0
    assert res["hbm_bytes_per_launch"] == int(want)
    assert res["source_sha256_16"] == bench.src_hash(bench.DECODE_SRCS)
    # the per-kernel table: the C2 step's split dispatches (mean of 100 and 300
    # KiB, doubled, in MB) and those after the first LMBA dispatch apart
    table = res["_table"].splitlines()
    c2 = [ln for ln in table if ln.startswith("| C2 step") and "decode_split" in ln]
    assert len(c2) == 1 and f"| 2 | {400.0 * 1024 / 1e6:.2f} | {6.0 * 1024 / 1e6:.2f} |" in c2[0]
    assert any(ln.startswith("| after") and "decode_split" in ln for ln in table)


def test_sq_table_per_kernel_shares(tmp_path):
    """One dispatch of 1000 cycles per XCD in 0.5 us (2 GHz) on 1024 SIMDs: 2
    resident waves per SIMD, matrix cores busy half the cycles, VALU issuing a
    quarter."""
    p = tmp_path / "sq.csv"
    with open(p, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Grid_Size",
                                          "Counter_Name", "Counter_Value",
                                          "Start_Timestamp", "End_Timestamp"])
        w.writeheader()
        name = "void kvsel::(anonymous namespace)::score_stats_reg_kernel<kvsel::bf16_t, 128, 4>(x)"
        vals = {"GRBM_GUI_ACTIVE": 8000.0, "SQ_WAVE_CYCLES": 2 * 1000 * 1024 / 4,
                "SQ_VALU_MFMA_BUSY_CYCLES": 0.5 * 1000 * 1024,
                "SQ_ACTIVE_INST_VALU": 0.25 * 1000 * 1024 / 4, "SQ_WAVES": 2048.0,
                "SQ_INSTS_VALU": 2048.0 * 300, "SQ_INSTS_MFMA": 2048.0 * 32}
        for k, v in vals.items():
            w.writerow({"Dispatch_Id": 7, "Kernel_Name": name, "Grid_Size": 131072,
                        "Counter_Name": k, "Counter_Value": v,
                        "Start_Timestamp": 1000, "End_Timestamp": 1500})
    row = bench.sq_table(str(p)).splitlines()[2]
    assert "score_stats_reg_kernel<kvsel::bf16_t, 128, 4>" in row
    assert "| 1 | 1000 | 0.5 | 2.00 | 2.00 | 0.50 | 0.25 | 0.00 | 300 | 32 |" in row


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_extras_start_includes_the_first_lmba_statistics_pass():
    """The extras open with LMBA, whose statistics pass uses the same kernels as
    the step's score: the cut steps back over that pass, and only that pass."""
    k = "void kvsel::(anonymous namespace)::"
    step = [k + "score_stats_reg_kernel<kvsel::bf16_t, 128, 4>(...)", k + "score_reduce_kernel(...)",
            k + "score_final_reg_kernel<kvsel::bf16_t, 128, 4>(...)", k + "select_topb_kernel<32>(...)",
            k + "compact_kernel<16>(...)", k + "decode_split_kernel<kvsel::bf16_t, 128, 4>(...)",
            k + "decode_combine_head_kernel<4, 128>(...)"]
    lmba = [k + "score_stats_reg_kernel<kvsel::bf16_t, 128, 4>(...)", k + "score_reduce_kernel(...)",
            k + "score_final_kernel<kvsel::bf16_t, 128, 4, true>(...)", k + "keep_mask_kernel(...)",
            k + "lmba_row_kernel<64>(...)"]
    assert bench._extras_start(step + lmba) == len(step)
    assert bench._extras_start(step) == len(step)
    # an LMBA call without its own statistics pass in front: nothing is taken back
    assert bench._extras_start(step + lmba[2:]) == len(step)
