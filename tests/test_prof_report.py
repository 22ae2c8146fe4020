"""Host logic of the rocprofv3 summary tool: counter scaling against the
calibration copy, per-step call counts, and the summary-file parser."""

import csv

from block_diffusion_draft_tap_amd import prof_report

FIELDS = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]


def _counter_csv(path, counter, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=FIELDS)
        w.writeheader()
        for i, (name, val) in enumerate(rows, start=1):
            w.writerow({"Dispatch_Id": i, "Kernel_Name": name, "Counter_Name": counter, "Counter_Value": val})


def test_traffic_scaling(tmp_path):
    copy = 1 << 20  # calibration kernel reads and writes 1 MiB
    fetch = tmp_path / "f.csv"
    write = tmp_path / "w.csv"
    mul = "void at::native::vectorized_elementwise_kernel<4, at::native::AUnaryFunctor<float, float, float, MulFunctor>"
    # the calibration copy is the last PyTorch multiply; the measured kernel's launches before it
    # (a warm-up) and the fills after it do not count
    _counter_csv(fetch, "FETCH_SIZE", [("void dfl::head", 50.0), ("void at::native::fill", 0.0), (mul, 512.0),
                                       ("void at::native::fill", 3.0), ("void dfl::head", 100.0),
                                       ("void dfl::head", 102.0)])
    _counter_csv(write, "WRITE_SIZE", [("void dfl::head", 9.0), ("void at::native::fill", 1024.0), (mul, 1024.0),
                                       ("void at::native::fill", 1.0), ("void dfl::head", 1.0),
                                       ("void dfl::head", 1.0)])
    v = prof_report.traffic_summary(str(fetch), str(write), "dfl::head", copy, 200 * 1024)
    # fetch counter reads half the true bytes -> scale 2; write exact -> scale 1
    assert v["fetch scale"] == "2.00000" and v["write scale"] == "1.00000"
    assert int(v["bytes per launch"]) == (101.0 * 2 + 1.0) * 1024
    assert v["launches"] == "2 (fetch pass), 2 (write pass)"
    assert v["kernel sources sha256[:16]"] == prof_report.kernel_sources_hash()


def test_kernel_sources_per_kernel():
    """A kernel's hash covers its own .hip file and the shared sources (headers, host launch
    code), not the files of other kernels; an unknown name covers every source."""
    every = prof_report.kernel_sources()
    attn = prof_report.kernel_sources("void dfl::attn_mfma_kernel<128, 3>(dfl::AttnParams)")
    assert "csrc/attention.hip" in attn and "csrc/dflash_api.cpp" in attn and "csrc/common.hpp" in attn
    assert "csrc/i4mm.hip" not in attn and "csrc/skinny.hip" not in attn and "csrc/gemv.hip" not in attn
    assert all(h in attn for h in every if h.endswith(".hpp"))
    sk = prof_report.kernel_sources("void dfl::(anonymous namespace)::skinny_kernel<1, 3>(dfl::SkinnyParams)")
    assert "csrc/skinny.hip" in sk and "csrc/attention.hip" not in sk
    assert prof_report.kernel_sources("not a kernel") == every
    assert prof_report.kernel_sources_hash("not a kernel") == prof_report.kernel_sources_hash()
    assert prof_report.kernel_sources_hash("attn_mfma_kernel<128, 3>") != prof_report.kernel_sources_hash()


def test_summary_parser_keeps_colons_in_keys(tmp_path):
    p = tmp_path / "s.md"
    p.write_text("# t\n\n- kernel sources sha256[:16]: abc\n- bytes per launch: 12\nnot a field: x\n")
    assert prof_report.read_summary(str(p)) == {"kernel sources sha256[:16]": "abc", "bytes per launch": "12"}


def test_stats_per_step(tmp_path):
    p = tmp_path / "k.csv"
    with open(p, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage", "MinNs", "MaxNs", "StdDev"])
        w.writerow(["head", 4, 400, 100, 0, 90, 110, 0])
        w.writerow(["layer", 20, 600, 30, 0, 20, 40, 0])
    t = prof_report.stats_table(str(p), per_kernel="head")
    assert "| `layer` | 20 | 5.00 |" in t and "| `head` | 4 | 1.00 |" in t and "60.0%" in t


def test_counter_summary_averages_and_conflict_share(tmp_path):
    p1 = tmp_path / "a.csv"
    p2 = tmp_path / "b.csv"
    with open(p1, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=FIELDS)
        w.writeheader()
        for i, (name, c, v) in enumerate([("void other", "SQ_LDS_IDX_ACTIVE", 5.0),
                                          ("void dfl::gemm_kernel<0, 0>", "SQ_LDS_IDX_ACTIVE", 100.0),
                                          ("void dfl::gemm_kernel<0, 0>", "SQ_LDS_BANK_CONFLICT", 30.0)], start=1):
            w.writerow({"Dispatch_Id": 7 if i > 1 else 1, "Kernel_Name": name, "Counter_Name": c, "Counter_Value": v})
    _counter_csv(p2, "SQ_VALU_MFMA_BUSY_CYCLES", [("void dfl::gemm_kernel<0, 0>", 40.0), ("void dfl::gemm_kernel<0, 0>", 60.0)])
    v = prof_report.counter_summary([str(p1), str(p2)], "gemm_kernel<0, 0>")
    assert v["SQ_LDS_IDX_ACTIVE per dispatch"] == "100"
    assert v["SQ_VALU_MFMA_BUSY_CYCLES per dispatch"] == "50"
    assert v["bank-conflict cycles / LDS-active cycles"] == "0.3000"
    assert v["dispatches per pass"] == "2"
