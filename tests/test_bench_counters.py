"""bench.py --import-counters on synthetic rocprofv3 counter files (no GPU):
each counter is scaled by what it reads for the runtime's 1 GiB device copy,
even when a torch copy kernel of the input generation reads more, and the
W1 and W2 GEMM launches are told apart by their template arguments."""
import csv
import json
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

FIELDS = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]
W1 = ("void moe::(anonymous namespace)::gemm_stream_kernel<2, 1, 4, 1, 128, true>(unsigned short const*, int const*, "
      "int const*, int, unsigned char const*, unsigned short const*, long, void*, int, int, int, int, int, int)")
W2 = W1.replace("<2, 1, 4,", "<2, 2, 4,")
TORCH_COPY = "void at::native::elementwise_kernel_manual_unroll<128, 4, at::native::bfloat16_copy_kernel_cuda>(int, F)"
RUNTIME_COPY = "__amd_rocclr_copyBuffer"


def write_csv(path, counter, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=FIELDS)
        w.writeheader()
        for i, (name, value) in enumerate(rows):
            w.writerow({"Dispatch_Id": i + 1, "Kernel_Name": name, "Counter_Name": counter, "Counter_Value": value})


def test_import_scales_by_the_runtime_copy(tmp_path, monkeypatch):
    # the 1 GiB copy reads as half its bytes for FETCH_SIZE and exactly for WRITE_SIZE; a torch copy kernel of
    # the input generation reads more than the calibration copy and must not be taken for it
    fetch = tmp_path / "fetch.csv"
    write = tmp_path / "write.csv"
    write_csv(fetch, "FETCH_SIZE", [(RUNTIME_COPY, 524288.0), (TORCH_COPY, 600000.0), (RUNTIME_COPY, 1000.0),
                                    (W1, 100000.0), (W2, 200000.0), (W1, 100002.0), (W2, 199998.0), (W1, 99998.0)])
    write_csv(write, "WRITE_SIZE", [(RUNTIME_COPY, 1048576.0), (TORCH_COPY, 2000000.0), (W1, 64.0), (W2, 128.0),
                                    (W1, 64.0), (W2, 128.0), (W1, 64.0)])
    traffic = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC", str(traffic))
    args = bench.parse(["--import-counters", str(fetch), str(write), "--workload", "int4-decode-T16-d12288-E16"])
    bench.import_counters(args)
    table = json.loads(traffic.read_text())
    w1 = table["moe_grouped_gemm_w1_streaming|int4-decode-T16-d12288-E16"]
    w2 = table["moe_grouped_gemm_w2_streaming|int4-decode-T16-d12288-E16"]
    assert w1["fetch_scale"] == pytest.approx(2.0) and w1["write_scale"] == pytest.approx(1.0)
    assert w1["fetch_bytes"] == int(100000.0 * 1024 * 2.0)   # median of the three W1 dispatches
    assert w1["write_bytes"] == 64 * 1024
    assert w2["fetch_bytes"] == int(199999.0 * 1024 * 2.0)   # median of the two W2 dispatches
    assert w2["bytes_per_launch"] == w2["fetch_bytes"] + w2["write_bytes"]
    assert w1["source_hash"] == bench.kernel_source_hash("moe_grouped_gemm_w1_streaming")


def test_import_needs_the_calibration_copy(tmp_path, monkeypatch):
    fetch = tmp_path / "fetch.csv"
    write = tmp_path / "write.csv"
    write_csv(fetch, "FETCH_SIZE", [(TORCH_COPY, 600000.0), (W1, 100000.0)])
    write_csv(write, "WRITE_SIZE", [(TORCH_COPY, 2000000.0), (W1, 64.0)])
    monkeypatch.setattr(bench, "TRAFFIC", str(tmp_path / "traffic.json"))
    args = bench.parse(["--import-counters", str(fetch), str(write), "--workload", "int4-decode-T16-d12288-E16"])
    with pytest.raises(SystemExit):
        bench.import_counters(args)


def test_source_hash_follows_code_not_comments(tmp_path):
    # counters stay valid across comment edits and are invalidated by code edits
    import shutil
    csrc = os.path.join(ROOT, "sparse_mixture_experts_03_amd", "csrc")
    for f in ("common.hpp", "launch.hpp", "moe_api.hip", "gemm_tiled.hip"):
        shutil.copy(os.path.join(csrc, f), tmp_path / f)
    base = bench.kernel_source_hash("moe_grouped_gemm_w1_tiled", csrc=str(tmp_path))
    assert base == bench.kernel_source_hash("moe_grouped_gemm_w1_tiled")
    src = (tmp_path / "gemm_tiled.hip").read_text()
    (tmp_path / "gemm_tiled.hip").write_text("// a new comment line\n" + src.replace("\n", "\n\n", 3) + "/* trailing */\n")
    assert bench.kernel_source_hash("moe_grouped_gemm_w1_tiled", csrc=str(tmp_path)) == base
    (tmp_path / "gemm_tiled.hip").write_text(src.replace("constexpr int kPpW = 3", "constexpr int kPpW = 2", 1))
    assert bench.kernel_source_hash("moe_grouped_gemm_w1_tiled", csrc=str(tmp_path)) != base
    assert bench.source_code_only('a = "// kept"; // dropped\n/* dropped */ b;') == 'a = "// kept"; b;'
