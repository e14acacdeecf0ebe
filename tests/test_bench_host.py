"""Host-side logic of bench.py (no GPU): the PMC traffic bookkeeping behind
the JSON line's roofline.traffic."""
import json
import os
import sys
import types

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def _csv(path, rows):
    with open(path, "w") as f:
        f.write("Dispatch_Id,Kernel_Name,Counter_Name,Counter_Value\n")
        for i, (kernel, value) in enumerate(rows):
            f.write(f'{i},"{kernel}",X,{value}\n')
    return str(path)


def test_traffic_report_scales_counters_by_the_copy_kernel(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "traffic.json"))
    gu = "void moe::gemv_gate_up<2048, 768, 128, 4, 4, true>(void const*, ...)"
    fetch = _csv(tmp_path / "f.csv", [(gu, 1000.0), ("void moe::gemv_down<...>", 7.0), (gu, 3000.0)])
    write = _csv(tmp_path / "w.csv", [(gu, 8.0), (gu, 12.0)])
    mib = bench.COPY_MIB * 2 ** 20
    # the copy kernel moves mib bytes each way: 2 bytes per fetch KiB, 1 per write KiB
    copy_f = _csv(tmp_path / "cf.csv", [("MulFunctor<float>", mib / 2048)] * 3)
    copy_w = _csv(tmp_path / "cw.csv", [("FillFunctor<float>", 1.0), ("MulFunctor<float>", mib / 1024)])
    args = types.SimpleNamespace(traffic_report=[fetch, write, copy_f, copy_w], config="c1",
                                 tokens=None, path="gemv")
    bench.traffic_report(args)

    entry = json.load(open(tmp_path / "traffic.json"))["c1:T16:gemv"]
    # only the gate/up dispatches count, averaged
    assert entry["fetch_kib_per_dispatch"] == 2000.0
    assert entry["write_kib_per_dispatch"] == 10.0
    assert entry["dispatches"] == [2, 2]
    assert entry["copy_calibration"]["fetch_bytes_per_kib"] == 2.0
    assert entry["copy_calibration"]["write_bytes_per_kib"] == 1.0
    assert entry["traffic_bytes_per_launch"] == 2000 * 1024 * 2 + 10 * 1024
    assert bench.recorded_traffic("c1", 16, "gemv") == entry["traffic_bytes_per_launch"]
    # other workloads have no record; changed kernel sources void this one
    assert bench.recorded_traffic("c1", 4, "gemv") is None
    monkeypatch.setattr(bench, "sources_sha", lambda family: "0" * 64)
    assert bench.recorded_traffic("c1", 16, "gemv") is None


def test_traffic_report_picks_the_mfma_kernel_at_prefill_sizes(tmp_path, monkeypatch):
    """The grouped bf16 path's gate/up and down passes share one launch
    (mfma_layer); the two-launch passes (streamed banks) and the FP8
    variant's launch (mfma_layer_f8) are not it."""
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "traffic.json"))
    gu = "void moe::mfma_layer<2048, 768>(unsigned short const*, ...)"
    dn = "void moe::mfma_pass<false, 2048, 768>(unsigned short const*, ...)"
    f8 = "void moe::mfma_layer_f8<2048, 768>(unsigned char const*, ...)"
    fetch = _csv(tmp_path / "f.csv", [(gu, 100.0), (dn, 900.0), (f8, 5000.0)])
    write = _csv(tmp_path / "w.csv", [(gu, 1.0), (dn, 9.0), (f8, 50.0)])
    copy_f = _csv(tmp_path / "cf.csv", [("MulFunctor", bench.COPY_MIB * 1024.0)])
    copy_w = _csv(tmp_path / "cw.csv", [("MulFunctor", bench.COPY_MIB * 1024.0)])
    args = types.SimpleNamespace(traffic_report=[fetch, write, copy_f, copy_w], config="c2",
                                 tokens=None, path="auto")
    bench.traffic_report(args)
    entry = json.load(open(tmp_path / "traffic.json"))["c2:T512:mfma"]
    assert entry["kernel"] == "mfma_layer<"
    assert entry["traffic_bytes_per_launch"] == 100 * 1024 + 1 * 1024


def test_traffic_hash_ignores_comments_but_not_code(tmp_path, monkeypatch):
    src = tmp_path / "csrc"
    src.mkdir()
    (src / "k.hip").write_text("// header\n__global__ void k(int* p) { p[0] = 1; /* store */ }\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "KERNEL_SOURCES", {"gemv": ["k.hip"]})
    (tmp_path / "block_fp8_routed_amd").mkdir()
    (tmp_path / "block_fp8_routed_amd" / "csrc").symlink_to(src)
    h0 = bench.sources_sha("gemv")
    (src / "k.hip").write_text("// a longer header\n/* block\n comment */\n"
                               "__global__ void k(int* p) {\n  p[0] = 1;  // store\n}\n")
    assert bench.sources_sha("gemv") == h0
    (src / "k.hip").write_text("// header\n__global__ void k(int* p) { p[0] = 2; }\n")
    assert bench.sources_sha("gemv") != h0


def test_traffic_report_picks_the_single_launch_layer(tmp_path, monkeypatch):
    """The single-launch decode layer runs as one kernel (decode_fused): its
    dispatches are the ones counted."""
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "traffic.json"))
    k = "void moe::decode_fused<2048, 768, 128, 4, 4, true, false>(moe::FusedArgs)"
    fetch = _csv(tmp_path / "f.csv", [(k, 500.0), ("void moe::gemv_gate_up<...>", 9.0)])
    write = _csv(tmp_path / "w.csv", [(k, 4.0)])
    mib = bench.COPY_MIB * 2 ** 20
    copy_f = _csv(tmp_path / "cf.csv", [("MulFunctor<float>", mib / 1024)])
    copy_w = _csv(tmp_path / "cw.csv", [("MulFunctor<float>", mib / 1024)])
    args = types.SimpleNamespace(traffic_report=[fetch, write, copy_f, copy_w], config="c1",
                                 tokens=None, path="gemv_fused")
    bench.traffic_report(args)
    entry = json.load(open(tmp_path / "traffic.json"))["c1:T16:gemv_fused"]
    assert entry["kernel"] == "decode_fused<"
    assert entry["traffic_bytes_per_launch"] == 504 * 1024


def test_traffic_report_follows_the_library_family_choice(tmp_path, monkeypatch):
    """Path auto: the dominant kernel is the one of the family the library
    takes for the call (GEMV up to 48 bf16 tokens, the one-launch grouped
    kernel above), read from the workspace layout, not from a copy of the
    rule."""
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "traffic.json"))
    gemv = "void moe::gemv_gate_up<2048, 768, 128, 4, 4, true>(void const*, ...)"
    layer = "void moe::mfma_layer<2048, 768>(unsigned short const*, ...)"
    fetch = _csv(tmp_path / "f.csv", [(gemv, 300.0), (layer, 7000.0)])
    write = _csv(tmp_path / "w.csv", [(gemv, 3.0), (layer, 70.0)])
    mib = bench.COPY_MIB * 2 ** 20
    copy_f = _csv(tmp_path / "cf.csv", [("MulFunctor<float>", mib / 1024)])
    copy_w = _csv(tmp_path / "cw.csv", [("MulFunctor<float>", mib / 1024)])
    for T, key, kernel in ((48, "c2:T48:gemv", "gemv_gate_up<"), (49, "c2:T49:mfma", "mfma_layer<")):
        args = types.SimpleNamespace(traffic_report=[fetch, write, copy_f, copy_w], config="c2",
                                     tokens=T, path="auto")
        bench.traffic_report(args)
        entry = json.load(open(tmp_path / "traffic.json"))[key]
        assert entry["kernel"] == kernel
