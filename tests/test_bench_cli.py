"""bench.py's host logic (no GPU): the one-GPU contract, the code hash that keys the
profiles, and the summaries it writes from rocprofv3 output."""
import csv
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_code_only_drops_comments_and_keeps_literals():
    text = ('int a = 1; // note "x"\n/* block\n comment */ const char* s = "// kept";'
            " char c = '\"';  int  b;\n")
    assert bench._code_only(text) == "int a = 1; const char* s = \"// kept\"; char c = '\"'; int b;"
    # edits to comments and spacing do not change the code
    assert bench._code_only("x = y; // one\n") == bench._code_only("x  =  y;   /* two */\n")
    assert bench._code_only("x = y;") != bench._code_only("x = z;")


def test_traffic_is_ignored_when_taken_on_other_code(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    path = tmp_path / "traffic_w.txt"
    path.write_text("kernel_source_sha256: 0000\ntraffic_bytes_per_call: 123\n")
    assert bench.traffic_per_call("w") is None
    path.write_text(f"kernel_source_sha256: {bench.kernel_source_hash()}\ntraffic_bytes_per_call: 123\n")
    assert bench.traffic_per_call("w") == 123.0


def test_counter_summary_derived_figures(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path / "profiles"))
    run = tmp_path / "pmc" / "host"
    run.mkdir(parents=True)
    kname = "void pa::(anonymous namespace)::pa_decode_balanced<128, 4, 1, 12, false, true>(pa::DecodeArgs)"
    values = {"SQ_LDS_BANK_CONFLICT": [10, 30], "SQ_LDS_IDX_ACTIVE": [110, 130],
              "SQ_WAVES": [3072, 3072], "SQ_INSTS_VALU": [3072 * 100, 3072 * 100],
              "TCC_EA0_RDREQ_sum": [1000, 1000], "TCC_EA0_RDREQ_128B_sum": [990, 990],
              "TCC_EA0_RDREQ_LEVEL_sum": [2_000_000, 2_000_000]}
    with open(run / "run_counter_collection.csv", "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for c, vs in values.items():
            for i, v in enumerate(vs):
                w.writerow({"Dispatch_Id": i, "Kernel_Name": kname, "Counter_Name": c, "Counter_Value": v})
    out = bench.summarize_counters([str(tmp_path / "pmc")], "w")
    text = open(out).read()
    assert f"kernel_source_sha256: {bench.kernel_source_hash()}" in text
    assert "pa_decode_balanced<128, 4, 1, 12, false, true>:" in text
    # conflict cycles over conflict-free active cycles: 40 / (240 - 40)
    assert "lds_bank_conflict_rate: 0.2000" in text
    assert "hbm_read_requests_128B_fraction: 0.9900" in text
    assert "mean_read_request_latency_l2_cycles: 2000" in text
    assert "sq_insts_valu_per_wave: 100" in text
    assert "waves_per_dispatch: 3072" in text


def test_counter_summary_without_values_fails(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path / "profiles"))
    (tmp_path / "empty").mkdir()
    with pytest.raises(SystemExit):
        bench.summarize_counters([str(tmp_path / "empty")], "w")


def test_resources_keyed_by_kernel_hash(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    rows = ("kernel  sgpr vgpr agpr scratch waves/simd sgpr_spill vgpr_spill lds\n"
            "pa_decode_balanced<128,4,1,12,0,1> 106 149 0 0 3 25 0 105664\n")
    (tmp_path / "resources.txt").write_text("kernel_source_sha256: 0000\n" + rows)
    assert bench.kernel_resources(["pa_decode_balanced<128,4,1,12,0,1>"]) is None
    (tmp_path / "resources.txt").write_text(f"kernel_source_sha256: {bench.kernel_source_hash()}\n" + rows)
    got = bench.kernel_resources(["pa_decode_balanced<128,4,1,12,0,1>", "absent<1>"])
    assert got == {"pa_decode_balanced<128,4,1,12,0,1>": dict(sgpr=106, vgpr=149, agpr=0, scratch=0,
                                                                **{"waves/simd": 3}, sgpr_spill=25,
                                                                vgpr_spill=0, lds=105664)}


def test_committed_resources_cover_the_benched_kernels():
    """profiles/resources.txt exists, and when it matches the current sources it lists
    the kernels the bench reports for each workload."""
    from decode_attention_paged_03_amd import workloads as W
    path = os.path.join(ROOT, "profiles", "resources.txt")
    assert os.path.exists(path)
    text = open(path).read()
    if f"kernel_source_sha256: {bench.kernel_source_hash()}" not in text:
        pytest.skip("resources.txt predates the current kernel sources")
    for name, spec in W.WORKLOADS.items():
        class _Wl:
            group = spec["query_heads"] // spec["kv_heads"]
            page_size = spec["page_size"]
            head_dim = spec["head_dim"]
            batch = spec["batch"]
            kv_heads = spec["kv_heads"]
        # the even split, and short contexts (one partition per sequence, 8 or 4 waves)
        for short, cus in ((False, 256), (True, 256), (True, 1)):
            names = bench.decode_kernel_names(_Wl, short, cus)
            got = bench.kernel_resources(names)
            assert got is not None and len(got) == len(names), (name, short, cus)


def test_cpu_baseline_fields():
    """Single-thread and all-thread oracle runs, the thread counts used and the host's
    core count reported separately."""
    from decode_attention_paged_03_amd import workloads as W
    wl = W.make_named("tiny")
    line = bench.cpu_baseline(wl, 0.05, reps=2)
    assert line["kind"] == "oracle" and line["unit"] == "GB/s" and line["value"] > 0
    assert line["single"]["threads"] == 1
    assert line["all"]["threads"] == line["cores"] == min(bench.host_cores(), bench.CPU_SHARE)
    assert line["host_cores"] == bench.host_cores()
    assert line["single"]["evaluations"] == 2
    assert "output rows" in line["sample"]
