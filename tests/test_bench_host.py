"""Host logic of bench.py (CPU only): the one-GPU refusal, the staleness
guard on recorded HBM traffic, and the rocprofv3 summary writers on small
synthetic CSV files."""

import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout.strip() == ""          # no JSON line for a refused run


def test_traffic_is_reported_only_for_matching_sources(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    name = "gpt2s_causal_bf16_b8h12n1024d64"
    assert bench.traffic_for(name) is None                     # nothing recorded
    rec = {"kernel_source_sha": bench.kernel_source_hash(), "hbm_bytes_per_launch": 123.0}
    (tmp_path / f"traffic_{name}.json").write_text(json.dumps(rec))
    assert bench.traffic_for(name) == 123.0
    rec["kernel_source_sha"] = "0" * 16                         # recorded for other kernel sources
    (tmp_path / f"traffic_{name}.json").write_text(json.dumps(rec))
    assert bench.traffic_for(name) is None


def test_kernel_source_hash_covers_the_forward_sources():
    """The recorded traffic belongs to the forward kernel: every local file
    the forward entry points are compiled from must be part of the hash."""
    import re
    dirs = [os.path.join(ROOT, "exact_io_aware_48_amd", "csrc"), os.path.join(ROOT, "include")]
    seen, todo = set(), [os.path.join(dirs[0], "fa_api.hip")]
    while todo:
        path = todo.pop()
        rel = os.path.relpath(path, ROOT)
        if rel in seen:
            continue
        seen.add(rel)
        for inc in re.findall(r'^#include "([^"]+)"', open(path).read(), re.M):
            todo += [os.path.join(d, inc) for d in dirs if os.path.exists(os.path.join(d, inc))]
    assert len(seen) >= 5
    assert seen <= set(bench.KERNEL_SOURCES), sorted(seen - set(bench.KERNEL_SOURCES))


def test_summarize_trace_writes_the_kernel_table(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path / "profiles"))
    d = tmp_path / "trace" / "host" / "123"
    d.mkdir(parents=True)
    (d / "kt_kernel_stats.csv").write_text(
        "Name,Calls,TotalDurationNs,AverageNs,Percentage,MinNs,MaxNs\n"
        "\"void fa::fa_fwd_kernel<64, 64, 4, 0, true, false, 0, false>(fa::Params)\",10,230000,23000,100.0,20000,31000\n")
    bench.summarize_trace(str(tmp_path / "trace"), "gpt2s_causal_bf16_b8h12n1024d64", "cmd")
    text = (tmp_path / "profiles" / "kernel_trace_gpt2s_causal_bf16_b8h12n1024d64.txt").read_text()
    row = next(ln for ln in text.splitlines() if ln.startswith("fa::fa_fwd_kernel"))
    calls, avg, lo, hi, share = row.split()[-5:]
    assert (int(calls), float(avg), float(lo), float(hi), float(share)) == (10, 23.0, 20.0, 31.0, 100.0)
    assert f"kernel sources sha: {bench.kernel_source_hash()}" in text


def test_backward_trace_summary_hashes_the_backward_sources(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path / "profiles"))
    d = tmp_path / "trace"
    d.mkdir()
    (d / "kt_kernel_stats.csv").write_text(
        "Name,Calls,TotalDurationNs,AverageNs,Percentage,MinNs,MaxNs\n"
        "\"void fa::fa_bwd_dq_kernel<64, 64, 4, 2, true>(fa::BwdParams)\",10,300000,30000,100.0,29000,36000\n")
    bench.summarize_trace(str(d), "gpt2s_causal_bf16_b8h12n1024d64", "cmd", "kernel_trace_backward")
    text = (tmp_path / "profiles" / "kernel_trace_backward_gpt2s_causal_bf16_b8h12n1024d64.txt").read_text()
    sha = bench.kernel_source_hash(bench.BWD_KERNEL_SOURCES)
    assert f"backward kernel sources sha: {sha}" in text and sha != bench.kernel_source_hash()
    assert all(os.path.exists(os.path.join(bench.ROOT, rel)) for rel in bench.BWD_KERNEL_SOURCES)


def test_summarize_pmc_scales_by_the_copy_calibration(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path / "profiles"))
    name = "gpt2s_causal_bf16_b8h12n1024d64"
    hdr = "Kernel_Name,Counter_Name,Counter_Value\n"
    fetch, write = tmp_path / "f", tmp_path / "w"
    fetch.mkdir()
    write.mkdir()
    # the copy of 256 MiB reads as 128 MiB in FETCH_SIZE (factor 2) and as 256 MiB in WRITE_SIZE
    (fetch / "a_counter_collection.csv").write_text(
        hdr + f"fa::fa_fwd_kernel<...>,FETCH_SIZE,1000\nfa::fa_fwd_kernel<...>,FETCH_SIZE,3000\n"
              f"__amd_rocclr_copyBuffer,FETCH_SIZE,{128 * 1024}\n")
    (write / "a_counter_collection.csv").write_text(
        hdr + f"fa::fa_fwd_kernel<...>,WRITE_SIZE,500\n__amd_rocclr_copyBuffer,WRITE_SIZE,{256 * 1024}\n")
    bench.summarize_pmc(str(fetch), str(write), name, "cmd")
    rec = json.loads((tmp_path / "profiles" / f"traffic_{name}.json").read_text())
    assert rec["copy_scale_fetch"] == pytest.approx(2.0)
    assert rec["copy_scale_write"] == pytest.approx(1.0)
    assert rec["hbm_bytes_per_launch"] == pytest.approx((2000 * 2.0 + 500 * 1.0) * 1024)
    assert rec["kernel_source_sha"] == bench.kernel_source_hash()


def test_roofline_block_bound_follows_the_lower_ceiling():
    from workloads import by_name
    # GPT-2-small shape: AI 254 FLOP/B, HBM ceiling 2032 < 2516.6 TFLOP/s -> HBM-bound, in GB/s
    w = by_name("gpt2s_causal_bf16_b8h12n1024d64")
    t = {"kernel_ms_mean": 0.025}
    blk = bench.roofline_block(w, t)
    assert blk["bound"] == "hbm" and blk["unit"] == "GB/s" and blk["peak"] == bench.HBM_GBPS
    gbs = w.compulsory_bytes / 25e-6 / 1e9
    assert abs(blk["achieved"] - gbs) < 0.1 and abs(blk["frac"] - gbs / 8000.0) < 1e-4
    # the same fraction as TFLOP/s over the HBM ceiling
    assert abs(blk["frac"] - blk["tflops"] / blk["ceilings_tflops"]["hbm"]) < 2e-3
    # long causal d = 128: AI 2040 -> MFMA-bound against the bf16 peak
    w = by_name("long_causal_bf16_b1h32n8192d128")
    blk = bench.roofline_block(w, {"kernel_ms_mean": 0.5})
    assert blk["bound"] == "mfma" and blk["unit"] == "TFLOP/s" and blk["peak"] == 2516.6
    assert abs(blk["achieved"] - w.flops / 0.5e-3 / 1e12) < 0.01
    # fp8 takes the fp8 peak
    blk = bench.roofline_block(by_name("wide_fp8_b2h8n16384d256"), {"kernel_ms_mean": 2.0})
    assert blk["bound"] == "mfma" and blk["peak"] == 5033.2


def test_cpu_share_respects_the_granted_threads(monkeypatch):
    cores = len(os.sched_getaffinity(0))
    monkeypatch.delenv("OMP_NUM_THREADS", raising=False)
    assert bench.cpu_share() == cores
    monkeypatch.setenv("OMP_NUM_THREADS", "1")
    assert bench.cpu_share() == 1
    monkeypatch.setenv("OMP_NUM_THREADS", str(cores + 100))
    assert bench.cpu_share() == cores


def test_headline_is_the_largest_metric_configuration():
    from workloads import WORKLOADS, by_name
    h = by_name(bench.HEADLINE)
    assert h.dtype == "bf16"
    assert all(h.flops >= w.flops for w in WORKLOADS if w.dtype == "bf16")


def test_summaries_recognise_both_forward_kernels():
    assert bench.is_forward_kernel("void fa::fa_fwd_kernel<64, 64, 4, 0, true, false, 0, false>(fa::Params)")
    assert bench.is_forward_kernel("void fa::fa_fwd_pipe_kernel<128, 64, 8, true>(fa::Params)")
    assert not bench.is_forward_kernel("void fa::fa_bwd_dq_kernel<128, 8, true>(fa::BwdParams)")
    assert not bench.is_forward_kernel("__amd_rocclr_copyBuffer")


def test_summarize_timelines_writes_each_workload(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    pct = [0.0, 1.0, 2.0, 3.0, 4.0]
    rec = {"workload": "gpt2s_causal_bf16_b8h12n1024d64", "workgroups": 768, "span_us": 22.5, "cus": 256,
           "workgroups_per_cu": {"3": 256}, "start_offset": pct, "prologue": pct, "main_loop": pct, "o_store": pct,
           "end": pct, "loop_sum_per_cu": pct, "last_end_per_cu": pct,
           "gap_between_sequential_workgroups_on_a_cu": None,
           "by_start_rank_on_cu": {"0": {"main_loop_p50": 17.5, "end_p50": 20.5}},
           "xcd": {"0": {"loop_sum_per_cu_mean": 43.8, "last_end": 22.1}}}
    src = tmp_path / "t.jsonl"
    src.write_text("noise\n" + json.dumps(rec) + "\n" + json.dumps(dict(rec, workload="bertl_bf16_b16h16n512d64",
                   gap_between_sequential_workgroups_on_a_cu=[0.2, 0.3, 0.4, 0.5, 0.6])) + "\n")
    bench.summarize_timelines(str(src), "cmd here")
    text = (tmp_path / "timeline_forward_workloads.txt").read_text()
    assert "command: cmd here" in text and f"kernel sources sha: {bench.kernel_source_hash()}" in text
    assert "== gpt2s_causal_bf16_b8h12n1024d64: 768 workgroups on 256 CUs {'3': 256}, span 22.5" in text
    assert "== bertl_bf16_b16h16n512d64" in text and "[0.2, 0.3, 0.4, 0.5, 0.6]" in text
    assert "ran side by side" in text and "0: loop 17.5 end 20.5" in text and "0: 43.8/22.1" in text


def test_counter_summary_records_the_source_hash(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    d = tmp_path / "sq"
    d.mkdir()
    (d / "sq_counter_collection.csv").write_text(
        "Kernel_Name,Counter_Name,Counter_Value\n"
        "\"fa::fa_fwd_kernel<64, 64, 4, 0, true, false, 0, false, 0>(fa::Params)\",SQ_INSTS_MFMA,100\n"
        "\"fa::fa_fwd_kernel<64, 64, 4, 0, true, false, 0, false, 0>(fa::Params)\",SQ_INSTS_VALU,1200\n")
    bench.summarize_counters([str(d)], "gpt2s_causal_bf16_b8h12n1024d64", "cmd")
    text = (tmp_path / "counters_gpt2s_causal_bf16_b8h12n1024d64.txt").read_text()
    assert f"kernel sources sha: {bench.kernel_source_hash()}" in text
    assert "VALU instructions per MFMA (the count includes the MFMAs): 12.00" in text
