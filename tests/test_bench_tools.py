"""CPU checks of the measurement tooling in bench.py: the byte counts the
roofline divides by, the kernel-source hash that keys traffic records, the
record lookup, and the summaries rendered from rocprofv3 output and from the
JSON lines of earlier runs (fixtures written here, no GPU)."""
import csv
import json
import os

import pytest

import bench
from speculative_sampling_verification_softmax_amd import synth


def test_algorithmic_bytes_at_headline():
    wl = synth.WORKLOADS["headline"]
    rows = 256 * 17
    logits = rows * 128256 * 2
    assert logits == 1_116_340_224
    assert bench.stats_bytes(wl) == logits + rows * 8
    # logits once, stats written and read back, tokens, uniforms, and the outputs
    # num_accepted, out_tokens, probs, num_emitted
    assert bench.step_bytes(wl) == (logits + 2 * rows * 8 + 256 * 8 * 4 + 256 * 9 * 4
                                    + 256 * 4 + 256 * 9 * 4 + 256 * 8 * 8 + 256 * 4)


def _write(path, text):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w") as fh:
        fh.write(text)


def test_source_hash_follows_the_kernel_sources(tmp_path, monkeypatch):
    _write(str(tmp_path / "a.hpp"), "int a;\n")
    _write(str(tmp_path / "b.hip"), "int b;\n")
    _write(str(tmp_path / "notes.txt"), "not a source\n")
    monkeypatch.setattr(bench, "CSRC", str(tmp_path))
    h = bench.kernel_sources_hash()
    assert len(h) == 16 and int(h, 16) >= 0
    assert bench.kernel_sources_hash() == h
    _write(str(tmp_path / "notes.txt"), "edited, still not a source\n")
    assert bench.kernel_sources_hash() == h
    _write(str(tmp_path / "b.hip"), "int b = 1;\n")
    assert bench.kernel_sources_hash() != h


def test_traffic_record_lookup(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    h = bench.kernel_sources_hash()
    _write(str(tmp_path / "profiles" / "traffic_x.md"),
           "# traffic\n\n"
           f"traffic-record: kernel=stats_kernel workload=headline sources={h} bytes=1117000000\n"
           f"traffic-record: kernel=filter_kernel workload=headline setting=k50-p0.9 "
           f"sources={h} bytes=2261000000\n"
           "traffic-record: kernel=stats_kernel workload=small sources=0000000000000000 bytes=1\n")
    assert bench.find_traffic("stats_kernel", "headline") == 1117000000.0
    assert bench.find_traffic("filter_kernel", "headline",
                              bench.filter_setting(50, 0.9)) == 2261000000.0
    assert bench.find_traffic("filter_kernel", "headline", bench.filter_setting(0, 0.9)) is None
    assert bench.find_traffic("stats_kernel", "small") is None  # measured on other sources


def test_trace_summary_lists_this_librarys_kernels(tmp_path):
    d = tmp_path / "tr"
    rows = [
        {"Name": "void spec::stats_kernel<512, 1, 4>(void const*, void const*)", "Calls": "10",
         "AverageNs": "160000.5", "MinNs": "155000", "MaxNs": "170000"},
        {"Name": "void at::native::elementwise_kernel<...>(int)", "Calls": "3",
         "AverageNs": "1000", "MinNs": "900", "MaxNs": "1100"},
        {"Name": "void spec_probe::read_rows<true>(uint4 const*)", "Calls": "5",
         "AverageNs": "159000", "MinNs": "150000", "MaxNs": "165000"},
    ]
    os.makedirs(d / "host")
    with open(d / "host" / "run_kernel_stats.csv", "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=list(rows[0]))
        w.writeheader()
        w.writerows(rows)
    out = bench.trace_summary(str(d), "the command")
    assert "| `spec::stats_kernel<512, 1, 4>` | 10 | 160000 | 155000 | 170000 |" in out
    assert "spec_probe::read_rows<true>" in out
    assert "elementwise_kernel" not in out
    assert "the command" in out and bench.kernel_sources_hash() in out


def _pmc(path, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for name, counter, value in rows:
            w.writerow({"Kernel_Name": name, "Counter_Name": counter, "Counter_Value": value})


def test_pmc_summary_calibrates_against_a_plain_copy(tmp_path):
    """FETCH_SIZE that counts half the bytes and WRITE_SIZE that counts all of
    them: the summary scales both by the copy's readings and writes a record
    with the stats kernel's measured bytes."""
    d = tmp_path / "pmc"
    copy_kib = (bench.COPY_MIB << 20) / 1024
    stats = "void spec::stats_kernel<512, 1, 4>(void const*)"
    draw = "void spec::verify_draw_kernel<1024, 1>(void const*)"
    copy = "void at::native::copyBuffer(int)"
    wl = synth.WORKLOADS["headline"]
    alg = bench.stats_bytes(wl)
    _pmc(str(d / "fetch" / "run_counter_collection.csv"),
         [(stats, "FETCH_SIZE", alg / 1024 / 2), (stats, "FETCH_SIZE", alg / 1024 / 2),
          (draw, "FETCH_SIZE", 60000.0)])
    _pmc(str(d / "write" / "run_counter_collection.csv"),
         [(stats, "WRITE_SIZE", 0.0), (stats, "WRITE_SIZE", 0.0), (draw, "WRITE_SIZE", 50.0)])
    _pmc(str(d / "fetch_copy" / "run_counter_collection.csv"),
         [(copy, "FETCH_SIZE", copy_kib / 2)] * 3 + [(copy, "FETCH_SIZE", 4.0)])
    _pmc(str(d / "write_copy" / "run_counter_collection.csv"),
         [(copy, "WRITE_SIZE", copy_kib)] * 3 + [(copy, "WRITE_SIZE", 8.0)])
    out = bench.pmc_summary(str(d), "two_call", "headline", "cmds")
    assert "FETCH_SIZE x 2.0000 x 1024 and WRITE_SIZE x 1.0000 x 1024" in out
    assert f"(1.0000 of algorithmic)" in out
    rec = [l for l in out.splitlines() if l.startswith("traffic-record:")]
    assert rec == [f"traffic-record: kernel=stats_kernel workload=headline "
                   f"sources={bench.kernel_sources_hash()} bytes={alg}"]


def test_summaries_from_json_lines(tmp_path):
    verify = {
        "metric": "m", "value": 1.3e6, "unit": "seqs/s", "ms_per_step": 0.1938,
        "achieved_GBps": 5762.0, "pct_of_peak": 72.0, "ms_per_step_cold": None,
        "config": {"workload": "headline", "path": "two_call"},
        "roofline": {"launch_us": 163.6, "frac": 0.853},
        "parity": {"draws": 1360, "flagged": 0, "failures": 0},
        "cpu_baseline": {"value": 1440.0, "cores": 16},
        "cpu_baseline_1thread": {"value": 100.0, "cores": 1},
    }
    f = tmp_path / "v.json"
    f.write_text("[bench] a log line\n" + json.dumps(verify) + "\n")
    out = bench.summary_from([str(f)], "cmd")
    assert "| headline | two_call | 193.8 | 1.3e+06 | 5762 (72.0 %) | 163.6 | 0.853 | — | " \
           "1360, 0, 0 | 1.44e+03 (16); 100 (1) |" in out
    phases = {"metric": "p", "config": {"mode": "phases", "workload": "batch1", "B": 1, "K": 4,
                                        "V": 32000, "logits": "f32", "path": "step",
                                        "draw": "split", "steps": 100, "repeats": 7},
              "phases": {"part: sweep of its items": {"n": 441, "median": 1.76, "p10": 1.7,
                                                      "p90": 1.8, "max": 1.84},
                         "empty": {"n": 0}}}
    g = tmp_path / "p.json"
    g.write_text(json.dumps(phases) + "\n")
    out = bench.summary_from([str(g)], "cmd")
    assert "| part: sweep of its items | 1.76 | 1.70 | 1.80 | 1.84 | 441 |" in out
    assert "empty" not in out


def test_overlap_plans_cover_the_batch():
    for B in (1, 2, 3, 17, 64, 100, 256):
        plans = bench.overlap_plans(B)
        for sizes, last_step in plans:
            assert sum(sizes) == B and min(sizes) > 0
    sizes = {tuple(s): ls for s, ls in bench.overlap_plans(256)}
    assert sizes == {(128, 128): False, (64, 64, 64, 64): False, (96, 96, 64): True,
                     (144, 80, 32): True}
    # the split-row tail: a last slice that spec_verify_step draws over several workgroups
    assert all(s[-1] <= bench.SPLIT_DRAW_MAX_B for s, ls in bench.overlap_plans(256) if ls)


def test_overlap_summary(tmp_path):
    rec = {"metric": "verify step time over batch slices", "config": {"mode": "overlap"},
           "plans": [{"plan": "one stream (two calls)", "us_per_step": 193.9,
                      "outputs_equal_one_stream": True},
                     {"plan": "128 + 128", "us_per_step": 209.5,
                      "outputs_equal_one_stream": False}]}
    f = tmp_path / "o.json"
    f.write_text(json.dumps(rec) + "\n")
    out = bench.summary_from([str(f)], "cmd")
    assert "| one stream (two calls) | 193.9 | yes |" in out
    assert "| 128 + 128 | 209.5 | NO |" in out


def test_more_than_one_gpu_is_refused():
    """--gpus above 1 (or a WORLD_SIZE above 1) ends at once with status 2 and
    a message, before any GPU call."""
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    for args, env in ((["--gpus", "2"], {}), (["--gpus", "1"], {"WORLD_SIZE": "4"})):
        r = subprocess.run([sys.executable, os.path.join(root, "bench.py")] + args,
                           capture_output=True, text=True, timeout=300,
                           env={**os.environ, **env})
        assert r.returncode == 2, r.stderr
        assert "one GPU" in r.stderr and r.stdout == ""
