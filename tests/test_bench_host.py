"""Host logic of bench.py (CPU only): the one-GPU guard and the rocprofv3 summaries
that the bench's `roofline.traffic` and `profiles/` come from, on synthetic
profiler output whose expected numbers are written out by hand."""
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

FWD = "void dsa::(anonymous namespace)::attn_fwd_kernel<__bf16, 128, true>(dsa::FwdArgs)"
COPY = "void at::native::bitwise_not_kernel(int*)"
PAIRS = 512 * 52 * 64 * 64 * 24


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def _run_dir(root, sub, cmd, src_hash, rows=None, counter=None, stats=None):
    d = os.path.join(root, sub)
    os.makedirs(os.path.join(d, "raw"), exist_ok=True)
    with open(os.path.join(d, "cmd.txt"), "w") as fh:
        fh.write(cmd + "\n")
    out = {"config": {"workload": "train_32k: one attention layer", "B": 1, "H": 24, "d": 128, "tokens": 32768,
                      "tile": [1, 8, 8], "k": 52},
           "source_hash": src_hash, "warmup": 1, "steps": 2, "phase_ms": {"fwd": 1.7}, "ms_per_step": 8.7,
           "value": 540.0, "fwd": {"ms": 1.7, "tflops": 790.0}, "counted_flop": {"pairs": PAIRS}}
    with open(os.path.join(d, "out.json"), "w") as fh:
        fh.write("profiler banner\n" + json.dumps(out) + "\n")
    if rows is not None:
        with open(os.path.join(d, "raw", "pmc_counter_collection.csv"), "w", newline="") as fh:
            w = csv.writer(fh)
            w.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
            for disp, name, value in rows:
                w.writerow([disp, name, counter, value])
    if stats is not None:
        with open(os.path.join(d, "raw", "kt_kernel_stats.csv"), "w", newline="") as fh:
            w = csv.writer(fh)
            w.writerow(["Name", "Calls", "TotalDurationNs", "AverageNs", "MinNs", "MaxNs"])
            for row in stats:
                w.writerow(row)


def test_summaries_scale_counters_by_the_copy_kernel(tmp_path):
    src = bench.source_hash()
    root = tmp_path / "run"
    prof = tmp_path / "prof"
    _run_dir(root, "trace", "rocprofv3 --kernel-trace ... -- python3 bench.py", src,
             stats=[(FWD, 3, 4.8e6, 1.6e6, 1.5e6, 1.7e6), (COPY, 1, 1e5, 1e5, 1e5, 1e5)])
    # FETCH_SIZE: the 1024 MiB copy reads 524,288 KiB on the counter -> scale 2.0;
    # the kernel reads 1000 KiB per dispatch (two dispatches: 900 and 1100)
    _run_dir(root, "fetch", "rocprofv3 --pmc FETCH_SIZE -- python3 bench.py --copy-probe-mib 1024", src,
             rows=[(1, FWD, 900.0), (2, FWD, 1100.0), (3, COPY, 524288.0)], counter="FETCH_SIZE")
    # WRITE_SIZE: the copy writes 1,048,576 KiB -> scale 1.0; the kernel 300 KiB
    _run_dir(root, "write", "rocprofv3 --pmc WRITE_SIZE -- python3 bench.py --copy-probe-mib 1024", src,
             rows=[(1, FWD, 300.0), (2, FWD, 300.0), (3, COPY, 1048576.0)], counter="WRITE_SIZE")
    # a counter pass: 32 MFMA per (wave, block) unit, four waves per (tile, block) pair
    units = PAIRS / (64 * 64) * 4
    _run_dir(root, "counters_1", "rocprofv3 --pmc SQ_INSTS_MFMA -- python3 bench.py", src,
             rows=[(1, FWD, 32 * units), (2, FWD, 32 * units)], counter="SQ_INSTS_MFMA")
    bench.summarize(str(root), prof_dir=str(prof))

    traffic = prof / "traffic_attn_fwd_kernel_train_32k.txt"
    vals = dict(line.split(":", 1) for line in traffic.read_text().splitlines() if ":" in line and line[0] != "#")
    assert float(vals["fetch_scale"]) == pytest.approx(2.0)
    assert float(vals["write_scale"]) == pytest.approx(1.0)
    assert float(vals["fetch_bytes_per_launch"]) == pytest.approx(1000 * 1024 * 2.0)
    assert float(vals["write_bytes_per_launch"]) == pytest.approx(300 * 1024 * 1.0)
    assert float(vals["hbm_bytes_per_launch"]) == pytest.approx(2000 * 1024 + 300 * 1024)
    # the bench reads it back only while the kernel sources are unchanged
    assert bench.load_traffic("attn_fwd_kernel", "train_32k", prof_dir=str(prof)) == pytest.approx(2300 * 1024)
    traffic.write_text(traffic.read_text().replace(src, "0" * 16))
    assert bench.load_traffic("attn_fwd_kernel", "train_32k", prof_dir=str(prof)) is None

    trace = (prof / "train_32k_kernel_trace.md").read_text()
    assert "| attn_fwd_kernel<bf16,128,full> | 3 | 1600.0 | 1500.0 | 1700.0 |" in trace
    assert "bitwise_not" not in trace                      # only the library's kernels
    counters = (prof / "counters_train_32k.md").read_text()
    assert "| SQ_INSTS_MFMA |" in counters and "| 32.0 |" in counters


def test_summaries_refuse_mixed_sources(tmp_path):
    root = tmp_path / "run"
    _run_dir(root, "trace", "c", "a" * 16, stats=[(FWD, 1, 1.0, 1.0, 1.0, 1.0)])
    _run_dir(root, "fetch", "c --copy-probe-mib 8", "a" * 16, rows=[(1, FWD, 1.0)], counter="FETCH_SIZE")
    _run_dir(root, "write", "c --copy-probe-mib 8", "b" * 16, rows=[(1, FWD, 1.0)], counter="WRITE_SIZE")
    with pytest.raises(SystemExit):
        bench.summarize(str(root), prof_dir=str(tmp_path / "prof"))


def test_kernel_labels():
    """Short kernel names in the profile summaries, from demangled and mangled symbols."""
    import bench
    cases = {
        "void dsa::(anonymous namespace)::attn_fwd_pair_kernel<128, true>(dsa::FwdArgs)": "attn_fwd_pair_kernel<bf16,128,full>",
        "_ZN3dsa12_GLOBAL__N_120attn_fwd_pair_kernelILi128ELb1EEEvNS_7FwdArgsE": "attn_fwd_pair_kernel<bf16,128,full>",
        "void dsa::(anonymous namespace)::attn_fwd_pair_kernel<64, false>(dsa::FwdArgs)": "attn_fwd_pair_kernel<bf16,64>",
        "void dsa::(anonymous namespace)::attn_fwd_kernel<__bf16, 128, true>(dsa::FwdArgs)": "attn_fwd_kernel<bf16,128,full>",
        "_ZN3dsa12_GLOBAL__N_115bwd_dkdv_kernelIDF16bLi128ELb1EEEvNS_8BwdArgsE": "bwd_dkdv_kernel<bf16,128,full>",
    }
    for raw, want in cases.items():
        assert bench._kernel_label(raw) == want, raw
