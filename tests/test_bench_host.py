"""Host-side logic of bench.py (no GPU): the --gpus contract, the kernel
groups that one w4a16 call is timed as, and the profiler and counter
summaries built from rocprofv3 CSV output."""
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
    assert "one GPU" in r.stdout


@pytest.mark.parametrize("name,role", [
    ("void w4a16::gemm_small_m_kernel<8, 2, 1, 4, 3, false>(w4a16::GemmArgs)", "main"),
    ("void w4a16::gemm_small_m_lds_kernel<8, 1, 4, 3, true>(w4a16::GemmArgs, int, int, int)", "main"),
    ("void w4a16::(anonymous namespace)::splitk_reduce_kernel<false>(w4a16::GemmArgs)", "reduce"),
    ("void w4a16::(anonymous namespace)::gemm_large_m_kernel<2, 4, 4, 4, 4, false>(w4a16::GemmArgs, int, int)", None),
    ("__amd_rocclr_copyBuffer", None),
])
def test_small_m_group_roles(name, role):
    assert bench.group_role("gemm_small_m", name) == role


def test_kernel_name_follows_the_library_plan():
    assert bench.kernel_name(1, 22016, 4096) == bench.kernel_name(64, 22016, 4096) == "gemm_small_m"
    assert bench.kernel_name(65, 22016, 4096) == bench.kernel_name(2048, 4096, 4096) == "gemm_large_m"
    assert bench.kernel_name(128, 4096, 4096) == "gemm_small_m"
    assert bench.kernel_name(128, 4096, 4096, "bf16") == "gemm_small_m"
    assert bench.kernel_name(256, 4096, 4096, "bf16") == "gemm_large_m"


def _write(path, text):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w") as f:
        f.write(text)


def test_prof_summary_per_call_time(tmp_path, monkeypatch):
    """Per-call time = (main kernels' + reduce kernel's total time) / main calls."""
    stats = tmp_path / "prof" / "host" / "run_kernel_stats.csv"
    _write(str(stats), "\n".join([
        '"Name","Calls","TotalDurationNs","AverageNs","Percentage","MinNs","MaxNs","StdDev"',
        '"void w4a16::gemm_small_m_kernel<4, 4, 2, 4, 2, false>(w4a16::GemmArgs)",100,1000000,10000,50,9000,11000,1',
        '"void w4a16::gemm_small_m_lds_kernel<8, 1, 4, 3, false>(w4a16::GemmArgs, int, int, int)",100,500000,5000,25,4000,6000,1',
        '"void w4a16::(anonymous namespace)::splitk_reduce_kernel<false>(w4a16::GemmArgs)",50,100000,2000,5,1500,2500,1',
        '"__amd_rocclr_copyBuffer",10,400000,40000,20,1000,90000,1']) + "\n")
    log = tmp_path / "bench.log"
    line = dict(metric="m", value=1.0, unit="GB/s",
                roofline=dict(avg_launch_us=8.1, kernel="gemm_small_m (...)", achieved=1.0,
                              unit="GB/s", frac=0.1))
    _write(str(log), "noise\n" + json.dumps(line) + "\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    os.makedirs(tmp_path / "profiles")
    monkeypatch.setattr(bench, "kernel_source_digest", lambda: "d")
    bench.prof_summary(str(tmp_path / "prof"), str(log), "decode7b", "f16", ["cmd"])
    text = (tmp_path / "profiles" / "gemm_small_m_decode7b.txt").read_text()
    rec = json.loads(text.split("data: ")[1])
    assert rec["calls"] == 200 and rec["reduce_dispatches"] == 50
    assert rec["profiler_us_per_call"] == pytest.approx(1.6e6 / 200 / 1e3)
    assert rec["bench_us_per_call"] == 8.1


def test_pmc_summary_scaling(tmp_path, monkeypatch):
    """Traffic per call = (counter KiB of the group's dispatches / calls) x
    (copy bytes / the copy's counter KiB), per direction."""
    def counters(path, counter, rows):
        body = ['"Dispatch_Id","Kernel_Name","Counter_Name","Counter_Value"']
        body += [f'{d},"{k}","{counter}",{v}' for d, k, v in rows]
        _write(path, "\n".join(body) + "\n")
    copy_kib = bench.COPY_MIB * 1024 / 2.0   # the counter reads half the bytes
    main = "void w4a16::gemm_small_m_kernel<4, 4, 2, 4, 2, false>(w4a16::GemmArgs)"
    red = "void w4a16::(anonymous namespace)::splitk_reduce_kernel<false>(w4a16::GemmArgs)"
    counters(str(tmp_path / "f" / "a_counter_collection.csv"), "FETCH_SIZE",
             [(1, "__amd_rocclr_copyBuffer", copy_kib), (2, main, 100.0), (3, main, 300.0),
              (4, red, 50.0)])
    counters(str(tmp_path / "w" / "a_counter_collection.csv"), "WRITE_SIZE",
             [(1, "__amd_rocclr_copyBuffer", copy_kib), (2, main, 10.0), (3, main, 10.0),
              (4, red, 20.0)])
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    os.makedirs(tmp_path / "profiles")
    monkeypatch.setattr(bench, "kernel_source_digest", lambda: "d")
    bench.pmc_summary(str(tmp_path / "f"), str(tmp_path / "w"), "decode7b", "f16", ["c1", "c2"])
    text = (tmp_path / "profiles" / "hbm_traffic_gemm_small_m_decode7b.txt").read_text()
    rec = json.loads(text.split("data: ")[1])
    assert rec["calls"] == [2, 2] and rec["reduce_dispatches"] == [1, 1]
    assert rec["fetch_kib_per_call"] == 225.0 and rec["write_kib_per_call"] == 20.0
    assert rec["traffic_bytes_per_launch"] == round((225.0 + 20.0) * 1024 * 2.0)
    monkeypatch.setattr(bench, "kernel_source_digest", lambda: "d")
    assert bench.load_traffic("gemm_small_m", "decode7b")["traffic_bytes_per_launch"] == \
        rec["traffic_bytes_per_launch"]
    monkeypatch.setattr(bench, "kernel_source_digest", lambda: "changed")
    assert bench.load_traffic("gemm_small_m", "decode7b") is None
