"""bench.py host logic on the CPU: the one-GPU refusal, the counter scaling of the traffic
summary (on small fabricated counter files), and the algorithmic byte model's parts."""
import csv
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import workloads as WL  # noqa: E402

pytestmark = pytest.mark.filterwarnings("ignore")


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr


def _counter_file(path, counter, rows):
    with open(path, "w", newline="") as f:
        wr = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        wr.writeheader()
        for name, v in rows:
            wr.writerow({"Kernel_Name": name, "Counter_Name": counter, "Counter_Value": v})


def test_traffic_summary_scales_by_the_copy_probe(tmp_path):
    attn = "void wd::k_attn<wd::bf16_t, 64, 1, true, 4>(wd::AttnParams)"
    selfattn = "void wd::k_attn<wd::bf16_t, 64, 1, false, 4>(wd::AttnParams)"
    copy_kib = bench.COPY_PROBE_BYTES / 1024
    # the counter reads half of the copy's bytes for fetches and all of them for writes
    _counter_file(tmp_path / "f.csv", "FETCH_SIZE", [(attn, 1000.0), (attn, 3000.0), (selfattn, 7.0),
                                                     ("__amd_rocclr_copyBuffer", copy_kib / 2),
                                                     ("__amd_rocclr_copyBuffer", 1.0)])
    _counter_file(tmp_path / "w.csv", "WRITE_SIZE", [(attn, 10.0), (attn, 30.0),
                                                     ("__amd_rocclr_copyBuffer", copy_kib)])
    out = bench.summarize_traffic(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), ["cmd"])
    assert out["dispatches"] == 2
    assert out["fetch_scale"] == pytest.approx(0.5) and out["write_scale"] == pytest.approx(1.0)
    assert out["hbm_fetch_bytes_per_launch"] == int(2000.0 * 1024 / 0.5)
    assert out["hbm_write_bytes_per_launch"] == int(20.0 * 1024)
    assert out["kernel_source_sha256"] == bench.attn_source_sha()


def test_cross_attention_bytes_per_launch_large_v3():
    w = WL.by_name("whisper_large_bf16_b64")
    assert bench.cross_attn_bytes_per_launch(w) == 64 * 20 * 1500 * 64 * 2 * 2 == 491_520_000


def test_traffic_summary_applies_to_its_own_workload_only():
    """The counter summary was taken on the large-v3 window's cross-attention; a
    bench line of any other workload reports no traffic figure."""
    assert bench.traffic_per_launch("whisper_small_f16_b16") is None
    assert bench.traffic_per_launch("qwen3asr_bf16_b8") is None
    t = bench.traffic_per_launch(bench.TRAFFIC_WORKLOAD)
    assert t is None or t > 0


def test_kernel_names_and_split_k_shapes():
    """Counter rows are labelled by kernel name (demangled or not) and launch shape: the
    split-K shapes restated in bench.py must name the instantiations the profiles show."""
    assert bench.canon_kernel("void wd::k_mgemv_sk<wd::bf16_t, 2, 4, 7, 1>(wd::MGemvParams)") == "k_mgemv_sk<2,4,7,1>"
    assert bench.canon_kernel("_ZN2wd10k_mgemv_skIDF16_Li1ELi1ELi4ELi1EEEvNS_11MGemvParamsE") == "k_mgemv_sk<1,1,4,1>"
    assert bench.canon_kernel("_ZN2wd6k_attnIDF16_Li64ELi1ELb1ELi8EEEvNS_10AttnParamsE") == "k_attn<64,1,true,8>"
    w = WL.by_name("whisper_large_bf16_b64")
    shapes = {r: bench.sk_shape(N, K, w.batch, e) for r, N, K, e in bench.projections(w)}
    assert shapes["self out"][:3] == (1, 4, 5) and shapes["q|k|v"][:3] == (2, 4, 5)
    assert shapes["fc1"][:3] == (2, 4, 7) and shapes["fc2"][3] == 24
    q = WL.by_name("qwen3asr_bf16_b8")
    qs = {r: bench.sk_shape(N, K, q.batch, e) for r, N, K, e in bench.projections(q)}
    assert qs["gate|up"][:3] == (1, 1, 16) and qs["out"][:3] == (1, 1, 8)


def test_counter_summary_scales_and_labels(tmp_path):
    w = WL.reduced(WL.by_name("whisper_large_bf16_b64"), layers=1)
    copy_kib = bench.COPY_PROBE_BYTES / 1024
    sk = "void wd::k_mgemv_sk<wd::bf16_t, 1, 4, 5, 1>(wd::MGemvParams)"
    ca = "void wd::k_attn<wd::bf16_t, 64, 1, true, 8>(wd::AttnParams)"

    def write(path, counter, rows):
        with open(path, "w", newline="") as f:
            wr = csv.DictWriter(f, fieldnames=["Kernel_Name", "Grid_Size", "Workgroup_Size", "Counter_Name",
                                               "Counter_Value"])
            wr.writeheader()
            for name, grid, v in rows:
                wr.writerow({"Kernel_Name": name, "Grid_Size": grid * 256, "Workgroup_Size": 256,
                             "Counter_Name": counter, "Counter_Value": v})
    write(tmp_path / "f.csv", "FETCH_SIZE", [(sk, 160, 3200.0), (ca, 1280, 480000.0),
                                             ("__amd_rocclr_copyBuffer", 1, copy_kib / 2)])
    write(tmp_path / "w.csv", "WRITE_SIZE", [(sk, 160, 2560.0), (ca, 1280, 640.0),
                                             ("__amd_rocclr_copyBuffer", 1, copy_kib)])
    md = bench.summarize_counters(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), w, 4, ["cmd"])
    line = [l for l in md.splitlines() if "k_mgemv_sk<1,4,5,1>" in l][0]
    assert "self out" in line and f"{3200 * 1024 * 2:,}" in line and f"{1280 * 1280 * 2:,}" in line
    line = [l for l in md.splitlines() if "k_attn<64,1,true,8>" in l][0]
    assert "cross-attention" in line and f"{bench.cross_attn_bytes_per_launch(w):,}" in line


def test_counter_summary_refuses_a_run_without_the_copy_probe(tmp_path):
    """Without the 256 MiB probe copy the scale would come from a small copy and inflate every
    figure thousands of times: both summaries refuse such a run."""
    w = WL.reduced(WL.by_name("qwen3asr_bf16_b8"), layers=1)
    sk = "void wd::k_mgemv_sk<wd::bf16_t, 1, 1, 16, 1>(wd::MGemvParams)"
    attn = "void wd::k_attn<wd::bf16_t, 64, 1, true, 8>(wd::AttnParams)"
    for path, counter in ((tmp_path / "f.csv", "FETCH_SIZE"), (tmp_path / "w.csv", "WRITE_SIZE")):
        _counter_file(path, counter, [(sk, 100.0), (attn, 100.0), ("__amd_rocclr_copyBuffer", 44.5)])
    with pytest.raises(SystemExit, match="copy probe"):
        bench.summarize_counters(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), w, 4, ["cmd"])
    with pytest.raises(SystemExit, match="copy probe"):
        bench.summarize_traffic(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), ["cmd"])
