"""Host-side logic of bench.py (no GPU): the FLOP convention against the
workload table's counts, the rocprofv3 counter bookkeeping behind the
roofline's ``traffic`` field, and the one-GPU guard."""

import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


@pytest.mark.parametrize("B,H,N,d,causal,gflop", [
    (8, 16, 1024, 64, False, 34.36),     # GPT-2-medium shape, non-causal
    (8, 16, 1024, 64, True, 17.18),      # causal: exactly half
    (1, 32, 4096, 128, True, 137.44),    # Llama-3.1-8B shape
    (1, 8, 16384, 128, True, 549.76),    # long context
    (1, 8, 32768, 128, True, 2199.02),
    (4, 16, 2048, 64, True, 34.36),      # training step forward
])
def test_forward_flop_count(B, H, N, d, causal, gflop):
    """4 N^2 d per (batch, head), halved when causal."""
    assert bench.fwd_flops(B, H, N, d, causal) / 1e9 == pytest.approx(gflop, abs=0.01)


def test_training_step_flops():
    """Forward plus 2.5x for the backward: 34.36 + 85.90 GFLOP."""
    f = bench.fwd_flops(4, 16, 2048, 64, True)
    assert 2.5 * f / 1e9 == pytest.approx(85.90, abs=0.01)


def _counter_csv(path, counter, rows):
    with open(path, "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for name, value in rows:
            w.writerow(dict(Kernel_Name=name, Counter_Name=counter, Counter_Value=value))


def test_pmc_summary_scales_by_the_copy(tmp_path, monkeypatch):
    """Bytes per launch = each counter's KiB scaled by what it reads for a copy
    of known size (FETCH_SIZE counting half of the copy's bytes: factor 2),
    averaged over the kernel's dispatches; entries are keyed by kernel and
    workload and by the sources' hash, and dropped once the sources differ."""
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "traffic.json"))
    copy_kib = 256 * 1024
    fetch = tmp_path / "fetch.csv"
    write = tmp_path / "write.csv"
    main = "void fa::bwd_main_kernel<64, true>(...)"
    _counter_csv(fetch, "FETCH_SIZE", [("__amd_rocclr_copyBuffer", copy_kib / 2),
                                       (main, 1000.0), (main, 3000.0)])
    _counter_csv(write, "WRITE_SIZE", [("__amd_rocclr_copyBuffer", copy_kib),
                                       (main, 500.0), (main, 500.0)])
    out = bench.pmc_summary(str(fetch), str(write), 256.0, "bwd_main_kernel",
                            "train_step_n2048", algorithmic_bytes=1e6)
    assert out["fetch_scale"] == pytest.approx(2.0)
    assert out["write_scale"] == pytest.approx(1.0)
    assert out["dispatches"] == 2
    assert out["bytes_per_launch"] == pytest.approx(2000.0 * 1024 * 2 + 500.0 * 1024)
    assert out["traffic_over_algorithmic"] == pytest.approx(out["bytes_per_launch"] / 1e6)
    # a second kernel / workload lands beside the first
    fwd = "void fa::fwd_bf16_kernel<128, 64, true>(...)"
    _counter_csv(fetch, "FETCH_SIZE", [("__amd_rocclr_copyBuffer", copy_kib / 2), (fwd, 10.0)])
    _counter_csv(write, "WRITE_SIZE", [("__amd_rocclr_copyBuffer", copy_kib), (fwd, 4.0)])
    bench.pmc_summary(str(fetch), str(write), 256.0, "fwd_bf16_kernel", "llama8b_n4096_causal")
    with open(bench.TRAFFIC_FILE) as fh:
        stored = json.load(fh)
    assert len(stored["entries"]) == 2
    assert stored["entries"][0]["source_hash"] == bench.source_hash("bwd_main_kernel")
    assert bench.load_traffic("bwd_main_kernel", "train_step_n2048") == \
        pytest.approx(out["bytes_per_launch"])
    assert bench.load_traffic("fwd_bf16_kernel", "llama8b_n4096_causal") == \
        pytest.approx(10.0 * 1024 * 2 + 4.0 * 1024)
    assert bench.load_traffic("fwd_bf16_kernel", "train_step_n2048") is None
    stored["entries"][0]["source_hash"] = "0" * 16
    with open(bench.TRAFFIC_FILE, "w") as fh:
        json.dump(stored, fh)
    assert bench.load_traffic("bwd_main_kernel", "train_step_n2048") is None


def test_algorithmic_bytes():
    """Forward: Q, K, V in and O out (2 bytes each) plus a 4-byte lse per row;
    backward: Q, K, V, O, dO, lse in and dQ, dK, dV out."""
    assert bench.fwd_algorithmic_bytes(1, 32, 4096, 128) == 4 * 32 * 4096 * 128 * 2 + 32 * 4096 * 4
    assert bench.bwd_algorithmic_bytes(4, 16, 2048, 64) == 8 * 64 * 2048 * 64 * 2 + 64 * 2048 * 4


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_cold_mode_times_one_call_per_repeat(monkeypatch):
    """--cold parses, and with the flush buffer set every timed repeat is one
    call (the buffer is written before each); warm repeats keep their length."""
    assert bench.main(["--cold", "--gpus", "2"]) == 2     # parsed, then refused before any GPU use
    monkeypatch.setattr(bench, "_cold_buf", None)
    assert bench._per_repeat(20) == 20
    monkeypatch.setattr(bench, "_cold_buf", object())
    assert bench._per_repeat(20) == 1
    assert bench.COLD_MIB * 2 ** 20 > 8 * 4 * 2 ** 20 + 256 * 2 ** 20   # past every L2 and the LLC
