"""Host logic of bench.py, without a GPU: the algorithmic flop and byte counts the
rooflines divide by, the sliding-window pair count, the seed offset, the refusal of
more than one GPU, and the ingest of rocprofv3 counter files (synthetic ones here)
into the traffic summary.
"""
import csv
import json
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_headline_algorithmic_counts():
    B, H, S, D = 2, 32, 8192, 128
    # two products of 2*S*S*D flop per (b, h): 4*B*H*S*S*D; causal counts half
    assert bench.fwd_flops(B, H, S, S, D) == 4.0 * B * H * S * S * D == 2199023255552.0
    assert bench.fwd_flops(B, H, S, S, D, causal=True) == 2199023255552.0 / 2
    # Q, K, V and O in bf16 once each (4 x 128 MiB) and the fp32 LSE (2 MiB)
    assert bench.fwd_bytes(B, H, S, D) == 4 * 134217728 + 2097152 == 538968064
    # e4m3 Q, K, V (one byte each), bf16 O, fp32 LSE
    assert bench.fp8_bytes(B, H, S, D) == 3 * 67108864 + 134217728 + 2097152 == 337641472
    # decode B1 H32 L32768 D128 f16: K and V, the f16 mask, q and out, the fp32 LSE
    assert bench.dec_bytes(1, 32, 32768, 128) == 536870912 + 2097152 + 16384 + 128 == 538984576


@pytest.mark.parametrize("S,w", [(1, 0), (7, 0), (7, 3), (64, 256), (300, 17), (513, 256)])
def test_window_pairs_brute_force(S, w):
    i = np.arange(S)[:, None]
    j = np.arange(S)[None, :]
    assert bench.window_pairs(S, w) == int(((j <= i) & (i - j <= w)).sum())


def test_seed_offset(monkeypatch):
    monkeypatch.setattr(bench, "SEED", 0)
    assert bench.sd(7) == 7
    monkeypatch.setattr(bench, "SEED", 5)
    assert bench.sd(7) == 12 and bench.sd(0) == 5


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def _counters(path, rows):
    """A rocprofv3-style counter_collection.csv with (kernel, counter, value) rows."""
    os.makedirs(path, exist_ok=True)
    with open(os.path.join(path, "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        for n, (k, c, v) in enumerate(rows):
            w.writerow([n + 1, k, c, v])


def test_ingest_scales_counters_by_the_copy_calibration(tmp_path, monkeypatch):
    """FETCH_SIZE / WRITE_SIZE are KiB per dispatch; each is scaled so that the 1 GiB
    copy reads as the bytes it moves, averaged over dispatches and summed over the
    kernels of a family (decode: split + merge)."""
    h = bench.kernel_source_hash()
    d = tmp_path / "counters"
    cp = "__amd_rocclr_copyBuffer"
    fill = "void at::native::vectorized_elementwise_kernel<8, at::native::FillFunctor<c10::Half> >(int)"
    # the copy's counters read half of the bytes it fetches and all it writes
    _counters(d / "fetch_copy", [(fill, "FETCH_SIZE", 20.0), (cp, "FETCH_SIZE", 2.0 ** 30 / 2 / 1024)])
    _counters(d / "write_copy", [(fill, "WRITE_SIZE", 9.0), (cp, "WRITE_SIZE", 2.0 ** 30 / 1024)])
    fk = "void mm::fwd_pipe_kernel<mm::BF16, 128, 0, 8>(mm::FwdParams)"
    _counters(d / "fetch_fwd", [(fk, "FETCH_SIZE", 1000.0), (fk, "FETCH_SIZE", 3000.0), (fill, "FETCH_SIZE", 7.0)])
    _counters(d / "write_fwd", [(fk, "WRITE_SIZE", 500.0)])
    sk = "void mm::decode_split_kernel<mm::F16, 128, true, 1, false>(mm::DecParams)"
    mk = "void mm::decode_merge_kernel<mm::F16, 128>(mm::DecParams)"
    _counters(d / "fetch_decode", [(sk, "FETCH_SIZE", 100.0), (sk, "FETCH_SIZE", 300.0), (mk, "FETCH_SIZE", 10.0)])
    _counters(d / "write_decode", [(sk, "WRITE_SIZE", 4.0), (mk, "WRITE_SIZE", 1.0)])
    pk = "void mm::fwd_fp8_kernel<128, false, 0, 8>(mm::FwdParams)"
    _counters(d / "fetch_fp8", [(pk, "FETCH_SIZE", 50.0)])
    _counters(d / "write_fp8", [(pk, "WRITE_SIZE", 25.0)])
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: h)
    bench.ingest(str(d))
    t = json.load(open(tmp_path / "profiles" / "traffic.json"))
    assert t["calibration"]["fetch_factor"] == 2.0 and t["calibration"]["write_factor"] == 1.0
    f = t["fwd_pipe_kernel"]
    assert f["fetch_bytes"] == 2000 * 1024 * 2 and f["write_bytes"] == 500 * 1024
    assert f["bytes_per_launch"] == f["fetch_bytes"] + f["write_bytes"]
    assert f["algorithmic_bytes"] == 538968064 and f["src_hash"] == h
    dec = t["decode"]
    assert dec["fetch_bytes"] == (200 + 10) * 1024 * 2 and dec["write_bytes"] == 5 * 1024
    p = t["fwd_fp8_kernel"]
    assert p["fetch_bytes"] == 50 * 1024 * 2 and p["write_bytes"] == 25 * 1024
    assert p["ratio_to_algorithmic"] == round((50 * 2048 + 25 * 1024) / 337641472, 3)
