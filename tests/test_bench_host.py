"""Host-side pieces of bench.py (no GPU): the algorithmic work a decode launch is
credited with, the one-GPU guard, and the HBM traffic record built from rocprofv3
counter files."""
import json
import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import mla_inputs as MI  # noqa: E402


def test_algorithmic_work_tiny_by_hand():
    w = MI.tiny()
    b, f, kv = bench.algorithmic_work(w)
    seq = [int(s) for s in w.seq_lens]
    assert seq == [37, 100]
    rows = 2 * 1 * 16
    assert kv == (37 + 100) * 1152
    assert b == kv + rows * (576 * 2 + 512 * 2 + 4) + (1 + 2) * 4 + 2 * 4
    assert f == (37 + 100) * 16 * (2 * 576 + 2 * 512)


def test_algorithmic_work_causal_q_len2():
    # q_len 2: row 0 sees seq - 1 tokens, row 1 sees seq
    w = MI.make_workload("c", 2, 2, 8, [10, 1], None, MI.KV_FP8, False, 5)
    b, f, kv = bench.algorithmic_work(w)
    assert kv == 11 * 584
    assert f == (9 + 10 + 0 + 1) * 8 * (2 * 576 + 2 * 512)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    msg = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in msg["error"]


def _csv(path, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w") as f:
        f.write("Dispatch_Id,Kernel_Name,Counter_Name,Counter_Value\n")
        for i, (k, c, v) in enumerate(rows):
            f.write(f"{i},{k},{c},{v}\n")


def test_traffic_record_scales_by_the_calibration_copy(tmp_path):
    fetch, write = str(tmp_path / "f"), str(tmp_path / "w")
    # a 64 MiB copy: FETCH_SIZE reads half of it (scale 2), WRITE_SIZE all of it
    _csv(os.path.join(fetch, "run_counter_collection.csv"),
         [("__amd_rocclr_copyBuffer", "FETCH_SIZE", 32768.0),
          ("void mla::decode_wide_kernel<false>(mla::DecodeParams)", "FETCH_SIZE", 100.0),
          ("void mla::decode_wide_kernel<false>(mla::DecodeParams)", "FETCH_SIZE", 104.0),
          ("void mla::decode_wide_kernel<false>(mla::DecodeParams)", "FETCH_SIZE", 102.0),
          ("mla::merge_kernel(mla::DecodeParams)", "FETCH_SIZE", 10.0),
          ("mla::head_gemm_kernel<128, 512>", "FETCH_SIZE", 999.0)])
    _csv(os.path.join(write, "run_counter_collection.csv"),
         [("__amd_rocclr_copyBuffer", "WRITE_SIZE", 65536.0),
          ("void mla::decode_wide_kernel<false>(mla::DecodeParams)", "WRITE_SIZE", 7.0),
          ("mla::merge_kernel(mla::DecodeParams)", "WRITE_SIZE", 3.0)])
    rec = bench.traffic_record_from_pmc(fetch, write, "full_head", 64, "cmd")
    assert rec["FETCH_SIZE"]["scale"] == 2.0 and rec["WRITE_SIZE"]["scale"] == 1.0
    assert rec["FETCH_SIZE"]["bytes_per_dispatch"] == {"decode_wide_kernel": 102 * 1024 * 2,
                                                        "merge_kernel": 10 * 1024 * 2}
    assert rec["hbm_bytes_per_launch"] == (102 + 10) * 2048 + (7 + 3) * 1024
    assert len(rec["decode_hip_sha256"]) == 64
