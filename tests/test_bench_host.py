"""bench.py's host logic (no GPU): the one-GPU guard, the traffic calibration
from counter files, and that the committed traffic records belong to the
attention sources as they stand (a record of other sources would be reported
as null traffic)."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

SCRATCH = os.path.join(ROOT, "_build", "bench_host")


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout.strip() == ""


def _csv(path, counter, rows):
    with open(path, "w") as f:
        f.write("Kernel_Name,Counter_Name,Counter_Value\n")
        for name, value in rows:
            f.write(f'"{name}",{counter},{value}\n')


def test_record_traffic_scales_by_the_copy_calibration():
    os.makedirs(SCRATCH, exist_ok=True)
    att = "void iqattn::(anonymous namespace)::iqattn_fast<64, 13, false, 0>(iqattn::DevParams)"
    copy = "__amd_rocclr_copyBuffer"
    fetch = os.path.join(SCRATCH, "fetch.csv")
    write = os.path.join(SCRATCH, "write.csv")
    # FETCH reads half of a 256 MiB copy (scale 2); WRITE reads it whole
    _csv(fetch, "FETCH_SIZE", [(att, 1000.0), (att, 1002.0), (copy, 131072.0), (copy, 5.0)])
    _csv(write, "WRITE_SIZE", [(att, 500.0), (copy, 262144.0)])
    rec = bench.record_traffic(fetch, write, "unit_case")
    assert rec["fetch"]["scale"] == 2.0 and rec["write"]["scale"] == 1.0
    assert rec["fetch"]["dispatches"] == 2
    assert rec["fetch"]["bytes_per_launch"] == 1001 * 1024 * 2
    assert rec["write"]["bytes_per_launch"] == 500 * 1024
    assert rec["hbm_bytes_per_launch"] == 1001 * 1024 * 2 + 500 * 1024
    assert rec["kernel_source_sha256_16"] == bench.kernel_source_hash()


def test_record_counters_derives_the_unit_shares():
    os.makedirs(SCRATCH, exist_ok=True)
    att = "void iqattn::(anonymous namespace)::iqattn_fast<64, 13, false, 0>(iqattn::DevParams)"
    path = os.path.join(SCRATCH, "pmc.csv")
    with open(path, "w") as f:
        f.write("Kernel_Name,Counter_Name,Counter_Value\n")
        for v in (1.0, 3.0):   # two dispatches: averaged
            f.write(f'"{att}",SQ_INSTS_VALU,{1024000 * v}\n')
            f.write(f'"{att}",SQ_INSTS_MFMA,{24000 * v}\n')
            f.write(f'"{att}",SQ_VALU_MFMA_BUSY_CYCLES,{1024 * 500 * v}\n')
            f.write(f'"{att}",GRBM_GUI_ACTIVE,{8 * 4000 * v}\n')
        f.write('"other_kernel",SQ_INSTS_VALU,99\n')
    rec = bench.record_counters(path, "unit_case")
    assert rec["valu_insts_per_launch"] == 2048000 - 48000
    # 2,000,000 VALU wave instructions x 4 cycles over 1,024 SIMDs and 8,000 cycles
    assert rec["valu_busy_share"] == round(4.0 * 2000000 / 1024 / 8000, 4)
    assert rec["mfma_busy_share"] == round(1000.0 / 8000, 4)
    assert rec["kernel_source_sha256_16"] == bench.kernel_source_hash()


COUNTER_SHAPES = ["deit_tiny_b1_h3_n197_d64", "deit_small_b64_h6_n197_d64", "vitb_b128_h12_n197_d64",
                  "swin_s_stage1_2048win_h3_n49_d32_relbias", "vitl384_b32_h16_n577_d64_lis",
                  "vitl384_b32_h16_n577_d64_lis_mfma"]


@pytest.mark.parametrize("name", COUNTER_SHAPES)
def test_committed_counter_records_match_the_sources(name):
    rec = json.load(open(os.path.join(ROOT, "profiles", f"counters_{name}.json")))
    assert rec["kernel_source_sha256_16"] == bench.kernel_source_hash(), \
        "attention sources changed since the counter record: re-record it"
    assert bench.load_counters(name) is not None
    assert 0.0 < rec["valu_busy_share"] < 1.5 and 0.0 < rec["mfma_busy_share"] < 1.0


@pytest.mark.parametrize("name", ["vitb_b128_h12_n197_d64", "vitl384_b32_h16_n577_d64_lis",
                                  "swin_s_stage1_2048win_h3_n49_d32_relbias",
                                  "deit_small_b64_h6_n197_d64", "deit_tiny_b1_h3_n197_d64",
                                  "vitl384_b32_h16_n577_d64_lis_mfma"])
def test_committed_traffic_records_match_the_sources(name):
    path = os.path.join(ROOT, "profiles", f"traffic_{name}.json")
    rec = json.load(open(path))
    assert rec["kernel_source_sha256_16"] == bench.kernel_source_hash(), \
        "attention sources changed since the traffic record: re-record it"
    assert bench.load_traffic(name) is not None
    # counted bytes within a few percent of the algorithmic 4 N d per head
    cfg = {"vitb_b128_h12_n197_d64": (1536, 197, 64), "vitl384_b32_h16_n577_d64_lis": (512, 577, 64),
           "vitl384_b32_h16_n577_d64_lis_mfma": (512, 577, 64),
           "swin_s_stage1_2048win_h3_n49_d32_relbias": (6144, 49, 32),
           "deit_small_b64_h6_n197_d64": (384, 197, 64), "deit_tiny_b1_h3_n197_d64": (3, 197, 64)}
    heads, n, d = cfg[name]
    # counted bytes within a few percent of the algorithmic 4 N d per head; the
    # three-head shape moves only 151 KB, so there the fixed per-dispatch bytes
    # (code, kernel arguments, table, queue words) count: within 128 KiB
    alg = 4.0 * n * d * heads
    if heads > 3:
        assert abs(rec["hbm_bytes_per_launch"] / alg - 1.0) < 0.08
    else:
        assert abs(rec["hbm_bytes_per_launch"] - alg) < 128 * 1024
