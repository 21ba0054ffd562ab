"""Host logic of bench.py (no GPU): the algorithmic byte counts behind the
roofline figures, format names in the JSON line, and the one-GPU rule.

The per-unit figures are the layer's packed sizes worked from the shapes:
a 4-bit g64 expert's gate and up projections are 2 x 512 x 2048 codes at
half a byte plus one 4-byte scale/bias word per group of 64
(1,048,576 + 131,072 = 1,179,648 B), its down projection 2048 x 512 codes
plus its words (524,288 + 65,536 = 589,824 B); the 4-bit router is
256 x 2048 codes plus words (262,144 + 32,768 = 294,912 B) and the gate row
one row of them (1,024 + 128 = 1,152 B).
"""
import os
import subprocess
import sys
from dataclasses import replace

import pytest

import synth
from synth.gen import Q2G64, Q3G64, Q4G64, Q5G64, Q6G64, Q8G64, S4G128

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_expert_bytes_of_the_headline_layer():
    spec = synth.CONFIGS[1]
    assert bench.expert_bytes(spec, Q4G64, spec.inter) == (1_179_648, 589_824)


@pytest.mark.parametrize("fmt,words_per_group", [(Q2G64, 4), (Q3G64, 6), (Q5G64, 10), (Q6G64, 12),
                                                 (Q8G64, 16)])
def test_expert_bytes_scale_with_the_code_width(fmt, words_per_group):
    """Codes: bits/8 bytes per weight (words_per_group uint32 words per row
    and group of 64); one 4-byte word per row and group for scale and bias."""
    spec = synth.CONFIGS[1]
    H, I = spec.hidden, spec.inter
    gu, dn = bench.expert_bytes(spec, fmt, I)
    assert gu == 2 * I * (H // 64) * (4 * words_per_group + 4)
    assert dn == H * (I // 64) * (4 * words_per_group + 4)


def test_symmetric_expert_bytes():
    """int4 symmetric g128: half a byte per weight, one 2-byte fp16 scale per
    row and group of 128, no bias."""
    spec = synth.CONFIGS[4]
    gu, dn = bench.expert_bytes(spec, S4G128, spec.inter)
    assert gu == 2 * 512 * 2048 // 2 + 2 * 512 * 16 * 2
    assert dn == 2048 * 512 // 2 + 2048 * 4 * 2


def test_router_bytes():
    assert bench.router_bytes(synth.CONFIGS[1]) == 294_912 + 1_152
    # W4A16: int4-symmetric g128 router, dense bf16 gate row
    assert bench.router_bytes(synth.CONFIGS[4]) == 256 * 2048 // 2 + 256 * 16 * 2 + 2048 * 2


def test_format_names():
    assert bench.fmt_name(Q4G64) == "affine 4-bit g64 bf16 scale/bias"
    assert bench.fmt_name(S4G128) == "symmetric 4-bit g128 fp16 scale"
    assert bench.fmt_name(synth.CONFIGS[4].gate_row) == "dense bf16"
    assert bench.fmt_name(replace(Q4G64, bits=6)) == "affine 6-bit g64 bf16 scale/bias"


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""


def test_prefill_algorithmic_counts_unique_experts_once():
    """A chunk's bytes: each selected expert's packed bytes once however many
    rows pick it, plus shared expert, router, gate row, x in and fp32 y out;
    flops per (row, slot), per row for the shared expert and the router."""
    import numpy as np
    spec = synth.CONFIGS[3]
    ids = np.array([[0, 1, 2, 3, 4, 5, 6, 7], [7, 6, 5, 4, 3, 2, 1, 0], [8, 1, 2, 3, 4, 5, 6, 7]], np.int32)
    a = bench.prefill_algorithmic(spec, ids)
    gu, dn = bench.expert_bytes(spec, spec.routed, spec.inter)
    H = spec.hidden
    assert a["unique_experts"] == 9
    assert a["bytes"] == 10 * (gu + dn) + bench.router_bytes(spec) + 3 * H * 2 + 3 * H * 4
    assert a["flop_routed"] == 2 * 3 * H * 512 * 3 * 8
    assert a["flop_shared"] == 2 * 3 * H * 512 * 3
    assert a["flop_router"] == 2 * 257 * H * 3


def test_host_threads_and_cpu_model():
    assert bench.host_threads() >= 1
    assert isinstance(bench.cpu_model(), str) and bench.cpu_model()


def test_mfma_summary_formula(tmp_path):
    """Busy fraction = MFMA busy cycles over (GRBM_GUI_ACTIVE / 8 XCDs) x 1024
    SIMDs; TFLOP/s = 512 flops per MOPS unit over the traced mean duration."""
    pmc = tmp_path / "p_counter_collection.csv"
    tr = tmp_path / "t_kernel_trace.csv"
    k = "void moe::k_grp_gemm<0, 0, 0>(moe::GroupedArgs)"
    pmc.write_text("Kernel_Name,Counter_Name,Counter_Value\n"
                   f'"{k}",GRBM_GUI_ACTIVE,800000\n'
                   f'"{k}",SQ_VALU_MFMA_BUSY_CYCLES,51200000\n'
                   f'"{k}",SQ_INSTS_VALU_MFMA_MOPS_F16,1000000\n')
    tr.write_text("Kernel_Name,Start_Timestamp,End_Timestamp\n" f'"{k}",1000,101000\n')
    md = bench.mfma_summary(str(pmc), str(tr), ["cmd"])
    row = [l for l in md.splitlines() if "k_grp_gemm" in l][0].split("|")
    # 51.2e6 / (1e5 x 1024) = 0.5; 512e6 flop / 100 us = 5.12 TFLOP/s
    assert row[-4].strip() == "0.500"
    assert row[-3].strip() == "5.1"
