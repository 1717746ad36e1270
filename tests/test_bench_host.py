"""Host-side checks of bench.py (no GPU): the algorithmic byte counts it
prices the rooflines with, the prefill tile accounting, and its refusal of
more than one GPU."""
import os
import subprocess
import sys

import bench
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_expert_bytes_match_the_block_formats():
    w = synth.WORKLOADS["decode_b1"]
    eg, ed = bench.expert_bytes(w)
    # IQ2X gate + up: 66 bytes per 256 weights; Q2K down: 84 bytes per 256
    assert eg == 2 * 2048 * (7168 // 256) * 66 == 7_569_408
    assert ed == 7168 * (2048 // 256) * 84 == 4_816_896
    assert eg + ed == 12_386_304
    # batch 1: 8 routed experts + bf16 shared gate, up, down + bf16 router
    assert w.k * (eg + ed) + 3 * w.I * w.H * 2 + w.E * w.H * 2 == 190_840_832
    # MXFP4: 17 bytes per 32 weights
    mg, md = bench.expert_bytes(w.with_(fmt="mxfp4"))
    assert (mg, md) == (2 * 2048 * 224 * 17, 7168 * 64 * 17)


def test_issued_rows_pad_each_tile_to_32_row_blocks():
    # tiles of up to 96 rows, each run in blocks of 32
    assert bench.issued_rows([0]) == 0
    assert bench.issued_rows([1]) == 32
    assert bench.issued_rows([32, 33]) == 32 + 64
    assert bench.issued_rows([96, 97]) == 96 + 96 + 32
    assert bench.issued_rows([200]) == 96 + 96 + 32


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""
