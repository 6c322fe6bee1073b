"""CPU check of the decode megakernel's weight and cache streaming order.

Each compute wave of the decode kernel streams, in task-queue order, the bytes of its CU's
weight tiles and attention history that do not depend on the step's activations, while the
I/O wave waits for the activations (AutoMegaKernel pages: page 1, "What's built", the one
persistent kernel per GPU that overlaps loads of later work with the wait on earlier work).
The iterator that orders those loads is a header shared by the device code and this check;
compiled for the host with the lowering, it walks every wave of every CU of the real lowering
of each workload shape and asserts that every load stays inside the CU's weight stream or the
chunk's cache rows below the position, that the issue side yields exactly as many loads as the
consumer takes, that every byte of every weight row a wave owns is loaded exactly once, and that
the quantisation scales each wave reads (whole dwords through the scalar cache) stay inside the
tile's scale block, each lane taking the scale of its own 128-column group (also when a row's
int4 scales start mid-dword, K/128 odd).
"""
from __future__ import annotations

import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "native", "ring_check.cpp")
CSRC = os.path.join(ROOT, "persistent_megakernel_amd", "csrc")

# hidden layers heads kv_heads head_dim intermediate vocab max_ctx wfmt pos
CASES = {
    "tiny_fp32": "64 2 4 2 16 176 256 64 0 20",
    "tiny_fp32_pos0": "64 2 4 2 16 176 256 64 0 0",
    "tiny_int4_odd_groups": "256 1 4 2 64 384 300 48 3 20",
    "smollm2_bf16": "576 30 9 3 64 1536 49152 64 1 40",
    "tinyllama_int8": "2048 22 32 4 64 5632 32000 1024 2 512",
    "tinyllama_int8_last": "2048 22 32 4 64 5632 32000 1024 2 1023",
    "llama7b_bf16": "4096 32 32 32 128 11008 32000 2080 1 2048",
    "llama7b_int8": "4096 32 32 32 128 11008 32000 2080 2 2050",
    "llama3_8b_int4": "4096 32 32 8 128 14336 128256 4128 3 4096",
    "tinyllama_int8_64cu": "2048 22 32 4 64 5632 32000 1024 2 700 64",
}


@pytest.fixture(scope="module")
def ring_check(tmp_path_factory):
    exe = str(tmp_path_factory.mktemp("ring") / "ring_check")
    subprocess.run(["g++", "-O2", "-std=c++17", "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-o", exe, SRC,
                    os.path.join(CSRC, "lower.cpp")], check=True)
    return exe


@pytest.mark.parametrize("case", list(CASES))
def test_ring_loads_in_bounds_and_complete(ring_check, case):
    r = subprocess.run([ring_check] + CASES[case].split(), capture_output=True, text=True, timeout=600)
    assert r.returncode == 0 and r.stdout.startswith("ok"), r.stdout + r.stderr
