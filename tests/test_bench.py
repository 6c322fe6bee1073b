"""bench.py on the CPU: its algorithmic byte and FLOP accounting against independent counts, the
measured-traffic table it reads from the profile summaries, and the one-GPU refusal."""
import json
import os
import subprocess
import sys

import numpy as np
import pytest

import amk_inputs as I

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def _stored_bytes(shape, master: np.ndarray) -> int:
    """Bytes of one projection as the kernel stores it, counted from the master tensor itself."""
    rows, cols = master.shape
    if shape.wfmt == I.WF_F32:
        return master.size * 4
    if shape.wfmt == I.WF_BF16:
        return master.size * 2
    if shape.wfmt == I.WF_INT8:
        return master.size + 2 * rows                  # codes + one fp16 scale per output row
    return master.size // 2 + 2 * rows * (cols // 128)  # nibbles + one fp16 scale per 128 inputs


@pytest.mark.parametrize("wfmt,act_f32,tied", [(I.WF_F32, True, False), (I.WF_BF16, False, True),
                                               (I.WF_INT8, False, False), (I.WF_INT4, False, False)])
def test_weight_bytes_count_every_stored_tensor_once(wfmt, act_f32, tied):
    shape = I.tiny_shape(hidden=256, intermediate=384, vocab=300, head_dim=64, n_heads=4, n_kv_heads=2,
                         wfmt=wfmt, act_f32=act_f32, tied=tied)
    w = I.make_weights(shape)
    act = 4 if act_f32 else 2
    total = 0
    for layer in w.layers:
        for name, t in layer.items():
            total += t.size * act if name.endswith("norm") else _stored_bytes(shape, t)
    lm = w.embed if tied else w.lm_head
    total += _stored_bytes(shape, lm)        # the LM head (the embedding matrix when tied)
    total += shape.hidden * act              # the final norm's gains
    total += shape.hidden * act              # one embedding row
    assert bench.weight_bytes(shape) == total


def test_kv_bytes_read_the_context_and_write_one_row():
    shape = I.SHAPES["tinyllama_int8"]
    row = shape.n_layers * 2 * shape.n_kv_heads * shape.head_dim * 2   # K and V, bf16, every layer
    assert bench.kv_bytes(shape, 0) == row
    assert bench.kv_bytes(shape, 512) == 513 * row


def test_prefill_flops_against_a_token_by_token_count():
    shape = I.tiny_shape(hidden=128, intermediate=192, vocab=100, head_dim=32, n_heads=4, n_kv_heads=2)
    n, pos0 = 7, 3
    want = 0
    for m in range(n):
        visible = pos0 + m + 1
        for _ in range(shape.n_layers):
            for rows, cols in [(shape.q_dim, shape.hidden), (shape.kv_dim, shape.hidden), (shape.kv_dim, shape.hidden),
                               (shape.hidden, shape.q_dim), (shape.intermediate, shape.hidden),
                               (shape.intermediate, shape.hidden), (shape.hidden, shape.intermediate)]:
                want += 2 * rows * cols
            want += shape.n_heads * visible * 2 * (2 * shape.head_dim)   # q.k and p.v
    want += 2 * shape.vocab * shape.hidden                              # LM head, last token only
    assert bench.prefill_flops(shape, n, pos0) == want


def test_traffic_table_covers_every_measured_workload():
    t = bench.traffic_table()
    for key in ("tinyllama_int8", "tinyllama_int8@0", "smollm2_135m_bf16", "llama7b_bf16", "llama7b_int8",
                "llama3_8b_int4", "prefill:tinyllama_int8:256"):
        assert key in t, key
    # measured traffic lies within a few percent above the algorithmic bytes of the same launch
    for key in ("llama7b_bf16", "tinyllama_int8"):
        shape = I.SHAPES[key]
        pos = bench.WORKLOADS[key][0]
        algo = bench.weight_bytes(shape) + bench.kv_bytes(shape, pos)
        assert 1.0 <= t[key] / algo < 1.1, (key, t[key], algo)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in json.loads(r.stdout.strip().splitlines()[-1])["error"]
