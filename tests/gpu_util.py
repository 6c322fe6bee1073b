"""Helpers of the GPU parity tests: run a workload through the HIP library and through the CPU
oracle on the same seeded inputs, and compare them the way the workload's tolerance says."""
from __future__ import annotations

import sys

import numpy as np

import amk_inputs as I


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def tol_of(shape) -> float:
    """fp32 workloads: max normwise relative error 1e-4; bf16/int workloads: max abs 2e-2."""
    return 1e-4 if shape.act_f32 else 2e-2


def logit_err(shape, got: np.ndarray, ref: np.ndarray) -> float:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if shape.act_f32:
        return float(np.max(np.abs(got - ref)) / max(np.max(np.abs(ref)), 1e-30))
    return float(np.max(np.abs(got - ref)))


def prefill_both(dec, ref, shape, n_pos: int) -> None:
    """Write the seeded N(0,1) cache contents of positions [0, n_pos) into both sides."""
    for l in range(shape.n_layers):
        kv = I.kv_prefill(shape, n_pos, l)
        if ref is not None:
            ref.set_kv(l, kv, 0)
        if dec is not None:
            dec.set_kv_prefix(l, kv)
