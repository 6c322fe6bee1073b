"""The CPU reference record that gates schedule-search candidates.

TEST INFRASTRUCTURE ONLY, like the rest of this package: it writes a file of expected values
computed by the oracle alone; the schedule search reads that file and never imports the oracle.

The record follows the pages' second optimisation loop (AutoMegaKernel pages: page 1, "Two
autoresearch loops", loop 2), whose proposals are checked against a CPU reference before any
timing: the model at a decode position pos0, its KV cache rows [0, pos0) filled with the
seeded synthetic prefix, is fed one seeded token and then decodes greedily for `steps` steps.
The record holds the tokens fed at each step (teacher forcing: a candidate is fed the same
tokens whatever it picks), the oracle's fp32 logits and greedy ids at each step, and the
top-2 margins.

    python -m oracle.search_reference --workload tinyllama_int8 --pos 512 --steps 4 --out ref.npz
"""
from __future__ import annotations

import argparse
import sys

import numpy as np

import amk_inputs as I

from . import OracleModel, prefill_model, run_protocol

FIRST_TOKEN_STREAM = 99   # the seeded stream the first token is drawn from


def record(workload: str, pos0: int, steps: int, weights: I.Weights | None = None) -> dict:
    """Teacher-forced reference of `steps` greedy steps from pos0 (see the module docstring)."""
    shape = I.SHAPES[workload]
    w = I.make_weights(shape) if weights is None else weights
    model = OracleModel(shape, w, max_ctx=max(shape.max_ctx, pos0 + steps + 1))
    try:
        if pos0:
            prefill_model(model, shape, pos0)
        tok0 = int(I.prompt_tokens(shape, 1, stream=FIRST_TOKEN_STREAM)[0])
        gen, logits, margins, inputs = run_protocol(model, shape, [tok0], steps, pos0=pos0)
    finally:
        model.close()
    return dict(workload=workload, pos0=int(pos0), inputs=np.asarray(inputs, np.int32),
                gen=np.asarray(gen, np.int32), logits=np.stack(logits).astype(np.float32),
                margins=np.asarray(margins, np.float64))


def save(rec: dict, path: str) -> None:
    np.savez(path, workload=np.array(rec["workload"]), pos0=np.int64(rec["pos0"]), inputs=rec["inputs"],
             gen=rec["gen"], logits=rec["logits"], margins=rec["margins"])


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--workload", default="tinyllama_int8", choices=sorted(I.SHAPES))
    ap.add_argument("--pos", type=int, default=None, help="decode position (default: the workload's prefill length)")
    ap.add_argument("--steps", type=int, default=4)
    ap.add_argument("--out", required=True)
    a = ap.parse_args(argv)
    pos0 = I.SHAPES[a.workload].prefill_ctx if a.pos is None else a.pos
    rec = record(a.workload, pos0, a.steps)
    save(rec, a.out)
    print(f"{a.workload} pos {pos0}: {a.steps} steps, ids {rec['gen'].tolist()}, "
          f"min margin {rec['margins'].min():.3e} -> {a.out}", flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
