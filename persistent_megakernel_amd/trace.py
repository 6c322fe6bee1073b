"""Per-task timestamp traces of the decode megakernel: where one launch spends its time.

A trace row per task (queue order) holds six realtime-counter values (100 MHz): compute start,
inputs observed, rows done (attention: the per-wave states stored; merge: the chunk weights
computed), end, the first wave's rows (GEMV) or positions (attention) done, outputs written
(amk_set_trace).
From them: per opcode the time spent waiting for inputs (producers on other CUs plus the
staging prologue), computing, in the epilogue, the skew between the first wave and the whole
workgroup at the end of the rows, and the closing barrier; per phase (opcode, layer) the moment
the last CU finished, i.e. the critical path of the launch; and per consuming opcode the hop:
from the last publication of a task's producers (their outputs written) to the task's inputs
observed, the cross-CU synchronisation cost of each dependency.

    python -m persistent_megakernel_amd.trace --workload tinyllama_int8 --pos 512
"""
from __future__ import annotations

import argparse
import json
import sys
from collections import defaultdict

import numpy as np

from . import _abi as A

TICK_US = 0.01          # one tick of the 100 MHz realtime counter
OPNAMES = {A.AMK_OP_QKV: "qkv", A.AMK_OP_ATTN: "attn", A.AMK_OP_MERGE: "merge", A.AMK_OP_OPROJ: "oproj",
           A.AMK_OP_GATEUP: "gateup", A.AMK_OP_DOWN: "down", A.AMK_OP_LM: "lm", A.AMK_OP_ARGMAX: "argmax",
           A.AMK_OP_ATTN_MERGE: "attn_merge"}


def summarize(sched, trace) -> dict:
    """sched: Python schedule (amk_ctx_schedule); trace: int array [n_tasks, 6] in queue order."""
    tr = np.asarray(trace, dtype=np.int64)
    order = [t for q in sched.queues for t in q]
    cu_of = [cu for cu, q in enumerate(sched.queues) for _ in q]
    t0 = int(tr[:, 0].min())
    rel = (tr - t0) * TICK_US
    by_op = defaultdict(lambda: defaultdict(list))
    phase = defaultdict(lambda: [np.inf, 0.0, 0.0])     # (op, layer) -> [first start, last inputs, last end]
    for k, tid in enumerate(order):
        t = sched.tasks[tid]
        op, layer = t.opcode, t.args[0]
        s, ready, done, end, w0, out = rel[k]
        d = by_op[OPNAMES.get(op, str(op))]
        d["wait"].append(ready - s)
        d["compute"].append(done - ready if op != A.AMK_OP_ARGMAX else 0.0)
        d["epilogue"].append(end - (done if op != A.AMK_OP_ARGMAX else ready))
        if op in (A.AMK_OP_QKV, A.AMK_OP_OPROJ, A.AMK_OP_GATEUP, A.AMK_OP_DOWN, A.AMK_OP_LM):
            d["wave_skew"].append(max(0.0, done - w0))
        d["close"].append(max(0.0, end - out))
        p = phase[(op, layer)]
        p[0] = min(p[0], s)
        p[1] = max(p[1], ready)
        p[2] = max(p[2], end)
    total = float(rel[:, 3].max())
    ops = {name: {k: round(float(np.mean(v)), 3) for k, v in d.items()} | {"tasks": len(d["wait"])}
           for name, d in by_op.items()}
    seq = sorted(phase.items(), key=lambda kv: kv[1][2])
    crit = []
    prev = 0.0
    for (op, layer), (s, ready, end) in seq:
        crit.append({"op": OPNAMES.get(op, str(op)), "layer": int(layer), "last_end_us": round(end, 3),
                     "span_us": round(end - prev, 3), "last_inputs_us": round(ready, 3)})
        prev = end
    return {"launch_us": round(total, 3), "ops_mean_us": ops, "phases": crit, "hops": hops(sched, tr),
            "n_cu": len(sched.queues), "cu_busy_end_us": round(float(np.median(rel[:, 3])), 3)}


def hops(sched, trace) -> dict:
    """Per consuming opcode: the hop of each task (inputs observed minus the latest 'outputs
    written' stamp of the producers of the counters it waits on), as the median over tasks, the
    median over phases of each phase's largest hop, and the share of phases whose slowest
    consumer runs on the CU of the phase's last producer."""
    tr = np.asarray(trace, dtype=np.int64)
    order = [t for q in sched.queues for t in q]
    row = {tid: k for k, tid in enumerate(order)}
    cu_of = {tid: cu for cu, q in enumerate(sched.queues) for tid in q}
    prods = defaultdict(list)
    for tid, t in enumerate(sched.tasks):
        for c in getattr(t, "signals", ()):
            prods[c].append(tid)
    per_task = defaultdict(list)
    per_phase = defaultdict(list)   # (op, layer) -> [(hop, consumer cu, last producer cu)]
    for tid, t in enumerate(sched.tasks):
        src = [p for (c, _) in getattr(t, "waits", ()) for p in prods.get(c, [])]
        if not src:
            continue
        last = max(src, key=lambda p: tr[row[p], 5])
        hop = float(tr[row[tid], 1] - tr[row[last], 5]) * TICK_US
        name = OPNAMES.get(t.opcode, str(t.opcode))
        per_task[name].append(hop)
        per_phase[(name, t.args[0])].append((hop, cu_of[tid], cu_of[last]))
    out = {}
    for name, v in per_task.items():
        phases = [ph for (n, _), ph in per_phase.items() if n == name]
        worst = [max(ph) for ph in phases]
        out[name] = {"median_us": round(float(np.median(v)), 3),
                     "phase_max_median_us": round(float(np.median([w[0] for w in worst])), 3),
                     "slowest_on_last_producer_cu": round(float(np.mean([w[1] == w[2] for w in worst])), 3)}
    return out


def main(argv=None) -> int:
    import torch
    import amk_inputs as I
    from . import Decoder, run_steps

    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", default="tinyllama_int8", choices=sorted(I.SHAPES))
    ap.add_argument("--pos", type=int, default=0)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--layers", type=int, default=0, help="override the layer count (0 = the workload's)")
    ap.add_argument("--phases", action="store_true", help="print every phase of the critical path")
    ap.add_argument("--cfg", nargs="*", default=[], help="lowering knobs, e.g. attn_chunks=8 tasks_lm=256")
    ap.add_argument("--raw", default=None, help="also save per-task records (op, layer, cu, 6 timestamps) to this .npz")
    args = ap.parse_args(argv)
    from . import schedule_config
    cfg = schedule_config(**{k: int(v) for k, v in (kv.split("=") for kv in args.cfg)}) if args.cfg else None
    shape = I.SHAPES[args.workload]
    if args.layers:
        shape = shape.replace(n_layers=args.layers)
    shape = shape.replace(max_ctx=max(shape.max_ctx, args.pos + args.steps + 1))
    w = I.make_weights(shape)
    dec = Decoder(shape, w, cfg=cfg)
    if args.pos:
        for l in range(shape.n_layers):
            dec.set_kv_prefix(l, I.kv_prefill(shape, args.pos, l))
    trace = dec.enable_trace()
    tok = int(I.prompt_tokens(shape, 1, stream=5)[0])
    run_steps(dec, [tok] * args.steps, args.pos, chain_from=1)
    torch.cuda.synchronize()
    sched = dec.schedule()
    res = summarize(sched, trace.cpu().numpy())
    res["cfg"] = args.cfg
    if args.raw:
        order = [t for q in sched.queues for t in q]
        cu = [c for c, q in enumerate(sched.queues) for _ in q]
        np.savez(args.raw, op=np.array([sched.tasks[t].opcode for t in order]),
                 layer=np.array([sched.tasks[t].args[0] for t in order]), cu=np.array(cu),
                 args=np.array([sched.tasks[t].args[1:] for t in order]), ts=trace.cpu().numpy())
    if not args.phases:
        res["phases"] = res["phases"][:12] + res["phases"][-4:]
    print(json.dumps(res, indent=1))
    st = dec.status()
    dec.close()
    return 1 if st else 0


if __name__ == "__main__":
    sys.exit(main())
