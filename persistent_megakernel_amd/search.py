"""Schedule search over the built-in lowering's knobs.

This is the pages' second optimisation loop (AutoMegaKernel pages: page 1, "Two autoresearch
loops", loop 2, whose edit surface is tiling, SM assignment, pipelining depth and page
allocation; page 3, "Autoresearch"). A candidate is an amk_schedule_config. Each one goes
through these steps:

1. Propose: change one knob of the incumbent, drawn from a seeded generator.
2. Lower and validate on the CPU. A schedule the validator rejects never reaches the GPU.
3. Rank: a static cost model estimates the launch time of the lowered DAG (a critical path with
   per-task costs). Only the best-ranked untried proposals are measured.
4. Gate on correctness on the GPU. Over a few chained greedy steps from the same state, the
   candidate's tokens must equal the incumbent's, and its logits must stay close to the
   incumbent's. (The GEMV rows reduce in a fixed order whatever their tiling, so only the
   attention split changes the floating-point order. Through a full-depth bf16 model that
   moves logits by up to about 0.1, so the bound is 0.25 absolute for bf16 activations and
   1e-3 of the largest logit for fp32. A schedule that races or reads stale inputs changes
   tokens or logits far beyond that.)
5. Time the candidate against the incumbent in interleaved blocks on one stream, both over the
   same decode positions. Keep it only if its median step time beats the incumbent's by more
   than `min_gain`.

The model and its inputs are the seeded synthetic workloads of `amk_inputs`.

    python -m persistent_megakernel_amd.search --workload tinyllama_int8 --budget 12
"""
from __future__ import annotations

import argparse
import dataclasses
import json
import random
import sys
import time
from typing import Dict, List, Optional, Tuple

from . import _abi as A

# The knobs and the values a proposal may give them (0 = the lowering's default).
KNOBS: Dict[str, Tuple[int, ...]] = {
    "tasks_qkv": (0, 128, 160, 192, 224),
    "tasks_o": (0, 64, 128, 192),
    "tasks_gateup": (0, 128, 176, 224),
    "tasks_down": (0, 128, 192),
    "tasks_lm": (0, 128, 192, 224),
    "attn_chunks": (0, 8, 16, 24, 32, 48, 64),
    "attn_group_tasks": (0, 2),
    "cu_assign": (0, 1),
}

Config = Dict[str, int]


def config_key(cfg: Config) -> Tuple[Tuple[str, int], ...]:
    return tuple(sorted((k, int(v)) for k, v in cfg.items() if v))


def propose(incumbent: Config, rng: random.Random, n: int) -> List[Config]:
    """n neighbours of the incumbent: each changes exactly one knob to another allowed value."""
    out = []
    names = sorted(KNOBS)
    for _ in range(n):
        k = rng.choice(names)
        vals = [v for v in KNOBS[k] if v != incumbent.get(k, 0)]
        c = dict(incumbent)
        c[k] = rng.choice(vals)
        out.append({kk: vv for kk, vv in c.items() if vv})
    return out


# ---------------------------------------------------------------- static cost model

@dataclasses.dataclass
class CostParams:
    """Per-task costs in microseconds, fitted to per-task traces and timings of the
    TinyLlama-shaped int8 decode on MI355X: a dependency hop (producer's store to the consumer's
    staged input) of about 3 us on the critical path; 111 ns per 1 KiB row part per wave with
    8 waves per CU; about 31 GB/s of weight streaming per CU when every CU streams; a fixed
    task overhead (barriers, epilogue) of about 0.5 us; attention about 1.1 us fixed plus 80 ns
    per position per wave per lane-reduction level (log2 of the lanes a head owns); a merge
    about 0.5 us plus 30 ns per chunk state gathered."""
    hop_us: float = 3.0
    part_us: float = 0.111
    waves: int = 8
    cu_gbps: float = 31.0
    task_us: float = 0.5
    attn_fixed_us: float = 1.1
    attn_level_us: float = 0.08
    merge_chunk_us: float = 0.03


def _row_bytes(shape, K: int) -> int:
    import amk_inputs as I
    if shape.wfmt == I.WF_F32:
        return 4 * K
    if shape.wfmt == I.WF_BF16:
        return 2 * K
    if shape.wfmt == I.WF_INT8:
        return K
    return K // 2


def task_cost(shape, task, pos: int, p: CostParams) -> float:
    """Estimated duration of one task once its inputs are in (microseconds)."""
    op = task.opcode
    args = tuple(task.args) + (0,) * (5 - len(task.args))
    layer, a0, a1, a2, a3 = args[:5]
    if op in (A.AMK_OP_QKV, A.AMK_OP_OPROJ, A.AMK_OP_GATEUP, A.AMK_OP_DOWN, A.AMK_OP_LM):
        rows = {A.AMK_OP_QKV: 4 * a1, A.AMK_OP_GATEUP: 2 * a1}.get(op, a1)
        K = shape.q_dim if op == A.AMK_OP_OPROJ else shape.intermediate if op == A.AMK_OP_DOWN else shape.hidden
        rb = _row_bytes(shape, K)
        parts = rows * ((rb + 1023) // 1024)
        compute = -(-parts // p.waves) * p.part_us
        stream = rows * rb / (p.cu_gbps * 1e3)
        return p.task_us + max(compute, stream)
    if op == A.AMK_OP_ATTN:
        n = pos + 1
        npos = n * (a2 + 1) // a3 - n * a2 // a3 if a3 else n
        nhp = 1
        while nhp < max(1, a1):
            nhp *= 2
        lanes = min(64 // nhp, shape.head_dim)
        levels = max(1, lanes.bit_length() - 1)
        return p.task_us + p.attn_fixed_us + -(-npos // p.waves) * p.attn_level_us * levels
    if op == A.AMK_OP_MERGE:
        return p.task_us + a1 * a3 * p.merge_chunk_us
    return p.task_us


def estimate_us(shape, sched, pos: int, p: Optional[CostParams] = None) -> float:
    """Critical path of the lowered schedule: a task starts when the task before it in its queue
    has ended and, for every counter it waits on, the last producer of that counter has ended
    plus one dependency hop; it then runs for task_cost(). Returns the last end (microseconds).
    The schedule must be acyclic (the validator's V3/V5 guarantee it)."""
    p = p or CostParams()
    tasks = sched.tasks
    prods: Dict[int, List[int]] = {}
    for i, t in enumerate(tasks):
        for c in t.signals:
            prods.setdefault(c, []).append(i)
    prev = {}
    for q in sched.queues:
        for a, b in zip(q[:-1], q[1:]):
            prev[b] = a
    deps = {i: ([prev[i]] if i in prev else []) + [j for (c, _) in t.waits for j in prods.get(c, [])]
            for i, t in enumerate(tasks)}
    end: Dict[int, float] = {}
    indeg = {i: len(d) for i, d in deps.items()}
    users: Dict[int, List[int]] = {}
    for i, d in deps.items():
        for j in d:
            users.setdefault(j, []).append(i)
    ready = [i for i, k in indeg.items() if k == 0]
    while ready:
        i = ready.pop()
        t = tasks[i]
        start = end[prev[i]] if i in prev else 0.0
        for (c, _) in t.waits:
            if prods.get(c):
                start = max(start, max(end[j] for j in prods[c]) + p.hop_us)
        end[i] = start + task_cost(shape, t, pos, p)
        for u in users.get(i, []):
            indeg[u] -= 1
            if indeg[u] == 0:
                ready.append(u)
    if len(end) != len(tasks):
        raise ValueError("schedule has a dependency cycle")
    return max(end.values()) if end else 0.0


# ---------------------------------------------------------------- lowering and validation

def lower(shape, cfg: Config, max_ctx: int, n_cu: int = 0):
    """Lower a configuration on the CPU: (accepted, schedule or None)."""
    from . import amk_lower, amk_lower_verdict, model_desc, schedule_config, AmkError
    desc = model_desc(shape, max_ctx)
    c = schedule_config(n_cu=n_cu, **cfg)
    try:
        v = amk_lower_verdict(desc, c)
    except AmkError:
        return False, None
    if not v.accepted:
        return False, None
    return True, amk_lower(desc, c)


def decide(t_inc: float, t_cand: float, min_gain: float) -> bool:
    """Keep the candidate when it is faster than the incumbent by more than min_gain (a fraction)."""
    return t_cand < t_inc * (1.0 - min_gain)


# ---------------------------------------------------------------- GPU legs

class Bench:
    """One decoder per configuration on the same weights and KV prefix, greedy steps chained on
    the device."""

    def __init__(self, shape, weights, pos0: int, max_ctx: int):
        import amk_inputs as I
        import torch
        self.torch, self.I = torch, I
        self.shape, self.w, self.pos0, self.max_ctx = shape, weights, pos0, max_ctx
        self.tok0 = int(I.prompt_tokens(shape, 1, stream=99)[0])
        self.prefix = [I.kv_prefill(shape, pos0, l) for l in range(shape.n_layers)] if pos0 else None

    def make(self, cfg: Config):
        from . import Decoder, schedule_config
        d = Decoder(self.shape, self.w, max_ctx=self.max_ctx, cfg=schedule_config(**cfg) if cfg else None)
        if self.prefix:
            for l, v in enumerate(self.prefix):
                d.set_kv_prefix(l, v)
        return d

    def run(self, dec, n: int, pos: int, logits: bool = False):
        """n chained greedy steps from pos; returns (tokens, logits or None) on the device."""
        torch = self.torch
        toks = torch.full((n + 1,), -1, dtype=torch.int32, device=dec.device)
        toks[0] = self.tok0
        lg = torch.empty((n, self.shape.vocab), dtype=torch.float32, device=dec.device) if logits else None
        for s in range(n):
            dec.step(toks[s:s + 1], pos + s, toks[s + 1:s + 2], lg[s] if logits else None)
        return toks[1:], lg

    def time_block(self, dec, n: int, pos: int) -> float:
        """Mean microseconds per step over n chained steps (events on the launch stream)."""
        torch = self.torch
        st = torch.cuda.current_stream()
        toks = torch.full((n + 1,), self.tok0, dtype=torch.int32, device=dec.device)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(st)
        for s in range(n):
            dec.step(toks[s:s + 1], pos + s, toks[s + 1:s + 2])
        b.record(st)
        torch.cuda.synchronize()
        if dec.status():
            raise RuntimeError(f"device status {dec.status()}")
        return a.elapsed_time(b) * 1e3 / n


def parity_ok(shape, ref, cand, tol: float) -> Tuple[bool, float]:
    """Tokens identical and logits within tol (absolute; fp32 models: relative to the largest
    logit magnitude)."""
    (t0, l0), (t1, l1) = ref, cand
    if not bool((t0 == t1).all()):
        return False, float("inf")
    d = (l0 - l1).abs().max().item()
    scale = max(1.0, l0.abs().max().item()) if shape.act_f32 else 1.0
    return d <= tol * scale, d


def search(workload: str, budget: int, seed: int = 0, pos0: Optional[int] = None, block: int = 50,
           rounds: int = 3, parity_steps: int = 4, min_gain: float = 0.005, rank_pool: int = 16,
           log=print) -> dict:
    """Run the loop; returns {"incumbent": cfg, "trials": [...], ...}."""
    import amk_inputs as I
    import torch
    torch.cuda.set_device(0)
    base = I.SHAPES[workload]
    pos0 = base.prefill_ctx if pos0 is None else pos0
    # every timing block runs over the same positions [pos0 + parity_steps, + block): the cache
    # keeps the workload's size unless that window does not fit (the cache size sets the
    # default attention split)
    max_ctx = max(base.max_ctx, pos0 + parity_steps + block + 1)
    shape = base.replace(max_ctx=max_ctx)
    tol = 1e-3 if shape.act_f32 else 0.25
    rng = random.Random(seed)
    log(f"[search] {workload}: weights, prefix to pos {pos0}")
    w = I.make_weights(shape)
    B = Bench(shape, w, pos0, max_ctx)

    inc_cfg: Config = {}
    ok, inc_sched = lower(shape, inc_cfg, max_ctx)
    if not ok:
        raise RuntimeError("the default schedule does not lower")
    inc_est = estimate_us(shape, inc_sched, pos0)
    inc = B.make(inc_cfg)
    ref = B.run(inc, parity_steps, pos0, logits=True)
    pos = pos0 + parity_steps
    B.time_block(inc, block, pos)   # warm-up
    trials = []
    tried = {config_key(inc_cfg)}
    for it in range(budget):
        # propose, lower, validate, rank by the cost model
        pool = []
        for c in propose(inc_cfg, rng, 4 * rank_pool):
            k = config_key(c)
            if k in tried or any(config_key(x[1]) == k for x in pool):
                continue
            ok, sc = lower(shape, c, max_ctx)
            if not ok:
                tried.add(k)
                trials.append({"cfg": c, "verdict": "rejected by lowering/validator"})
                continue
            pool.append((estimate_us(shape, sc, pos0), c))
            if len(pool) >= rank_pool:
                break
        if not pool:
            log("[search] no untried proposal left")
            break
        pool.sort(key=lambda x: x[0])
        est, cfg = pool[0]
        tried.add(config_key(cfg))
        rec = {"cfg": cfg, "estimate_us": round(est, 1)}
        cand = B.make(cfg)
        try:
            ok_p, dl = parity_ok(shape, ref, B.run(cand, parity_steps, pos0, logits=True), tol)
            rec["parity_max_logit_diff"] = dl
            if not ok_p:
                rec["verdict"] = "failed the parity gate"
            else:
                ti, tc = [], []
                B.time_block(cand, block, pos)   # warm-up
                for _ in range(rounds):
                    ti.append(B.time_block(inc, block, pos))
                    tc.append(B.time_block(cand, block, pos))
                ti.sort(); tc.sort()
                mi, mc = ti[len(ti) // 2], tc[len(tc) // 2]
                rec.update({"incumbent_us": round(mi, 2), "candidate_us": round(mc, 2)})
                if decide(mi, mc, min_gain):
                    rec["verdict"] = "kept"
                    inc.close()
                    inc, inc_cfg, inc_est, cand = cand, cfg, est, None
                    ref = B.run(inc, parity_steps, pos0, logits=True)
                else:
                    rec["verdict"] = "reverted"
        finally:
            if cand is not None:
                cand.close()
        trials.append(rec)
        log(f"[search] {it}: {json.dumps(rec)}")
    t_final = []
    for _ in range(rounds):
        t_final.append(B.time_block(inc, block, pos))
    t_final.sort()
    inc.close()
    return {"workload": workload, "pos": pos0, "incumbent": inc_cfg, "incumbent_estimate_us": round(inc_est, 1),
            "incumbent_us": round(t_final[len(t_final) // 2], 2), "trials": trials, "seed": seed}


def main(argv=None) -> int:
    import amk_inputs as I
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--workload", default="tinyllama_int8", choices=sorted(I.SHAPES))
    ap.add_argument("--budget", type=int, default=12, help="candidates measured on the GPU")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--pos", type=int, default=None, help="decode position (default: the workload's prefill length)")
    ap.add_argument("--block", type=int, default=50, help="steps per timing block")
    ap.add_argument("--out", default=None, help="write the result JSON here")
    args = ap.parse_args(argv)
    t0 = time.time()
    res = search(args.workload, args.budget, args.seed, args.pos, args.block,
                 log=lambda m: print(m, file=sys.stderr, flush=True))
    res["wall_s"] = round(time.time() - t0, 1)
    s = json.dumps(res)
    if args.out:
        with open(args.out, "w") as f:
            f.write(s + "\n")
    print(s)
    return 0


if __name__ == "__main__":
    sys.exit(main())
