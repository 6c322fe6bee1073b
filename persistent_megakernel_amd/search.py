"""Schedule search over the built-in lowering's knobs.

This is the pages' second optimisation loop (AutoMegaKernel pages: page 1, "Two autoresearch
loops", loop 2, whose edit surface is tiling, SM assignment, pipelining depth and page
allocation, and whose proposals are checked against a CPU reference; page 3, "Autoresearch").
A candidate is an amk_schedule_config. Each one goes through these steps:

1. Propose: change one knob of the incumbent, drawn from a seeded generator.
2. Lower and validate on the CPU. A schedule the validator rejects never reaches the GPU.
3. Rank: a static cost model estimates the launch time of the lowered DAG (a critical path with
   per-task costs). Only the best-ranked untried proposals are measured.
4. Gate on correctness against the CPU reference: a record of the float64 reference model's
   teacher-forced decode from the same state (the tokens fed at each step, its fp32 logits,
   greedy ids and top-2 margins), written beforehand by a separate reference program and read
   here from a file (`load_reference`). The candidate is fed the same tokens; its logits must
   lie within the parity bar (fp32 activations: max normwise relative error 1e-4; bf16
   activations: max absolute error 2e-2 at one layer, 0.25 with RMS 0.05 deeper, where one
   different bf16 rounding of one activation already moves the logits by about 0.08), each id
   must be the lowest-index argmax of its own logits, and each id must equal the reference's
   wherever the reference's top-2 margin exceeds both 2e-2 and twice that step's error. The
   default schedule passes the same gate before the loop starts.
5. Time the candidate against the incumbent in interleaved blocks on one stream, both over the
   same decode positions. Keep it only if its median step time beats the incumbent's by more
   than `min_gain`.

`calibrate` measures a fixed spread of configurations on the GPU, each gated the same way;
`refit` then refits the cost model's parameters to those times on the CPU and reports
Spearman's rank correlation of estimate and measurement, in sample and on configurations held
out of the fit.

The model and its inputs are the seeded synthetic workloads of `amk_inputs`.

    python -m oracle.search_reference --workload tinyllama_int8 --pos 512 --out ref.npz
    python -m persistent_megakernel_amd.search --reference ref.npz --budget 12
    python -m persistent_megakernel_amd.search --reference ref.npz --calibrate --out cal.json
    python -m persistent_megakernel_amd.search --refit cal.json
"""
from __future__ import annotations

import argparse
import dataclasses
import json
import math
import random
import sys
import time
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

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
    "prefetch_groups": (0, -1, 2),
    "merge_fusion": (0, 1),
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


def ahead_groups(cfg: Config) -> int:
    """Weight-load groups a GEMV task has in flight before its inputs arrive (the kernel's
    reading of prefetch_groups: 0 means the default of one, -1 none)."""
    g = int(cfg.get("prefetch_groups", 0))
    return 1 if g == 0 else max(0, g)


# ---------------------------------------------------------------- static cost model

@dataclasses.dataclass
class CostParams:
    """Per-task costs in microseconds. The defaults are fitted (`calibrate`, then `refit`) to
    measured launch times of 18 lowerings of the TinyLlama-shaped int8 decode at position 512
    on MI355X; the terms are:
    * a dependency hop (producer's store to the consumer's staged input) of hop_us on the
      critical path, plus ahead_hop_us for every weight-load group the consuming GEMV wave has
      in flight (its input polls return behind those loads, in order);
    * part_us per 1 KiB row part per wave with `waves` waves per CU, or cu_gbps of weight
      streaming per CU when every CU streams, whichever is slower; each load group issued
      before the inputs arrive takes ahead_us off that;
    * a fixed task overhead (barriers, epilogue) of task_us;
    * attention: attn_fixed_us plus, per position per wave, attn_mac_us per multiply-add a lane
      does (head_dim x heads / 64) and attn_level_us per lane-reduction level (log2 of the
      lanes a head owns);
    * a merge: merge_chunk_us per chunk state gathered."""
    hop_us: float = 4.05
    part_us: float = 0.111
    waves: int = 8
    cu_gbps: float = 28.5
    task_us: float = 0.29
    attn_fixed_us: float = 1.18
    attn_mac_us: float = 0.027
    attn_level_us: float = 0.0405
    merge_chunk_us: float = 0.0304
    ahead_us: float = 0.73
    ahead_hop_us: float = 0.34


FIT_FIELDS = ("hop_us", "cu_gbps", "task_us", "attn_fixed_us", "attn_mac_us", "attn_level_us", "merge_chunk_us",
              "ahead_us", "ahead_hop_us")

GEMV_OPS = (A.AMK_OP_QKV, A.AMK_OP_OPROJ, A.AMK_OP_GATEUP, A.AMK_OP_DOWN, A.AMK_OP_LM)


def _row_bytes(shape, K: int) -> int:
    import amk_inputs as I
    if shape.wfmt == I.WF_F32:
        return 4 * K
    if shape.wfmt == I.WF_BF16:
        return 2 * K
    if shape.wfmt == I.WF_INT8:
        return K
    return K // 2


def task_cost(shape, task, pos: int, p: CostParams, ahead: int = 1) -> float:
    """Estimated duration of one task once its inputs are in (microseconds)."""
    op = task.opcode
    args = tuple(task.args) + (0,) * (5 - len(task.args))
    layer, a0, a1, a2, a3 = args[:5]
    if op in GEMV_OPS:
        rows = {A.AMK_OP_QKV: 4 * a1, A.AMK_OP_GATEUP: 2 * a1}.get(op, a1)
        K = shape.q_dim if op == A.AMK_OP_OPROJ else shape.intermediate if op == A.AMK_OP_DOWN else shape.hidden
        rb = _row_bytes(shape, K)
        parts = rows * ((rb + 1023) // 1024)
        compute = -(-parts // p.waves) * p.part_us
        stream = rows * rb / (p.cu_gbps * 1e3)
        body = max(compute, stream)
        return p.task_us + max(0.0, body - ahead * p.ahead_us)
    if op in (A.AMK_OP_ATTN, A.AMK_OP_ATTN_MERGE):
        n = pos + 1
        npos = n * (a2 + 1) // a3 - n * a2 // a3 if a3 else n
        nhp = 1
        while nhp < max(1, a1):
            nhp *= 2
        lanes = min(64 // nhp, shape.head_dim)
        levels = max(1, lanes.bit_length() - 1)
        macs = shape.head_dim * max(1, a1) / 64.0
        att = p.task_us + p.attn_fixed_us + -(-npos // p.waves) * (p.attn_mac_us * macs + p.attn_level_us * levels)
        # the fused form also merges every chunk state of its heads (no task of its own)
        return att + (max(1, a1) * a3 * p.merge_chunk_us if op == A.AMK_OP_ATTN_MERGE else 0.0)
    if op == A.AMK_OP_MERGE:
        return p.task_us + a1 * a3 * p.merge_chunk_us
    return p.task_us


class Plan:
    """A lowered schedule prepared for repeated cost estimates: a topological order, each task's
    queue predecessor, waits and signals, and its cost features at one decode position."""

    def __init__(self, shape, sched, pos: int):
        tasks = sched.tasks
        self.shape, self.pos, self.tasks = shape, pos, tasks
        prods: Dict[int, List[int]] = {}
        for i, t in enumerate(tasks):
            for c in t.signals:
                prods.setdefault(c, []).append(i)
        prev = {}
        for q in sched.queues:
            for a, b in zip(q[:-1], q[1:]):
                prev[b] = a
        indeg = [0] * len(tasks)
        users: Dict[int, List[int]] = {}
        for i, t in enumerate(tasks):
            deps = ([prev[i]] if i in prev else []) + [j for (c, _) in t.waits for j in prods.get(c, [])]
            indeg[i] = len(deps)
            for j in deps:
                users.setdefault(j, []).append(i)
        ready = [i for i in range(len(tasks)) if indeg[i] == 0]
        order = []
        while ready:
            i = ready.pop()
            order.append(i)
            for u in users.get(i, []):
                indeg[u] -= 1
                if indeg[u] == 0:
                    ready.append(u)
        if len(order) != len(tasks):
            raise ValueError("schedule has a dependency cycle")
        # a waiter depends on every producer of its counters, so in this order a counter's
        # producers all come before its first waiter
        self.order = order
        self.prev = [prev.get(i, -1) for i in range(len(tasks))]
        self.waits = [tuple(c for (c, _) in t.waits if c in prods) for t in tasks]
        self.signals = [tuple(t.signals) for t in tasks]
        self.gemv = [t.opcode in GEMV_OPS for t in tasks]


def plan_estimate(plan: Plan, p: Optional[CostParams] = None, ahead: int = 1) -> float:
    """Critical path of a prepared schedule: a task starts when the task before it in its queue
    has ended and, for every counter it waits on, the last producer of that counter has ended
    plus one dependency hop (longer into a GEMV task by its prefetched load groups); it then
    runs for task_cost(). Returns the last end (microseconds)."""
    p = p or CostParams()
    end = [0.0] * len(plan.tasks)
    cend: Dict[int, float] = {}
    for i in plan.order:
        j = plan.prev[i]
        start = end[j] if j >= 0 else 0.0
        hop = p.hop_us + (ahead * p.ahead_hop_us if plan.gemv[i] else 0.0)
        for c in plan.waits[i]:
            v = cend[c] + hop
            if v > start:
                start = v
        e = start + task_cost(plan.shape, plan.tasks[i], plan.pos, p, ahead)
        end[i] = e
        for c in plan.signals[i]:
            if e > cend.get(c, -1.0):
                cend[c] = e
    return max(end) if end else 0.0


class DepthPlan:
    """Estimates for a deep model from its lowerings at two and three layers: the lowered DAG
    repeats layer by layer, so past the first layer the critical path grows by the same amount
    per layer (to within the first layer's start-up)."""

    def __init__(self, shape, cfg: Config, max_ctx: int, pos: int, n_cu: int = 0):
        self.n_layers = shape.n_layers
        depths = (shape.n_layers,) if shape.n_layers <= 3 else (2, 3)
        self.plans = []
        for d in depths:
            ok, sc = lower(shape.replace(n_layers=d), cfg, max_ctx, n_cu)
            if not ok:
                raise ValueError(f"{cfg} does not lower")
            self.plans.append(Plan(shape.replace(n_layers=d), sc, pos))

    def estimate(self, p: Optional[CostParams] = None, ahead: int = 1) -> float:
        if len(self.plans) == 1:
            return plan_estimate(self.plans[0], p, ahead)
        e2, e3 = (plan_estimate(pl, p, ahead) for pl in self.plans)
        return e2 + (self.n_layers - 2) * (e3 - e2)


def estimate_us(shape, sched, pos: int, p: Optional[CostParams] = None, ahead: int = 1) -> float:
    """plan_estimate of a lowered schedule (the validator's V3/V5 guarantee it is acyclic)."""
    return plan_estimate(Plan(shape, sched, pos), p, ahead)


def spearman(a: Sequence[float], b: Sequence[float]) -> float:
    """Spearman's rank correlation (ties take their average rank)."""
    def ranks(x):
        x = np.asarray(x, dtype=np.float64)
        order = np.argsort(x, kind="stable")
        r = np.empty(len(x))
        i = 0
        while i < len(x):
            j = i
            while j + 1 < len(x) and x[order[j + 1]] == x[order[i]]:
                j += 1
            r[order[i:j + 1]] = (i + j) / 2.0
            i = j + 1
        return r
    ra, rb = ranks(a), ranks(b)
    if len(ra) < 2 or ra.std() == 0 or rb.std() == 0:
        return float("nan")
    return float(np.corrcoef(ra, rb)[0, 1])


def _est(plan, p, ahead):
    return plan.estimate(p, ahead) if isinstance(plan, DepthPlan) else plan_estimate(plan, p, ahead)


def fit_cost_params(items, p0: Optional[CostParams] = None, fields: Sequence[str] = FIT_FIELDS,
                    sweeps: int = 6) -> CostParams:
    """Refit the cost model to measured launches by coordinate descent over multiplicative steps.

    items: (Plan or DepthPlan, ahead groups, measured microseconds) tuples. The loss is the sum of squared log
    ratios of estimate to measurement; each sweep tries, for each field in turn, the current value
    scaled by a few factors and keeps the best."""
    p = dataclasses.replace(p0 or CostParams())

    def loss(q):
        return sum((math.log(max(_est(pl, q, ah), 1e-9)) - math.log(m)) ** 2 for pl, ah, m in items)

    best = loss(p)
    for _ in range(sweeps):
        improved = False
        for f in fields:
            for fac in (0.6, 0.8, 0.92, 1.08, 1.25, 1.6):
                cur = getattr(p, f)
                q = dataclasses.replace(p, **{f: cur * fac if cur else 0.05 * fac})
                lq = loss(q)
                if lq < best - 1e-12:
                    best, p, improved = lq, q, True
        if not improved:
            break
    return p


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


# ---------------------------------------------------------------- the CPU reference and the gate

@dataclasses.dataclass
class Reference:
    """The CPU reference's teacher-forced record: tokens fed at pos0, pos0+1, ..., and at each
    step the reference's fp32 logits, greedy id and top-2 margin."""
    workload: str
    pos0: int
    inputs: List[int]
    gen: List[int]
    logits: np.ndarray
    margins: List[float]

    @classmethod
    def from_record(cls, rec: dict) -> "Reference":
        return cls(str(rec["workload"]), int(rec["pos0"]), [int(t) for t in rec["inputs"]],
                   [int(t) for t in rec["gen"]], np.asarray(rec["logits"], dtype=np.float32),
                   [float(m) for m in rec["margins"]])


def load_reference(path: str) -> Reference:
    with np.load(path, allow_pickle=False) as z:
        return Reference.from_record({k: z[k] for k in z.files})


GATE_MARGIN = 2e-2


def gate_bounds(shape) -> Tuple[str, float, Optional[float]]:
    """(kind, max error, max RMS or None) of the parity bar for this shape."""
    if shape.act_f32:
        return "rel", 1e-4, None
    if shape.n_layers <= 1:
        return "abs", 2e-2, None
    return "abs", 0.25, 0.05


def gate(shape, ref: Reference, logits: np.ndarray, ids: Sequence[int]) -> Tuple[bool, dict]:
    """Check a teacher-forced run (per-step fp32 logits and ids, fed ref.inputs) against the
    reference; returns (passed, details)."""
    kind, bound, rms_bound = gate_bounds(shape)
    logits = np.asarray(logits, dtype=np.float64)
    R = np.asarray(ref.logits, dtype=np.float64)
    n = len(ref.inputs)
    if logits.shape != R.shape or len(ids) != n:
        return False, {"reason": "shape mismatch"}
    err, rms, abs_err = [], [], []
    for s in range(n):
        d = np.abs(logits[s] - R[s])
        a = float(d.max()) if d.size else 0.0
        abs_err.append(a)
        err.append(a / max(float(np.abs(R[s]).max()), 1e-30) if kind == "rel" else a)
        rms.append(float(np.sqrt(np.mean(d * d))) if d.size else 0.0)
    info = {"max_err": max(err), "max_rms": max(rms), "err_kind": kind,
            "ids_equal": [int(i) for i in ids] == ref.gen}
    if not all(np.isfinite(logits).ravel()):
        info["reason"] = "non-finite logits"
        return False, info
    if max(err) > bound or (rms_bound is not None and max(rms) > rms_bound):
        info["reason"] = "logits outside the parity bar"
        return False, info
    for s in range(n):
        row = logits[s]
        if int(ids[s]) != int(np.flatnonzero(row == row.max())[0]):
            info["reason"] = f"step {s}: id is not the argmax of the candidate's own logits"
            return False, info
        if int(ids[s]) != ref.gen[s] and ref.margins[s] >= max(GATE_MARGIN, 2 * abs_err[s]):
            info["reason"] = f"step {s}: id {int(ids[s])} != reference {ref.gen[s]} at margin {ref.margins[s]:.3e}"
            return False, info
    return True, info


# ---------------------------------------------------------------- GPU legs

class Bench:
    """One decoder per configuration on the same weights and KV prefix as the reference."""

    def __init__(self, shape, weights, ref: Reference, max_ctx: int):
        import amk_inputs as I
        import torch
        self.torch, self.I = torch, I
        self.shape, self.w, self.ref, self.max_ctx = shape, weights, ref, max_ctx
        self.pos0 = ref.pos0
        self.prefix = [I.kv_prefill(shape, ref.pos0, l) for l in range(shape.n_layers)] if ref.pos0 else None

    def make(self, cfg: Config):
        from . import Decoder, schedule_config
        d = Decoder(self.shape, self.w, max_ctx=self.max_ctx, cfg=schedule_config(**cfg) if cfg else None)
        if self.prefix:
            for l, v in enumerate(self.prefix):
                d.set_kv_prefix(l, v)
        return d

    def check(self, dec) -> Tuple[bool, dict]:
        """Teacher-forced run over the reference's inputs from pos0, then the gate. The run
        rewrites cache rows from pos0 on, which every later step rewrites before reading."""
        from . import run_steps
        torch = self.torch
        n = len(self.ref.inputs)
        lg = torch.zeros((n, self.shape.vocab), dtype=torch.float32, device=dec.device)
        ids = run_steps(dec, self.ref.inputs, self.pos0, logits=lg)
        torch.cuda.synchronize()
        if dec.status():
            return False, {"reason": f"device status {dec.status()}"}
        return gate(self.shape, self.ref, lg.cpu().numpy(), ids.cpu().numpy().tolist())

    def time_block(self, dec, n: int, pos: int) -> float:
        """Mean microseconds per step over n chained steps (events on the launch stream)."""
        torch = self.torch
        st = torch.cuda.current_stream()
        toks = torch.full((n + 1,), self.ref.inputs[0], dtype=torch.int32, device=dec.device)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(st)
        for s in range(n):
            dec.step(toks[s:s + 1], pos + s, toks[s + 1:s + 2])
        b.record(st)
        torch.cuda.synchronize()
        if dec.status():
            raise RuntimeError(f"device status {dec.status()}")
        return a.elapsed_time(b) * 1e3 / n


def _setup(ref: Reference, block: int):
    """Shape (cache sized for the timing window after the reference's steps), weights, Bench."""
    import amk_inputs as I
    import torch
    torch.cuda.set_device(0)
    base = I.SHAPES[ref.workload]
    steps = len(ref.inputs)
    # every timing block runs over the same positions [pos0 + steps, + block): the cache keeps
    # the workload's size unless that window does not fit (the cache size sets the default
    # attention split)
    max_ctx = max(base.max_ctx, ref.pos0 + steps + block + 1)
    shape = base.replace(max_ctx=max_ctx)
    w = I.make_weights(shape)
    return shape, w, Bench(shape, w, ref, max_ctx), max_ctx


def _median(x):
    x = sorted(x)
    return x[len(x) // 2]


def search(reference: Reference, budget: int, seed: int = 0, block: int = 50, rounds: int = 3,
           min_gain: float = 0.005, rank_pool: int = 16, params: Optional[CostParams] = None,
           log=print) -> dict:
    """Run the loop from the default schedule; returns {"incumbent": cfg, "trials": [...], ...}."""
    ref = reference
    rng = random.Random(seed)
    log(f"[search] {ref.workload}: weights, prefix to pos {ref.pos0}")
    shape, w, B, max_ctx = _setup(ref, block)
    pos0 = ref.pos0
    pos = pos0 + len(ref.inputs)

    inc_cfg: Config = {}
    ok, inc_sched = lower(shape, inc_cfg, max_ctx)
    if not ok:
        raise RuntimeError("the default schedule does not lower")
    inc_est = estimate_us(shape, inc_sched, pos0, params, ahead_groups(inc_cfg))
    inc = B.make(inc_cfg)
    ok, info = B.check(inc)
    if not ok:
        inc.close()
        raise RuntimeError(f"the default schedule fails the reference gate: {info}")
    log(f"[search] default schedule: {json.dumps(info)}")
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
            pool.append((estimate_us(shape, sc, pos0, params, ahead_groups(c)), c))
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
            ok_p, info = B.check(cand)
            rec["gate"] = info
            if not ok_p:
                rec["verdict"] = "failed the reference gate"
            else:
                ti, tc = [], []
                B.time_block(cand, block, pos)   # warm-up
                for _ in range(rounds):
                    ti.append(B.time_block(inc, block, pos))
                    tc.append(B.time_block(cand, block, pos))
                mi, mc = _median(ti), _median(tc)
                rec.update({"incumbent_us": round(mi, 2), "candidate_us": round(mc, 2)})
                if decide(mi, mc, min_gain):
                    rec["verdict"] = "kept"
                    inc.close()
                    inc, inc_cfg, inc_est, cand = cand, cfg, est, None
                else:
                    rec["verdict"] = "reverted"
        finally:
            if cand is not None:
                cand.close()
        trials.append(rec)
        log(f"[search] {it}: {json.dumps(rec)}")
    t_final = [B.time_block(inc, block, pos) for _ in range(rounds)]
    inc.close()
    return {"workload": ref.workload, "pos": pos0, "incumbent": inc_cfg, "incumbent_estimate_us": round(inc_est, 1),
            "incumbent_us": round(_median(t_final), 2), "trials": trials, "seed": seed}


# Configurations that spread the launch time: attention splits and groupings, the prefetch depth,
# coarser GEMV tilings, plain round-robin placement.
CALIBRATION_CONFIGS: List[Config] = [
    {}, {"prefetch_groups": -1}, {"prefetch_groups": 2},
    {"attn_chunks": 1}, {"attn_chunks": 4}, {"attn_chunks": 8}, {"attn_chunks": 32},
    {"attn_group_tasks": 2}, {"attn_chunks": 1, "attn_group_tasks": 2}, {"attn_chunks": 4, "attn_group_tasks": 2},
    {"tasks_qkv": 64}, {"tasks_o": 32}, {"tasks_gateup": 64}, {"tasks_down": 64}, {"tasks_lm": 64},
    {"tasks_qkv": 32, "tasks_gateup": 32, "tasks_down": 32, "tasks_o": 32},
    {"cu_assign": 1}, {"prefetch_groups": -1, "attn_chunks": 8},
    {"merge_fusion": 1}, {"merge_fusion": 1, "attn_chunks": 4},
]


def calibrate(reference: Reference, configs: Sequence[Config] = tuple(CALIBRATION_CONFIGS), block: int = 30,
              rounds: int = 3, log=print) -> dict:
    """Measure each configuration on the GPU, each gated against the reference first; returns
    the measurement record that `refit` reads."""
    ref = reference
    shape, w, B, max_ctx = _setup(ref, block)
    pos = ref.pos0 + len(ref.inputs)
    rows = []
    for cfg in configs:
        ok, sc = lower(shape, cfg, max_ctx)
        if not ok:
            rows.append({"cfg": cfg, "verdict": "rejected by lowering/validator"})
            continue
        dec = B.make(cfg)
        try:
            ok_g, info = B.check(dec)
            if not ok_g:
                rows.append({"cfg": cfg, "verdict": "failed the reference gate", "gate": info})
                continue
            B.time_block(dec, block, pos)   # warm-up
            ts = [B.time_block(dec, block, pos) for _ in range(rounds)]
        finally:
            dec.close()
        rows.append({"cfg": cfg, "verdict": "measured", "gate_max_err": info["max_err"],
                     "measured_us": round(_median(ts), 2), "spread_us": round(max(ts) - min(ts), 2)})
        log(f"[calibrate] {json.dumps(rows[-1])}")
    return {"workload": ref.workload, "pos": ref.pos0, "max_ctx": max_ctx, "block": block, "rounds": rounds,
            "configs": rows}


def refit(record: dict, params: Optional[CostParams] = None) -> dict:
    """Refit the cost model to a calibration record (CPU only) and report how well it ranks the
    measured configurations: Spearman's rho of estimate and measurement with the starting
    parameters, with parameters fitted to all points (in sample), and on the odd-numbered
    configurations with parameters fitted to the even-numbered ones (held out)."""
    import amk_inputs as I
    p0 = params or CostParams()
    shape = I.SHAPES[record["workload"]].replace(max_ctx=record["max_ctx"])
    pos = record["pos"]
    rows = [dict(r) for r in record["configs"] if r["verdict"] == "measured"]
    items = [(DepthPlan(shape, r["cfg"], record["max_ctx"], pos), ahead_groups(r["cfg"]), float(r["measured_us"]))
             for r in rows]

    def est(q, sel):
        return [_est(pl, q, ah) for pl, ah, _ in sel]

    meas = [m for _, _, m in items]
    p_all = fit_cost_params(items, p0)
    even, odd = items[0::2], items[1::2]
    p_even = fit_cost_params(even, p0)
    for r, e0, e1 in zip(rows, est(p0, items), est(p_all, items)):
        r["estimate_us"], r["fitted_estimate_us"] = round(e0, 1), round(e1, 1)
    return {"workload": record["workload"], "pos": pos, "n_measured": len(items), "configs": rows,
            "rho_start": spearman(est(p0, items), meas),
            "rho_fitted_in_sample": spearman(est(p_all, items), meas),
            "rho_held_out": spearman(est(p_even, odd), [m for _, _, m in odd]),
            "params_start": dataclasses.asdict(p0), "params_fitted": dataclasses.asdict(p_all)}


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--reference", default=None,
                    help="the CPU reference record (.npz: workload, pos0, inputs, gen, logits, margins)")
    ap.add_argument("--budget", type=int, default=12, help="candidates measured on the GPU")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--block", type=int, default=50, help="steps per timing block")
    ap.add_argument("--calibrate", action="store_true",
                    help="measure the calibration spread (GPU) and write the measurement record")
    ap.add_argument("--refit", default=None, metavar="RECORD",
                    help="refit the cost model to a measurement record (CPU only)")
    ap.add_argument("--out", default=None, help="write the result JSON here")
    args = ap.parse_args(argv)
    t0 = time.time()
    log = lambda m: print(m, file=sys.stderr, flush=True)
    if args.refit:
        with open(args.refit) as f:
            res = refit(json.loads(f.read()))
    else:
        if not args.reference:
            ap.error("--reference is required to measure on the GPU")
        ref = load_reference(args.reference)
        if args.calibrate:
            res = calibrate(ref, block=args.block, log=log)
        else:
            res = search(ref, args.budget, args.seed, args.block, log=log)
    res["wall_s"] = round(time.time() - t0, 1)
    s = json.dumps(res)
    if args.out:
        with open(args.out, "w") as f:
            f.write(s + "\n")
    print(s)
    return 0


if __name__ == "__main__":
    sys.exit(main())
