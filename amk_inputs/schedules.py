"""Schedule containers and seeded random schedules.

A schedule is the static task DAG the megakernel walks: per-CU queues of tasks, monotone
counters that tasks signal (+1 each) and wait on (value >= threshold), and the memory each
task touches, so that a validator can decide deadlock and race freedom before launch (the
AutoMegaKernel pages, page 2, "Statically verified schedule IR", and page 4, "Methodologie":
thresholds within [1, producers], an acyclic producer/consumer graph, per-SM queues that are
linear extensions, full waits on multi-producer counters, writers of a read that precede it).

This module only holds the data and draws random schedules; it implements none of the
validation rules.

Access flags: bit 0 = write, bit 1 = performed after the task's signals ("post" accesses).
Region kinds: 0 = plain memory, 1 = flag-carrying (each element written once per launch, the
reader detects the write from the data itself), 2 = read-only during a launch.
"""
from __future__ import annotations

import dataclasses
import random
from typing import List, Tuple

ACC_WRITE, ACC_POST = 1, 2
REGION_PLAIN, REGION_LL, REGION_RO = 0, 1, 2


@dataclasses.dataclass
class Task:
    waits: List[Tuple[int, int]] = dataclasses.field(default_factory=list)      # (counter, threshold)
    signals: List[int] = dataclasses.field(default_factory=list)                # counters (+1 each)
    accesses: List[Tuple[int, int, int, int]] = dataclasses.field(default_factory=list)  # (region, flags, lo, hi)
    opcode: int = 0
    args: Tuple[int, ...] = (0, 0, 0, 0, 0)


@dataclasses.dataclass
class Schedule:
    n_queues: int
    n_counters: int
    n_regions: int
    tasks: List[Task]
    queues: List[List[int]]
    region_kind: List[int] = None
    inputs: List[Tuple[int, int, int]] = dataclasses.field(default_factory=list)   # (region, lo, hi)
    outputs: List[Tuple[int, int, int]] = dataclasses.field(default_factory=list)
    ll_protocol: bool = False

    def __post_init__(self):
        if self.region_kind is None:
            self.region_kind = [REGION_PLAIN] * self.n_regions

    def copy(self) -> "Schedule":
        return Schedule(self.n_queues, self.n_counters, self.n_regions,
                        [Task(list(t.waits), list(t.signals), list(t.accesses), t.opcode, tuple(t.args))
                         for t in self.tasks],
                        [list(q) for q in self.queues], list(self.region_kind), list(self.inputs),
                        list(self.outputs), self.ll_protocol)


# ---------------------------------------------------------------- random schedules

SPAN = 16   # region element range [0, SPAN)


def _valid_schedule(rng: random.Random, ll: bool = False) -> Schedule:
    """Valid by construction: tasks 0..n-1 are in a topological order; every queue lists its
    tasks in that order; every wait is a full wait on a counter whose producers all come
    earlier; every read is of a declared input or of a range written by a producer of a
    counter the reader waits on; every task writes its own range."""
    n = rng.randint(2, 12)
    nq = rng.randint(1, 4)
    nr = rng.randint(1, 4)
    nc = rng.randint(1, 6)
    tasks = [Task() for _ in range(n)]
    # counters: producers are a random set of tasks below a cut, consumers above it
    prods = {}
    for c in range(nc):
        if n < 2:
            break
        hi = rng.randint(1, n - 1)
        k = rng.randint(1, min(3, hi))
        ps = sorted(rng.sample(range(hi), k))
        prods[c] = ps
        for p in ps:
            tasks[p].signals.append(c)
    # each task writes one range of its own: region r, element [slot, slot+1)
    # (with the flag protocol every producer writes into region 0, the flag-carrying one)
    slots = {}
    for i, t in enumerate(tasks):
        if rng.random() < 0.8 or (ll and t.signals):
            r = 0 if (ll and t.signals) else rng.randrange(nr)
            lo = i if i < SPAN else SPAN - 1
            if (r, lo) in slots:
                continue
            slots[(r, lo)] = i
            t.accesses.append((r, ACC_WRITE, lo, lo + 1))
    written_by = {}
    for (r, lo), i in slots.items():
        written_by.setdefault(i, []).append((r, lo))
    inputs = []
    for r in range(nr):
        lo = SPAN + 0
        inputs.append((r, SPAN, SPAN + 4))
    for i, t in enumerate(tasks):
        cands = [c for c, ps in prods.items() if ps and max(ps) < i]
        waits = rng.sample(cands, min(len(cands), rng.randint(0, 2)))
        for c in waits:
            t.waits.append((c, len(prods[c])))
            if ll:   # observe every producer's flag-carrying write
                for p in prods[c]:
                    for (r, lo) in written_by.get(p, []):
                        if r == 0:
                            t.accesses.append((0, 0, lo, lo + 1))
        # reads: of something a waited producer wrote, or of an input
        n_reads = rng.randint(0, 2)
        for _ in range(n_reads):
            srcs = [(r, lo) for c in waits for p in prods[c] for (r, lo) in written_by.get(p, [])]
            if srcs and rng.random() < 0.7:
                r, lo = rng.choice(srcs)
                t.accesses.append((r, 0, lo, lo + 1))
            else:
                r = rng.randrange(1, nr) if (ll and nr > 1) else (rng.randrange(nr) if not ll else None)
                if r is None:
                    continue
                a = rng.randint(SPAN, SPAN + 3)
                t.accesses.append((r, 0, a, a + 1))
    queues = [[] for _ in range(nq)]
    for i in range(n):
        queues[rng.randrange(nq)].append(i)
    outputs = []
    plain_slots = sorted(k for k in slots.items() if not (ll and k[0][0] == 0))
    if plain_slots and rng.random() < 0.6:
        (r, lo), _ = rng.choice(plain_slots)
        outputs.append((r, lo, lo + 1))
    kinds = [REGION_PLAIN] * nr
    if ll:
        kinds[0] = REGION_LL
        inputs = [x for x in inputs if x[0] != 0]
    return Schedule(nq, nc, nr, tasks, queues, kinds, inputs, outputs, ll_protocol=ll)


def _mutate(s: Schedule, rng: random.Random) -> None:
    kind = rng.randrange(13)
    ts = s.tasks
    all_waits = [(i, j) for i, t in enumerate(ts) for j in range(len(t.waits))]
    if kind == 0 and all_waits:                                   # lower a threshold
        i, j = rng.choice(all_waits)
        c, t = ts[i].waits[j]
        ts[i].waits[j] = (c, max(0, t - rng.randint(1, 2)))
    elif kind == 1 and all_waits:                                 # raise a threshold
        i, j = rng.choice(all_waits)
        c, t = ts[i].waits[j]
        ts[i].waits[j] = (c, t + rng.randint(1, 2))
    elif kind == 2 and all_waits:                                 # threshold 0
        i, j = rng.choice(all_waits)
        ts[i].waits[j] = (ts[i].waits[j][0], 0)
    elif kind == 3:                                               # swap two entries of a queue
        q = rng.choice(s.queues)
        if len(q) >= 2:
            a, b = rng.sample(range(len(q)), 2)
            q[a], q[b] = q[b], q[a]
    elif kind == 4 and len(s.queues) > 1:                         # move an entry to another queue
        src = rng.choice([q for q in s.queues if q] or [s.queues[0]])
        if src:
            x = src.pop(rng.randrange(len(src)))
            dst = rng.choice(s.queues)
            dst.insert(rng.randint(0, len(dst)), x)
    elif kind == 5 and all_waits:                                 # drop a wait
        i, j = rng.choice(all_waits)
        del ts[i].waits[j]
    elif kind == 6:                                               # back-edge: an early task waits on a late signal
        sig = [(i, c) for i, t in enumerate(ts) for c in t.signals]
        if sig:
            i, c = rng.choice(sig)
            victim = rng.randrange(0, i + 1)
            p = sum(1 for t in ts if c in t.signals)
            ts[victim].waits.append((c, p))
    elif kind == 7:                                               # alias a write onto another task's range
        ws = [(i, a) for i, t in enumerate(ts) for a in t.accesses if a[1] & ACC_WRITE]
        if len(ws) >= 2:
            (i, a), (k, b) = rng.sample(ws, 2)
            ts[i].accesses.append((b[0], ACC_WRITE, b[2], b[3]))
    elif kind == 8:                                               # duplicate a task id in a queue
        q = rng.choice(s.queues)
        if q:
            q.insert(rng.randint(0, len(q)), rng.choice(q))
    elif kind == 9:                                               # drop a task from its queue
        q = rng.choice(s.queues)
        if q:
            q.pop(rng.randrange(len(q)))
    elif kind == 10:                                              # drop a write
        ws = [(i, j) for i, t in enumerate(ts) for j, a in enumerate(t.accesses) if a[1] & ACC_WRITE]
        if ws:
            i, j = rng.choice(ws)
            del ts[i].accesses[j]
    elif kind == 11:                                              # read an element nobody writes
        i = rng.randrange(len(ts))
        r = rng.randrange(s.n_regions)
        if s.region_kind[r] == REGION_PLAIN:
            ts[i].accesses.append((r, 0, SPAN + 8, SPAN + 9))
    else:                                                         # move an access after the signals
        ax = [(i, j) for i, t in enumerate(ts) for j, a in enumerate(t.accesses)]
        if ax:
            i, j = rng.choice(ax)
            r, f, lo, hi = ts[i].accesses[j]
            ts[i].accesses[j] = (r, f | ACC_POST, lo, hi)


def random_schedule(seed: int) -> Schedule:
    """A small schedule (<= 12 tasks, <= 4 queues, <= 6 counters, <= 4 regions): valid by
    construction, then mutated 1-3 times with probability 0.8. Every fourth seed uses the
    flag protocol (region 0 flag-carrying, waiters read every producer's flag-carrying write)."""
    rng = random.Random(seed * 7919 + 17)
    s = _valid_schedule(rng, ll=(seed % 4 == 3))
    if rng.random() < 0.8:
        for _ in range(rng.randint(1, 3)):
            _mutate(s, rng)
    return s


def corpus(n: int = 200, first_seed: int = 0) -> List[Schedule]:
    return [random_schedule(first_seed + i) for i in range(n)]
