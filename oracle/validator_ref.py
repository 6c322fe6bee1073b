"""Reference schedule validator (plain Python, small schedules). TEST INFRASTRUCTURE.

It decides the same verdict (accepted, rule mask) as the library's validator, from the same
rules, with none of its code: explicit reachability sets instead of vector clocks, and
brute-force interval coverage instead of sweeps.

The checks follow the AutoMegaKernel pages (page 2, "Statically verified schedule IR" and its
Table 1; page 4, "Methodologie", the safety gate): wait thresholds within [1, #producers];
an acyclic producer/consumer graph; per-SM queues that are linear extensions of the DAG; full
waits on multi-producer counters; every writer of a read is a predecessor; happens-before
respected by memory accesses; output reachability and referential integrity. The reading of
each rule (precise form, gating) is:

  V0 integrity   ids in range, every task in exactly one queue exactly once, lo < hi, no
                 duplicate signal, no write to a read-only region, no declared input/output
                 or post access on a flag-carrying region. If V0 fails nothing else is checked.
  V1             a wait threshold outside [1, P(c)], P(c) = number of tasks signalling c.
  V2             a partial wait (1 <= t < P(c)) on a counter with P(c) > 1.
  V3             the producer->waiter graph has a cycle (a self-wait included).
  V4             the union graph U (producer->waiter edges plus queue order) has a cycle while
                 the producer->waiter graph has none: a queue is not a linear extension.
  V5             (only without V3/V4) two accesses of different tasks to overlapping ranges of
                 one region, at least one a write, unordered by happens-before; on a
                 flag-carrying region any two overlapping writes.
  V6             a declared output not covered by writes.
  V7             (only without V3/V4) a read not covered by declared inputs and by writes that
                 happen before it; on a flag-carrying region a write overlapping a read that
                 does not happen before it.
  V8             (flag-protocol schedules only) a task waits on a counter one of whose
                 producers writes nothing the task reads from a flag-carrying region, so the
                 wait could not be observed through the data.

Happens-before is reachability in U where each task is split in two nodes, pre -> post; a
task's signals leave from pre, its waits enter pre, queue order goes from post to the next
task's pre; accesses flagged post sit on the post node.
"""
from __future__ import annotations

from amk_inputs.schedules import ACC_POST, ACC_WRITE, REGION_LL, REGION_RO, Schedule

V = {f"V{i}": 1 << i for i in range(9)}


def _covered(lo, hi, intervals):
    """Is [lo, hi) inside the union of the intervals? (element by element; small spans)."""
    for x in range(lo, hi):
        if not any(a <= x < b for a, b in intervals):
            return False
    return True


def _has_cycle(n, succ):
    color = [0] * n
    for s in range(n):
        if color[s]:
            continue
        stack = [(s, iter(succ[s]))]
        color[s] = 1
        while stack:
            u, it = stack[-1]
            nxt = next(it, None)
            if nxt is None:
                color[u] = 2
                stack.pop()
            elif color[nxt] == 1:
                return True
            elif color[nxt] == 0:
                color[nxt] = 1
                stack.append((nxt, iter(succ[nxt])))
    return False


def validate(s: Schedule):
    """-> (accepted, rule_mask)."""
    n = len(s.tasks)
    mask = 0
    # ---- V0
    seen = [0] * n
    bad = False
    for q in s.queues:
        for t in q:
            if not (0 <= t < n):
                bad = True
            else:
                seen[t] += 1
    if len(s.queues) != s.n_queues or any(c != 1 for c in seen):
        bad = True
    if len(s.region_kind) != s.n_regions or any(k not in (0, 1, 2) for k in s.region_kind):
        bad = True
    for t in s.tasks:
        for c, _ in t.waits:
            if not (0 <= c < s.n_counters):
                bad = True
        if len(set(t.signals)) != len(t.signals) or any(not (0 <= c < s.n_counters) for c in t.signals):
            bad = True
        for r, f, lo, hi in t.accesses:
            if not (0 <= r < s.n_regions) or not lo < hi or f & ~3:
                bad = True
            elif s.region_kind[r] == REGION_RO and f & ACC_WRITE:
                bad = True
            elif s.region_kind[r] == REGION_LL and f & ACC_POST:
                bad = True
    for r, lo, hi in list(s.inputs) + list(s.outputs):
        if not (0 <= r < s.n_regions) or not lo < hi or s.region_kind[r] == REGION_LL:
            bad = True
    if bad:
        return False, V["V0"]

    prod = {c: [] for c in range(s.n_counters)}
    for i, t in enumerate(s.tasks):
        for c in t.signals:
            prod[c].append(i)
    # ---- V1, V2
    for t in s.tasks:
        for c, th in t.waits:
            P = len(prod[c])
            if th < 1 or th > P:
                mask |= V["V1"]
            if P > 1 and 1 <= th < P:
                mask |= V["V2"]
    # ---- V3: producer -> waiter graph over tasks
    csucc = [set() for _ in range(n)]
    for b, t in enumerate(s.tasks):
        for c, _ in t.waits:
            for a in prod[c]:
                csucc[a].add(b)
    v3 = _has_cycle(n, [list(x) for x in csucc])
    # ---- V4: union graph with split nodes pre(i) = 2i, post(i) = 2i + 1
    usucc = [set() for _ in range(2 * n)]
    for i in range(n):
        usucc[2 * i].add(2 * i + 1)
    for q in s.queues:
        for a, b in zip(q, q[1:]):
            usucc[2 * a + 1].add(2 * b)
    for a in range(n):
        for b in csucc[a]:
            usucc[2 * a].add(2 * b)
    ucyc = _has_cycle(2 * n, [list(x) for x in usucc])
    if v3:
        mask |= V["V3"]
    if ucyc and not v3:
        mask |= V["V4"]
    acyclic = not v3 and not ucyc

    def node(i, flags):
        return 2 * i + (1 if flags & ACC_POST else 0)

    reach = None
    if acyclic:
        reach = []
        for x in range(2 * n):
            vis, st = set(), [x]
            while st:
                u = st.pop()
                for v in usucc[u]:
                    if v not in vis:
                        vis.add(v)
                        st.append(v)
            reach.append(vis)

    def hb(x, y):
        return y in reach[x]

    acc = [(i, r, f, lo, hi) for i, t in enumerate(s.tasks) for (r, f, lo, hi) in t.accesses]
    # ---- V5
    if acyclic:
        for k1 in range(len(acc)):
            i, r, f, lo, hi = acc[k1]
            for k2 in range(k1 + 1, len(acc)):
                j, r2, f2, lo2, hi2 = acc[k2]
                if i == j or r != r2 or not (lo < hi2 and lo2 < hi):
                    continue
                if not ((f | f2) & ACC_WRITE):
                    continue
                if s.region_kind[r] == REGION_LL and (f & ACC_WRITE) and (f2 & ACC_WRITE):
                    mask |= V["V5"]
                    continue
                x, y = node(i, f), node(j, f2)
                if not hb(x, y) and not hb(y, x):
                    mask |= V["V5"]
    # ---- V6
    for r, lo, hi in s.outputs:
        ws = [(a, b) for (_, rr, f, a, b) in acc if rr == r and f & ACC_WRITE]
        if not _covered(lo, hi, ws):
            mask |= V["V6"]
    # ---- V7
    if acyclic:
        for (j, r, f, lo, hi) in acc:
            if f & ACC_WRITE:
                continue
            y = node(j, f)
            before = []
            for (i, r2, f2, lo2, hi2) in acc:
                if i == j or r2 != r or not (f2 & ACC_WRITE):
                    continue
                if hb(node(i, f2), y):
                    before.append((lo2, hi2))
                elif s.region_kind[r] == REGION_LL and lo2 < hi and lo < hi2:
                    mask |= V["V7"]
            ins = [(a, b) for (rr, a, b) in s.inputs if rr == r]
            if not _covered(lo, hi, before + ins):
                mask |= V["V7"]
    # ---- V8
    if s.ll_protocol:
        for b, t in enumerate(s.tasks):
            reads = [(r, lo, hi) for (r, f, lo, hi) in t.accesses
                     if not f & ACC_WRITE and s.region_kind[r] == REGION_LL]
            for c, _ in t.waits:
                for a in prod[c]:
                    if a == b:
                        continue
                    writes = [(r, lo, hi) for (r, f, lo, hi) in s.tasks[a].accesses
                              if f & ACC_WRITE and s.region_kind[r] == REGION_LL]
                    if not any(r1 == r2 and l1 < h2 and l2 < h1 for (r1, l1, h1) in writes for (r2, l2, h2) in reads):
                        mask |= V["V8"]
    return mask == 0, mask
