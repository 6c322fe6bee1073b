"""Brute-force interleaving enumeration of a small schedule. TEST INFRASTRUCTURE.

This is the independent judge of safety for the validator's property tests: it explores every
interleaving the counter protocol allows and reports whether any can deadlock or race. Safety
here is exactly what the AutoMegaKernel pages promise a validated schedule has (page 1, tweet
and "Deadlock-free by construction"; page 4, "De Safety Gate"): no reachable state where the
GPU would wait forever, and no two conflicting memory accesses in flight at once.

Model: every queue runs its tasks in order. A task is waiting until all of its waits hold
(counter value >= threshold), then runs its pre part (pre accesses in flight), then emits its
signals (+1 per signalled counter), then runs its post part (post accesses in flight), then the
queue moves on. A state is final when every queue is exhausted.

  deadlock: a reachable non-final state with no enabled step;
  race:     a reachable state where two different tasks have conflicting accesses in flight
            (same region, overlapping ranges, at least one write).

Schedules that fail the validator's integrity rule (a task missing from every queue or listed
twice, out-of-range ids) are reported unsafe as malformed.
"""
from __future__ import annotations

from amk_inputs.schedules import ACC_POST, ACC_WRITE, Schedule

WAIT, PRE, POST = 0, 1, 2


def _conflict(a, b):
    r, f, lo, hi = a
    r2, f2, lo2, hi2 = b
    return r == r2 and lo < hi2 and lo2 < hi and bool((f | f2) & ACC_WRITE)


def explore(s: Schedule, max_states: int = 200000):
    """-> dict(safe, deadlock, race, malformed, states)."""
    n = len(s.tasks)
    seen = [0] * n
    for q in s.queues:
        for t in q:
            if not (0 <= t < n):
                return dict(safe=False, deadlock=False, race=False, malformed=True, states=0)
            seen[t] += 1
    for t in s.tasks:
        if any(not (0 <= c < s.n_counters) for c, _ in t.waits) or any(not (0 <= c < s.n_counters) for c in t.signals):
            return dict(safe=False, deadlock=False, race=False, malformed=True, states=0)
    if any(c != 1 for c in seen):
        return dict(safe=False, deadlock=False, race=False, malformed=True, states=0)

    pre_acc = [[a for a in t.accesses if not a[1] & ACC_POST] for t in s.tasks]
    post_acc = [[a for a in t.accesses if a[1] & ACC_POST] for t in s.tasks]
    Q = s.queues
    start = tuple((0, WAIT) for _ in Q)
    stack = [start]
    visited = {start}
    deadlock = race = False

    def counters(state):
        cnt = [0] * s.n_counters
        for qi, (pc, ph) in enumerate(state):
            for k in range(pc + (1 if ph == POST else 0)):
                for c in s.tasks[Q[qi][k]].signals:
                    cnt[c] += 1
        return cnt

    while stack:
        st = stack.pop()
        # race check on this state
        inflight = []
        for qi, (pc, ph) in enumerate(st):
            if pc < len(Q[qi]) and ph in (PRE, POST):
                t = Q[qi][pc]
                inflight.append((t, pre_acc[t] if ph == PRE else post_acc[t]))
        for x in range(len(inflight)):
            for y in range(x + 1, len(inflight)):
                tx, ax = inflight[x]
                ty, ay = inflight[y]
                if tx != ty and any(_conflict(a, b) for a in ax for b in ay):
                    race = True
        cnt = counters(st)
        succ = []
        for qi, (pc, ph) in enumerate(st):
            if pc >= len(Q[qi]):
                continue
            t = s.tasks[Q[qi][pc]]
            if ph == WAIT:
                if all(cnt[c] >= th for c, th in t.waits):
                    succ.append(qi)
            else:
                succ.append(qi)
        final = all(pc >= len(Q[qi]) for qi, (pc, _) in enumerate(st))
        if not final and not succ:
            deadlock = True
        for qi in succ:
            pc, ph = st[qi]
            nxt = (pc, PRE) if ph == WAIT else (pc, POST) if ph == PRE else (pc + 1, WAIT)
            ns = st[:qi] + (nxt,) + st[qi + 1:]
            if ns not in visited:
                visited.add(ns)
                if len(visited) > max_states:
                    raise RuntimeError("state space too large")
                stack.append(ns)
    return dict(safe=not (deadlock or race), deadlock=deadlock, race=race, malformed=False, states=len(visited))
