"""Hand-written schedules, one rejected case per validator rule and accepted look-alikes.

Each entry: (name, schedule, expected accepted, expected rule mask). Rule bits: V0 = 1 ... V8 = 256.
"""
from amk_inputs.schedules import ACC_POST, ACC_WRITE, REGION_LL, REGION_PLAIN, REGION_RO, Schedule, Task

W, R, P = ACC_WRITE, 0, ACC_POST


def _s(tasks, queues, n_counters=4, n_regions=2, kinds=None, inputs=(), outputs=(), ll=False):
    return Schedule(len(queues), n_counters, n_regions, tasks, queues,
                    list(kinds) if kinds else [REGION_PLAIN] * n_regions, list(inputs), list(outputs), ll)


def corpus():
    out = []

    def add(name, s, mask):
        out.append((name, s, mask == 0, mask))

    # producer a (queue 0) writes r0[0,1) and signals c0; consumer b (queue 1) waits and reads it
    def base(**kw):
        a = Task(signals=[0], accesses=[(0, W, 0, 1)])
        b = Task(waits=[(0, 1)], accesses=[(0, R, 0, 1), (1, W, 0, 1)])
        return _s([a, b], [[0], [1]], outputs=[(1, 0, 1)], **kw)

    add("base", base(), 0)
    s = base(); s.queues = [[0, 1], [1]]; add("V0 task in two queues", s, 1)
    s = base(); s.queues = [[0], []]; add("V0 task in no queue", s, 1)
    s = base(); s.tasks[1].waits = [(9, 1)]; add("V0 counter out of range", s, 1)
    s = base(); s.tasks[0].accesses = [(0, W, 3, 3)]; add("V0 empty range", s, 1)
    s = base(); s.tasks[0].signals = [0, 0]; add("V0 duplicate signal", s, 1)
    s = base(kinds=[REGION_RO, REGION_PLAIN]); add("V0 write to read-only region", s, 1)
    s = base(kinds=[REGION_LL, REGION_PLAIN], inputs=[(0, 4, 5)]); add("V0 declared input on flag region", s, 1)
    s = base(); s.tasks[1].waits = [(0, 0)]; add("V1 threshold zero", s, 2)
    s = base(); s.tasks[1].waits = [(0, 2)]; add("V1 threshold above producers", s, 2)
    s = base(); s.tasks[1].waits = [(0, 1), (3, 1)]; add("V1 wait on a counter nobody signals", s, 2)

    # two producers of c0
    a1 = Task(signals=[0], accesses=[(0, W, 0, 1)])
    a2 = Task(signals=[0], accesses=[(0, W, 1, 2)])
    b = Task(waits=[(0, 2)], accesses=[(0, R, 0, 2)])
    add("full wait on two producers", _s([a1, a2, b], [[0], [1], [2]]), 0)
    b = Task(waits=[(0, 1)], accesses=[(0, R, 0, 2)])
    # a partial wait: the union graph still holds edges from both producers, so only V2 fires
    add("V2 partial wait", _s([a1, a2, b], [[0], [1], [2]]), 4)
    b = Task(waits=[(0, 1)])
    add("V2 partial wait, no data", _s([Task(signals=[0]), Task(signals=[0]), b], [[0], [1], [2]]), 4)

    add("V3 self wait", _s([Task(signals=[0], waits=[(0, 1)])], [[0]]), 8)
    x = Task(signals=[0], waits=[(1, 1)])
    y = Task(signals=[1], waits=[(0, 1)])
    add("V3 two-task cycle", _s([x, y], [[0], [1]]), 8)
    # queue order contradicts the counter DAG: q0 = [b, a] while b waits on a
    a = Task(signals=[0])
    b = Task(waits=[(0, 1)])
    add("V4 queue against the DAG", _s([a, b], [[1, 0]]), 16)
    add("queue along the DAG", _s([a, b], [[0, 1]]), 0)
    # the cross-queue cycle: A = [a1, a2], B = [b1, b2], a2 -> b1 and b2 -> a1. Each counter
    # edge alone is acyclic and each queue pair is unordered by the counter edges, yet the
    # queues deadlock.
    a1 = Task(waits=[(1, 1)]); a2 = Task(signals=[0]); b1 = Task(waits=[(0, 1)]); b2 = Task(signals=[1])
    add("V4 cross-queue cycle", _s([a1, a2, b1, b2], [[0, 1], [2, 3]]), 16)

    add("V5 unordered writes",
        _s([Task(accesses=[(0, W, 0, 4)]), Task(accesses=[(0, W, 3, 8)])], [[0], [1]]), 32)
    add("V5 unordered write and read",
        _s([Task(accesses=[(0, W, 0, 4)]), Task(accesses=[(0, R, 2, 3)])], [[0], [1]], inputs=[(0, 0, 4)]), 32)
    add("same queue orders writes",
        _s([Task(accesses=[(0, W, 0, 4)]), Task(accesses=[(0, W, 3, 8)])], [[0, 1]]), 0)
    s = base(); s.tasks[0].accesses = [(0, W | P, 0, 1)]
    add("V5 write after the signal is not released", s, 32 | 128)
    s = base(); s.tasks[1].accesses = [(0, R | P, 0, 1), (1, W, 0, 1)]
    add("read after the consumer's own signals is still ordered", s, 0)

    s = base(); s.outputs = [(1, 0, 2)]; add("V6 output not covered", s, 64)
    s = base(); s.tasks[1].accesses = [(0, R, 0, 2), (1, W, 0, 1)]
    add("V7 read beyond what was written", s, 128)
    s = base(inputs=[(0, 1, 2)]); s.tasks[1].accesses = [(0, R, 0, 2), (1, W, 0, 1)]
    add("read covered by writes and inputs", s, 0)
    # write-after-read is fine on plain memory when ordered
    rd = Task(signals=[0], accesses=[(0, R, 0, 1)])
    wr = Task(waits=[(0, 1)], accesses=[(0, W, 0, 1)])
    add("ordered write after read", _s([rd, wr], [[0], [1]], inputs=[(0, 0, 1)]), 0)

    # flag protocol: region 0 carries flags
    def llbase():
        a = Task(signals=[0], accesses=[(0, W, 0, 2)])
        b = Task(waits=[(0, 1)], accesses=[(0, R, 0, 2), (1, W, 0, 1)])
        return _s([a, b], [[0], [1]], kinds=[REGION_LL, REGION_PLAIN], outputs=[(1, 0, 1)], ll=True)

    add("flag protocol base", llbase(), 0)
    s = llbase(); s.tasks[1].accesses = [(0, R, 5, 6), (1, W, 0, 1)]
    add("V8 wait not observable in the data", s, 128 | 256)
    s = llbase(); s.tasks.append(Task(accesses=[(0, W, 1, 2)])); s.queues[0].insert(0, 2)
    add("V5 flag region written twice, even in queue order", s, 32)
    s = llbase(); s.tasks[1].waits = []
    add("V7 flag read without ordering", s, 32 | 128)
    s = llbase(); s.tasks[0].accesses = [(0, W | P, 0, 2)]
    add("V0 post write on flag region", s, 1)
    return out
