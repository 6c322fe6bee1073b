"""The CPU executor of schedules (amk_vm_run): the counter protocol on host threads with a
happens-before race detector and an exact deadlock check, no device.

Pinned against the brute-force interleaver (every interleaving of a small schedule) and the
validator: a problem the executor reports must be reachable; deadlocks must match exactly
(counters only grow, so a wait once satisfied stays satisfied and whether a schedule deadlocks
does not depend on the interleaving); accepted schedules, and the built-in lowering of every
workload, must run clean."""
import random

import pytest

import amk_inputs as I
from amk_inputs import schedules as S
from oracle import interleave as IL

import schedule_corpus


@pytest.fixture(scope="module")
def M():
    import persistent_megakernel_amd as M
    M.lib()
    return M


def _clean(r):
    return (r["completed"] and not r["deadlocked"] and not r["races"] and not r["uncovered_reads"]
            and not r["unwritten_outputs"] and not r["ll_rewrites"] and r["task"] == -1)


def _runs(M, s, n=3, delay=5):
    return [M.amk_vm_run(s, seed=k, max_delay_us=delay, watchdog_ms=5000) for k in range(n)]


def test_valid_by_construction_schedules_run_clean(M):
    for seed in range(150):
        s = S._valid_schedule(random.Random(seed), ll=bool(seed % 2))
        for r in _runs(M, s):
            assert _clean(r), (seed, r)


def test_random_corpus_agrees_with_the_interleaver(M):
    """Deadlock: equal to the interleaver's. Races: never one the interleaver cannot reach, and
    most reachable ones are found in three jittered runs. Accepted schedules run clean."""
    n_race = n_found = 0
    for seed in range(1200):
        s = S.random_schedule(seed)
        v = M.amk_validate(s)
        if v.rule_mask & 1:          # structurally broken: the executor refuses it (see below)
            continue
        il = IL.explore(s)
        rs = _runs(M, s)
        for r in rs:
            assert r["completed"] != r["deadlocked"], (seed, r)
            assert bool(r["deadlocked"]) == il["deadlock"], (seed, r, il)
            assert not (r["races"] and not il["race"]), (seed, r, il)
            if v.accepted:
                assert _clean(r), (seed, r)
        if il["race"] and not il["deadlock"]:
            n_race += 1
            n_found += any(r["races"] for r in rs)
    assert n_race >= 30
    assert n_found >= 0.85 * n_race, (n_found, n_race)


def test_rejections_have_a_dynamic_symptom(M):
    """Rules whose violation the executor can observe on its own: a cycle (V3/V4) deadlocks, an
    uncovered output (V6) is reported after a complete run, an unordered conflict (V5) is a race
    or, on a flag-carrying region, a second write in the launch."""
    seen = set()
    for seed in range(600):
        s = S.random_schedule(seed)
        m = M.amk_validate(s).rule_mask
        if m & 0b111:                 # V0-V2 change what the waits mean; skip those
            continue
        r = M.amk_vm_run(s, seed=seed, max_delay_us=5, watchdog_ms=5000)
        if m & 0b11000:
            assert r["deadlocked"] and r["task"] >= 0, (seed, hex(m), r)
            seen.add("cycle")
            continue
        if m & (1 << 5):
            assert r["races"] or r["ll_rewrites"], (seed, hex(m), r)
            seen.add("V5")
        if m & (1 << 6):
            assert r["unwritten_outputs"], (seed, hex(m), r)
            seen.add("V6")
        if m & (1 << 7):
            # (the validator also counts a flag-carrying element written twice here)
            assert r["uncovered_reads"] or r["races"] or r["ll_rewrites"], (seed, hex(m), r)
            seen.add("V7")
    assert seen == {"cycle", "V5", "V6", "V7"}


@pytest.mark.parametrize("name,sched,acc,mask", schedule_corpus.corpus(), ids=lambda x: x if isinstance(x, str) else "")
def test_hand_corpus(M, name, sched, acc, mask):
    il = IL.explore(sched)
    structural = il["malformed"] or any(a[2] >= a[3] or not 0 <= a[0] < sched.n_regions
                                        for t in sched.tasks for a in t.accesses)
    if structural:                      # the executor refuses what it cannot run
        assert mask & 1
        with pytest.raises(M.AmkError):
            M.amk_vm_run(sched)
        return
    for r in _runs(M, sched, n=2):
        assert bool(r["deadlocked"]) == il["deadlock"], (name, r, il)
        assert not (r["races"] and not il["race"]), (name, r, il)
        if acc:
            assert _clean(r), (name, r)


def test_self_wait_deadlocks_and_names_the_task(M):
    a = S.Task(signals=[0], accesses=[(0, S.ACC_WRITE, 0, 1)])
    b = S.Task(waits=[(1, 1)], signals=[1])                       # waits on its own signal
    c = S.Task(waits=[(0, 1)], accesses=[(0, 0, 0, 1)])
    s = S.Schedule(2, 2, 1, [a, b, c], [[0, 1], [2]])
    r = M.amk_vm_run(s, watchdog_ms=5000)
    assert r["deadlocked"] and not r["completed"] and r["task"] == 1


def test_threshold_above_producers_deadlocks(M):
    a = S.Task(signals=[0], accesses=[(0, S.ACC_WRITE, 0, 1)])
    b = S.Task(waits=[(0, 2)], accesses=[(0, 0, 0, 1)])
    r = M.amk_vm_run(S.Schedule(2, 1, 1, [a, b], [[0], [1]]), watchdog_ms=5000)
    assert r["deadlocked"] and r["task"] == 1


def test_post_access_races_with_the_waiter(M):
    # the producer writes after its signal: the waiter's read is not ordered after that write
    a = S.Task(signals=[0], accesses=[(0, S.ACC_WRITE | S.ACC_POST, 0, 1)])
    b = S.Task(waits=[(0, 1)], accesses=[(0, 0, 0, 1)])
    s = S.Schedule(2, 1, 1, [a, b], [[0], [1]])
    # whichever runs first, the pair is unordered (a read first is also a read of nothing yet)
    assert all(r["races"] == 1 and r["task"] in (0, 1) for r in _runs(M, s, n=4))
    # the same write before the signal is ordered
    s.tasks[0].accesses = [(0, S.ACC_WRITE, 0, 1)]
    assert all(_clean(r) for r in _runs(M, s, n=4))


def test_flag_region_written_twice_is_reported_even_when_ordered(M):
    a = S.Task(signals=[0], accesses=[(0, S.ACC_WRITE, 0, 1)])
    b = S.Task(waits=[(0, 1)], signals=[1], accesses=[(0, 0, 0, 1), (0, S.ACC_WRITE, 0, 1)])
    s = S.Schedule(2, 2, 1, [a, b], [[0], [1]], region_kind=[S.REGION_LL])
    r = M.amk_vm_run(s, watchdog_ms=5000)
    assert r["completed"] and not r["races"] and r["ll_rewrites"] == 1 and (r["task"], r["other"]) == (1, 0)
    s.region_kind = [S.REGION_PLAIN]
    assert _clean(M.amk_vm_run(s, watchdog_ms=5000))


def test_shadow_budget_leaves_regions_unchecked(M):
    a = S.Task(signals=[0], accesses=[(0, S.ACC_WRITE, 0, 100)])
    b = S.Task(waits=[(0, 1)], accesses=[(0, 0, 0, 100), (1, S.ACC_WRITE, 0, 10)])
    s = S.Schedule(2, 1, 2, [a, b], [[0], [1]])
    r = M.amk_vm_run(s, max_elements=50, watchdog_ms=5000)   # region 0 does not fit, region 1 does
    assert r["completed"] and r["unchecked"] == 200 and not r["races"]


def test_malformed_schedules_are_refused(M):
    a = S.Task(signals=[0])
    for s in (S.Schedule(2, 1, 1, [a], [[0], [0]]),          # a task in two queues
              S.Schedule(1, 1, 1, [a, S.Task()], [[0]]),      # a task in none
              S.Schedule(1, 1, 1, [S.Task(waits=[(3, 1)])], [[0]]),
              S.Schedule(1, 1, 1, [S.Task(accesses=[(0, 0, 2, 2)])], [[0]])):
        with pytest.raises(M.AmkError):
            M.amk_vm_run(s)


@pytest.mark.parametrize("name,n_cu", [("tiny_fp32", 16), ("tiny_fp32", 256), ("tinyllama_int8", 64)])
def test_builtin_lowering_runs_clean(M, name, n_cu):
    sc = M.amk_lower(M.model_desc(I.SHAPES[name]), M.schedule_config(n_cu=n_cu))
    r = M.amk_vm_run(sc, seed=3, max_delay_us=0, watchdog_ms=20000)
    assert _clean(r), r
    assert r["unchecked"] == 0


@pytest.mark.slow
@pytest.mark.parametrize("name", ["smollm2_135m_bf16", "tinyllama_int8", "llama7b_int8"])
def test_builtin_lowering_runs_clean_on_256_queues(M, name):
    sc = M.amk_lower(M.model_desc(I.SHAPES[name]), M.schedule_config(n_cu=256))
    assert _clean(M.amk_vm_run(sc, seed=5, watchdog_ms=60000))


def test_lowering_with_a_dropped_wait_is_caught_by_both_checkers(M):
    sc = M.amk_lower(M.model_desc(I.SHAPES["tiny_fp32"]), M.schedule_config(n_cu=16))
    rng = random.Random(11)
    waiters = [i for i, t in enumerate(sc.tasks) if t.waits]
    hits = 0
    for i in rng.sample(waiters, 12):
        s = sc.copy()
        s.tasks[i].waits.pop(rng.randrange(len(s.tasks[i].waits)))
        v = M.amk_validate(s)
        if v.accepted:               # the dropped wait was implied by another one
            continue
        rs = _runs(M, s, n=3, delay=20)
        # a missing ordering shows as a race, a read before its producer ran, or (with flags) nothing
        # observable on the CPU: the flag protocol would still order it on the device
        hits += any(r["races"] or r["uncovered_reads"] for r in rs)
        assert not any(r["deadlocked"] for r in rs)
    assert hits >= 4


def _lowered_mutants(M, n, seed):
    sc = M.amk_lower(M.model_desc(I.SHAPES["tiny_fp32"]), M.schedule_config(n_cu=16))
    rng = random.Random(seed)
    for _ in range(n):
        s = sc.copy()
        for _ in range(rng.randint(1, 2)):
            S._mutate(s, rng)
        yield s


@pytest.mark.parametrize("n,seed", [(150, 1), pytest.param(1000, 2, marks=pytest.mark.slow)])
def test_mutants_of_the_lowering_agree_with_the_validator(M, n, seed):
    """Beyond brute-force sizes (149 tasks on 16 queues): mutants of the real lowering. Whatever
    the validator accepts runs clean; whatever deadlocks or races, the validator rejected."""
    counts = {"accepted": 0, "deadlock": 0, "race": 0, "refused": 0}
    for s in _lowered_mutants(M, n, seed):
        v = M.amk_validate(s)
        try:
            rs = _runs(M, s, n=2, delay=2)
        except M.AmkError:
            assert v.rule_mask & 1
            counts["refused"] += 1
            continue
        for r in rs:
            if v.accepted:
                assert _clean(r), (hex(v.rule_mask), r)
            if r["deadlocked"]:
                # V1 (threshold), V3 or V4; or V0, after which nothing else is checked
                assert v.rule_mask & 0b11011, hex(v.rule_mask)
            if r["races"]:
                assert not v.accepted
        counts["accepted"] += v.accepted
        counts["deadlock"] += any(r["deadlocked"] for r in rs)
        counts["race"] += any(r["races"] for r in rs)
    assert all(counts[k] > 0 for k in counts), counts
