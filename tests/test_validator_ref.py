"""The reference validator and the brute-force interleaver, checked against each other and
against a hand corpus with one case per rule."""
import pytest

from amk_inputs import schedules as S
from oracle import interleave as IL
from oracle import validator_ref as VR

import schedule_corpus


@pytest.mark.parametrize("name,sched,acc,mask", schedule_corpus.corpus(), ids=lambda x: x if isinstance(x, str) else "")
def test_hand_corpus(name, sched, acc, mask):
    assert VR.validate(sched) == (acc, mask), name


@pytest.mark.parametrize("name,sched,acc,mask", schedule_corpus.corpus(), ids=lambda x: x if isinstance(x, str) else "")
def test_hand_corpus_accepted_cases_are_safe(name, sched, acc, mask):
    r = IL.explore(sched)
    if acc:
        assert r["safe"], name
    if "deadlock" in name or "V4" in name or "V3" in name:
        assert r["deadlock"] or r["malformed"]


def test_cross_queue_cycle_deadlocks_in_the_interleaver():
    # the case a counter-DAG-only check would accept
    s = [c for c in schedule_corpus.corpus() if c[0] == "V4 cross-queue cycle"][0][1]
    assert IL.explore(s)["deadlock"]


def test_random_corpus_no_false_accepts():
    """200 seeded schedules of at most 12 tasks: accepted implies safe under every
    interleaving (deadlock-free and race-free); false rejects are allowed and counted."""
    n_safe = n_acc = false_rej = 0
    masks = 0
    for seed in range(200):
        s = S.random_schedule(seed)
        acc, mask = VR.validate(s)
        r = IL.explore(s)
        masks |= mask
        n_safe += r["safe"]
        n_acc += acc
        assert not (acc and not r["safe"]), f"false accept at seed {seed}: {r}"
        false_rej += (not acc) and r["safe"]
    assert masks == 0x1FF                          # every rule fires somewhere in the corpus
    assert 40 <= n_safe <= 160 and n_acc > 20
    assert false_rej < n_safe


def test_valid_by_construction_schedules_are_accepted_and_safe():
    import random
    for seed in range(200):
        s = S._valid_schedule(random.Random(seed), ll=bool(seed % 2))
        assert VR.validate(s) == (True, 0), seed
        assert IL.explore(s)["safe"], seed
