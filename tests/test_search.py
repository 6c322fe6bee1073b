"""Schedule search (the pages' second optimisation loop): proposals, the keep/revert rule, the
static cost model and the lowering filter on the CPU; one short search on the GPU, whose kept
candidates must have passed the parity gate."""
import random

import pytest

import amk_inputs as I
from amk_inputs.schedules import Schedule, Task
from persistent_megakernel_amd import _abi as A
from persistent_megakernel_amd import search as S


def test_proposals_change_exactly_one_knob_within_its_domain():
    inc = {"tasks_o": 128, "attn_chunks": 16}
    props = S.propose(inc, random.Random(7), 200)
    assert props == S.propose(inc, random.Random(7), 200)   # seeded
    for c in props:
        diff = [k for k in S.KNOBS if c.get(k, 0) != inc.get(k, 0)]
        assert len(diff) == 1
        k = diff[0]
        assert c.get(k, 0) in S.KNOBS[k]
        assert all(v != 0 for v in c.values())   # defaults are left out of the dict
    assert {k for c in props for k in S.KNOBS if c.get(k, 0) != inc.get(k, 0)} == set(S.KNOBS)


def test_keep_only_beyond_the_noise_margin():
    assert S.decide(100.0, 99.0, 0.005)
    assert not S.decide(100.0, 99.6, 0.005)
    assert not S.decide(100.0, 101.0, 0.0)
    assert S.config_key({"a": 0, "b": 3}) == S.config_key({"b": 3})


def _chain(n_phases: int, per_phase: int, n_queues: int) -> Schedule:
    """n_phases phases of per_phase tasks; every task of phase p waits for all of phase p-1."""
    tasks, queues = [], [[] for _ in range(n_queues)]
    for p in range(n_phases):
        for i in range(per_phase):
            t = Task(waits=[(p - 1, per_phase)] if p else [], signals=[p], opcode=A.AMK_OP_ARGMAX,
                     args=(0, 0, 0, 0, 0))
            queues[i % n_queues].append(len(tasks))
            tasks.append(t)
    return Schedule(n_queues, n_phases, 1, tasks, queues)


def test_cost_model_critical_path_of_a_chain():
    shape = I.SHAPES["tiny_fp32"]
    p = S.CostParams()
    # k phases of independent tasks on as many queues: k task costs and k - 1 hops
    for k in (1, 2, 5):
        est = S.estimate_us(shape, _chain(k, 4, 4), 0, p)
        assert est == pytest.approx(k * p.task_us + (k - 1) * p.hop_us)
    # two tasks of a phase on one queue run one after the other
    est = S.estimate_us(shape, _chain(1, 4, 2), 0, p)
    assert est == pytest.approx(2 * p.task_us)


def test_cost_model_rejects_a_cycle():
    t0 = Task(waits=[(1, 1)], signals=[0], opcode=A.AMK_OP_ARGMAX)
    t1 = Task(waits=[(0, 1)], signals=[1], opcode=A.AMK_OP_ARGMAX)
    with pytest.raises(ValueError):
        S.estimate_us(I.SHAPES["tiny_fp32"], Schedule(2, 2, 1, [t0, t1], [[0], [1]]), 0)


@pytest.mark.slow
def test_cost_model_orders_attention_splits_as_measured():
    # on MI355X (TinyLlama-shaped int8 at position 512): one task per query head is slower the
    # fewer context chunks it has, and all of them are slower than the default split
    shape = I.SHAPES["tinyllama_int8"]
    est = {}
    for name, cfg in {"default": {}, "c1h": {"attn_chunks": 1, "attn_group_tasks": 2},
                      "c4h": {"attn_chunks": 4, "attn_group_tasks": 2}}.items():
        ok, sc = S.lower(shape, cfg, shape.max_ctx)
        assert ok
        est[name] = S.estimate_us(shape, sc, 512)
    assert est["c1h"] > est["c4h"] > est["default"] > 0


def test_lowering_filter_rejects_an_impossible_split():
    # a merge of 1000 chunk states per head does not fit the kernel's LDS staging
    shape = I.SHAPES["tinyllama_int8"]
    ok, sc = S.lower(shape, {"attn_chunks": 1000}, shape.max_ctx)
    assert not ok and sc is None


@pytest.mark.gpu
def test_short_search_keeps_only_parity_checked_candidates():
    res = S.search("tiny_fp32", budget=3, seed=1, pos0=4, block=8, rounds=1, parity_steps=3, log=lambda m: None)
    assert res["incumbent_us"] > 0
    assert len(res["trials"]) >= 1
    for t in res["trials"]:
        assert t["verdict"] in ("kept", "reverted", "failed the parity gate", "rejected by lowering/validator")
        if t["verdict"] in ("kept", "reverted"):
            assert t["parity_max_logit_diff"] <= 1e-3 * 100   # relative bound times logit scale
            assert t["incumbent_us"] > 0 and t["candidate_us"] > 0
    kept = [t["cfg"] for t in res["trials"] if t["verdict"] == "kept"]
    assert res["incumbent"] == (kept[-1] if kept else {})
