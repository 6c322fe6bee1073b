"""Schedule search (the pages' second optimisation loop): proposals, the keep/revert rule, the
static cost model, its refit, the reference gate and the lowering filter on the CPU; one short
search and one calibration on the GPU, every measured candidate gated against the oracle."""
import dataclasses
import random

import numpy as np
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


def test_prefetch_knob_range_and_reading():
    from persistent_megakernel_amd import AmkError, amk_lower, model_desc, schedule_config
    shape = I.SHAPES["tiny_fp32"]
    for g in (-1, 0, 1, 2):
        amk_lower(model_desc(shape), schedule_config(prefetch_groups=g))
    for g in (-2, 3):
        with pytest.raises(AmkError):
            amk_lower(model_desc(shape), schedule_config(prefetch_groups=g))
    assert [S.ahead_groups({"prefetch_groups": g}) for g in (-1, 0, 1, 2)] == [0, 1, 1, 2]
    assert S.ahead_groups({}) == 1


def test_cost_model_prefetch_shortens_gemv_tasks_only():
    shape = I.SHAPES["tinyllama_int8"].replace(n_layers=2)
    ok, sc = S.lower(shape, {}, shape.max_ctx)
    assert ok
    # prefetched groups shorten GEMV tasks and lengthen the hops into them
    p = dataclasses.replace(S.CostParams(), ahead_hop_us=0.0)
    e0, e1, e2 = (S.estimate_us(shape, sc, 512, p, a) for a in (0, 1, 2))
    assert e0 > e1 > e2
    q = dataclasses.replace(S.CostParams(), ahead_us=0.0)
    f0, f1, f2 = (S.estimate_us(shape, sc, 512, q, a) for a in (0, 1, 2))
    assert f0 < f1 < f2
    gemv = [t for t in sc.tasks if t.opcode == A.AMK_OP_GATEUP]   # a body longer than one group's saving
    attn = [t for t in sc.tasks if t.opcode == A.AMK_OP_ATTN]
    assert S.task_cost(shape, gemv[0], 512, p, 0) - S.task_cost(shape, gemv[0], 512, p, 1) == pytest.approx(p.ahead_us)
    assert S.task_cost(shape, attn[0], 512, p, 0) == S.task_cost(shape, attn[0], 512, p, 2)


def test_spearman_against_brute_force():
    rng = np.random.default_rng(3)
    assert S.spearman([1, 2, 3, 4], [10, 20, 30, 40]) == pytest.approx(1.0)
    assert S.spearman([1, 2, 3, 4], [4, 3, 2, 1]) == pytest.approx(-1.0)
    for _ in range(20):
        a, b = rng.normal(size=9), rng.normal(size=9)
        # no ties: 1 - 6 sum d^2 / (n (n^2 - 1))
        ra, rb = np.argsort(np.argsort(a)), np.argsort(np.argsort(b))
        n = len(a)
        want = 1 - 6 * float(((ra - rb) ** 2).sum()) / (n * (n * n - 1))
        assert S.spearman(a, b) == pytest.approx(want)
    # ties take the average rank
    assert S.spearman([1, 1, 2], [1, 2, 3]) == pytest.approx(np.corrcoef([0.5, 0.5, 2], [0, 1, 2])[0, 1])


def test_depth_plan_extrapolation_is_exact_for_a_repeating_dag():
    shape = I.SHAPES["tinyllama_int8"].replace(n_layers=6)
    for cfg in ({}, {"attn_chunks": 4, "attn_group_tasks": 2}, {"prefetch_groups": 2}):
        ok, sc = S.lower(shape, cfg, shape.max_ctx)
        assert ok
        a = S.ahead_groups(cfg)
        full = S.estimate_us(shape, sc, 512, None, a)
        assert S.DepthPlan(shape, cfg, shape.max_ctx, 512).estimate(None, a) == pytest.approx(full, rel=1e-9)


def test_refit_recovers_a_planted_cost_model():
    """Times generated by the model itself with other parameters: the refit ranks them (two of
    them lie within 0.1 % of each other) and brings the estimates within a few percent."""
    shape = I.SHAPES["tinyllama_int8"].replace(n_layers=2)
    truth = dataclasses.replace(S.CostParams(), hop_us=1.7, cu_gbps=45.0, ahead_us=0.9, attn_level_us=0.15,
                                ahead_hop_us=0.1)
    items = []
    for cfg in ({}, {"prefetch_groups": -1}, {"prefetch_groups": 2}, {"attn_chunks": 1}, {"attn_chunks": 8},
                {"tasks_qkv": 32}, {"tasks_gateup": 64}, {"attn_group_tasks": 2}):
        cfg = {"attn_group_tasks": 1, **cfg}   # grouped attention unless the case says otherwise
        ok, sc = S.lower(shape, cfg, shape.max_ctx)
        assert ok
        pl = S.Plan(shape, sc, 512)
        items.append((pl, S.ahead_groups(cfg), S.plan_estimate(pl, truth, S.ahead_groups(cfg))))
    start = [S.plan_estimate(pl, S.CostParams(), a) for pl, a, _ in items]
    fit = S.fit_cost_params(items, S.CostParams())
    est = [S.plan_estimate(pl, fit, a) for pl, a, _ in items]
    meas = [m for _, _, m in items]
    assert S.spearman(est, meas) >= 0.9
    assert max(abs(e / m - 1) for e, m in zip(est, meas)) < 0.06 < max(abs(e / m - 1) for e, m in zip(start, meas))


def _ref(shape, logits, gen, margins):
    return S.Reference("x", 0, list(range(len(gen))), list(gen), np.asarray(logits, np.float32), list(margins))


def test_gate_rules():
    bf = I.SHAPES["tinyllama_int8"]             # bf16 activations, full depth: 0.25 abs, 0.05 RMS
    one = bf.replace(n_layers=1)                # one layer: 2e-2
    f32 = I.SHAPES["tiny_fp32"]                 # fp32: 1e-4 normwise
    rng = np.random.default_rng(5)
    L = rng.normal(size=(3, 50)).astype(np.float32)
    L[:, 7] += 10.0                             # a clear winner: margin of several units
    gen = [7, 7, 7]
    ref = _ref(bf, L, gen, [5.0, 5.0, 5.0])
    assert S.gate(bf, ref, L, gen)[0]
    ok, info = S.gate(bf, ref, L + 0.2, gen)                    # within 0.25 abs but RMS 0.2 > 0.05
    assert not ok and "parity bar" in info["reason"]
    bump = L.copy(); bump[:, 3] += 0.2                         # one logit 0.2 off: RMS small
    assert S.gate(bf, ref, bump, gen)[0]
    assert not S.gate(one, ref, bump, gen)[0]                  # one layer: 2e-2
    ok, info = S.gate(bf, ref, L, [7, 3, 7])                   # not the argmax of its own logits
    assert not ok and "argmax" in info["reason"]
    # a different winner is allowed only where the reference's margin is small
    R = L.copy(); R[1, 9] = R[1, 7] - 0.005                  # the reference picks 7 by 0.005
    cand = R.copy(); cand[1, 9] += 0.01                        # the candidate picks 9
    assert S.gate(bf, _ref(bf, R, gen, [5.0, 0.005, 5.0]), cand, [7, 9, 7])[0]
    assert not S.gate(bf, _ref(bf, R, gen, [5.0, 5.0, 5.0]), cand, [7, 9, 7])[0]
    # fp32: relative to the largest reference logit
    rf = _ref(f32, L, gen, [5.0] * 3)
    scale = np.abs(L).max(axis=1, keepdims=True)
    assert S.gate(f32, rf, L + 0.5e-4 * scale, gen)[0]
    assert not S.gate(f32, rf, L + 2e-4 * scale, gen)[0]
    bad = L.copy(); bad[0, 0] = np.nan
    assert not S.gate(bf, ref, bad, gen)[0]


def test_reference_record_round_trip(tmp_path):
    from oracle import search_reference as R
    rec = R.record("tiny_fp32", 4, 3)
    assert rec["logits"].shape == (3, I.SHAPES["tiny_fp32"].vocab)
    # teacher forcing: each fed token after the first is the reference's previous greedy id
    assert rec["inputs"].tolist()[1:] == rec["gen"].tolist()[:-1]
    assert rec["gen"].tolist() == [int(np.argmax(r)) for r in rec["logits"]]
    path = str(tmp_path / "ref.npz")
    R.save(rec, path)
    ref = S.load_reference(path)
    assert (ref.workload, ref.pos0, ref.inputs) == ("tiny_fp32", 4, rec["inputs"].tolist())
    assert np.array_equal(ref.logits, rec["logits"])
    assert S.gate(I.SHAPES["tiny_fp32"], ref, rec["logits"], rec["gen"].tolist())[0]


@pytest.mark.gpu
def test_short_search_keeps_only_oracle_checked_candidates():
    from oracle import search_reference as R
    ref = S.Reference.from_record(R.record("tiny_fp32", 4, 3))
    res = S.search(ref, budget=3, seed=1, block=8, rounds=1, log=lambda m: None)
    assert res["incumbent_us"] > 0
    assert len(res["trials"]) >= 1
    for t in res["trials"]:
        assert t["verdict"] in ("kept", "reverted", "failed the reference gate", "rejected by lowering/validator")
        if t["verdict"] in ("kept", "reverted"):
            assert t["gate"]["max_err"] <= 1e-4 and t["gate"]["ids_equal"]
            assert t["incumbent_us"] > 0 and t["candidate_us"] > 0
    kept = [t["cfg"] for t in res["trials"] if t["verdict"] == "kept"]
    assert res["incumbent"] == (kept[-1] if kept else {})


@pytest.mark.gpu
def test_calibration_measures_gated_configurations():
    from oracle import search_reference as R
    ref = S.Reference.from_record(R.record("tiny_fp32", 4, 3))
    cfgs = [{}, {"prefetch_groups": -1}, {"prefetch_groups": 2}, {"cu_assign": 1}, {"tasks_qkv": 2, "tasks_gateup": 2}]
    rec = S.calibrate(ref, cfgs, block=8, rounds=1, log=lambda m: None)
    rows = rec["configs"]
    assert [r["cfg"] for r in rows] == cfgs
    for r in rows:
        assert r["verdict"] == "measured", r
        assert r["gate_max_err"] <= 1e-4 and r["measured_us"] > 0
    fit = S.refit(rec)
    assert fit["n_measured"] == len(cfgs) and -1.0 <= fit["rho_fitted_in_sample"] <= 1.0
