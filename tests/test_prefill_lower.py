"""The prefill lowering on the CPU: every workload's schedule is accepted by the validator at
several chunk sizes, runs clean on the CPU executor, and a schedule with a wait removed is
rejected; sizes outside one launch are refused."""
import random

import pytest

import amk_inputs as I


@pytest.fixture(scope="module")
def M():
    import persistent_megakernel_amd as M
    M.lib()
    return M


@pytest.mark.parametrize("name", ["tiny_fp32", "smollm2_135m_bf16", "tinyllama_int8"])
@pytest.mark.parametrize("n", [1, 63, 64, 65, 256])
def test_prefill_schedule_accepted(M, name, n):
    v = M.amk_lower_prefill(M.model_desc(I.SHAPES[name]), 256, n, python=False)
    assert v.accepted, (name, n, hex(v.rule_mask), v.task, v.region)


@pytest.mark.slow
@pytest.mark.parametrize("name", ["llama7b_bf16", "llama3_8b_int4"])
def test_prefill_schedule_accepted_large(M, name):
    v = M.amk_lower_prefill(M.model_desc(I.SHAPES[name]), 256, 256, python=False)
    assert v.accepted, (name, hex(v.rule_mask))


@pytest.mark.parametrize("n_cu,n", [(1, 3), (7, 64), (16, 130), (256, 200)])
def test_prefill_schedule_runs_clean_on_the_executor(M, n_cu, n):
    s = M.amk_lower_prefill(M.model_desc(I.SHAPES["tiny_fp32"]), n_cu, n)
    for seed in range(3):
        r = M.amk_vm_run(s, seed=seed, max_delay_us=3, watchdog_ms=10000)
        assert r["completed"] and not r["races"] and not r["uncovered_reads"] and not r["unwritten_outputs"], r


def _splits(sh, K, nm, n_cu):
    """K splits of an O or down tile: whole K stages over the CUs the phase's tiles leave idle."""
    kt = 128 if sh.act_f32 else 256
    tiles = nm * (sh.hidden // 64)
    return max(1, min(8, n_cu // tiles, -(-K // kt)))


def test_prefill_schedule_structure(M):
    """One embedding phase, then five phases per layer (the norms fused into the GEMMs that
    consume them), each waiting on all of the previous one; an O or down phase with fewer tiles
    than CUs is split along K, its parts signalling one counter per tile that the tile's sum
    task waits on; LM tiles and one argmax."""
    sh = I.SHAPES["tiny_fp32"]
    n_cu, nm = 16, 2
    s = M.amk_lower_prefill(M.model_desc(sh), n_cu, 100)
    ops = [t.opcode for t in s.tasks]
    nqkv = sh.n_heads + 2 * sh.n_kv_heads
    tiles = nm * (sh.hidden // 64)
    so = _splits(sh, sh.n_heads * sh.head_dim, nm, n_cu)
    sd = _splits(sh, sh.intermediate, nm, n_cu)
    assert (so, sd) == (1, 2)
    resid = lambda ns: tiles if ns == 1 else tiles * (ns + 1)
    per_layer = nm * (nqkv + sh.n_heads + sh.intermediate // 16) + resid(so) + resid(sd)
    n_lm = ops.count(7)
    assert ops.count(8) == 1 and n_lm >= 1 and ops.count(1) == nm
    assert len(ops) == nm + sh.n_layers * per_layer + n_lm + 1
    assert ops.count(11) == sh.n_layers * tiles * sd and ops.count(12) == sh.n_layers * tiles
    assert ops.count(6) == 0 and ops.count(4) == sh.n_layers * tiles
    assert len({c for t in s.tasks for c in t.signals}) == 1 + (5 + tiles) * sh.n_layers + 1
    # every wait is a full wait on its counter: the phase before, or a tile's K splits
    producers = {}
    for i, t in enumerate(s.tasks):
        for c in t.signals:
            producers[c] = producers.get(c, 0) + 1
    for t in s.tasks:
        for c, th in t.waits:
            assert th == producers[c]
            if t.opcode == 12:
                assert th == sd


def test_prefill_k_split_of_the_benchmarked_shape(M):
    """TinyLlama int8, 256 tokens on 256 CUs: 128 O and 128 down tiles, each split in two (one
    round of the CUs); 64 tokens: in eight. Tiles past the split bound stay whole."""
    sh = I.SHAPES["tinyllama_int8"]
    for n, ns in ((256, 2), (64, 8)):
        s = M.amk_lower_prefill(M.model_desc(sh), 256, n)
        ops = [t.opcode for t in s.tasks]
        tiles = (n // 64) * (sh.hidden // 64)
        assert ops.count(9) == ops.count(11) == sh.n_layers * tiles * ns, n
        assert ops.count(10) == ops.count(12) == sh.n_layers * tiles, n
        assert ops.count(4) == ops.count(6) == 0
    s = M.amk_lower_prefill(M.model_desc(sh), 64, 256)   # 128 tiles on 64 CUs: no split
    ops = [t.opcode for t in s.tasks]
    assert ops.count(4) == ops.count(6) == sh.n_layers * 128 and ops.count(9) == 0


def test_prefill_schedule_without_a_wait(M):
    """Dropping a queue's first wait on a counter is rejected unless the queue order already
    orders every access it guarded (e.g. the norm task of the same M-tile earlier in the same
    queue); whatever the validator still accepts runs clean on the executor."""
    s = M.amk_lower_prefill(M.model_desc(I.SHAPES["tiny_fp32"]), 8, 70)
    first = []
    for q in s.queues:
        seen = set()
        for i in q:
            for c, _ in s.tasks[i].waits:
                if c not in seen:
                    first.append(i)
                    seen.add(c)
    rejected = 0
    for i in first:
        m = s.copy()
        m.tasks[i].waits = []
        if not M.amk_validate(m).accepted:
            rejected += 1
            continue
        for seed in range(3):
            r = M.amk_vm_run(m, seed=seed, max_delay_us=20, watchdog_ms=10000)
            assert r["completed"] and not r["races"] and not r["uncovered_reads"], (i, r)
    assert rejected >= 0.9 * len(first), (rejected, len(first))


@pytest.mark.parametrize("n", [0, -1, 257])
def test_prefill_sizes_outside_one_launch_are_refused(M, n):
    with pytest.raises(M.AmkError):
        M.amk_lower_prefill(M.model_desc(I.SHAPES["tiny_fp32"]), 256, n)
