"""Host side of libamk.so, no GPU: the library loads and exports every call include/amk.h
declares; the C++ validator's verdicts equal the reference validator's bit for bit; the
built-in lowering of every workload (and of the lowering knobs the GPU tests use) is accepted;
shapes the kernel does not implement are refused before anything reaches a device."""
import ctypes as C
import os
import re

import pytest

import amk_inputs as I
from amk_inputs import schedules as S
from oracle import validator_ref as VR

import schedule_corpus

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def M():
    import persistent_megakernel_amd as M
    M.lib()
    return M


def test_exports_every_declared_symbol(M):
    hdr = open(os.path.join(ROOT, "include", "amk.h")).read()
    names = set(re.findall(r"^\s*(?:amk_status|void|uint32_t|const\s+\w+\s*\*|const char\s*\*)\s+(amk_\w+)\s*\(",
                           hdr, re.M))
    assert {"amk_validate", "amk_create", "amk_decode_step", "amk_destroy"} <= names
    lib = C.CDLL(M._abi.LIB_PATH)
    for n in sorted(names):
        assert hasattr(lib, n), n
        assert n in M._abi.SIGNATURES, n
    assert M.amk_version().startswith("amk-mi355x")


@pytest.mark.parametrize("name,sched,acc,mask", schedule_corpus.corpus(), ids=lambda x: x if isinstance(x, str) else "")
def test_cpp_validator_equals_reference_on_hand_corpus(M, name, sched, acc, mask):
    v = M.amk_validate(sched)
    assert (bool(v.accepted), v.rule_mask) == (acc, mask), name


def test_cpp_validator_equals_reference_on_random_schedules(M):
    for seed in range(400):
        s = S.random_schedule(seed)
        v = M.amk_validate(s)
        assert (bool(v.accepted), v.rule_mask) == VR.validate(s), seed
        assert bool(v.accepted) == (v.rule_mask == 0)


@pytest.mark.parametrize("name", sorted(I.SHAPES))
def test_builtin_lowering_accepted(M, name):
    v = M.amk_lower_verdict(M.model_desc(I.SHAPES[name]))
    assert v.accepted and v.rule_mask == 0


@pytest.mark.parametrize("kw", [dict(n_cu=1), dict(n_cu=7, cu_assign=1), dict(attn_chunks=3, attn_group_tasks=1),
                                dict(tasks_qkv=3, tasks_o=5, tasks_gateup=2, tasks_down=9, tasks_lm=4)])
def test_tiny_lowering_knobs_accepted_and_agree_with_reference(M, kw):
    """The Python reference validator, run on the lowered schedule itself, agrees."""
    sched = M.amk_lower(M.model_desc(I.SHAPES["tiny_fp32"]), M.schedule_config(**kw))
    assert VR.validate(sched) == (True, 0)
    assert M.amk_validate(sched).accepted


def test_lowered_schedule_round_trip_and_mutation_rejected(M):
    """A lowered schedule copied back into C is accepted; dropping one full wait (so a reader
    is no longer ordered after its producers) is rejected by both validators."""
    sched = M.amk_lower(M.model_desc(I.SHAPES["tiny_fp32"]), M.schedule_config(n_cu=4))
    assert M.amk_validate(sched).accepted
    bad = sched.copy()
    i = next(k for k, t in enumerate(bad.tasks) if t.opcode == M.A.AMK_OP_OPROJ and t.waits)
    bad.tasks[i].waits = []
    v = M.amk_validate(bad)
    assert not v.accepted
    assert (bool(v.accepted), v.rule_mask) == VR.validate(bad)


@pytest.mark.parametrize("kw,status", [
    (dict(head_dim=32), 2),                         # head_dim not in {16, 64, 128}
    (dict(n_kv_heads=3), 2),                        # n_heads not a multiple of n_kv_heads
    (dict(intermediate=180), 2),                    # not a multiple of 16
    (dict(wfmt=I.WF_BF16), 2),                      # fp32 activations with bf16 weights
    (dict(hidden=0), 1),
])
def test_unsupported_shapes_refused(M, kw, status):
    shape = I.tiny_shape(**kw)
    with pytest.raises(M.AmkError) as e:
        M.amk_lower(M.model_desc(shape))
    assert e.value.status == status


def test_merge_fusion_lowering(M):
    """The fusion-grouping knob for split-context attention: on request each head group's merge
    runs inside its last chunk's task (AMK_OP_ATTN_MERGE, waiting on the other chunks' states);
    the schedule is accepted by the validator and completes under the CPU executor with no race.
    The default keeps separate merge tasks; the fused form is refused where the last chunk's LDS
    stage cannot hold every chunk state of its heads (grouped Llama-3-8B heads at 4096), and
    values outside the knob's range are refused."""
    A = M.A
    sh = I.SHAPES["tinyllama_int8"].replace(n_layers=2)
    d = M.model_desc(sh, max_ctx=1024)
    dflt = M.amk_lower(d, M.schedule_config(n_cu=64))
    ops = [t.opcode for t in dflt.tasks]
    assert A.AMK_OP_MERGE in ops and A.AMK_OP_ATTN_MERGE not in ops
    fused = M.amk_lower(d, M.schedule_config(n_cu=64, merge_fusion=1))
    ops = [t.opcode for t in fused.tasks]
    n_att = ops.count(A.AMK_OP_ATTN) + ops.count(A.AMK_OP_ATTN_MERGE)
    assert A.AMK_OP_MERGE not in ops and ops.count(A.AMK_OP_ATTN_MERGE) == sh.n_layers * sh.n_heads
    assert n_att == [t.opcode for t in dflt.tasks].count(A.AMK_OP_ATTN)
    for t in fused.tasks:
        if t.opcode == A.AMK_OP_ATTN_MERGE:
            nc = t.args[4]
            assert nc > 1 and t.args[3] == nc - 1 and len(t.waits) == 3   # q, current k/v, other chunks
    assert M.amk_validate(fused).accepted == 1
    for seed in range(2):
        r = M.amk_vm_run(fused, seed=seed, max_delay_us=30)
        assert r["completed"] == 1 and r["races"] == 0 and r["uncovered_reads"] == 0, r
    big = M.model_desc(I.SHAPES["llama3_8b_int4"], max_ctx=4128)
    with pytest.raises(M.AmkError):
        M.amk_lower(big, M.schedule_config(merge_fusion=1))
    with pytest.raises(M.AmkError):
        M.amk_lower(d, M.schedule_config(merge_fusion=3))
