"""Per-task timestamp traces of the decode and prefill kernels on the GPU.

Tracing must not change what a launch computes: a traced decode launch and a traced prefill
launch give logits and tokens bit-identical to untraced ones. Every task's timestamps must be
ordered the way the kernels take them, and a CU's tasks must follow one another in queue order.
Decode slots: 0 start, 1 inputs observed, 2 rows done (GEMV; attention: per-wave states stored;
merge: chunk weights computed), 3 end, 4 the first wave's rows (GEMV) or positions (attention)
done, 5 outputs written. Prefill slots: 0 start, 1 inputs ready, 2 computed,
3 signalled. (The pages measure per-tile cross-SM synchronisation this way: AutoMegaKernel pages,
page 2, "Performance ceiling and gap".)
"""
from __future__ import annotations

import numpy as np
import pytest

import amk_inputs as I
from gpu_util import log

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def M():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import persistent_megakernel_amd as M
    M.lib()
    return M


def _decode(M, dec, toks, pos0):
    lg = torch.zeros((len(toks), dec.shape.vocab), dtype=torch.float32, device="cuda")
    out = M.run_steps(dec, toks, pos0, logits=lg)
    torch.cuda.synchronize()
    assert dec.status() == 0
    return lg.cpu().numpy(), out.cpu().numpy()


@pytest.mark.parametrize("name,pos0", [("tiny_fp32", 0), ("tinyllama_int8", 300)])
def test_traced_decode_is_bit_identical_and_ordered(M, name, pos0):
    shape = I.SHAPES[name]
    if name != "tiny_fp32":
        shape = shape.replace(n_layers=2)
    log(f"case traced decode {name} pos {pos0}")
    w = I.make_weights(shape)
    dec = M.Decoder(shape, w)
    if pos0:
        for l in range(shape.n_layers):
            dec.set_kv_prefix(l, I.kv_prefill(shape, pos0, l))
    toks = [int(t) for t in I.prompt_tokens(shape, 3, stream=4)]
    lg0, ids0 = _decode(M, dec, toks, pos0)
    trace = dec.enable_trace()
    lg1, ids1 = _decode(M, dec, toks, pos0)   # the same steps again, traced
    sched = dec.schedule()
    dec.close()
    np.testing.assert_array_equal(lg1, lg0)
    np.testing.assert_array_equal(ids1, ids0)
    tr = trace.cpu().numpy()   # the last traced launch: every task's slots
    order = [t for q in sched.queues for t in q]
    assert tr.shape[0] == len(order)
    k = 0
    for q in sched.queues:
        prev_end = None
        for tid in q:
            op = sched.tasks[tid].opcode
            s, ready, done, end, w0, out = (int(x) for x in tr[k])
            k += 1
            assert s > 0 and s <= ready <= out <= end, (op, tr[k - 1])
            if op in (1, 4, 5, 6, 7):   # GEMV ops
                assert ready <= w0 <= done <= out, (op, tr[k - 1])
            elif op in (2, 9):          # attention (9: with the merge fused)
                assert ready <= w0 <= done <= out, (op, tr[k - 1])
            elif op == 3:               # merge
                assert ready <= done <= out, (op, tr[k - 1])
            if prev_end is not None:
                assert prev_end <= s, "a CU's tasks overlap in its trace"
            prev_end = end
    log(f"{name}: {len(order)} tasks traced, launch span {(tr[:, 3].max() - tr[:, 0].min()) * 0.01:.1f} us")


def test_traced_prefill_is_bit_identical_and_ordered(M):
    shape = I.SHAPES["tinyllama_int8"].replace(n_layers=2)
    log("case traced prefill tinyllama_int8 2 layers, 64 tokens")
    w = I.make_weights(shape)
    n = 64
    toks = torch.tensor(I.prompt_tokens(shape, n, stream=7), dtype=torch.int32, device="cuda")

    def run(dec):
        tout = torch.zeros(1, dtype=torch.int32, device="cuda")
        lg = torch.zeros(shape.vocab, dtype=torch.float32, device="cuda")
        dec.prefill(toks, 0, tout, lg)
        torch.cuda.synchronize()
        assert dec.status() == 0
        return lg.cpu().numpy(), int(tout.item())

    dec = M.Decoder(shape, w)
    lg0, t0 = run(dec)
    tr_dev, sched = dec.enable_prefill_trace(n, len(dec.schedule().queues))   # the context's CU count
    lg1, t1 = run(dec)
    dec.close()
    np.testing.assert_array_equal(lg1, lg0)
    assert t1 == t0
    tr = tr_dev.cpu().numpy()
    k = 0
    for q in sched.queues:
        prev = None
        for _ in q:
            s, ready, done, sig = (int(x) for x in tr[k])
            k += 1
            assert 0 < s <= ready <= done <= sig, tr[k - 1]
            if prev is not None:
                assert prev <= s
            prev = sig
    assert k == tr.shape[0]
