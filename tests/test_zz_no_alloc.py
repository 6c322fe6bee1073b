"""The allocation-free decode entry point (amk_decode_step_static) against amk_decode_step,
through the C ABI: the same context, the same inputs, bit-identical logits and tokens, on two
calls in a row whose second call is a smaller model (the static flag-word array keeps the
first call's contents, which must not leak into the second)."""
from __future__ import annotations

import numpy as np
import pytest

import amk_inputs as I

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def M():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import persistent_megakernel_amd as M
    M.lib()
    return M


def _both(M, shape, tokens):
    """Run the token list (one step per position) through both entry points on one context;
    returns (regular logits, static logits, regular ids, static ids) as numpy arrays."""
    w = I.make_weights(shape)
    dec = M.Decoder(shape, w)
    n = len(tokens)
    st = torch.cuda.current_stream().cuda_stream
    tin = torch.tensor(tokens, dtype=torch.int32, device="cuda")
    out = {}
    for name, fn in (("regular", M.amk_decode_step), ("static", M.amk_decode_step_static)):
        lg = torch.zeros((n, shape.vocab), dtype=torch.float32, device="cuda")
        ids = torch.full((n,), -1, dtype=torch.int32, device="cuda")
        for p in range(n):
            rc = fn(dec.ctx, tin[p:p + 1].data_ptr(), p, ids[p:p + 1].data_ptr(), lg[p].data_ptr(), st)
            assert rc == 0, (name, p, rc)
        torch.cuda.synchronize()
        out[name] = (lg.cpu().numpy(), ids.cpu().numpy())
    assert dec.status() == 0
    dec.close()
    return out["regular"][0], out["static"][0], out["regular"][1], out["static"][1]


def test_static_entry_point_equals_decode_step_on_two_calls():
    import persistent_megakernel_amd as M
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    M.lib()
    big = I.SHAPES["smollm2_135m_bf16"].replace(n_layers=4, max_ctx=32)
    small = I.SHAPES["tiny_fp32"]
    for shape, n in ((big, 6), (small, 3)):
        toks = [int(t) for t in I.prompt_tokens(shape, n, stream=4)]
        lr, ls, ir, is_ = _both(M, shape, toks)
        print(f"{shape.name}: {n} steps, max |logit difference| {float(np.max(np.abs(lr - ls))):.3e}, ids {ir.tolist()}")
        assert np.array_equal(lr, ls), shape.name
        assert np.array_equal(ir, is_), shape.name


def test_static_entry_point_argument_errors(M):
    shape = I.SHAPES["tiny_fp32"]
    dec = M.Decoder(shape, I.make_weights(shape))
    t = torch.zeros(2, dtype=torch.int32, device="cuda")
    for pos in (-1, dec.max_ctx):
        assert M.amk_decode_step_static(dec.ctx, t.data_ptr(), pos, t.data_ptr()) == M._abi.AMK_E_INVALID_ARG
    assert M.amk_decode_step_static(dec.ctx, 0, 0, t.data_ptr()) == M._abi.AMK_E_INVALID_ARG
    assert M.amk_decode_step_static(0, t.data_ptr(), 0, t.data_ptr()) == M._abi.AMK_E_INVALID_ARG
    dec.close()
