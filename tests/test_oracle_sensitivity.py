"""How far one rounding decision moves the logits of a full-depth workload (oracle only, CPU).

The decode step rounds every activation to bf16. Two correct evaluations that differ only in
fp32 summation order make a few different rounding decisions, and in a 22-layer random-init
model one such one-ulp change propagates to every later layer. This test measures that effect
on the oracle itself: it perturbs one element of the input token's embedding row by one bf16
ulp and reports the largest logit change. It pins two facts the GPU parity bars rest on: the
change exceeds 2e-2 (so 2e-2 cannot be required at full depth of this workload), and it stays
well below the full-depth bar (a few flips fit inside it).
"""
import numpy as np
import pytest

import amk_inputs as I
import oracle

FULL_DEPTH_ABS = 0.25   # same value as the GPU parity tests' full-depth bar


@pytest.mark.slow
def test_one_ulp_flip_moves_full_depth_logits():
    shape = I.SHAPES["tinyllama_int8"]
    w = I.make_weights(shape)
    tok = int(I.prompt_tokens(shape, 1, stream=1)[0])
    a = oracle.OracleModel(shape, w)
    _, base, _ = a.step(tok, 0)
    a.close()
    emb = w.embed.copy()
    emb[tok, 5] = np.uint16(int(emb[tok, 5]) + 1)   # one bf16 ulp (same sign, next magnitude)
    w2 = I.Weights(embed=emb, final_norm=w.final_norm, lm_head=w.lm_head, layers=w.layers)
    b = oracle.OracleModel(shape, w2)
    _, pert, _ = b.step(tok, 0)
    b.close()
    delta = float(np.max(np.abs(pert.astype(np.float64) - base)))
    print(f"one-ulp input flip: max abs logit change {delta:.4f}")
    assert delta > 2e-2
    assert 3 * delta < FULL_DEPTH_ABS



TWO_LAYER_ABS = 0.075   # same value as the prefill tests' two-layer bar: three one-ulp flips


@pytest.mark.slow
def test_one_ulp_flip_moves_two_layer_logits():
    """The same effect two layers deep (the TinyLlama-shaped width, int8): one one-ulp change of
    one input element moves the logits by more than 1e-2 and at most a third of the two-layer
    bar, so 2e-2 is within a single rounding flip there, and three flips fit the bar."""
    shape = I.SHAPES["tinyllama_int8"].replace(n_layers=2, max_ctx=16)
    w = I.make_weights(shape)
    tok = 1234
    a = oracle.OracleModel(shape, w)
    _, base, _ = a.step(tok, 0)
    a.close()
    deltas = []
    for k in (5, 77, 1000, 2047):
        emb = w.embed.copy()
        emb[tok, k] = np.uint16(int(emb[tok, k]) + 1)
        w2 = I.Weights(embed=emb, final_norm=w.final_norm, lm_head=w.lm_head, layers=w.layers)
        b = oracle.OracleModel(shape, w2)
        _, pert, _ = b.step(tok, 0)
        b.close()
        deltas.append(float(np.max(np.abs(pert.astype(np.float64) - base))))
    print(f"two layers, one-ulp input flips: max abs logit changes {deltas}")
    assert min(deltas) > 1e-2
    assert 3 * max(deltas) <= TWO_LAYER_ABS
