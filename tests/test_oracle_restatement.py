"""The whole decode step, restated a second time in float64 NumPy and compared with the C oracle.

This is a differential pin of the oracle's wiring: an independent plain NumPy statement of the
standard Llama step (RMSNorm, QKV projections, rotary embedding on half-split pairs, grouped
query attention over the cache, O projection and residual, RMSNorm, SwiGLU MLP and residual,
final RMSNorm, LM head, greedy argmax; AutoMegaKernel pages: page 3, "How it works", layer 1,
and page 1, "What's built"), with activations rounded where the method stores them. It shares
nothing with oracle.c: matrix products are numpy's, the bf16 rounding is done on the float64
bit pattern (not by the oracle's frexp/nearbyint route), fp32 rounding is numpy's cast, the
logistic is scipy's, and the int8/int4 quantiser is restated from its definition. Agreement
to float64 summation-order noise on every logit, and identical greedy tokens, over the tiny
fp32 protocol (23 steps), the first two steps of the SmolLM2-shaped bf16 model and short runs
of small int8 and int4 models, pins every wire of the step at once.
"""
from __future__ import annotations

import numpy as np
import pytest
import scipy.special

import amk_inputs as I
import oracle as O


# ---------------------------------------------------------------- storage rounding

def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bf16 value, ties to even, from the float64 bits:
    keep sign, exponent and the top 7 of the 52 mantissa bits. Valid for zero and for results
    in bf16's normal range, which is asserted."""
    x = np.asarray(x, dtype=np.float64)
    nz = x[x != 0]
    assert np.all(np.isfinite(nz)) and (nz.size == 0 or (np.min(np.abs(nz)) >= 2.0 ** -126
                                                         and np.max(np.abs(nz)) < 3.38e38))
    b = x.view(np.uint64)
    drop = np.uint64(45)
    lsb = (b >> drop) & np.uint64(1)
    r = (b + (np.uint64((1 << 44) - 1) + lsb)) & ~np.uint64((1 << 45) - 1)
    return r.view(np.float64)


def f32_round(x: np.ndarray) -> np.ndarray:
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def master_f64(a: np.ndarray) -> np.ndarray:
    """fp32 master as is; bf16 bits widened (exact)."""
    return I.bf16_bits_to_f32(a).astype(np.float64) if a.dtype == np.uint16 else a.astype(np.float64)


# ---------------------------------------------------------------- quantiser, from its definition

def quantize(w_bf16: np.ndarray, group: int, qmax: int):
    """Symmetric absmax: scale = fp16(fp32(absmax) / qmax) per row (group 0) or per (row,
    group of columns); code = clamp(round-half-even(fp32(w) / fp32(scale)), -qmax, qmax), zero
    scale -> zero codes. Returns dequantisation pieces (codes as float64, scales as float64)."""
    w = I.bf16_bits_to_f32(w_bf16)                       # exact fp32 values
    rows, cols = w.shape
    g = group or cols
    wg = w.reshape(rows, cols // g, g)
    amax = np.max(np.abs(wg), axis=2).astype(np.float32)
    s = (amax / np.float32(qmax)).astype(np.float32).astype(np.float16).astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        t = (wg / s[:, :, None]).astype(np.float32)
    q = np.clip(np.rint(t), -qmax, qmax)
    q[np.broadcast_to(s[:, :, None] == 0, q.shape)] = 0
    return q.reshape(rows, cols).astype(np.float64), s.astype(np.float64)


class Proj:
    """y = W h: exact products, float64 sums; int8 scales the row sum, int4 each group sum."""

    def __init__(self, master: np.ndarray, wfmt: int):
        self.wfmt = wfmt
        if wfmt in (I.WF_F32, I.WF_BF16):
            self.w = master_f64(master)
        else:
            self.group = 128 if wfmt == I.WF_INT4 else 0
            self.q, self.s = quantize(master, self.group, 7 if self.group else 127)

    def __call__(self, h: np.ndarray) -> np.ndarray:
        if self.wfmt in (I.WF_F32, I.WF_BF16):
            return self.w @ h
        if not self.group:
            return (self.q @ h) * self.s[:, 0]
        rows, cols = self.q.shape
        parts = np.einsum("rgk,gk->rg", self.q.reshape(rows, cols // 128, 128), h.reshape(cols // 128, 128))
        return np.sum(parts * self.s, axis=1)


# ---------------------------------------------------------------- the step

class NumpyModel:
    def __init__(self, shape: I.ModelShape, w: I.Weights):
        self.s = shape
        self.rnd = f32_round if shape.act_f32 else bf16_round
        f = shape.wfmt
        self.embed = master_f64(w.embed)
        self.final_norm = master_f64(w.final_norm)
        self.lm = Proj(w.lm(), f)
        self.layers = []
        for t in w.layers:
            self.layers.append(dict(attn_norm=master_f64(t["attn_norm"]), mlp_norm=master_f64(t["mlp_norm"]),
                                    **{n: Proj(t[n], f) for n in ("wq", "wk", "wv", "wo", "wg", "wu", "wd")}))
        self.K = np.zeros((shape.n_layers, shape.n_kv_heads, shape.max_ctx, shape.head_dim))
        self.V = np.zeros_like(self.K)

    def norm(self, x, g):
        eps = float(np.float32(self.s.rms_eps))   # the model description's fp32 value
        return self.rnd(x * (1.0 / np.sqrt(np.dot(x, x) / x.size + eps)) * g)

    def rope(self, u, pos):
        """u: [heads, hd]; pair (i, i + hd/2) rotated by pos * theta^(-2i/hd)."""
        hd = self.s.head_dim
        i = np.arange(hd // 2, dtype=np.float64)
        ang = pos * float(np.float32(self.s.rope_theta)) ** (-(2.0 * i) / hd)
        c, s = np.cos(ang), np.sin(ang)
        a, b = u[:, : hd // 2], u[:, hd // 2:]
        return np.concatenate([a * c - b * s, b * c + a * s], axis=1)

    def step(self, tok: int, pos: int):
        S = self.s
        hd, nH, nKV = S.head_dim, S.n_heads, S.n_kv_heads
        x = self.embed[tok].copy()
        for l, P in enumerate(self.layers):
            h = self.norm(x, P["attn_norm"])
            q = self.rnd(self.rope(P["wq"](h).reshape(nH, hd), pos))
            k = self.rnd(self.rope(P["wk"](h).reshape(nKV, hd), pos))
            v = self.rnd(P["wv"](h).reshape(nKV, hd))
            self.K[l, :, pos] = k
            self.V[l, :, pos] = v
            o = np.empty((nH, hd))
            for head in range(nH):
                g = head * nKV // nH
                sc = self.K[l, g, : pos + 1] @ q[head] / np.sqrt(hd)
                p = np.exp(sc - np.max(sc))
                o[head] = self.rnd((p @ self.V[l, g, : pos + 1]) / np.sum(p))
            x = self.rnd(x + P["wo"](o.reshape(-1)))
            h = self.norm(x, P["mlp_norm"])
            G, U = P["wg"](h), P["wu"](h)
            a = self.rnd(G * scipy.special.expit(G) * U)
            x = self.rnd(x + P["wd"](a))
        logits = self.lm(self.norm(x, self.final_norm))
        l32 = logits.astype(np.float32)
        tok = int(np.flatnonzero(l32 == l32.max())[0])
        return logits, tok


def _compare(shape, w, tokens, pos0=0, prefill=0, teacher=True):
    ref = O.OracleModel(shape, w)
    npm = NumpyModel(shape, w)
    if prefill:
        for l in range(shape.n_layers):
            kv = I.kv_prefill(shape, prefill, l)
            ref.set_kv(l, kv, 0)
            kvf = kv if shape.act_f32 else I.bf16_bits_to_f32(kv)
            npm.K[l, :, :prefill] = kvf[0]
            npm.V[l, :, :prefill] = kvf[1]
    worst = 0.0
    for i, t in enumerate(tokens):
        lo, _, to = ref.step(int(t), pos0 + i)
        ln, tn = npm.step(int(t), pos0 + i)
        scale = float(np.max(np.abs(lo)))
        err = float(np.max(np.abs(lo - ln))) / scale
        worst = max(worst, err)
        assert err <= 1e-9, f"step {i}: logits differ by {err:.3e} of max |logit|"
        assert to == tn, f"step {i}: greedy token {to} vs {tn}"
    ref.close()
    return worst


def _protocol_tokens(shape, w):
    """The tiny protocol's inputs: the prompt, then the oracle's own greedy tokens."""
    ref = O.OracleModel(shape, w)
    _, _, _, inputs = O.run_protocol(ref, shape, I.prompt_tokens(shape), shape.n_generate)
    ref.close()
    return inputs


def test_bf16_round_matches_torch_on_fp32_values():
    import torch
    rng = np.random.default_rng(11)
    x32 = (rng.standard_normal(4000) * 10.0 ** rng.integers(-30, 30, 4000)).astype(np.float32)
    want = torch.from_numpy(x32).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(bf16_round(x32.astype(np.float64)), want)
    # from double: slightly above a tie rounds up (no double rounding through fp32)
    assert bf16_round(np.array([1 + 2 ** -8 + 2 ** -40]))[0] == 1 + 2 ** -7
    assert bf16_round(np.array([1 + 2 ** -8]))[0] == 1.0


def test_restatement_tiny_fp32_protocol():
    shape = I.SHAPES["tiny_fp32"]
    w = I.make_weights(shape)
    toks = _protocol_tokens(shape, w)
    assert len(toks) == 23
    worst = _compare(shape, w, toks)
    print(f"tiny fp32, 23 steps: worst normwise logit difference {worst:.2e}")


@pytest.mark.slow
def test_restatement_smollm2_bf16_first_steps():
    shape = I.SHAPES["smollm2_135m_bf16"]
    w = I.make_weights(shape)
    worst = _compare(shape, w, I.prompt_tokens(shape)[:2])
    print(f"smollm2 bf16, 2 steps: worst normwise logit difference {worst:.2e}")


@pytest.mark.parametrize("wfmt", [I.WF_INT8, I.WF_INT4])
def test_restatement_quantised_with_history(wfmt):
    shape = I.tiny_shape(hidden=256, n_heads=4, n_kv_heads=2, head_dim=64, intermediate=384, vocab=300,
                         wfmt=wfmt, act_f32=False, max_ctx=48, seed=21 + wfmt)
    w = I.make_weights(shape)
    worst = _compare(shape, w, [3, 299, 17, 150], pos0=20, prefill=20)
    print(f"wfmt {wfmt}: worst normwise logit difference {worst:.2e}")
