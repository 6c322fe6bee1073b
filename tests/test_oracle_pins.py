"""Pins of the CPU oracle against facts fixed independently of it: closed forms, library
routines (numpy/torch casts, numpy matmul, scipy's logistic), brute force and invariants of
the decode step. Each test names the plausible oracle mistake it would catch."""
from fractions import Fraction
import math

import numpy as np
import pytest
import scipy.special

import amk_inputs as I
import oracle as O

F32, BF16, F16 = O.FMT_F32, O.FMT_BF16, O.FMT_F16


# ---------------------------------------------------------------- rounding

def test_round_f32_matches_numpy_cast():
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.standard_normal(2000) * 10.0 ** rng.integers(-40, 38, 2000),
                        [1e-45, 1.4e-45, 3e-39, -7e-42, 3.5e38, -3.41e38, 1.0 + 2.0 ** -24, 1.0 + 3 * 2.0 ** -24]])
    got = O.round_to(x, F32)
    with np.errstate(over="ignore"):
        want = x.astype(np.float32).astype(np.float64)
    np.testing.assert_array_equal(got, want)          # catches a wrong mantissa width or tie rule


def test_round_f16_matches_numpy_cast():
    rng = np.random.default_rng(2)
    x = np.concatenate([rng.standard_normal(2000) * 10.0 ** rng.integers(-9, 5, 2000),
                        [65504.0, 65519.99, 65520.0, -70000.0, 6.1e-5, 5.96e-8, 2.98e-8, 2.99e-8, 1 + 2 ** -11]])
    got = O.round_to(x, F16)
    with np.errstate(over="ignore"):
        want = x.astype(np.float16).astype(np.float64)   # numpy rounds double->half directly, to nearest even
    np.testing.assert_array_equal(got, want)          # catches subnormal spacing or overflow mistakes


def test_round_bf16_matches_torch_on_fp32_inputs():
    rng = np.random.default_rng(3)
    x32 = (rng.standard_normal(5000) * 10.0 ** rng.integers(-30, 30, 5000)).astype(np.float32)
    got = O.round_to(x32.astype(np.float64), BF16)
    import torch
    want = torch.from_numpy(x32).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(got, want)


def test_round_bf16_exact_ties_from_double():
    # 1 + 2^-8 lies exactly between bf16 neighbours 1 and 1 + 2^-7: ties go to the even one (1).
    # 1 + 3*2^-8 lies between 1 + 2^-7 (odd) and 1 + 2^-6 (even): goes up. Slightly above a
    # tie must round up (a double-rounding via fp32 would not see the extra bit at 2^-40).
    cases = {1 + 2 ** -8: 1.0, 1 + 3 * 2 ** -8: 1 + 2 ** -6, 1 + 2 ** -8 + 2 ** -40: 1 + 2 ** -7,
             -(1 + 2 ** -8): -1.0, 3.0e38 * 1.2: math.inf}
    for x, want in cases.items():
        assert O.round_to([x], BF16)[0] == want


# ---------------------------------------------------------------- RMSNorm

def test_rmsnorm_constant_power_of_two_input_gives_signed_gains():
    n = 64
    s = np.where(np.arange(n) % 3 == 0, -1.0, 1.0)
    g = 1.0 + 0.02 * np.random.default_rng(4).standard_normal(n)
    for c in (2.0 ** -6, 1.0, 2.0 ** 9):
        h = O.rmsnorm(c * s, g, 0.0, F32)
        np.testing.assert_array_equal(h, O.round_to(s * g, F32))   # x/rms(x) is exactly +-1 here


def test_rmsnorm_is_invariant_to_power_of_two_scaling():
    rng = np.random.default_rng(5)
    x = rng.standard_normal(576)
    g = 1 + 0.02 * rng.standard_normal(576)
    base = O.rmsnorm(x, g, 0.0, BF16)
    for k in (-20, -3, 7, 40):
        np.testing.assert_array_equal(O.rmsnorm(x * 2.0 ** k, g, 0.0, BF16), base)


def test_rmsnorm_unit_gain_output_has_unit_mean_square():
    rng = np.random.default_rng(6)
    for n in (16, 2048, 5632):
        h = O.rmsnorm(rng.standard_normal(n) * 3.7, np.ones(n), 0.0, F32)
        assert abs(np.sum(h * h) / n - 1.0) < 4 * 2.0 ** -24   # catches dividing by n-1 or a missing sqrt


def test_rmsnorm_eps_dominates_tiny_inputs():
    n, eps = 64, 1e-5
    x = np.full(n, 1e-9)
    h = O.rmsnorm(x, np.ones(n), eps, F32)
    want = O.round_to(x / math.sqrt(1e-18 + eps), F32)          # eps added inside the root
    np.testing.assert_allclose(h, want, rtol=1e-6)
    np.testing.assert_array_equal(O.rmsnorm(np.zeros(n), np.ones(n), eps, F32), np.zeros(n))


# ---------------------------------------------------------------- RoPE

def test_rope_position_zero_is_identity():
    u = np.random.default_rng(7).standard_normal(128)
    np.testing.assert_array_equal(O.rope(u, 0, 1e4), u)


def test_rope_half_split_pairs_and_frequencies():
    # hd = 4, theta = 100: pair 0 is (0, 2) at frequency 1, pair 1 is (1, 3) at 100^(-1/2) = 0.1.
    p = 3
    e0 = O.rope([1.0, 0.0, 0.0, 0.0], p, 100.0)
    np.testing.assert_allclose(e0, [math.cos(p), 0.0, math.sin(p), 0.0], atol=1e-15)
    e1 = O.rope([0.0, 1.0, 0.0, 0.0], p, 100.0)
    np.testing.assert_allclose(e1, [0.0, math.cos(0.1 * p), 0.0, math.sin(0.1 * p)], atol=1e-15)
    e3 = O.rope([0.0, 0.0, 0.0, 1.0], p, 100.0)                  # second member rotates the other way
    np.testing.assert_allclose(e3, [0.0, -math.sin(0.1 * p), 0.0, math.cos(0.1 * p)], atol=1e-15)


def test_rope_preserves_pair_norms_and_encodes_relative_position():
    rng = np.random.default_rng(8)
    hd = 64
    q, k = rng.standard_normal(hd), rng.standard_normal(hd)
    for p, s in ((5, 2), (512, 100), (4095, 7)):
        rq = O.rope(q, p, 1e4)
        pn = lambda u: u[: hd // 2] ** 2 + u[hd // 2:] ** 2
        np.testing.assert_allclose(pn(rq), pn(q), rtol=1e-12)
        lhs = float(np.dot(rq, O.rope(k, s, 1e4)))
        rhs = float(np.dot(O.rope(q, p - s, 1e4), k))
        assert abs(lhs - rhs) < 1e-9 * (1 + abs(rhs))
    np.testing.assert_allclose(O.rope(O.rope(q, 30, 5e5), 12, 5e5), O.rope(q, 42, 5e5), atol=1e-12)


# ---------------------------------------------------------------- attention

def test_attention_single_key_returns_value_exactly():
    rng = np.random.default_rng(9)
    for hd in (16, 64, 128):
        v = I.bf16_bits_to_f32(I.f32_to_bf16_bits(rng.standard_normal((1, hd)).astype(np.float32)))
        o = O.attention(rng.standard_normal(hd), rng.standard_normal((1, hd)), v, BF16)
        np.testing.assert_array_equal(o, v[0].astype(np.float64))


def test_attention_weights_sum_to_one_exactly():
    rng = np.random.default_rng(10)
    n, hd = 333, 64
    o = O.attention(rng.standard_normal(hd), rng.standard_normal((n, hd)), np.ones((n, hd)), F32)
    np.testing.assert_array_equal(o, np.ones(hd))


def test_attention_equal_keys_average_values():
    rng = np.random.default_rng(11)
    n, hd = 17, 16
    K = np.tile(rng.standard_normal(hd), (n, 1))
    V = rng.standard_normal((n, hd)).astype(np.float32)
    o = O.attention(rng.standard_normal(hd), K, V, F32)
    np.testing.assert_allclose(o, V.astype(np.float64).mean(0), rtol=2e-7, atol=1e-7)


def test_attention_two_keys_is_logistic_with_sqrt_hd_scale():
    hd = 64
    for t in (-3.0, 0.25, 2.0):
        q = np.zeros(hd); q[0] = 1.0
        K = np.zeros((2, hd)); K[1, 0] = t * math.sqrt(hd)      # scores 0 and t after the 1/sqrt(hd) scale
        V = np.zeros((2, hd), dtype=np.float32); V[0, 1] = 1.0; V[1, 2] = 1.0
        o = O.attention(q, K.astype(np.float32), V, F32)
        p1 = scipy.special.expit(t)
        np.testing.assert_allclose([o[1], o[2]], [1 - p1, p1], rtol=1e-7)


# ---------------------------------------------------------------- SwiGLU and argmax

def test_swiglu_closed_forms():
    assert O.swiglu(0.0, 3.0, F32) == 0.0
    for g, u in ((0.5, 2.0), (-1.25, 0.75), (8.0, -0.3), (-30.0, 1.0)):
        want = float(np.float32(g * scipy.special.expit(g) * u))
        assert O.swiglu(g, u, F32) == pytest.approx(want, rel=2 ** -23)
    assert O.swiglu(60.0, 1.0, F32) == 60.0                       # silu(z) -> z for large z


def test_argmax_lowest_index_wins_ties_and_nan_fails():
    v = np.array([0.5, 2.0, -1.0, 2.0, 2.0], dtype=np.float32)
    assert O.argmax_f32(v) == 1
    v[0] = np.nan
    assert O.argmax_f32(v) == -1
    assert O.argmax_f32(np.array([-np.inf, -3.0], dtype=np.float32)) == 1


# ---------------------------------------------------------------- quantisation

def _brute_nearest_even(t: float, qmax: int) -> int:
    """The integer nearest to t (ties to even), clamped, found by trying every candidate."""
    ft = Fraction(t)
    best = None
    # the minimiser is within one of t, or an endpoint when t is out of range
    window = set(range(max(-qmax, math.floor(t) - 2), min(qmax, math.ceil(t) + 2) + 1)) | {-qmax, qmax}
    for c in sorted(window):
        d = abs(ft - c)
        if best is None or d < best[0] or (d == best[0] and c % 2 == 0):
            best = (d, c)
    return best[1]


@pytest.mark.parametrize("group,qmax", [(0, 127), (128, 7)])
def test_quantize_matches_brute_force_definition(group, qmax):
    rng = np.random.default_rng(12 + qmax)
    rows, cols = 6, 256
    w32 = (rng.standard_normal((rows, cols)) * 0.02).astype(np.float32)
    w32[1] *= 100.0                                 # a row with larger magnitude
    w32[2, :128] *= 0.01                            # a quiet first group
    w32[3] = 0.0                                    # an all-zero row
    wb = I.f32_to_bf16_bits(w32)
    wf = I.bf16_bits_to_f32(wb)
    q, s = O.quantize(wb, group, qmax)
    g = group or cols
    for r in range(rows):
        for b in range(cols // g):
            blk = wf[r, b * g:(b + 1) * g]
            a = np.float32(np.max(np.abs(blk)))
            s_want = np.float16(np.float32(a) / np.float32(qmax))          # numpy's own casts
            s_got = s[r, b] if group else s[r]
            assert np.float32(s_got) == np.float32(s_want)
            for k in range(g):
                if s_want == 0:
                    assert q[r, b * g + k] == 0
                    continue
                t = float(np.float32(blk[k]) / np.float32(s_want))
                assert q[r, b * g + k] == _brute_nearest_even(t, qmax), (r, b, k)


@pytest.mark.parametrize("group,qmax", [(0, 127), (128, 7)])
def test_quantize_error_bound_and_extremes(group, qmax):
    rng = np.random.default_rng(20 + qmax)
    wb = I.f32_to_bf16_bits((rng.standard_normal((64, 512)) * 0.02).astype(np.float32))
    wf = I.bf16_bits_to_f32(wb).astype(np.float64)
    q, s = O.quantize(wb, group, qmax)
    assert q.min() >= -qmax and q.max() <= qmax
    sc = np.repeat(s, group, axis=1) if group else s[:, None]
    err = np.abs(wf - sc * q)
    # unclamped codes are within half a step; the absmax element of each group lands on +-qmax
    unclamped = np.abs(q) < qmax
    assert np.all(err[unclamped] <= np.broadcast_to(sc, err.shape)[unclamped] * 0.5 * (1 + 1e-6))
    gsz = group or 512
    blocks = np.abs(wf).reshape(64, 512 // gsz, gsz)
    arg = blocks.argmax(axis=2)
    qb = np.abs(q.reshape(64, 512 // gsz, gsz))
    assert np.all(np.take_along_axis(qb, arg[..., None], axis=2) == qmax)


# ---------------------------------------------------------------- whole-step invariants

def _model(shape, weights):
    return O.OracleModel(shape, weights)


def _ones_pattern(n, k):
    return np.where((np.arange(n) * 7 + k) % 5 < 2, -1.0, 1.0)


def test_zero_layer_model_is_lm_head_times_normalised_embedding():
    shape = I.tiny_shape(n_layers=0, rms_eps=0.0)
    w = I.make_weights(shape)
    emb = np.stack([_ones_pattern(shape.hidden, t) * 2.0 ** (t % 5 - 2) for t in range(shape.vocab)]).astype(np.float32)
    w.embed = emb
    w.final_norm = np.ones(shape.hidden, dtype=np.float32)
    m = _model(shape, w)
    for t in (0, 3, 77):
        lg, lg32, tok = m.step(t, 0)
        want = w.lm_head.astype(np.float64) @ _ones_pattern(shape.hidden, t)   # numpy matmul
        np.testing.assert_allclose(lg, want, rtol=1e-12, atol=1e-15)
        assert tok == int(np.argmax(lg32))


def test_zero_layer_int8_lm_head_applies_row_scales_after_the_sum():
    shape = I.tiny_shape(n_layers=0, rms_eps=0.0, wfmt=I.WF_INT8, act_f32=False)
    w = I.make_weights(shape)
    emb = np.stack([_ones_pattern(shape.hidden, t) for t in range(shape.vocab)]).astype(np.float32)
    w.embed = I.f32_to_bf16_bits(emb)
    w.final_norm = I.f32_to_bf16_bits(np.ones(shape.hidden, dtype=np.float32))
    m = _model(shape, w)
    q, s = m.codes(O.W_LM_HEAD)
    q_ind, s_ind = O.quantize(w.lm_head, 0, 127)
    np.testing.assert_array_equal(q, q_ind)
    lg, _, _ = m.step(9, 0)
    h = _ones_pattern(shape.hidden, 9)
    np.testing.assert_allclose(lg, (q.astype(np.float64) @ h) * s.astype(np.float64), rtol=1e-13)


def _wiring_shape(**kw):
    base = dict(n_layers=1, n_heads=4, n_kv_heads=4, head_dim=16, hidden=64, rms_eps=0.0)
    base.update(kw)
    return I.tiny_shape(**base)


def test_one_layer_closed_form_wiring():
    """W_v = W_o = I and W_q = W_k = W_g = 0: attention returns the mean of the cached values
    (uniform scores), the MLP adds nothing, and the residual stream carries the sums."""
    shape = _wiring_shape()
    H = shape.hidden
    w = I.make_weights(shape)
    L = w.layers[0]
    L["wq"][:] = 0; L["wk"][:] = 0; L["wg"][:] = 0
    L["wv"][:] = np.eye(H, dtype=np.float32); L["wo"][:] = np.eye(H, dtype=np.float32)
    L["attn_norm"][:] = 1.0
    emb = np.stack([_ones_pattern(H, t) * (1 + t % 3) for t in range(shape.vocab)]).astype(np.float32)
    w.embed = emb
    m = _model(shape, w)
    x0, x1 = emb[5].astype(np.float64), emb[11].astype(np.float64)
    h0, h1 = _ones_pattern(H, 5), _ones_pattern(H, 11)        # RMSNorm of +-c patterns with g = 1
    gf = w.final_norm.astype(np.float64)

    def final_logits(x):
        hn = (x / np.sqrt(np.mean(x * x))) * gf
        return w.lm_head.astype(np.float64) @ hn.astype(np.float32).astype(np.float64)

    lg, _, _ = m.step(5, 0)                                       # attention over one key: o = v = h0
    np.testing.assert_allclose(lg, final_logits(x0 + h0), rtol=1e-6, atol=1e-7)
    lg, _, _ = m.step(11, 1)                                      # uniform over two keys: o = (h0 + h1)/2
    np.testing.assert_allclose(lg, final_logits(x1 + (h0 + h1) / 2), rtol=1e-6, atol=1e-7)


def test_one_layer_mlp_closed_form_wiring():
    """The MLP block alone, with every operand distinguishable: W_o = 0 (attention adds
    nothing), attention-norm gains of 3 and MLP-norm gains g_m in {0.5, ..., 1.5}, so
    RMSNorm(x) of the +-c embedding pattern is exactly +-g_m; W_g and W_u pick different
    elements with different coefficients (G_j = alpha_j h[j mod H], U_j = beta_j h[(j+7) mod H]);
    W_d sums a over j = i (mod H) times gamma. The expected logits come from numpy matmuls and
    scipy's logistic: silu(G) = G * expit(G), a = fp32(silu(G) U), x' = fp32(x + W_d a).
    Catches: the SiLU applied to the up projection, the MLP norm taking the attention gains or
    being dropped, the down residual dropped, the SwiGLU product's operands crossed."""
    shape = _wiring_shape()
    H, Imid = shape.hidden, shape.intermediate
    w = I.make_weights(shape)
    L = w.layers[0]
    L["wq"][:] = 0; L["wk"][:] = 0; L["wo"][:] = 0
    L["attn_norm"][:] = 3.0
    gm = (1.0 + 0.25 * (np.arange(H) % 5 - 2)).astype(np.float32)
    L["mlp_norm"][:] = gm
    j = np.arange(Imid)
    alpha = (0.5 + 0.25 * (j % 7)).astype(np.float32)
    beta = (-1.0 + 0.5 * (j % 5)).astype(np.float32)
    beta[beta == 0] = 0.75                                        # every U_j non-zero
    wg = np.zeros((Imid, H), np.float32); wg[j, j % H] = alpha
    wu = np.zeros((Imid, H), np.float32); wu[j, (j + 7) % H] = beta
    gamma = np.float32(0.375)
    wd = np.zeros((H, Imid), np.float32); wd[j % H, j] = gamma
    L["wg"][:] = wg; L["wu"][:] = wu; L["wd"][:] = wd
    emb = np.stack([_ones_pattern(H, t) * (1 + t % 3) for t in range(shape.vocab)]).astype(np.float32)
    w.embed = emb
    m = _model(shape, w)
    gf = w.final_norm.astype(np.float64)
    for pos, t in enumerate((5, 11)):                             # c = 3 and c = 3: norm != identity
        x = emb[t].astype(np.float64)
        h = _ones_pattern(H, t) * gm.astype(np.float64)           # RMSNorm(+-c) * g_m, exact
        G = wg.astype(np.float64) @ h
        U = wu.astype(np.float64) @ h
        a = (G * scipy.special.expit(G) * U).astype(np.float32).astype(np.float64)
        x1 = (x + wd.astype(np.float64) @ a).astype(np.float32).astype(np.float64)
        hn = ((x1 / np.sqrt(np.mean(x1 * x1))) * gf).astype(np.float32).astype(np.float64)
        want = w.lm_head.astype(np.float64) @ hn
        lg, _, _ = m.step(t, pos)
        np.testing.assert_allclose(lg, want, rtol=1e-6, atol=1e-7)


def test_one_layer_cache_rows_hold_each_steps_keys_and_values():
    """With W_k = W_v = I the cache row written at position p holds RoPE_p(h_p) and h_p."""
    shape = _wiring_shape()
    H, hd = shape.hidden, shape.head_dim
    w = I.make_weights(shape)
    L = w.layers[0]
    L["wk"][:] = np.eye(H, dtype=np.float32); L["wv"][:] = np.eye(H, dtype=np.float32)
    L["attn_norm"][:] = 1.0
    w.embed = np.stack([_ones_pattern(H, t) * (1 + t % 3) for t in range(shape.vocab)]).astype(np.float32)
    m = _model(shape, w)
    toks = [5, 11, 2]
    for p, t in enumerate(toks):
        m.step(t, p)
    for p, t in enumerate(toks):
        h = _ones_pattern(H, t)
        for g in range(shape.n_kv_heads):
            hv = h[g * hd:(g + 1) * hd]
            np.testing.assert_array_equal(m.get_kv(0, 1, g, p, 1)[0], hv.astype(np.float32))
            want_k = O.round_to(O.rope(hv, p, shape.rope_theta), F32)
            np.testing.assert_array_equal(m.get_kv(0, 0, g, p, 1)[0], want_k.astype(np.float32))


def test_gqa_equals_mha_with_duplicated_kv_heads():
    """Query head h reads KV group floor(h * nKV / nH): a GQA model and the MHA model whose KV
    heads repeat each group for its consecutive query heads give identical logits."""
    gqa = I.tiny_shape(n_layers=2, n_heads=4, n_kv_heads=2)
    mha = gqa.replace(n_kv_heads=4)
    wg = I.make_weights(gqa)
    wm = I.make_weights(gqa)
    hd = gqa.head_dim
    for l in range(gqa.n_layers):
        for n in ("wk", "wv"):
            src = wg.layers[l][n]
            wm.layers[l][n] = np.concatenate([src[(h // 2) * hd:(h // 2 + 1) * hd] for h in range(4)])
    a, b = _model(gqa, wg), _model(mha, wm)
    for pos, tok in enumerate([3, 9, 250, 17, 4]):
        la, _, ta = a.step(tok, pos)
        lb, _, tb = b.step(tok, pos)
        np.testing.assert_array_equal(la, lb)
        assert ta == tb


def test_cache_rows_beyond_position_are_never_read():
    shape = I.tiny_shape(n_layers=2)
    w = I.make_weights(shape)
    a, b = _model(shape, w), _model(shape, w)
    nan = np.full((2, shape.n_kv_heads, shape.max_ctx - 4, shape.head_dim), np.nan, dtype=np.float32)
    for l in range(shape.n_layers):
        b.set_kv(l, nan, pos0=4)
    for pos, tok in enumerate([1, 2, 3, 4]):
        la, _, _ = a.step(tok, pos)
        lb, _, _ = b.step(tok, pos)
        np.testing.assert_array_equal(la, lb)


def test_step_is_idempotent_at_a_fixed_position():
    shape = I.tiny_shape()
    m = _model(shape, I.make_weights(shape))
    m.step(5, 0)
    first = m.step(7, 1)[0]
    again = m.step(7, 1)[0]                                       # rewrites the same cache row
    np.testing.assert_array_equal(first, again)


@pytest.mark.parametrize("wfmt,group", [(I.WF_INT8, 0), (I.WF_INT4, 128)])
def test_quantised_model_equals_fp32_model_on_dequantised_weights(wfmt, group):
    """The int model scales once after each (group) sum; the fp32 model multiplies the exact
    dequantised weights s*q. Both are evaluated in double, so they agree to rounding noise."""
    qshape = I.tiny_shape(hidden=256, n_heads=4, n_kv_heads=2, head_dim=64, intermediate=384, vocab=300,
                          wfmt=wfmt, act_f32=False)
    fshape = qshape.replace(wfmt=I.WF_F32)
    wq = I.make_weights(qshape)
    qm = _model(qshape, wq)
    wf = I.Weights(embed=I.bf16_bits_to_f32(wq.embed), final_norm=I.bf16_bits_to_f32(wq.final_norm),
                   lm_head=None, layers=[])
    kinds = dict(wq=O.W_WQ, wk=O.W_WK, wv=O.W_WV, wo=O.W_WO, wg=O.W_WG, wu=O.W_WU, wd=O.W_WD)

    def deq(kind, layer):
        q, s = qm.codes(kind, layer)
        sc = np.repeat(s, group, axis=1) if group else s[:, None]
        return (q.astype(np.float64) * sc).astype(np.float32)      # exact: <= 11 + 7 bits

    wf.lm_head = deq(O.W_LM_HEAD, 0)
    for l in range(qshape.n_layers):
        d = {n: deq(k, l) for n, k in kinds.items()}
        d["attn_norm"] = I.bf16_bits_to_f32(wq.layers[l]["attn_norm"])
        d["mlp_norm"] = I.bf16_bits_to_f32(wq.layers[l]["mlp_norm"])
        wf.layers.append(d)
    fm = _model(fshape, wf)
    for pos, tok in enumerate([1, 200, 33, 7]):
        la, _, ta = qm.step(tok, pos)
        lb, _, tb = fm.step(tok, pos)
        np.testing.assert_allclose(la, lb, rtol=1e-9, atol=1e-12)
        assert ta == tb


def test_protocol_step_count_and_teacher_forcing():
    shape = I.SHAPES["tiny_fp32"]
    m = _model(shape, I.make_weights(shape))
    prompt = I.prompt_tokens(shape)
    gen, logits, margins, inputs = O.run_protocol(m, shape, prompt, shape.n_generate)
    assert len(logits) == len(prompt) + shape.n_generate - 1 == 23
    assert len(gen) == 16 and inputs[: len(prompt)] == list(prompt)
    assert inputs[len(prompt):] == gen[:-1]
    m2 = _model(shape, I.make_weights(shape))
    gen2, logits2, _, _ = O.run_protocol(m2, shape, prompt, shape.n_generate, forced=gen)
    assert gen2 == gen
    for a, b in zip(logits, logits2):
        np.testing.assert_array_equal(a, b)
