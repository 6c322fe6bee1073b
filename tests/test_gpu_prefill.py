"""Parity of the prompt prefill (amk_prefill, matrix-core GEMM tiles over many tokens per launch)
with the CPU oracle, called through the C ABI.

The prefill of tokens t_0 .. t_{n-1} at positions pos0 .. pos0+n-1 is defined as n chained
decode steps fed those tokens: the oracle runs exactly that, step by step, and the GPU must
match its K/V cache rows for every prompt position and the logits and greedy token of the last
step. Bars, as for the decode path:
  * fp32 workloads: logits within 1e-4 max normwise relative error, greedy token identical,
    cache rows within 1e-4 normwise relative error per (layer, K or V);
  * bf16 / int workloads limited to one or two layers at full width: logits within 2e-2 max
    absolute error, the token identical wherever the oracle's top-2 margin exceeds 2e-2; the
    first layer's cache rows within 2 bf16 ulps (|d| <= 2^-7 |ref| + 1e-3: its inputs are
    exact, the GPU sums in fp32 in another order and may round a value next to a rounding
    boundary the other way), later layers' within 1e-2 normwise relative error (their inputs
    already carry those one-ulp differences, which the projections sum);
  * two TinyLlama-shaped layers over a 256-token prompt: logits within 0.075 (three one-ulp
    flips two layers deep, pinned on the CPU), cache rows as above;
  * the full-depth int8 workload: logits within 0.25 max absolute and 0.05 RMS error (the
    decode path's full-depth bar), the token the argmax of the GPU's own logits.
"""
from __future__ import annotations

import numpy as np
import pytest

import amk_inputs as I
import oracle
from gpu_util import log, logit_err, prefill_both, tol_of

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

MARGIN = 2e-2
# two-layer bar for long prompts: three one-ulp rounding flips of the first layer's outputs (one
# moves TinyLlama-width logits by about 0.02 two layers deep; pinned on the CPU by
# test_oracle_sensitivity.py::test_one_ulp_flip_moves_two_layer_logits)
TWO_LAYER_ABS = 0.075


@pytest.fixture(scope="module")
def M():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import persistent_megakernel_amd as M
    M.lib()
    return M


def _oracle_prefill(ref, shape, tokens, pos0):
    """The definition: one oracle decode step per prompt token. -> (logits64, logits32, token)."""
    out = None
    for i, t in enumerate(tokens):
        out = ref.step(int(t), pos0 + i)
    return out


def _kv_rows(dec, layer, kv, g, pos0, n):
    t = dec.kv[layer, kv, g, pos0:pos0 + n, :]
    if t.dtype == torch.bfloat16:
        t = t.float()
    return t.cpu().numpy().astype(np.float64)


def _check_kv(M, dec, ref, shape, pos0, n, label):
    worst = 0.0
    for l in range(shape.n_layers):
        for kv in range(2):
            for g in range(shape.n_kv_heads):
                got = _kv_rows(dec, l, kv, g, pos0, n)
                want = ref.get_kv(l, kv, g, pos0, n).astype(np.float64)
                if shape.act_f32:
                    err = float(np.max(np.abs(got - want)) / max(np.max(np.abs(want)), 1e-30))
                    assert err <= 1e-4, f"{label}: layer {l} kv {kv} group {g} normwise rel err {err:.3e}"
                elif l == 0:
                    bound = 2.0 ** -7 * np.abs(want) + 1e-3
                    bad = np.abs(got - want) > bound
                    assert not bad.any(), (f"{label}: layer {l} kv {kv} group {g}: {int(bad.sum())} values "
                                           f"beyond 2 ulps, worst {float(np.max(np.abs(got - want))):.3e}")
                    err = float(np.max(np.abs(got - want)))
                else:
                    err = float(np.max(np.abs(got - want)) / max(np.max(np.abs(want)), 1e-30))
                    assert err <= 1e-2, f"{label}: layer {l} kv {kv} group {g} normwise rel err {err:.3e}"
                worst = max(worst, err)
    return worst


def _run(M, shape, n, pos0=0, history=0, max_ctx=None, seed_stream=3, w=None, check_kv=True):
    w = w if w is not None else I.make_weights(shape)
    ref = oracle.OracleModel(shape, w, max_ctx=max_ctx)
    dec = M.Decoder(shape, w, max_ctx=max_ctx)
    if history:
        prefill_both(dec, ref, shape, history)
    tokens = I.prompt_tokens(shape, n, stream=seed_stream)
    lg64, lg32, tok = _oracle_prefill(ref, shape, tokens, pos0)
    tin = torch.tensor(tokens, dtype=torch.int32, device="cuda")
    tout = torch.full((1,), -7, dtype=torch.int32, device="cuda")
    lg = torch.zeros(shape.vocab, dtype=torch.float32, device="cuda")
    dec.prefill(tin, pos0, tout, lg)
    torch.cuda.synchronize()
    assert dec.status() == 0
    glog = lg.cpu().numpy()
    gtok = int(tout.item())
    err = logit_err(shape, glog, lg32)
    kv_err = _check_kv(M, dec, ref, shape, pos0, n, shape.name) if check_kv else None
    margin = oracle.top2_margin(lg32)
    return dict(ref=ref, dec=dec, tok=tok, gtok=gtok, err=err, kv_err=kv_err, margin=margin, glog=glog,
                tokens=tokens, ref32=lg32)


def _close(r):
    r["dec"].close()
    r["ref"].close()


def _assert_token(r, label):
    if r["gtok"] != r["tok"]:
        assert r["margin"] < max(MARGIN, 2 * r["err"]), f"{label}: token {r['gtok']} != oracle {r['tok']} at margin {r['margin']:.3e}"
        log(f"{label}: picked {r['gtok']} over oracle {r['tok']} at margin {r['margin']:.3e} (allowed)")
    assert r["gtok"] == int(np.flatnonzero(r["glog"] == r["glog"].max())[0])


# ------------------------------------------------------------------ fp32

@pytest.mark.parametrize("n,pos0,history", [(1, 0, 0), (8, 0, 0), (64, 0, 0), (65, 0, 0), (200, 7, 7), (300, 5, 5)])
def test_tiny_fp32_prefill(M, n, pos0, history):
    """Inside one M-tile, exactly one, one plus a row, several with a history before them, and
    two launches (256 + 44 tokens)."""
    shape = I.SHAPES["tiny_fp32"]
    log(f"case prefill tiny_fp32 n={n} pos0={pos0}")
    r = _run(M, shape, n, pos0=pos0, history=history, max_ctx=320)
    log(f"tiny_fp32 n={n}: logits err {r['err']:.3e}, kv err {r['kv_err']:.3e}")
    assert r["err"] <= tol_of(shape)
    assert r["gtok"] == r["tok"]
    _close(r)


def test_tiny_fp32_decode_continues_from_prefilled_rows(M):
    """Decode steps after a prefill read the cache rows it wrote: the chained continuation
    equals the oracle's."""
    shape = I.SHAPES["tiny_fp32"]
    log("case prefill then decode tiny_fp32")
    r = _run(M, shape, 37, max_ctx=64)
    dec, ref = r["dec"], r["ref"]
    tok, gtok = r["tok"], r["gtok"]
    assert gtok == tok
    buf = torch.tensor([gtok, -1], dtype=torch.int32, device="cuda")
    lg = torch.zeros(shape.vocab, dtype=torch.float32, device="cuda")
    for s in range(6):
        pos = 37 + s
        _, ref32, tok = ref.step(tok, pos)
        dec.step(buf[0:1], pos, buf[1:2], lg)
        torch.cuda.synchronize()
        assert logit_err(shape, lg.cpu().numpy(), ref32) <= tol_of(shape)
        assert int(buf[1].item()) == tok
        buf[0] = buf[1]
    _close(r)


def test_tiny_fp32_repeated_prefill_is_identical(M):
    """The counters of a schedule keep growing from launch to launch; results do not change."""
    shape = I.SHAPES["tiny_fp32"]
    w = I.make_weights(shape)
    dec = M.Decoder(shape, w, max_ctx=128)
    tin = torch.tensor(I.prompt_tokens(shape, 70, stream=5), dtype=torch.int32, device="cuda")
    outs = []
    for _ in range(4):
        tout = torch.zeros(1, dtype=torch.int32, device="cuda")
        lg = torch.zeros(shape.vocab, dtype=torch.float32, device="cuda")
        dec.prefill(tin, 3, tout, lg)
        torch.cuda.synchronize()
        outs.append((int(tout.item()), lg.cpu().numpy().copy(), dec.kv.clone()))
    assert dec.status() == 0
    for t, l, kv in outs[1:]:
        assert t == outs[0][0]
        assert np.array_equal(l, outs[0][1])
        assert torch.equal(kv, outs[0][2])
    dec.close()


def test_bad_token_is_replaced_and_flagged(M):
    shape = I.SHAPES["tiny_fp32"]
    w = I.make_weights(shape)
    dec = M.Decoder(shape, w, max_ctx=64)
    ref = oracle.OracleModel(shape, w, max_ctx=64)
    toks = list(I.prompt_tokens(shape, 6, stream=9))
    bad = list(toks)
    bad[2] = shape.vocab + 5
    toks[2] = 0
    _, lg32, tok = _oracle_prefill(ref, shape, toks, 0)
    tout = torch.zeros(1, dtype=torch.int32, device="cuda")
    lg = torch.zeros(shape.vocab, dtype=torch.float32, device="cuda")
    dec.prefill(torch.tensor(bad, dtype=torch.int32, device="cuda"), 0, tout, lg)
    torch.cuda.synchronize()
    assert dec.status() & 2
    assert logit_err(shape, lg.cpu().numpy(), lg32) <= tol_of(shape)
    assert int(tout.item()) == tok
    dec.close()
    ref.close()


def test_invalid_arguments_are_refused(M):
    shape = I.SHAPES["tiny_fp32"]
    dec = M.Decoder(shape, I.make_weights(shape), max_ctx=32)
    t = torch.zeros(40, dtype=torch.int32, device="cuda")
    o = torch.zeros(1, dtype=torch.int32, device="cuda")
    for tok, pos0 in ((t[:33], 0), (t[:10], 23), (t[:1], -1)):
        with pytest.raises(M.AmkError) as e:
            dec.prefill(tok, pos0, o)
        assert e.value.status == M._abi.AMK_E_INVALID_ARG
    rc = M.amk_prefill(dec.ctx, t.data_ptr(), 0, 0, o.data_ptr())
    assert rc == M._abi.AMK_E_INVALID_ARG
    dec.close()


# ------------------------------------------------------------------ bf16 / int8 / int4, limited depth

@pytest.mark.parametrize("name,layers,n,pos0", [
    ("smollm2_135m_bf16", 2, 40, 0),     # K = 576: a partial K stage; 9 query heads over 3 groups; tied LM
    ("tinyllama_int8", 2, 70, 100),      # int8 per-row scales; two M-tiles after 100 history rows
    ("llama7b_bf16", 1, 33, 64),         # head_dim 128: 128-column QKV tiles; 32 KV heads
    ("llama3_8b_int4", 1, 20, 16),       # int4 group scales; head_dim 128; 128k vocabulary
])
def test_limited_depth_prefill(M, name, layers, n, pos0):
    shape = I.SHAPES[name].replace(n_layers=layers)
    log(f"case prefill {name} layers={layers} n={n} pos0={pos0}")
    r = _run(M, shape, n, pos0=pos0, history=pos0, max_ctx=pos0 + n + 8)
    log(f"{name}: logits err {r['err']:.3e}, kv err {r['kv_err']:.3e}, margin {r['margin']:.3e}")
    assert r["err"] <= tol_of(shape)
    _assert_token(r, name)
    _close(r)


@pytest.mark.parametrize("wfmt", [I.WF_INT8, I.WF_INT4], ids=["int8", "int4"])
def test_two_layer_tinyllama_256_tokens_wide_gateup(M, wfmt):
    """Two TinyLlama-shaped layers, a 256-token prompt in one launch: at 256 tokens the
    lowering gives gate/up tiles of 176 weight rows (88 j), the wide GEMM tile, staged 128
    input columns at a time. Every row of such a tile must be staged: the SwiGLU output feeds
    the second layer, whose K/V rows and the logits are held at the limited-depth bar."""
    shape = I.SHAPES["tinyllama_int8"].replace(n_layers=2, wfmt=wfmt, name=f"tinyllama_2l_w{wfmt}")
    n = 256
    log(f"case prefill {shape.name} n={n} (wide gate/up tiles)")
    r = _run(M, shape, n, max_ctx=264, seed_stream=11)
    log(f"{shape.name}: logits err {r['err']:.3e}, kv err {r['kv_err']:.3e}, margin {r['margin']:.3e}")
    assert r["err"] <= TWO_LAYER_ABS
    _assert_token(r, shape.name)
    _close(r)


def test_full_depth_tinyllama_int8_prefill(M):
    shape = I.SHAPES["tinyllama_int8"]
    n = 24
    log(f"case prefill tinyllama_int8 full depth n={n}")
    r = _run(M, shape, n, max_ctx=64, check_kv=False)
    rms = float(np.sqrt(np.mean((r["glog"].astype(np.float64) - r["ref32"].astype(np.float64)) ** 2)))
    log(f"tinyllama_int8 full depth: logits max abs err {r['err']:.3e}, rms {rms:.3e}, margin {r['margin']:.3e}")
    assert r["err"] <= 0.25 and rms <= 0.05
    _assert_token(r, "tinyllama_int8 full depth")
    _close(r)


def test_full_depth_tinyllama_int8_prefill_in_the_benchmarked_configuration(M):
    """The prefill the benchmark times: TinyLlama-shaped int8 at full depth, a 256-token prompt
    at position 0 in one launch (four M-tiles, gate/up tiles of 176 weight rows). The oracle's 256 chained
    steps decide the logits (full-depth bar); the K/V rows of the first layer, whose inputs are
    exact, are checked at 16 sampled positions across the four M-tiles."""
    shape = I.SHAPES["tinyllama_int8"]
    n = 256
    log(f"case prefill tinyllama_int8 full depth n={n} (benchmarked launch)")
    r = _run(M, shape, n, max_ctx=1024, seed_stream=7, check_kv=False)
    rms = float(np.sqrt(np.mean((r["glog"].astype(np.float64) - r["ref32"].astype(np.float64)) ** 2)))
    worst = 0.0
    for p in np.linspace(0, n - 1, 16).astype(int):
        for kv in range(2):
            for g in range(shape.n_kv_heads):
                got = _kv_rows(r["dec"], 0, kv, g, int(p), 1)
                want = r["ref"].get_kv(0, kv, g, int(p), 1).astype(np.float64)
                assert np.all(np.abs(got - want) <= 2.0 ** -7 * np.abs(want) + 1e-3), (p, kv, g)
                worst = max(worst, float(np.max(np.abs(got - want))))
    log(f"tinyllama_int8 full depth n={n}: logits max abs err {r['err']:.3e}, rms {rms:.3e}, "
        f"layer-0 kv worst {worst:.3e}, margin {r['margin']:.3e}")
    assert r["err"] <= 0.25 and rms <= 0.05
    _assert_token(r, "tinyllama_int8 full depth 256")
    _close(r)
