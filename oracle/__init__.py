"""CPU oracle of the batch-1 greedy decode step (plain C in fp64, see oracle.c) and of the
schedule validator (validator_ref.py, interleave.py).

TEST INFRASTRUCTURE ONLY: only tests/, __graft_entry__.smoke() and the cpu_baseline leg of
bench.py may import this package. It shares no code with the GPU path; the only module both
sides use is the seeded input generator amk_inputs.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess
import threading

import numpy as np

import amk_inputs as I

_HERE = os.path.dirname(os.path.abspath(__file__))
# AMK_ORACLE_LIB points the wrapper at another build of oracle.c (the mutation tests use it)
LIB_PATH = os.environ.get("AMK_ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")
SRC_PATH = os.path.join(_HERE, "oracle.c")

FMT_F32, FMT_BF16, FMT_F16 = 0, 1, 2
W_EMBED, W_FINAL_NORM, W_LM_HEAD = 0, 1, 2
W_ATTN_NORM, W_WQ, W_WK, W_WV, W_WO, W_MLP_NORM, W_WG, W_WU, W_WD = range(10, 19)
_KIND = dict(attn_norm=W_ATTN_NORM, wq=W_WQ, wk=W_WK, wv=W_WV, wo=W_WO, mlp_norm=W_MLP_NORM,
             wg=W_WG, wu=W_WU, wd=W_WD)


def build(force: bool = False) -> str:
    """Compile liboracle.so with gcc (plain C, OpenMP over output rows, no fast-math)."""
    if force or not os.path.exists(LIB_PATH):
        tmp = LIB_PATH + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
               "-Wall", "-o", tmp, SRC_PATH, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, LIB_PATH)
    return LIB_PATH


class _Desc(C.Structure):
    _fields_ = [("hidden", C.c_int), ("n_layers", C.c_int), ("n_heads", C.c_int), ("n_kv_heads", C.c_int),
                ("head_dim", C.c_int), ("intermediate", C.c_int), ("vocab", C.c_int), ("max_ctx", C.c_int),
                ("tied", C.c_int), ("wfmt", C.c_int), ("act_f32", C.c_int),
                ("rope_theta", C.c_double), ("rms_eps", C.c_double)]


_lib = None
_lock = threading.Lock()


def lib() -> C.CDLL:
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                build()
            L = C.CDLL(LIB_PATH)
            dp, fp, ip = C.POINTER(C.c_double), C.POINTER(C.c_float), C.POINTER(C.c_int)
            L.orc_round.restype = C.c_double
            L.orc_round.argtypes = [C.c_double, C.c_int]
            L.orc_quantize.restype = C.c_int
            L.orc_quantize.argtypes = [C.c_void_p, C.c_int64, C.c_int64, C.c_int, C.c_int, C.c_void_p, C.c_void_p]
            L.orc_set_threads.argtypes = [C.c_int]
            L.orc_set_threads.restype = C.c_int
            L.orc_rmsnorm.restype = None
            L.orc_rmsnorm.argtypes = [dp, dp, C.c_int, C.c_double, C.c_int, dp]
            L.orc_rope.restype = None
            L.orc_rope.argtypes = [dp, C.c_int, C.c_int, C.c_double]
            L.orc_attention.restype = None
            L.orc_attention.argtypes = [dp, fp, fp, C.c_int, C.c_int, C.c_int, dp, dp]
            L.orc_swiglu.restype = C.c_double
            L.orc_swiglu.argtypes = [C.c_double, C.c_double, C.c_int]
            L.orc_argmax_f32.restype = C.c_int
            L.orc_argmax_f32.argtypes = [fp, C.c_int64]
            L.orc_create.restype = C.c_void_p
            L.orc_create.argtypes = [C.POINTER(_Desc)]
            L.orc_destroy.restype = None
            L.orc_destroy.argtypes = [C.c_void_p]
            L.orc_set_weight.restype = C.c_int
            L.orc_set_weight.argtypes = [C.c_void_p, C.c_int, C.c_int, C.c_void_p]
            L.orc_set_kv.restype = C.c_int
            L.orc_set_kv.argtypes = [C.c_void_p, C.c_int, C.c_int, C.c_int, C.c_int, C.c_int, fp]
            L.orc_get_kv.restype = C.c_int
            L.orc_get_kv.argtypes = [C.c_void_p, C.c_int, C.c_int, C.c_int, C.c_int, C.c_int, fp]
            L.orc_step.restype = C.c_int
            L.orc_step.argtypes = [C.c_void_p, C.c_int, C.c_int, dp, fp, ip]
            L.orc_get_codes.restype = C.c_int
            L.orc_get_codes.argtypes = [C.c_void_p, C.c_int, C.c_int, C.c_void_p, C.c_void_p]
            L.orc_rounding_mode_is_nearest.restype = C.c_int
            _lib = L
    return _lib


def set_threads(n: int) -> int:
    """Threads of the oracle's OpenMP loops from now on; returns the count in effect."""
    return int(lib().orc_set_threads(int(n)))


def _dp(a):
    return a.ctypes.data_as(C.POINTER(C.c_double))


def _fp(a):
    return a.ctypes.data_as(C.POINTER(C.c_float))


# ---------------------------------------------------------------- single ops

def round_to(x, fmt: int) -> np.ndarray:
    f = lib().orc_round
    x = np.asarray(x, dtype=np.float64)
    return np.array([f(float(v), fmt) for v in x.ravel()], dtype=np.float64).reshape(x.shape)


def quantize(master_bf16: np.ndarray, group: int, qmax: int):
    """(codes int8 [rows, cols], scales fp32 [rows] or [rows, cols/group])."""
    w = np.ascontiguousarray(master_bf16, dtype=np.uint16)
    rows, cols = w.shape
    q = np.empty((rows, cols), dtype=np.int8)
    ns = rows * (cols // group) if group else rows
    s = np.empty(ns, dtype=np.float32)
    rc = lib().orc_quantize(w.ctypes.data, rows, cols, group, qmax, q.ctypes.data, s.ctypes.data)
    if rc:
        raise ValueError("orc_quantize failed (%d)" % rc)
    return q, (s.reshape(rows, cols // group) if group else s)


def rmsnorm(x, g, eps, act_fmt) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float64)
    g = np.ascontiguousarray(g, dtype=np.float64)
    h = np.empty_like(x)
    lib().orc_rmsnorm(_dp(x), _dp(g), x.size, float(eps), act_fmt, _dp(h))
    return h


def rope(u, pos: int, theta: float) -> np.ndarray:
    u = np.array(u, dtype=np.float64, copy=True)
    lib().orc_rope(_dp(u), u.size, int(pos), float(theta))
    return u


def attention(q, K, V, act_fmt) -> np.ndarray:
    q = np.ascontiguousarray(q, dtype=np.float64)
    K = np.ascontiguousarray(K, dtype=np.float32)
    V = np.ascontiguousarray(V, dtype=np.float32)
    n, hd = K.shape
    o = np.empty(hd, dtype=np.float64)
    scratch = np.empty(max(n, 1), dtype=np.float64)
    lib().orc_attention(_dp(q), _fp(K), _fp(V), n, hd, act_fmt, _dp(o), _dp(scratch))
    return o


def swiglu(g: float, u: float, act_fmt: int) -> float:
    return lib().orc_swiglu(float(g), float(u), act_fmt)


def argmax_f32(v) -> int:
    v = np.ascontiguousarray(v, dtype=np.float32)
    return lib().orc_argmax_f32(_fp(v), v.size)


# ---------------------------------------------------------------- whole model

class OracleModel:
    """The decode step of one model shape on the CPU. Master weights are borrowed (kept alive
    here); int8/int4 codes are quantised by the oracle itself."""

    def __init__(self, shape: I.ModelShape, weights: I.Weights, max_ctx: int | None = None):
        self.shape = shape
        self.max_ctx = max_ctx or shape.max_ctx
        self.act_fmt = FMT_F32 if shape.act_f32 else FMT_BF16
        # theta and eps as the model description carries them (fp32 values)
        d = _Desc(shape.hidden, shape.n_layers, shape.n_heads, shape.n_kv_heads, shape.head_dim,
                  shape.intermediate, shape.vocab, self.max_ctx, int(shape.tied), shape.wfmt,
                  int(shape.act_f32), float(np.float32(shape.rope_theta)), float(np.float32(shape.rms_eps)))
        L = lib()
        self._h = L.orc_create(C.byref(d))
        if not self._h:
            raise ValueError("orc_create rejected the shape")
        self._keep = []

        def put(kind, layer, arr):
            a = np.ascontiguousarray(arr)
            self._keep.append(a)
            rc = L.orc_set_weight(self._h, kind, layer, a.ctypes.data)
            if rc:
                raise ValueError("orc_set_weight(%d, %d) failed" % (kind, layer))

        put(W_EMBED, 0, weights.embed)
        put(W_FINAL_NORM, 0, weights.final_norm)
        if not shape.tied:
            put(W_LM_HEAD, 0, weights.lm_head)
        for l, t in enumerate(weights.layers):
            for name, arr in t.items():
                put(_KIND[name], l, arr)
        if not shape.wfmt in (I.WF_INT8, I.WF_INT4):
            # fp32/bf16 weights are borrowed: keep the arrays alive (done via _keep)
            pass

    def close(self):
        if getattr(self, "_h", None):
            lib().orc_destroy(self._h)
            self._h = None
            self._keep = []

    def __del__(self):
        try:
            self.close()
        except Exception:   # interpreter shutdown: the library may already be gone
            pass

    def set_kv(self, layer: int, kv_vals: np.ndarray, pos0: int = 0):
        """kv_vals: [2][nKV][n][hd] act-format values (fp32 or bf16 bits)."""
        a = kv_vals
        if a.dtype == np.uint16:
            a = I.bf16_bits_to_f32(a)
        a = np.ascontiguousarray(a, dtype=np.float32)
        for kv in range(2):
            for g in range(self.shape.n_kv_heads):
                blk = np.ascontiguousarray(a[kv, g])
                rc = lib().orc_set_kv(self._h, layer, kv, g, pos0, blk.shape[0], _fp(blk))
                if rc:
                    raise ValueError("orc_set_kv failed")

    def get_kv(self, layer: int, kv: int, grp: int, pos0: int, n: int) -> np.ndarray:
        out = np.empty((n, self.shape.head_dim), dtype=np.float32)
        rc = lib().orc_get_kv(self._h, layer, kv, grp, pos0, n, _fp(out))
        if rc:
            raise ValueError("orc_get_kv failed")
        return out

    def codes(self, kind: int, layer: int = 0):
        s = self.shape
        rows, cols = {W_LM_HEAD: (s.vocab, s.hidden), W_WQ: (s.q_dim, s.hidden), W_WK: (s.kv_dim, s.hidden),
                      W_WV: (s.kv_dim, s.hidden), W_WO: (s.hidden, s.q_dim), W_WG: (s.intermediate, s.hidden),
                      W_WU: (s.intermediate, s.hidden), W_WD: (s.hidden, s.intermediate)}[kind]
        group = 128 if s.wfmt == I.WF_INT4 else 0
        q = np.empty((rows, cols), dtype=np.int8)
        sc = np.empty(rows * (cols // group) if group else rows, dtype=np.float32)
        if lib().orc_get_codes(self._h, kind, layer, q.ctypes.data, sc.ctypes.data):
            raise ValueError("no codes")
        return q, (sc.reshape(rows, -1) if group else sc)

    def step(self, token: int, pos: int):
        """-> (logits float64 [V], logits fp32 [V], greedy token)."""
        V = self.shape.vocab
        lg = np.empty(V, dtype=np.float64)
        lg32 = np.empty(V, dtype=np.float32)
        t = C.c_int(-2)
        rc = lib().orc_step(self._h, int(token), int(pos), _dp(lg), _fp(lg32), C.byref(t))
        if rc not in (0, 2):
            raise ValueError("orc_step failed (%d)" % rc)
        return lg, lg32, t.value


def top2_margin(logits32: np.ndarray) -> float:
    """Gap between the largest and second-largest fp32 logit."""
    v = np.sort(np.asarray(logits32, dtype=np.float64))
    return float(v[-1] - v[-2]) if v.size > 1 else float("inf")


def prefill_model(model: OracleModel, shape: I.ModelShape, n_pos: int, seed: int | None = None):
    for l in range(shape.n_layers):
        model.set_kv(l, I.kv_prefill(shape, n_pos, l, seed), 0)


def run_protocol(model: OracleModel, shape: I.ModelShape, prompt, n_generate: int, pos0: int = 0,
                 forced=None):
    """Feed the prompt one token per step from pos0, then decode greedily.

    The first generated token comes from the last prompt step, so P prompt tokens and N
    generated tokens take P + N - 1 steps. With `forced` (a list of tokens, teacher forcing)
    the generated tokens fed back are taken from it instead of the model's own choices.
    Returns (generated tokens, per-step fp32 logits, per-step top-2 margins, input tokens)."""
    prompt = list(int(t) for t in prompt)
    gen, logits, margins, inputs = [], [], [], []
    tok = prompt[0]
    pos = pos0
    n_steps = len(prompt) + n_generate - 1
    for s in range(n_steps):
        inputs.append(tok)
        _, lg32, t = model.step(tok, pos)
        logits.append(lg32)
        margins.append(top2_margin(lg32))
        pos += 1
        if s + 1 < len(prompt):
            tok = prompt[s + 1]
        else:
            gen.append(t)
            tok = forced[len(gen) - 1] if forced is not None else t
    return gen, logits, margins, inputs
