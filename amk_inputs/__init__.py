"""Seeded synthetic inputs for the batch-1 decode step: model shapes, master weights,
prompt tokens and pre-filled KV caches.

This module is shared by the CPU oracle and the GPU path. It holds no arithmetic of the
decode step or of the weight quantisation: it only draws random numbers and rounds the
fp32 draws to the storage format named by each workload (bf16 masters, bf16 KV).

Workloads (the five model shapes of the batch-1 decode benchmark; Llama-family
transformers as described on the AutoMegaKernel pages, "What's built" and "Results"):

  tiny_fp32          hidden 64, 2 layers, 4/2 heads (hd 16), I 176, vocab 256, fp32
  smollm2_135m_bf16  hidden 576, 30 layers, 9/3 heads (hd 64), I 1536, vocab 49152, tied, bf16
  tinyllama_int8     hidden 2048, 22 layers, 32/4 heads (hd 64), I 5632, vocab 32000, int8 W8A16
  llama7b_bf16       hidden 4096, 32 layers, 32/32 heads (hd 128), I 11008, vocab 32000, bf16
  llama7b_int8       the same master as llama7b_bf16, int8 W8A16
  llama3_8b_int4     hidden 4096, 32 layers, 32/8 heads (hd 128), I 14336, vocab 128256,
                     int4 g128, rope theta 5e5

Seeding: every tensor (or 16M-element chunk of one) is drawn from
numpy.random.Generator(PCG64(SeedSequence([seed, layer, tensor_id, chunk]))), so any tensor
can be regenerated alone and the draw is the same on every machine.
"""
from __future__ import annotations

import dataclasses
from concurrent.futures import ThreadPoolExecutor
import os

import numpy as np

# weight formats (the same integers as the C headers of both sides)
WF_F32, WF_BF16, WF_INT8, WF_INT4 = 0, 1, 2, 3

# tensor ids used in seeds
T_EMBED, T_FINAL_NORM, T_LM_HEAD = 0, 1, 2
T_ATTN_NORM, T_WQ, T_WK, T_WV, T_WO, T_MLP_NORM, T_WG, T_WU, T_WD = 10, 11, 12, 13, 14, 15, 16, 17, 18
T_TOKENS, T_KV = 100, 101

LAYER_TENSORS = ("attn_norm", "wq", "wk", "wv", "wo", "mlp_norm", "wg", "wu", "wd")
_TID = dict(attn_norm=T_ATTN_NORM, wq=T_WQ, wk=T_WK, wv=T_WV, wo=T_WO, mlp_norm=T_MLP_NORM,
            wg=T_WG, wu=T_WU, wd=T_WD)

_CHUNK = 1 << 24


@dataclasses.dataclass(frozen=True)
class ModelShape:
    name: str
    hidden: int
    n_layers: int
    n_heads: int
    n_kv_heads: int
    head_dim: int
    intermediate: int
    vocab: int
    tied: bool
    wfmt: int
    act_f32: bool
    rope_theta: float
    rms_eps: float = 1e-5
    seed: int = 0
    # decode protocol
    prompt_len: int = 0       # prompt tokens fed one launch each from pos 0
    n_generate: int = 0       # greedy tokens generated
    prefill_ctx: int = 0      # KV positions [0, prefill_ctx) pre-filled with N(0,1)
    max_ctx: int = 0

    @property
    def q_dim(self) -> int:
        return self.n_heads * self.head_dim

    @property
    def kv_dim(self) -> int:
        return self.n_kv_heads * self.head_dim

    def tensor_shape(self, name: str):
        H, I, V = self.hidden, self.intermediate, self.vocab
        return {
            "embed": (V, H), "final_norm": (H,), "lm_head": (V, H),
            "attn_norm": (H,), "mlp_norm": (H,),
            "wq": (self.q_dim, H), "wk": (self.kv_dim, H), "wv": (self.kv_dim, H),
            "wo": (H, self.q_dim), "wg": (I, H), "wu": (I, H), "wd": (H, I),
        }[name]

    def replace(self, **kw) -> "ModelShape":
        return dataclasses.replace(self, **kw)


def _shape(name, H, L, nH, nKV, hd, I, V, tied, wfmt, act_f32, theta, seed, **kw):
    s = ModelShape(name, H, L, nH, nKV, hd, I, V, tied, wfmt, act_f32, theta, 1e-5, seed, **kw)
    if not s.max_ctx:
        s = s.replace(max_ctx=s.prefill_ctx + s.prompt_len + s.n_generate + 16)
    return s


SHAPES = {
    "tiny_fp32": _shape("tiny_fp32", 64, 2, 4, 2, 16, 176, 256, False, WF_F32, True, 1e4, 1001,
                        prompt_len=8, n_generate=16),
    "smollm2_135m_bf16": _shape("smollm2_135m_bf16", 576, 30, 9, 3, 64, 1536, 49152, True, WF_BF16, False,
                                1e4, 1002, prompt_len=16, n_generate=32),
    "tinyllama_int8": _shape("tinyllama_int8", 2048, 22, 32, 4, 64, 5632, 32000, False, WF_INT8, False,
                             1e4, 1003, prefill_ctx=512, n_generate=16, max_ctx=1024),
    "llama7b_bf16": _shape("llama7b_bf16", 4096, 32, 32, 32, 128, 11008, 32000, False, WF_BF16, False,
                           1e4, 1004, prefill_ctx=2048, n_generate=16),
    "llama7b_int8": _shape("llama7b_int8", 4096, 32, 32, 32, 128, 11008, 32000, False, WF_INT8, False,
                           1e4, 1004, prefill_ctx=2048, n_generate=16),
    "llama3_8b_int4": _shape("llama3_8b_int4", 4096, 32, 32, 8, 128, 14336, 128256, False, WF_INT4, False,
                             5e5, 1005, prefill_ctx=4096, n_generate=16),
}


def _rng(*key) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(k) for k in key])))


def _workers() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def _normal_f32(shape, std, mean, key, threads: bool = True) -> np.ndarray:
    """N(mean, std^2) in fp32, drawn in 16M-element chunks with per-chunk seeds (on a thread
    pool when `threads`; the values do not depend on it)."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.float32)
    chunks = [(c, min(_CHUNK, n - c * _CHUNK)) for c in range((n + _CHUNK - 1) // _CHUNK)]

    def fill(cl):
        c, m = cl
        g = _rng(*key, c)
        seg = out[c * _CHUNK: c * _CHUNK + m]
        g.standard_normal(m, dtype=np.float32, out=seg)
        seg *= np.float32(std)
        if mean:
            seg += np.float32(mean)

    if len(chunks) == 1 or not threads:
        for cl in chunks:
            fill(cl)
    else:
        with ThreadPoolExecutor(_workers()) as ex:
            list(ex.map(fill, chunks))
    return out.reshape(shape)


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (round-to-nearest-even, via torch's CPU cast); return uint16 bits."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bits to fp32 (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _master(shape: ModelShape, a32: np.ndarray) -> np.ndarray:
    """Master storage: fp32 for fp32 weights, bf16 bits (uint16) otherwise."""
    if shape.wfmt == WF_F32:
        return a32
    return f32_to_bf16_bits(a32)


def make_tensor(shape: ModelShape, name: str, layer: int = 0, seed: int | None = None,
                threads: bool = True) -> np.ndarray:
    seed = shape.seed if seed is None else seed
    shp = shape.tensor_shape(name)
    if name in ("attn_norm", "mlp_norm", "final_norm"):
        tid = _TID.get(name, T_FINAL_NORM)
        a = _normal_f32(shp, 0.02, 1.0, (seed, layer, tid), threads)
    else:
        tid = {"embed": T_EMBED, "lm_head": T_LM_HEAD, **_TID}[name]
        a = _normal_f32(shp, 0.02, 0.0, (seed, layer, tid), threads)
    return _master(shape, a)


@dataclasses.dataclass
class Weights:
    """Master weights, row-major [out, in]; fp32 arrays or bf16 bits (uint16)."""
    embed: np.ndarray
    final_norm: np.ndarray
    lm_head: np.ndarray | None          # None when tied to embed
    layers: list                        # list of dicts keyed by LAYER_TENSORS

    def lm(self) -> np.ndarray:
        return self.embed if self.lm_head is None else self.lm_head

    def nbytes(self) -> int:
        n = self.embed.nbytes + self.final_norm.nbytes + (0 if self.lm_head is None else self.lm_head.nbytes)
        return n + sum(t.nbytes for d in self.layers for t in d.values())


def make_weights(shape: ModelShape, seed: int | None = None) -> Weights:
    """Every tensor of the model, drawn on a thread pool (one tensor per job; each tensor's
    draw depends only on its own seed key, so the result is the same for any pool size)."""
    seed = shape.seed if seed is None else seed
    jobs = [(n, l) for l in range(shape.n_layers) for n in LAYER_TENSORS]
    jobs += [("embed", 0), ("final_norm", 0)] + ([] if shape.tied else [("lm_head", 0)])
    with ThreadPoolExecutor(_workers()) as ex:
        out = dict(zip(jobs, ex.map(lambda j: make_tensor(shape, j[0], j[1], seed, threads=False), jobs)))
    return Weights(
        embed=out[("embed", 0)],
        final_norm=out[("final_norm", 0)],
        lm_head=None if shape.tied else out[("lm_head", 0)],
        layers=[{n: out[(n, l)] for n in LAYER_TENSORS} for l in range(shape.n_layers)],
    )


def prompt_tokens(shape: ModelShape, n: int | None = None, seed: int | None = None, stream: int = 0) -> np.ndarray:
    """Uniform token ids in [0, vocab)."""
    seed = shape.seed if seed is None else seed
    n = (shape.prompt_len or 1) if n is None else n
    return _rng(seed, stream, T_TOKENS).integers(0, shape.vocab, size=n, dtype=np.int64).astype(np.int32)


def kv_prefill(shape: ModelShape, n_pos: int, layer: int, seed: int | None = None) -> np.ndarray:
    """Cache contents for positions [0, n_pos) of one layer: [2][nKV][n_pos][hd], N(0,1).

    Returned as fp32 values for fp32-activation shapes, else bf16 bits (uint16)."""
    seed = shape.seed if seed is None else seed
    a = _normal_f32((2, shape.n_kv_heads, n_pos, shape.head_dim), 1.0, 0.0, (seed, layer, T_KV))
    return a if shape.act_f32 else f32_to_bf16_bits(a)


def tiny_shape(**kw) -> ModelShape:
    """A small shape for unit tests (fp32 by default); keyword arguments override fields."""
    base = dict(name="tiny_custom", hidden=64, n_layers=2, n_heads=4, n_kv_heads=2, head_dim=16,
                intermediate=176, vocab=256, tied=False, wfmt=WF_F32, act_f32=True, rope_theta=1e4,
                rms_eps=1e-5, seed=7, prompt_len=8, n_generate=16, prefill_ctx=0, max_ctx=64)
    base.update(kw)
    return ModelShape(**base)
