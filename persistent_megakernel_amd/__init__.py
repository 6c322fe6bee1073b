"""MI355X batch-1 persistent decode megakernel: Python binding of libamk.so.

The functions here carry the names of the C calls in include/amk.h and only marshal
arguments: the lowering, the validator, the weight quantiser/repack and the whole decode
step run in the library (host C++ and hand-written HIP for gfx950). PyTorch provides device
memory and streams and nothing else.

    from persistent_megakernel_amd import Decoder
    dec = Decoder(shape, weights)                # amk_create: validate, quantise, repack
    dec.step(tok_in, pos, tok_out, logits)       # amk_decode_step: one launch = one token
"""
from __future__ import annotations

import ctypes as C
from typing import Optional

import numpy as np

from . import _abi as A
from ._abi import (AMK_BF16, AMK_F32, AMK_INT4_G128, AMK_INT8_PC, AmkError, STATUS_BAD_TOKEN,  # noqa: F401
                   STATUS_TIMEOUT, check, lib)

__all__ = ["amk_validate", "amk_lower", "amk_create", "amk_decode_step", "amk_decode_step_static", "amk_destroy",
           "amk_quantize", "amk_read_probe", "amk_device_status", "amk_ctx_schedule", "amk_set_trace", "amk_version", "Decoder",
           "model_desc", "schedule_config", "AmkError", "amk_vm_run",
           "amk_prefill", "amk_lower_prefill", "amk_set_prefill_trace"]


# ---------------------------------------------------------------- descriptors

def model_desc(shape, max_ctx: Optional[int] = None) -> A.amk_model_desc:
    """amk_model_desc of a model shape (any object with the ModelShape fields)."""
    return A.amk_model_desc(C.sizeof(A.amk_model_desc), shape.hidden, shape.n_layers, shape.n_heads,
                            shape.n_kv_heads, shape.head_dim, shape.intermediate, shape.vocab,
                            int(max_ctx or shape.max_ctx), int(bool(shape.tied)), float(shape.rope_theta),
                            float(shape.rms_eps), int(shape.wfmt), int(bool(shape.act_f32)))


def schedule_config(**kw) -> A.amk_schedule_config:
    """amk_schedule_config with the named knobs set (others 0 = default)."""
    c = A.amk_schedule_config()
    c.struct_size = C.sizeof(A.amk_schedule_config)
    for k, v in kw.items():
        if not hasattr(c, k):
            raise TypeError(f"unknown schedule knob {k!r}")
        setattr(c, k, int(v))
    return c


# ---------------------------------------------------------------- schedules <-> C

class CSchedule:
    """An amk_schedule view over ctypes arrays built from a Python schedule (the arrays live as
    long as this object)."""

    def __init__(self, s):
        tasks, waits, sigs, accs = [], [], [], []
        for t in s.tasks:
            args = tuple(t.args) + (0,) * (5 - len(t.args))
            tk = A.amk_task()
            tk.opcode = t.opcode
            tk.layer = args[0]
            for k in range(4):
                tk.arg[k] = args[1 + k]
            tk.wait_off, tk.wait_cnt = len(waits), len(t.waits)
            waits.extend(t.waits)
            tk.sig_off, tk.sig_cnt = len(sigs), len(t.signals)
            sigs.extend(t.signals)
            tk.acc_off, tk.acc_cnt = len(accs), len(t.accesses)
            accs.extend(t.accesses)
            tasks.append(tk)
        qoff = [0]
        qt = []
        for q in s.queues:
            qt.extend(q)
            qoff.append(len(qt))

        def arr(ctype, items, conv=lambda x: x):
            a = (ctype * max(1, len(items)))()
            for i, x in enumerate(items):
                a[i] = conv(x)
            return a

        self._tasks = arr(A.amk_task, tasks)
        self._qoff = arr(C.c_uint32, qoff)
        self._qt = arr(C.c_uint32, [q & 0xffffffff for q in qt])
        self._waits = arr(A.amk_wait, waits, lambda w: A.amk_wait(w[0] & 0xffffffff, w[1] & 0xffffffff))
        self._sigs = arr(C.c_uint32, [c & 0xffffffff for c in sigs])
        self._accs = arr(A.amk_access, accs, lambda a: A.amk_access(a[0], a[1], a[2], a[3]))
        self._kinds = arr(C.c_uint32, list(s.region_kind))
        self._ins = arr(A.amk_range, s.inputs, lambda r: A.amk_range(r[0], 0, r[1], r[2]))
        self._outs = arr(A.amk_range, s.outputs, lambda r: A.amk_range(r[0], 0, r[1], r[2]))
        v = A.amk_schedule()
        v.struct_size = C.sizeof(A.amk_schedule)
        v.flags = A.AMK_SCHED_LL_PROTOCOL if getattr(s, "ll_protocol", False) else 0
        v.n_tasks, v.n_queues, v.n_counters, v.n_regions = len(tasks), len(s.queues), s.n_counters, s.n_regions
        v.n_waits, v.n_signals, v.n_accesses = len(waits), len(sigs), len(accs)
        v.n_inputs, v.n_outputs = len(s.inputs), len(s.outputs)
        v.tasks, v.queue_off, v.queue_tasks = self._tasks, self._qoff, self._qt
        v.waits, v.signals, v.accesses = self._waits, self._sigs, self._accs
        v.region_kind, v.inputs, v.outputs = self._kinds, self._ins, self._outs
        self.view = v


def schedule_from_c(p) -> "object":
    """A Python schedule (amk_inputs.schedules.Schedule) copied from an amk_schedule view."""
    from amk_inputs import schedules as S
    v = p.contents if hasattr(p, "contents") else p
    tasks = []
    for i in range(v.n_tasks):
        t = v.tasks[i]
        tasks.append(S.Task(
            waits=[(v.waits[t.wait_off + k].counter, v.waits[t.wait_off + k].threshold) for k in range(t.wait_cnt)],
            signals=[v.signals[t.sig_off + k] for k in range(t.sig_cnt)],
            accesses=[(a.region, a.flags, a.lo, a.hi) for a in
                      (v.accesses[t.acc_off + k] for k in range(t.acc_cnt))],
            opcode=t.opcode, args=(t.layer, t.arg[0], t.arg[1], t.arg[2], t.arg[3])))
    queues = [[v.queue_tasks[k] for k in range(v.queue_off[q], v.queue_off[q + 1])] for q in range(v.n_queues)]
    return S.Schedule(v.n_queues, v.n_counters, v.n_regions, tasks, queues,
                      [v.region_kind[r] for r in range(v.n_regions)],
                      [(r.region, r.lo, r.hi) for r in (v.inputs[k] for k in range(v.n_inputs))],
                      [(r.region, r.lo, r.hi) for r in (v.outputs[k] for k in range(v.n_outputs))],
                      ll_protocol=bool(v.flags & A.AMK_SCHED_LL_PROTOCOL))


# ---------------------------------------------------------------- calls

def amk_version() -> str:
    return lib().amk_version().decode()


def amk_validate(sched) -> A.amk_verdict:
    """Validate a schedule (Python Schedule, CSchedule or amk_schedule view) on the CPU."""
    if isinstance(sched, A.amk_schedule):
        view, keep = sched, None
    elif isinstance(sched, CSchedule):
        view, keep = sched.view, sched
    else:
        keep = CSchedule(sched)
        view = keep.view
    out = A.amk_verdict()
    check("amk_validate", lib().amk_validate(C.byref(view), C.byref(out)))
    del keep
    return out


def amk_vm_run(sched, seed: int = 0, max_delay_us: int = 0, watchdog_ms: int = 0, max_elements: int = 0) -> dict:
    """Run a Python schedule on the CPU executor (amk_vm_run): the counter protocol on host
    threads, checked with a happens-before race detector. Returns the outcome as a dict."""
    cs = CSchedule(sched)
    o = A.amk_vm_opts()
    o.struct_size = C.sizeof(A.amk_vm_opts)
    o.seed, o.max_delay_us, o.watchdog_ms, o.max_elements = seed, max_delay_us, watchdog_ms, max_elements
    r = A.amk_vm_result()
    check("amk_vm_run", lib().amk_vm_run(C.byref(cs.view), C.byref(o), C.byref(r)))
    return {k: getattr(r, k) for k, _ in A.amk_vm_result._fields_}


def amk_lower(desc: A.amk_model_desc, cfg: Optional[A.amk_schedule_config] = None):
    """The built-in lowering as a Python schedule (the C copy is freed here)."""
    p = C.POINTER(A.amk_schedule)()
    check("amk_lower", lib().amk_lower(C.byref(desc), C.byref(cfg) if cfg is not None else None, C.byref(p)))
    try:
        return schedule_from_c(p)
    finally:
        lib().amk_schedule_free(p)


def amk_lower_verdict(desc: A.amk_model_desc, cfg: Optional[A.amk_schedule_config] = None) -> A.amk_verdict:
    """Lower and validate in C without copying the schedule to Python (large models)."""
    p = C.POINTER(A.amk_schedule)()
    check("amk_lower", lib().amk_lower(C.byref(desc), C.byref(cfg) if cfg is not None else None, C.byref(p)))
    try:
        out = A.amk_verdict()
        check("amk_validate", lib().amk_validate(p, C.byref(out)))
        return out
    finally:
        lib().amk_schedule_free(p)


def amk_create(desc, weights, kv_cache_ptr: int, sched=None, cfg=None, stream: int = 0):
    """-> (ctx handle, verdict). Raises AmkError (with .verdict) when the call fails."""
    ctx = C.c_void_p()
    verdict = A.amk_verdict()
    keep = None
    sp = None
    if sched is not None:
        keep = sched if isinstance(sched, CSchedule) else CSchedule(sched)
        sp = C.byref(keep.view)
    st = lib().amk_create(C.byref(desc), C.byref(weights), C.c_void_p(kv_cache_ptr), sp,
                          C.byref(cfg) if cfg is not None else None, C.c_void_p(stream), C.byref(verdict),
                          C.byref(ctx))
    if st != A.AMK_OK:
        e = AmkError("amk_create", st)
        e.verdict = verdict
        raise e
    return ctx.value, verdict


def amk_decode_step(ctx: int, token_in_ptr: int, pos: int, token_out_ptr: int, logits_ptr: int = 0,
                    stream: int = 0) -> int:
    """Enqueue one decode launch; returns the amk_status (does not raise, for hot loops)."""
    return lib().amk_decode_step(C.c_void_p(ctx), C.c_void_p(token_in_ptr), int(pos), C.c_void_p(token_out_ptr),
                                 C.c_void_p(logits_ptr or None), C.c_void_p(stream))


def amk_decode_step_static(ctx: int, token_in_ptr: int, pos: int, token_out_ptr: int, logits_ptr: int = 0,
                           stream: int = 0) -> int:
    """amk_decode_step with the step's flag-carrying words in the library's static per-device
    array (allocates nothing); returns the amk_status."""
    return lib().amk_decode_step_static(C.c_void_p(ctx), C.c_void_p(token_in_ptr), int(pos), C.c_void_p(token_out_ptr),
                                        C.c_void_p(logits_ptr or None), C.c_void_p(stream))


def amk_prefill(ctx: int, tokens_ptr: int, pos0: int, n_tokens: int, token_out_ptr: int, logits_ptr: int = 0,
                stream: int = 0) -> int:
    """Enqueue the prefill launches of n_tokens prompt tokens; returns the amk_status."""
    return lib().amk_prefill(C.c_void_p(ctx), C.c_void_p(tokens_ptr), int(pos0), int(n_tokens),
                             C.c_void_p(token_out_ptr), C.c_void_p(logits_ptr or None), C.c_void_p(stream))


def amk_lower_prefill(desc: A.amk_model_desc, n_cu: int, n_tokens: int, python: bool = True):
    """The prefill schedule of one launch, as a Python schedule (python=True) or its verdict."""
    p = C.POINTER(A.amk_schedule)()
    check("amk_lower_prefill", lib().amk_lower_prefill(C.byref(desc), int(n_cu), int(n_tokens), C.byref(p)))
    try:
        if python:
            return schedule_from_c(p)
        out = A.amk_verdict()
        check("amk_validate", lib().amk_validate(p, C.byref(out)))
        return out
    finally:
        lib().amk_schedule_free(p)


def amk_device_status(ctx: int) -> int:
    return int(lib().amk_device_status(C.c_void_p(ctx)))


def amk_ctx_schedule(ctx: int):
    return schedule_from_c(lib().amk_ctx_schedule(C.c_void_p(ctx)))


def amk_set_trace(ctx: int, trace_ptr: int, capacity: int) -> None:
    check("amk_set_trace", lib().amk_set_trace(C.c_void_p(ctx), C.c_void_p(trace_ptr or None), int(capacity)))


def amk_set_prefill_trace(ctx: int, trace_ptr: int, capacity: int) -> None:
    check("amk_set_prefill_trace", lib().amk_set_prefill_trace(C.c_void_p(ctx), C.c_void_p(trace_ptr or None),
                                                               int(capacity)))


def amk_destroy(ctx: Optional[int]) -> None:
    lib().amk_destroy(C.c_void_p(ctx) if ctx else None)


def amk_quantize(wfmt: int, master_ptr: int, rows: int, cols: int, codes_ptr: int, scales_ptr: int,
                 stream: int = 0) -> None:
    check("amk_quantize", lib().amk_quantize(int(wfmt), C.c_void_p(master_ptr), int(rows), int(cols),
                                             C.c_void_p(codes_ptr), C.c_void_p(scales_ptr), C.c_void_p(stream)))


def amk_read_probe(buf_ptr: int, nbytes: int, out_ptr: int, stream: int = 0) -> None:
    check("amk_read_probe", lib().amk_read_probe(C.c_void_p(buf_ptr), int(nbytes), C.c_void_p(out_ptr),
                                                 C.c_void_p(stream)))


# ---------------------------------------------------------------- a model on the device

class Decoder:
    """A model resident on the current GPU: the library's repacked weights plus a caller-owned
    KV cache (a torch tensor [L][2][nKV][max_ctx][hd] in the activation type).

    `weights` holds master weights as numpy arrays (fp32, or bf16 bits as uint16), the layout
    of amk_inputs.Weights; they are copied to the device for amk_create and released after it.
    """

    def __init__(self, shape, weights, max_ctx: Optional[int] = None, cfg=None, sched=None, device: str = "cuda"):
        import torch
        self.torch = torch
        self.shape = shape
        self.max_ctx = int(max_ctx or shape.max_ctx)
        self.device = torch.device(device)
        act = torch.float32 if shape.act_f32 else torch.bfloat16
        self.act_dtype = act
        s = shape
        self.kv = torch.zeros((s.n_layers, 2, s.n_kv_heads, self.max_ctx, s.head_dim), dtype=act, device=self.device)
        self.desc = model_desc(shape, self.max_ctx)
        self.cfg = cfg
        stream = torch.cuda.current_stream(self.device)

        def dev(a):
            t = torch.from_numpy(np.ascontiguousarray(a))
            if t.dtype == torch.uint16:
                t = t.view(torch.int16)
            return t.to(self.device)

        tmp = []

        def ptr(a):
            t = dev(a)
            tmp.append(t)
            return t.data_ptr()

        names = ("attn_norm", "wq", "wk", "wv", "wo", "mlp_norm", "wg", "wu", "wd")
        arrays = {n: (C.c_void_p * s.n_layers)() for n in names}
        w = A.amk_weights()
        w.struct_size = C.sizeof(A.amk_weights)
        w.embed = ptr(weights.embed)
        w.final_norm = ptr(weights.final_norm)
        w.lm_head = ptr(weights.lm_head) if weights.lm_head is not None else None
        for l, d in enumerate(weights.layers):
            for n in names:
                arrays[n][l] = ptr(d[n])
        for n in names:
            setattr(w, n, C.cast(arrays[n], C.POINTER(C.c_void_p)))
        torch.cuda.synchronize(self.device)
        self.ctx, self.verdict = amk_create(self.desc, w, self.kv.data_ptr(), sched=sched, cfg=cfg,
                                            stream=stream.cuda_stream)
        del tmp
        self.tok = torch.zeros(2, dtype=torch.int32, device=self.device)

    def set_kv_prefix(self, layer: int, vals) -> None:
        """Write cache positions [0, n) of one layer from [2][nKV][n][hd] (fp32 values or bf16
        bits as uint16)."""
        torch = self.torch
        t = torch.from_numpy(np.ascontiguousarray(vals))
        if t.dtype == torch.uint16:
            t = t.view(torch.int16).view(torch.bfloat16)
        n = t.shape[2]
        self.kv[layer, :, :, :n, :].copy_(t.to(self.device, self.act_dtype))

    def step(self, token_in, pos: int, token_out, logits=None, stream=None) -> None:
        """One decode launch. token_in/token_out: device int32 tensors (one element used);
        logits: device fp32 [vocab] or None."""
        torch = self.torch
        st = (stream or torch.cuda.current_stream(self.device)).cuda_stream
        rc = amk_decode_step(self.ctx, token_in.data_ptr(), pos, token_out.data_ptr(),
                             logits.data_ptr() if logits is not None else 0, st)
        check("amk_decode_step", rc)

    def prefill(self, tokens, pos0: int, token_out, logits=None, stream=None) -> None:
        """Prompt prefill (amk_prefill). tokens: device int32 [n]; token_out: device int32 (one
        element used); logits: device fp32 [vocab] or None."""
        torch = self.torch
        st = (stream or torch.cuda.current_stream(self.device)).cuda_stream
        rc = amk_prefill(self.ctx, tokens.data_ptr(), pos0, tokens.numel(), token_out.data_ptr(),
                         logits.data_ptr() if logits is not None else 0, st)
        check("amk_prefill", rc)

    def status(self) -> int:
        return amk_device_status(self.ctx)

    def enable_trace(self):
        """Allocate a trace buffer and make later steps record per-task timestamps into it;
        returns the device uint64 tensor [n_tasks, 6] (see amk_set_trace)."""
        n = len(self.schedule().tasks)
        self.trace = self.torch.zeros((n, A.TRACE_SLOTS), dtype=self.torch.int64, device=self.device)
        amk_set_trace(self.ctx, self.trace.data_ptr(), self.trace.numel())
        return self.trace

    def enable_prefill_trace(self, n_tokens: int, n_cu: int):
        """Record per-task timestamps of later prefill launches of n_tokens (<= 256) tokens;
        returns (device int64 tensor [n_tasks, 4], the launch's schedule)."""
        sched = amk_lower_prefill(self.desc, n_cu, ((n_tokens + 63) // 64) * 64)
        self.pf_trace = self.torch.zeros((len(sched.tasks), 4), dtype=self.torch.int64, device=self.device)
        amk_set_prefill_trace(self.ctx, self.pf_trace.data_ptr(), self.pf_trace.numel())
        return self.pf_trace, sched

    def schedule(self):
        return amk_ctx_schedule(self.ctx)

    def close(self) -> None:
        if getattr(self, "ctx", None):
            amk_destroy(self.ctx)
            self.ctx = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def run_steps(dec: Decoder, inputs, pos0: int, chain_from: int | None = None, logits=None):
    """Launch one decode step per input position, back to back on the current stream.

    inputs: host list of token ids fed at pos0, pos0+1, ...; from step `chain_from` on (if
    given) each step instead reads the token the previous step wrote, on the device (greedy
    decoding with no host round trip). logits: optional device fp32 [n_steps, vocab].
    Returns the device int32 tensor of the tokens each step produced."""
    torch = dec.torch
    n = len(inputs)
    tin = torch.tensor(list(inputs), dtype=torch.int32).to(dec.device)
    tout = torch.full((max(n, 1),), -1, dtype=torch.int32, device=dec.device)
    for s in range(n):
        src = tin[s:s + 1] if chain_from is None or s < chain_from or s == 0 else tout[s - 1:s]
        dec.step(src, pos0 + s, tout[s:s + 1], logits[s] if logits is not None else None)
    return tout[:n]
