"""ctypes declarations of libamk.so (include/amk.h): structs, enums and the exported calls.

Argument marshalling only. Every step of the decode path runs inside the library; if the
library is missing, loading raises instead of falling back to anything else.
"""
from __future__ import annotations

import ctypes as C
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("AMK_LIB") or os.path.join(HERE, "libamk.so")

# amk_status
AMK_OK, AMK_E_INVALID_ARG, AMK_E_UNSUPPORTED, AMK_E_REJECTED = 0, 1, 2, 3
AMK_E_OOM, AMK_E_HIP, AMK_E_NOT_RESIDENT, AMK_E_DEVICE_TIMEOUT = 4, 5, 6, 7
STATUS_NAMES = {0: "AMK_OK", 1: "AMK_E_INVALID_ARG", 2: "AMK_E_UNSUPPORTED", 3: "AMK_E_REJECTED",
                4: "AMK_E_OOM", 5: "AMK_E_HIP", 6: "AMK_E_NOT_RESIDENT", 7: "AMK_E_DEVICE_TIMEOUT"}

# amk_wfmt
AMK_F32, AMK_BF16, AMK_INT8_PC, AMK_INT4_G128 = 0, 1, 2, 3

# access flags, region kinds, schedule flags
AMK_ACC_WRITE, AMK_ACC_POST = 1, 2
AMK_REGION_PLAIN, AMK_REGION_LL, AMK_REGION_RO = 0, 1, 2
AMK_SCHED_LL_PROTOCOL = 1

# opcodes
AMK_OP_QKV, AMK_OP_ATTN, AMK_OP_MERGE, AMK_OP_OPROJ = 1, 2, 3, 4
AMK_OP_GATEUP, AMK_OP_DOWN, AMK_OP_LM, AMK_OP_ARGMAX = 5, 6, 7, 8
AMK_OP_ATTN_MERGE = 9

# device status bits
STATUS_TIMEOUT, STATUS_BAD_TOKEN = 1, 2
TRACE_SLOTS = 6


class amk_model_desc(C.Structure):
    _fields_ = [("struct_size", C.c_uint32), ("hidden", C.c_int32), ("n_layers", C.c_int32),
                ("n_heads", C.c_int32), ("n_kv_heads", C.c_int32), ("head_dim", C.c_int32),
                ("intermediate", C.c_int32), ("vocab", C.c_int32), ("max_ctx", C.c_int32),
                ("tied_embeddings", C.c_int32), ("rope_theta", C.c_float), ("rms_eps", C.c_float),
                ("wfmt", C.c_int32), ("act_f32", C.c_int32)]


class amk_weights(C.Structure):
    _fields_ = [("struct_size", C.c_uint32), ("embed", C.c_void_p), ("final_norm", C.c_void_p),
                ("lm_head", C.c_void_p)] + [
        (n, C.POINTER(C.c_void_p)) for n in
        ("attn_norm", "wq", "wk", "wv", "wo", "mlp_norm", "wg", "wu", "wd")]


class amk_task(C.Structure):
    _fields_ = [("opcode", C.c_uint32), ("layer", C.c_uint32), ("arg", C.c_uint32 * 4),
                ("wait_off", C.c_uint32), ("wait_cnt", C.c_uint32), ("sig_off", C.c_uint32),
                ("sig_cnt", C.c_uint32), ("acc_off", C.c_uint32), ("acc_cnt", C.c_uint32)]


class amk_wait(C.Structure):
    _fields_ = [("counter", C.c_uint32), ("threshold", C.c_uint32)]


class amk_access(C.Structure):
    _fields_ = [("region", C.c_uint32), ("flags", C.c_uint32), ("lo", C.c_uint64), ("hi", C.c_uint64)]


class amk_range(C.Structure):
    _fields_ = [("region", C.c_uint32), ("pad", C.c_uint32), ("lo", C.c_uint64), ("hi", C.c_uint64)]


class amk_schedule(C.Structure):
    _fields_ = [("struct_size", C.c_uint32), ("flags", C.c_uint32), ("n_tasks", C.c_uint32),
                ("n_queues", C.c_uint32), ("n_counters", C.c_uint32), ("n_regions", C.c_uint32),
                ("n_waits", C.c_uint32), ("n_signals", C.c_uint32), ("n_accesses", C.c_uint32),
                ("n_inputs", C.c_uint32), ("n_outputs", C.c_uint32),
                ("tasks", C.POINTER(amk_task)), ("queue_off", C.POINTER(C.c_uint32)),
                ("queue_tasks", C.POINTER(C.c_uint32)), ("waits", C.POINTER(amk_wait)),
                ("signals", C.POINTER(C.c_uint32)), ("accesses", C.POINTER(amk_access)),
                ("region_kind", C.POINTER(C.c_uint32)), ("inputs", C.POINTER(amk_range)),
                ("outputs", C.POINTER(amk_range))]


class amk_verdict(C.Structure):
    _fields_ = [("accepted", C.c_int32), ("rule_mask", C.c_uint32), ("task", C.c_int32),
                ("counter", C.c_int32), ("region", C.c_int32)]


class amk_schedule_config(C.Structure):
    _fields_ = [("struct_size", C.c_uint32), ("n_cu", C.c_int32), ("tasks_qkv", C.c_int32),
                ("tasks_o", C.c_int32), ("tasks_gateup", C.c_int32), ("tasks_down", C.c_int32),
                ("tasks_lm", C.c_int32), ("attn_chunks", C.c_int32), ("attn_group_tasks", C.c_int32),
                ("cu_assign", C.c_int32), ("prefetch_groups", C.c_int32), ("merge_fusion", C.c_int32)]


class amk_vm_opts(C.Structure):
    _fields_ = [("struct_size", C.c_uint32), ("seed", C.c_uint32), ("max_delay_us", C.c_uint32),
                ("watchdog_ms", C.c_uint32), ("max_elements", C.c_uint64)]


class amk_vm_result(C.Structure):
    _fields_ = [("completed", C.c_int32), ("deadlocked", C.c_int32), ("races", C.c_uint32),
                ("uncovered_reads", C.c_uint32), ("unwritten_outputs", C.c_uint32), ("task", C.c_int32),
                ("other", C.c_int32), ("unchecked", C.c_uint64), ("ll_rewrites", C.c_uint32), ("pad", C.c_uint32)]


# every symbol include/amk.h declares, with (restype, argtypes)
_P = C.c_void_p
SIGNATURES = {
    "amk_validate": (C.c_int, [C.POINTER(amk_schedule), C.POINTER(amk_verdict)]),
    "amk_lower": (C.c_int, [C.POINTER(amk_model_desc), C.POINTER(amk_schedule_config),
                            C.POINTER(C.POINTER(amk_schedule))]),
    "amk_schedule_free": (None, [C.POINTER(amk_schedule)]),
    "amk_create": (C.c_int, [C.POINTER(amk_model_desc), C.POINTER(amk_weights), _P,
                             C.POINTER(amk_schedule), C.POINTER(amk_schedule_config), _P,
                             C.POINTER(amk_verdict), C.POINTER(_P)]),
    "amk_decode_step": (C.c_int, [_P, _P, C.c_int32, _P, _P, _P]),
    "amk_decode_step_static": (C.c_int, [_P, _P, C.c_int32, _P, _P, _P]),
    "amk_device_status": (C.c_uint32, [_P]),
    "amk_ctx_schedule": (C.POINTER(amk_schedule), [_P]),
    "amk_set_trace": (C.c_int, [_P, _P, C.c_uint64]),
    "amk_destroy": (None, [_P]),
    "amk_quantize": (C.c_int, [C.c_int32, _P, C.c_int64, C.c_int64, _P, _P, _P]),
    "amk_read_probe": (C.c_int, [_P, C.c_uint64, _P, _P]),
    "amk_version": (C.c_char_p, []),
    "amk_vm_run": (C.c_int, [C.POINTER(amk_schedule), C.POINTER(amk_vm_opts), C.POINTER(amk_vm_result)]),
    "amk_prefill": (C.c_int, [_P, _P, C.c_int32, C.c_int32, _P, _P, _P]),
    "amk_set_prefill_trace": (C.c_int, [_P, _P, C.c_uint64]),
    "amk_lower_prefill": (C.c_int, [C.POINTER(amk_model_desc), C.c_int32, C.c_int32,
                                    C.POINTER(C.POINTER(amk_schedule))]),
}

_lib = None


class AmkError(RuntimeError):
    def __init__(self, call: str, status: int):
        super().__init__(f"{call} returned {STATUS_NAMES.get(status, status)}")
        self.status = status


def lib() -> C.CDLL:
    """Load libamk.so (built by persistent_megakernel_amd.build). Raises if it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run persistent_megakernel_amd/build.py "
                              "(or __graft_entry__.build())")
        L = C.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def check(call: str, status: int) -> None:
    if status != AMK_OK:
        raise AmkError(call, status)
