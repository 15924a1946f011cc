"""ctypes binding of libmoe.so (include/moe.h).

Argument marshalling only: torch tensors supply device pointers and the
current HIP stream; every step of the layer runs in the library's kernels.
There is no fallback: if libmoe.so is missing or a call fails, an exception is
raised.
"""
from __future__ import annotations

import ctypes as C
import os
import threading

_HERE = os.path.dirname(os.path.abspath(__file__))
# MOE_LIBRARY names an alternative build of the same C ABI (e.g. a tuning build).
LIB_PATH = os.environ.get("MOE_LIBRARY") or os.path.join(_HERE, "libmoe.so")

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = range(5)
MOE_DT_F32, MOE_DT_BF16 = 0, 1
MOE_ACT_SWIGLU, MOE_ACT_RELU = 0, 1
MOE_F_LOGITS_GIVEN, MOE_F_VALIDATE_ONLY, MOE_F_NONDETERMINISTIC_COMBINE, MOE_F_BF16_ROWS = 1, 2, 4, 8
MOE_ATOMIC_AUTO, MOE_ATOMIC_DENSE, MOE_ATOMIC_EXPERT_CENTRIC = 0, 1, 2

EXPORTED = ("moe_route_topk", "moe_permute", "moe_permute_workspace_size", "moe_grouped_ffn",
            "moe_grouped_ffn_workspace_size", "moe_combine", "moe_layer_forward",
            "moe_workspace_size", "moe_replica_split", "moe_layer_forward_replica",
            "moe_replica_workspace_size", "moe_mwq_group", "moe_mwq_group_workspace_size",
            "moe_grouped_ffn_mwq", "moe_grouped_ffn_mwq_workspace_size", "moe_layer_forward_mwq",
            "moe_mwq_workspace_size", "moe_layer_forward_floe", "moe_floe_workspace_size",
            "moe_atomic_layer_forward", "moe_atomic_workspace_size", "moe_atomic_schedule",
            "moe_layer_forward_noalloc", "moe_noalloc_scratch_bytes",
            "moe_set_stage_events", "moe_status_string", "moe_last_error")


class MoeError(RuntimeError):
    def __init__(self, status, fn, detail):
        self.status = status
        super().__init__("%s -> %s: %s" % (fn, _STATUS.get(status, status), detail))


_STATUS = {0: "MOE_OK", 1: "MOE_ERR_INVALID_ARG", 2: "MOE_ERR_UNSUPPORTED",
           3: "MOE_ERR_WORKSPACE", 4: "MOE_ERR_HIP"}


class W4(C.Structure):
    _fields_ = [("q", C.c_void_p), ("scale", C.c_void_p), ("zero", C.c_void_p)]


class Experts(C.Structure):
    _fields_ = [("dtype", C.c_int), ("w_gate", C.c_void_p), ("w_up", C.c_void_p),
                ("w_down", C.c_void_p), ("q_gate", C.POINTER(W4)), ("q_up", C.POINTER(W4)),
                ("q_down", C.POINTER(W4))]


class LayerDesc(C.Structure):
    _fields_ = [("d_model", C.c_int), ("d_ff", C.c_int), ("n_experts", C.c_int),
                ("top_k", C.c_int), ("act", C.c_int), ("act_dtype", C.c_int),
                ("w_router", C.c_void_p), ("b_router", C.c_void_p), ("routed", Experts),
                ("n_shared", C.c_int), ("d_ff_shared", C.c_int), ("shared", Experts)]


class Replica(C.Structure):
    _fields_ = [("expert", C.c_int), ("q_gate", C.POINTER(W4)), ("q_up", C.POINTER(W4)),
                ("q_down", C.POINTER(W4))]


class WMwq(C.Structure):
    _fields_ = [("q2", C.c_void_p), ("s2", C.c_void_p), ("z2", C.c_void_p), ("p3", C.c_void_p),
                ("a3", C.c_void_p), ("p4", C.c_void_p), ("a4", C.c_void_p)]


class MwqExperts(C.Structure):
    _fields_ = [("gate", C.POINTER(WMwq)), ("up", C.POINTER(WMwq)), ("down", C.POINTER(WMwq))]


class MwqGroups(C.Structure):
    _fields_ = [("group_idx", C.c_void_p), ("counts", C.c_void_p), ("offsets", C.c_void_p),
                ("row_assign", C.c_void_p), ("assign_row", C.c_void_p)]


class FloeExperts(C.Structure):
    _fields_ = [("up", C.POINTER(WMwq)), ("w_gate", C.c_void_p), ("w_down_t", C.c_void_p),
                ("threshold", C.c_void_p)]


class FloeAux(C.Structure):
    _fields_ = [("up_out", C.c_void_p), ("kept", C.c_void_p), ("channels", C.c_void_p)]


class AtomicLayerDesc(C.Structure):
    _fields_ = [("d_model", C.c_int), ("grid_rows", C.c_int), ("grid_cols", C.c_int),
                ("top_k", C.c_int), ("w_row", C.c_void_p), ("w_col", C.c_void_p),
                ("w_in", C.c_void_p), ("w_out", C.c_void_p), ("n_shared", C.c_int),
                ("d_ff_shared", C.c_int), ("shared", Experts), ("w_out_rows", C.c_void_p),
                ("schedule", C.c_int)]


class AtomicAux(C.Structure):
    _fields_ = [("logp_row", C.c_void_p), ("logp_col", C.c_void_p), ("idx", C.c_void_p),
                ("gates", C.c_void_p), ("counts", C.c_void_p), ("offsets", C.c_void_p),
                ("row_assign", C.c_void_p), ("assign_row", C.c_void_p), ("lis", C.c_void_p)]


class Aux(C.Structure):
    _fields_ = [("logits", C.c_void_p), ("idx", C.c_void_p), ("gates", C.c_void_p),
                ("counts", C.c_void_p), ("offsets", C.c_void_p), ("row_assign", C.c_void_p),
                ("assign_row", C.c_void_p), ("lis", C.c_void_p)]


_lib = None
_lock = threading.Lock()


def lib():
    """Load libmoe.so; raises if it has not been built."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise ImportError("libmoe.so not built (%s); run __graft_entry__.build()" % LIB_PATH)
            L = C.CDLL(LIB_PATH)
            p, i, u, sz = C.c_void_p, C.c_int, C.c_uint, C.c_size_t
            L.moe_route_topk.argtypes = [p, i, p, p, i, i, i, i, p, p, p, u, p]
            L.moe_permute.argtypes = [p, i, i, i, p, p, p, p, p, p, sz, u, p]
            L.moe_permute_workspace_size.argtypes = [i, i, i]
            L.moe_permute_workspace_size.restype = sz
            L.moe_grouped_ffn.argtypes = [p, i, i, i, i, i, i, i, C.POINTER(Experts), p, p, p, p,
                                          p, sz, u, p]
            L.moe_grouped_ffn_workspace_size.argtypes = [i, i, i, i, i, i, C.POINTER(Experts)]
            L.moe_grouped_ffn_workspace_size.restype = sz
            L.moe_combine.argtypes = [p, p, i, i, i, p, p, i, u, p]
            L.moe_layer_forward.argtypes = [C.POINTER(LayerDesc), p, i, p, i, C.POINTER(Aux), p,
                                            sz, u, p]
            L.moe_workspace_size.argtypes = [C.POINTER(LayerDesc), i, C.POINTER(sz)]
            L.moe_layer_forward_noalloc.argtypes = [C.POINTER(LayerDesc), p, i, p, i,
                                                    C.POINTER(Aux), u, p]
            L.moe_noalloc_scratch_bytes.argtypes = []
            L.moe_noalloc_scratch_bytes.restype = sz
            L.moe_replica_split.argtypes = [p, p, p, p, i, i, i, i, p, p, p, p, p, p, u, p]
            L.moe_layer_forward_replica.argtypes = [C.POINTER(LayerDesc), C.POINTER(Replica), p, i,
                                                    p, i, C.POINTER(Aux), p, p, sz, u, p]
            L.moe_replica_workspace_size.argtypes = [C.POINTER(LayerDesc), i, C.POINTER(sz)]
            L.moe_mwq_group.argtypes = [p, p, i, i, i, C.POINTER(MwqGroups), p, sz, u, p]
            L.moe_mwq_group_workspace_size.argtypes = [i, i, i]
            L.moe_mwq_group_workspace_size.restype = sz
            L.moe_grouped_ffn_mwq.argtypes = [p, i, i, i, i, i, i, C.POINTER(MwqExperts), p, p, p,
                                              p, p, sz, u, p]
            L.moe_grouped_ffn_mwq_workspace_size.argtypes = [i, i, i]
            L.moe_grouped_ffn_mwq_workspace_size.restype = sz
            L.moe_layer_forward_mwq.argtypes = [C.POINTER(LayerDesc), C.POINTER(MwqExperts), p, p,
                                                i, p, i, C.POINTER(Aux), C.POINTER(MwqGroups), p,
                                                sz, u, p]
            L.moe_mwq_workspace_size.argtypes = [C.POINTER(LayerDesc), i, C.POINTER(sz)]
            L.moe_layer_forward_floe.argtypes = [C.POINTER(LayerDesc), C.POINTER(FloeExperts),
                                                 p, i, p, i, C.POINTER(Aux), C.POINTER(FloeAux),
                                                 p, sz, u, p]
            L.moe_floe_workspace_size.argtypes = [C.POINTER(LayerDesc), i, C.POINTER(sz)]
            L.moe_atomic_layer_forward.argtypes = [C.POINTER(AtomicLayerDesc), p, i, p, i,
                                                   C.POINTER(AtomicAux), p, sz, u, p]
            L.moe_atomic_workspace_size.argtypes = [C.POINTER(AtomicLayerDesc), i,
                                                    C.POINTER(sz)]
            L.moe_atomic_schedule.argtypes = [C.POINTER(AtomicLayerDesc), i, C.POINTER(i)]
            L.moe_set_stage_events.argtypes = [C.POINTER(C.c_void_p), i]
            L.moe_set_stage_events.restype = C.c_int
            L.moe_status_string.argtypes = [i]
            L.moe_status_string.restype = C.c_char_p
            L.moe_last_error.argtypes = []
            L.moe_last_error.restype = C.c_char_p
            for f in ("moe_route_topk", "moe_permute", "moe_grouped_ffn", "moe_combine",
                      "moe_layer_forward", "moe_workspace_size", "moe_replica_split",
                      "moe_layer_forward_noalloc",
                      "moe_layer_forward_replica", "moe_replica_workspace_size",
                      "moe_mwq_group", "moe_grouped_ffn_mwq", "moe_layer_forward_mwq",
                      "moe_mwq_workspace_size", "moe_layer_forward_floe",
                      "moe_floe_workspace_size", "moe_atomic_layer_forward",
                      "moe_atomic_workspace_size", "moe_atomic_schedule"):
                getattr(L, f).restype = C.c_int
            _lib = L
    return _lib


def check(status, fn):
    if status != MOE_OK:
        raise MoeError(status, fn, lib().moe_last_error().decode())
    return status
