"""ctypes binding of libkos.so: argument marshalling only.

Every step of every operation runs in the library's HIP kernels; this module
only turns torch tensors into device pointers and the current torch stream
into a hipStream_t.  Importing it fails loudly if the library is not built.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, c_char_p, c_int32, c_int64, c_size_t, c_uint32, c_void_p

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libkos.so")

# status codes (include/kos.h)
KOS_OK, KOS_ERR_ARG, KOS_ERR_SHAPE, KOS_ERR_ALIGN, KOS_ERR_WORKSPACE, KOS_ERR_HIP, \
    KOS_ERR_UNSUPPORTED, KOS_ERR_TIMEOUT, KOS_ERR_CAPACITY = range(9)
STATUS_NAMES = ["OK", "ERR_ARG", "ERR_SHAPE", "ERR_ALIGN", "ERR_WORKSPACE", "ERR_HIP",
                "ERR_UNSUPPORTED", "ERR_TIMEOUT", "ERR_CAPACITY"]
KOS_BF16, KOS_F32 = 0, 1
MODE_FUSED, MODE_FIXED, MODE_UNFUSED = 0, 1, 2
RS_BAND, RS_ROW = 0, 1
POLICY_DEFAULT, POLICY_SWAPPED = 0, 1

# Every symbol include/kos.h declares.
EXPORTS = [
    "kos_opts_default", "kos_workspace_bytes", "kos_workspace_init", "kos_workspace_status",
    "kos_last_error", "kos_device_cu_count", "kos_ag_gemm", "kos_gemm_rs",
    "kos_ag_gemm_mx", "kos_gemm_rs_mx", "kos_ag_gemm_wt", "kos_gemm_rs_wt",
    "kos_moe_dispatch", "kos_moe_combine", "kos_workspace_trace", "kos_ag_gemm_noalloc", "kos_moe_layer",
    "kos_moe_layer_bwd",
]


class KosError(RuntimeError):
    def __init__(self, status: int, msg: str):
        name = STATUS_NAMES[status] if 0 <= status < len(STATUS_NAMES) else str(status)
        super().__init__(f"KOS_{name}: {msg}")
        self.status = status


class Opts(ctypes.Structure):
    _fields_ = [("mode", c_int32), ("n_movers", c_int32), ("rs_order", c_int32),
                ("grid", c_int32), ("spin_limit", c_uint32), ("peer_link", c_int32),
                ("trace", c_int32), ("policy", c_int32)]


class TraceRec(ctypes.Structure):
    _fields_ = [("t0", ctypes.c_uint64), ("dt", c_uint32), ("tag", c_uint32)]


TRACE_RECORDS = 512     # KOS_TRACE_RECORDS: records per workgroup
TRACE_MAX_WG = 256      # KOS_TRACE_MAX_WG
TRACE_LAUNCHES = 4      # KOS_TRACE_LAUNCHES: slots, one per launch of a call
TRACE_KINDS = {1: "move", 2: "tile", 3: "wait", 4: "reduce", 5: "route", 6: "scan", 7: "push", 8: "fold",
               9: "tile_down"}
TRACE_CLOCK = 10        # KOS_TR_CLOCK: record 1, shader-clock cycles over the lifetime


class DeviceError(ctypes.Structure):
    _fields_ = [("status", c_int32), ("entry", c_uint32)]


class MoeShape(ctypes.Structure):
    _fields_ = [("world", c_int32), ("rank", c_int32), ("tokens", c_int32),
                ("hidden", c_int32), ("experts", c_int32), ("topk", c_int32),
                ("ffn", c_int32), ("reserved", c_int32)]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built: run __graft_entry__.build() "
                          "(hipcc --offload-arch=gfx950); there is no fallback path")
    lib = ctypes.CDLL(LIB_PATH)
    P = c_void_p
    PP = POINTER(c_void_p)
    sig = {
        "kos_opts_default": (None, [POINTER(Opts)]),
        "kos_workspace_bytes": (c_size_t, []),
        "kos_workspace_init": (c_int32, [P, c_size_t, P]),
        "kos_workspace_status": (c_int32, [P, P, POINTER(DeviceError)]),
        "kos_last_error": (c_char_p, []),
        "kos_device_cu_count": (c_int32, []),
        "kos_workspace_trace": (c_int32, [P, P, c_size_t, P]),
        "kos_ag_gemm": (c_int32, [c_int32, c_int32, c_int64, c_int64, c_int64, P, PP, P, P, P,
                                  c_int32, POINTER(Opts), P, c_size_t, P]),
        "kos_gemm_rs": (c_int32, [c_int32, c_int32, c_int64, c_int64, c_int64, P, P, PP, P, P,
                                  POINTER(Opts), P, c_size_t, P]),
        "kos_ag_gemm_noalloc": (c_int32, [c_int32, c_int32, c_int64, c_int64, c_int64, P, PP, P, P, P,
                                          c_int32, POINTER(Opts), P, P]),
        "kos_ag_gemm_wt": (c_int32, [c_int32, c_int32, c_int64, c_int64, c_int64, P, PP, P, P, P,
                                     c_int32, POINTER(Opts), P, c_size_t, P]),
        "kos_gemm_rs_wt": (c_int32, [c_int32, c_int32, c_int64, c_int64, c_int64, P, P, PP, P, P,
                                     POINTER(Opts), P, c_size_t, P]),
        "kos_ag_gemm_mx": (c_int32, [c_int32, c_int32, c_int64, c_int64, c_int64, P, P, PP, PP, P, P,
                                     P, P, P, c_int32, POINTER(Opts), P, c_size_t, P]),
        "kos_gemm_rs_mx": (c_int32, [c_int32, c_int32, c_int64, c_int64, c_int64, P, P, P, P, PP, P, P,
                                     POINTER(Opts), P, c_size_t, P]),
        "kos_moe_dispatch": (c_int32, [POINTER(MoeShape), P, P, PP, P, P, P, P, P, PP, POINTER(c_int64),
                                       P, c_int64, P, P, POINTER(Opts), P, c_size_t, P]),
        "kos_moe_layer": (c_int32, [POINTER(MoeShape), P, P, PP, P, P, P, P, PP, P, P, P, P, PP, POINTER(c_int64),
                                    P, c_int64, P, P, P, P, P, P, PP, POINTER(c_int64), P, POINTER(Opts), P,
                                    c_size_t, P]),
        "kos_moe_combine": (c_int32, [POINTER(MoeShape), P, P, P, c_int64, P, P, P, P, P, P, P, P,
                                      PP, P, P, P, P, PP, POINTER(c_int64), P, POINTER(Opts), P, c_size_t, P]),
        "kos_moe_layer_bwd": (c_int32, [POINTER(MoeShape), P, P, P, P, P, P, P, c_int64, P, P, P, PP, P, P, P,
                                        P, P, PP, PP, POINTER(c_int64), P, P, P, P, P, PP, PP, POINTER(c_int64),
                                        P, P, POINTER(Opts), P, c_size_t, P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name, None)
        if fn is None:
            continue
        fn.restype = res
        fn.argtypes = args
    return lib


lib = _load()


def check(status: int) -> None:
    if status != KOS_OK:
        raise KosError(status, lib.kos_last_error().decode(errors="replace"))


def opts(mode=MODE_FUSED, n_movers=-1, rs_order=RS_BAND, grid=0, spin_limit=0, peer_link=0,
         trace=False, policy=0) -> Opts:
    o = Opts()
    lib.kos_opts_default(ctypes.byref(o))
    o.mode, o.n_movers, o.rs_order, o.grid = mode, n_movers, rs_order, grid
    o.spin_limit, o.peer_link, o.trace, o.policy = spin_limit, peer_link, int(bool(trace)), policy
    return o


def ptr_array(ptrs) -> ctypes.Array:
    """Host array of device pointers (None -> NULL)."""
    arr = (c_void_p * len(ptrs))()
    for i, p in enumerate(ptrs):
        arr[i] = p
    return arr
