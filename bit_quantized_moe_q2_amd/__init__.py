"""Python binding of libds4q.so: the routed-MoE expert FFN on Q2_K / Q4_1
block-quantised weights for MI355X (gfx950).

Argument marshalling only: every function takes torch tensors that already
live on the GPU, passes their device pointers and the current HIP stream to
the C entry point of the same name (declared in ``include/ds4q.h``), and
raises :class:`Ds4qError` on a non-zero status.  No computation happens here
and there is no CPU fallback: if the library is not built, :func:`load`
raises.
"""
from __future__ import annotations

import ctypes
import os

__all__ = [
    "TYPE_F32", "TYPE_F16", "TYPE_Q4_1", "TYPE_Q2_K", "TYPE_IQ2_XXS", "TYPE_BF16",
    "F_ACCUMULATE", "F_RMSNORM_INPUT", "Ds4qError", "MoeLayer", "RouteOut", "load",
    "ds4q_abi_version", "ds4q_strerror", "ds4q_dequant", "ds4q_matvec", "ds4q_route",
    "ds4q_route_workspace_size", "ds4q_moe_workspace_size", "ds4q_moe_decode",
    "ds4q_moe_decode_static", "ds4q_moe_decode_phases", "PHASE_ROUTE", "PHASE_GATEUP", "PHASE_DOWN", "PHASE_ALL",
    "ds4q_moe_prefill", "ds4q_moe_stack", "ds4q_steer", "ds4q_act_encode", "ds4q_act_decode",
    "ds4q_timing_enable", "ds4q_timing_read",
    "QK", "BLOCK_BYTES", "row_bytes",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libds4q.so")

TYPE_F32, TYPE_F16, TYPE_Q4_1, TYPE_Q2_K, TYPE_IQ2_XXS, TYPE_BF16 = 0, 1, 3, 10, 16, 30
SCRATCH_BYTES = 24 << 20  # DS4Q_SCRATCH_BYTES
F_ACCUMULATE, F_RMSNORM_INPUT = 0x1, 0x2
PHASE_ROUTE, PHASE_GATEUP, PHASE_DOWN, PHASE_ALL = 0x1, 0x2, 0x4, 0x7
QK = {TYPE_Q2_K: 256, TYPE_Q4_1: 32}
BLOCK_BYTES = {TYPE_Q2_K: 84, TYPE_Q4_1: 20}


def row_bytes(qtype: int, cols: int) -> int:
    return cols // QK[qtype] * BLOCK_BYTES[qtype]


class Ds4qError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn}: {ds4q_strerror(status)} ({status})")


class MoeLayer(ctypes.Structure):
    """Mirror of ds4q_moe_layer."""
    _fields_ = [("n_embd", ctypes.c_int32), ("n_ff", ctypes.c_int32),
                ("n_expert", ctypes.c_int32), ("n_expert_used", ctypes.c_int32),
                ("type_gate", ctypes.c_int32), ("type_up", ctypes.c_int32),
                ("type_down", ctypes.c_int32),
                ("gate", ctypes.c_void_p), ("up", ctypes.c_void_p), ("down", ctypes.c_void_p),
                ("flags", ctypes.c_uint32), ("norm_eps", ctypes.c_float),
                ("steer_dir", ctypes.c_void_p), ("steer_scale", ctypes.c_float),
                ("imatrix_in", ctypes.c_void_p), ("imatrix_down", ctypes.c_void_p)]

    @classmethod
    def from_tensors(cls, gate, up, down, n_embd, n_ff, n_expert, k, type_gate,
                     type_up=None, type_down=None, flags=0, norm_eps=1e-6,
                     steer_dir=None, steer_scale=0.0):
        L = cls(n_embd, n_ff, n_expert, k, type_gate,
                type_gate if type_up is None else type_up,
                type_gate if type_down is None else type_down,
                _ptr(gate), _ptr(up), _ptr(down), flags, norm_eps, _ptr(steer_dir), steer_scale)
        L._keep = (gate, up, down, steer_dir)  # keep the tensors alive with the struct
        return L

    def set_imatrix(self, imatrix_in, imatrix_down):
        """Accumulate the layer's imatrix statistics into device f32 tensors
        [n_expert][n_embd] and [n_expert][n_ff] (None: not collected)."""
        self.imatrix_in = _ptr(imatrix_in)
        self.imatrix_down = _ptr(imatrix_down)
        self._keep_stats = (imatrix_in, imatrix_down)

    def set_steering(self, steer_dir, steer_scale):
        """Steer this layer's MoE output with a device f32 [n_embd] direction
        (None switches steering off)."""
        self.steer_dir = _ptr(steer_dir)
        self.steer_scale = steer_scale
        self._keep = self._keep[:3] + (steer_dir,)


class RouteOut(ctypes.Structure):
    """Mirror of ds4q_route_out (device pointers, any may be 0)."""
    _fields_ = [("topk_ids", ctypes.c_void_p), ("topk_w", ctypes.c_void_p),
                ("expert_counts", ctypes.c_void_p), ("expert_offsets", ctypes.c_void_p),
                ("sorted_pairs", ctypes.c_void_p)]

    @classmethod
    def from_tensors(cls, topk_ids=None, topk_w=None, expert_counts=None, expert_offsets=None,
                     sorted_pairs=None):
        r = cls(_ptr(topk_ids), _ptr(topk_w), _ptr(expert_counts), _ptr(expert_offsets),
                _ptr(sorted_pairs))
        r._keep = (topk_ids, topk_w, expert_counts, expert_offsets, sorted_pairs)
        return r


_lib = None


def load():
    """Load libds4q.so (built in-tree by ``__graft_entry__.build()``)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build()")
    L = ctypes.CDLL(LIB_PATH)
    P, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    LP, RP = ctypes.POINTER(MoeLayer), ctypes.POINTER(RouteOut)
    sig = {
        "ds4q_abi_version": (ctypes.c_int, []),
        "ds4q_strerror": (ctypes.c_char_p, [ctypes.c_int]),
        "ds4q_dequant": (ctypes.c_int, [i32, P, i64, i64, i32, P, P]),
        "ds4q_matvec": (ctypes.c_int, [i32, P, i64, i64, P, i32, P, P]),
        "ds4q_route_workspace_size": (sz, [i32, i32, i32]),
        "ds4q_route": (ctypes.c_int, [P, i32, i32, i32, RP, P, sz, P]),
        "ds4q_moe_workspace_size": (sz, [LP, i32, i32]),
        "ds4q_moe_decode": (ctypes.c_int, [LP, P, P, i32, P, RP, P, sz, P]),
        "ds4q_moe_decode_static": (ctypes.c_int, [LP, P, P, i32, P, RP, P]),
        "ds4q_moe_decode_phases": (ctypes.c_int, [LP, P, P, i32, P, RP, P, sz, ctypes.c_uint32, P]),
        "ds4q_moe_prefill": (ctypes.c_int, [LP, P, i32, P, i32, P, RP, P, sz, P]),
        "ds4q_moe_stack": (ctypes.c_int, [LP, i32, i32, P, P, i32, P, sz, P]),
        "ds4q_steer": (ctypes.c_int, [P, ctypes.c_float, P, i32, i32, P, ctypes.c_uint32, P]),
        "ds4q_act_encode": (ctypes.c_int, [P, i64, i32, P, P]),
        "ds4q_act_decode": (ctypes.c_int, [P, i64, i32, P, P]),
        "ds4q_timing_enable": (ctypes.c_int, [ctypes.c_int]),
        "ds4q_timing_read": (ctypes.c_int, [P, ctypes.c_int, P, P, ctypes.c_int,
                                            ctypes.POINTER(ctypes.c_int)]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(L, name)
        fn.restype, fn.argtypes = res, args
    _lib = L
    return L


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def _check(fn: str, rc: int):
    if rc != 0:
        raise Ds4qError(fn, rc)


def ds4q_abi_version() -> int:
    return load().ds4q_abi_version()


def ds4q_strerror(status: int) -> str:
    return load().ds4q_strerror(status).decode()


def ds4q_dequant(src_type, src, rows, cols, dst_type, dst, stream=None):
    _check("ds4q_dequant", load().ds4q_dequant(src_type, _ptr(src), rows, cols, dst_type,
                                               _ptr(dst), _stream(stream)))


def ds4q_matvec(w_type, w, rows, cols, x, n_tok, y, stream=None):
    _check("ds4q_matvec", load().ds4q_matvec(w_type, _ptr(w), rows, cols, _ptr(x), n_tok,
                                             _ptr(y), _stream(stream)))


def ds4q_route_workspace_size(n_tok, n_expert, k) -> int:
    return load().ds4q_route_workspace_size(n_tok, n_expert, k)


def ds4q_route(logits, n_tok, n_expert, k, out: RouteOut, workspace, workspace_bytes=None,
               stream=None):
    wb = workspace.numel() * workspace.element_size() if workspace_bytes is None else workspace_bytes
    _check("ds4q_route", load().ds4q_route(_ptr(logits), n_tok, n_expert, k, ctypes.byref(out),
                                           _ptr(workspace), wb, _stream(stream)))


def ds4q_moe_workspace_size(layer: MoeLayer, max_tok: int, mode: int) -> int:
    return load().ds4q_moe_workspace_size(ctypes.byref(layer), max_tok, mode)


def _ws_bytes(workspace, workspace_bytes):
    if workspace_bytes is not None:
        return workspace_bytes
    return 0 if workspace is None else workspace.numel() * workspace.element_size()


def ds4q_moe_decode(layer: MoeLayer, x, logits, n_tok, y, route: RouteOut | None, workspace,
                    workspace_bytes=None, stream=None):
    _check("ds4q_moe_decode", load().ds4q_moe_decode(
        ctypes.byref(layer), _ptr(x), _ptr(logits), n_tok, _ptr(y),
        ctypes.byref(route) if route is not None else None, _ptr(workspace),
        _ws_bytes(workspace, workspace_bytes), _stream(stream)))


def ds4q_moe_decode_static(layer: MoeLayer, x, logits, n_tok, y, route: RouteOut | None,
                           stream=None):
    _check("ds4q_moe_decode_static", load().ds4q_moe_decode_static(
        ctypes.byref(layer), _ptr(x), _ptr(logits), n_tok, _ptr(y),
        ctypes.byref(route) if route is not None else None, _stream(stream)))


def ds4q_moe_decode_phases(layer: MoeLayer, x, logits, n_tok, y, route: RouteOut | None,
                           workspace, phases, workspace_bytes=None, stream=None):
    _check("ds4q_moe_decode_phases", load().ds4q_moe_decode_phases(
        ctypes.byref(layer), _ptr(x), _ptr(logits), n_tok, _ptr(y),
        ctypes.byref(route) if route is not None else None, _ptr(workspace),
        _ws_bytes(workspace, workspace_bytes), phases, _stream(stream)))


def ds4q_moe_prefill(layer: MoeLayer, x, x_type, logits, n_tok, y, route: RouteOut | None,
                     workspace, workspace_bytes=None, stream=None):
    _check("ds4q_moe_prefill", load().ds4q_moe_prefill(
        ctypes.byref(layer), _ptr(x), x_type, _ptr(logits), n_tok, _ptr(y),
        ctypes.byref(route) if route is not None else None, _ptr(workspace),
        _ws_bytes(workspace, workspace_bytes), _stream(stream)))


def ds4q_moe_stack(layers, mode, x, logits, n_tok, workspace, workspace_bytes=None, stream=None):
    arr = (MoeLayer * len(layers))(*layers)
    _check("ds4q_moe_stack", load().ds4q_moe_stack(
        arr, len(layers), mode, _ptr(x), _ptr(logits), n_tok, _ptr(workspace),
        _ws_bytes(workspace, workspace_bytes), _stream(stream)))


def ds4q_steer(dir_, scale, y, n_rows, n_embd, out, flags=0, stream=None):
    _check("ds4q_steer", load().ds4q_steer(_ptr(dir_), float(scale), _ptr(y), n_rows, n_embd,
                                           _ptr(out), flags, _stream(stream)))


def ds4q_act_encode(src, n, bits, dst, stream=None):
    _check("ds4q_act_encode", load().ds4q_act_encode(_ptr(src), n, bits, _ptr(dst), _stream(stream)))


def ds4q_act_decode(src, n, bits, dst, stream=None):
    _check("ds4q_act_decode", load().ds4q_act_decode(_ptr(src), n, bits, _ptr(dst), _stream(stream)))


def ds4q_timing_enable(on: bool):
    _check("ds4q_timing_enable", load().ds4q_timing_enable(1 if on else 0))


def ds4q_timing_read() -> dict:
    """{launch site: (total_ms, count)} since the last read."""
    n_max, name_len = 32, 32
    names = ctypes.create_string_buffer(n_max * name_len)
    tot = (ctypes.c_double * n_max)()
    cnt = (ctypes.c_int64 * n_max)()
    n = ctypes.c_int(0)
    _check("ds4q_timing_read", load().ds4q_timing_read(
        ctypes.cast(names, ctypes.c_void_p), name_len, ctypes.cast(tot, ctypes.c_void_p),
        ctypes.cast(cnt, ctypes.c_void_p), n_max, ctypes.byref(n)))
    out = {}
    for i in range(n.value):
        nm = names.raw[i * name_len:(i + 1) * name_len].split(b"\0", 1)[0].decode()
        out[nm] = (tot[i], cnt[i])
    return out
