"""ds4q oracle — TEST INFRASTRUCTURE ONLY.

ctypes binding of ``ds4q_oracle.c``: a plain, slow fp64 CPU statement of the
routed-MoE expert path on Q2_K / Q4_1 weights.  Only ``tests/``, the smoke
check and the benchmark's CPU-baseline leg may import this package; the GPU
library never does.  See ``ds4q_oracle.h`` for the page citations and the
readings taken where the pages are silent.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ds4q_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libds4q_oracle.so")

Q4_1 = 3
Q2_K = 10
QK = {Q2_K: 256, Q4_1: 32}
BLOCK_BYTES = {Q2_K: 84, Q4_1: 20}

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (-O2, no fast-math, no FP contraction)."""
    if force or not os.path.exists(_LIB_PATH):
        cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
               "-fno-fast-math", "-Wall", "-o", _LIB_PATH + ".tmp", _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(_LIB_PATH + ".tmp", _LIB_PATH)
    return _LIB_PATH


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        L = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        i64, i32 = ctypes.c_int64, ctypes.c_int32
        L.orc_f16_value.restype = ctypes.c_double
        L.orc_f16_value.argtypes = [ctypes.c_uint16]
        L.orc_bf16_rne.restype = ctypes.c_uint16
        L.orc_bf16_rne.argtypes = [ctypes.c_float]
        L.orc_f32_to_bf16.argtypes = [P, P, i64]
        L.orc_q2k_decode_block.argtypes = [P, P]
        L.orc_q41_decode_block.argtypes = [P, P]
        L.orc_dequant_f32.argtypes = [ctypes.c_int, P, i64, i64, P]
        L.orc_dequant_bf16.argtypes = [ctypes.c_int, P, i64, i64, P]
        L.orc_q2k_encode_block.argtypes = [P, P, P, ctypes.c_uint16, ctypes.c_uint16, P]
        L.orc_q41_encode_block.argtypes = [P, ctypes.c_uint16, ctypes.c_uint16, P]
        L.orc_q41_reencode.argtypes = [P, P, P, i64, ctypes.c_int, ctypes.c_int, P]
        L.orc_matvec.argtypes = [ctypes.c_int, P, i64, i64, P, P]
        L.orc_route.argtypes = [P, i32, i32, i32, P, P]
        L.orc_group.argtypes = [P, i32, i32, i32, P, P, P]
        L.orc_expert_ffn.argtypes = [P, i32, P, P]
        L.orc_moe.argtypes = [P, P, P, i32, P, ctypes.c_int]
        L.orc_rmsnorm.argtypes = [P, i32, ctypes.c_double, P]
        L.orc_stack.argtypes = [P, i32, ctypes.c_int, P, P, i32, ctypes.c_double, ctypes.c_int,
                                P, ctypes.c_double]
        L.orc_steer_f64.argtypes = [P, ctypes.c_double, P, i32, i32]
        L.orc_moe_imatrix.argtypes = [P, P, P, i32, P, P, ctypes.c_int]
        L.orc_expert_swiglu.argtypes = [P, i32, P, P]
        L.orc_steer.argtypes = [P, ctypes.c_double, P, i32, i32, P, P]
        L.orc_f16_rne.restype = ctypes.c_uint16
        L.orc_f16_rne.argtypes = [ctypes.c_float]
        L.orc_e4m3_rne.restype = ctypes.c_uint8
        L.orc_e4m3_rne.argtypes = [ctypes.c_float]
        L.orc_e4m3_value.restype = ctypes.c_double
        L.orc_e4m3_value.argtypes = [ctypes.c_uint8]
        _lib = L
    return _lib


def _p(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


class _Layer(ctypes.Structure):
    _fields_ = [("n_embd", ctypes.c_int32), ("n_ff", ctypes.c_int32),
                ("n_expert", ctypes.c_int32), ("n_expert_used", ctypes.c_int32),
                ("type_gate", ctypes.c_int32), ("type_up", ctypes.c_int32),
                ("type_down", ctypes.c_int32),
                ("gate", ctypes.c_void_p), ("up", ctypes.c_void_p), ("down", ctypes.c_void_p)]


class Layer:
    """Host-side expert weights of one layer: uint8 arrays [E][rows][block bytes...]."""

    def __init__(self, n_embd, n_ff, n_expert, k, qtype, gate, up, down,
                 type_up=None, type_down=None):
        self.gate = np.ascontiguousarray(gate, dtype=np.uint8)
        self.up = np.ascontiguousarray(up, dtype=np.uint8)
        self.down = np.ascontiguousarray(down, dtype=np.uint8)
        self.s = _Layer(n_embd, n_ff, n_expert, k, qtype,
                        qtype if type_up is None else type_up,
                        qtype if type_down is None else type_down,
                        self.gate.ctypes.data, self.up.ctypes.data, self.down.ctypes.data)


def f16_value(bits: int) -> float:
    return lib().orc_f16_value(bits)


def bf16_rne(a: np.ndarray) -> np.ndarray:
    a = np.ascontiguousarray(a, dtype=np.float32)
    out = np.empty(a.shape, dtype=np.uint16)
    lib().orc_f32_to_bf16(_p(a), _p(out), a.size)
    return out


def q2k_decode_block(blk: np.ndarray) -> np.ndarray:
    blk = np.ascontiguousarray(blk, dtype=np.uint8)
    assert blk.size == 84
    out = np.empty(256, dtype=np.float32)
    lib().orc_q2k_decode_block(_p(blk), _p(out))
    return out


def q41_decode_block(blk: np.ndarray) -> np.ndarray:
    blk = np.ascontiguousarray(blk, dtype=np.uint8)
    assert blk.size == 20
    out = np.empty(32, dtype=np.float32)
    lib().orc_q41_decode_block(_p(blk), _p(out))
    return out


def dequant_f32(qtype: int, src: np.ndarray, rows: int, cols: int) -> np.ndarray:
    src = np.ascontiguousarray(src, dtype=np.uint8)
    out = np.empty((rows, cols), dtype=np.float32)
    rc = lib().orc_dequant_f32(qtype, _p(src), rows, cols, _p(out))
    if rc:
        raise ValueError(f"orc_dequant_f32 rc={rc}")
    return out


def dequant_bf16(qtype: int, src: np.ndarray, rows: int, cols: int) -> np.ndarray:
    src = np.ascontiguousarray(src, dtype=np.uint8)
    out = np.empty((rows, cols), dtype=np.uint16)
    rc = lib().orc_dequant_bf16(qtype, _p(src), rows, cols, _p(out))
    if rc:
        raise ValueError(f"orc_dequant_bf16 rc={rc}")
    return out


def q2k_encode_block(sc, mn, q, d_bits: int, dmin_bits: int) -> np.ndarray:
    sc = np.ascontiguousarray(sc, dtype=np.uint8)
    mn = np.ascontiguousarray(mn, dtype=np.uint8)
    q = np.ascontiguousarray(q, dtype=np.uint8)
    out = np.empty(84, dtype=np.uint8)
    lib().orc_q2k_encode_block(_p(sc), _p(mn), _p(q), d_bits, dmin_bits, _p(out))
    return out


def q41_encode_block(q, d_bits: int, m_bits: int) -> np.ndarray:
    q = np.ascontiguousarray(q, dtype=np.uint8)
    out = np.empty(20, dtype=np.uint8)
    lib().orc_q41_encode_block(_p(q), d_bits, m_bits, _p(out))
    return out


def q41_reencode(codes, scale_bits, min_bits, group: int, bits: int) -> np.ndarray:
    codes = np.ascontiguousarray(codes, dtype=np.uint8).reshape(-1)
    scale_bits = np.ascontiguousarray(scale_bits, dtype=np.uint16).reshape(-1)
    min_bits = np.ascontiguousarray(min_bits, dtype=np.uint16).reshape(-1)
    out = np.empty(codes.size // 32 * 20, dtype=np.uint8)
    rc = lib().orc_q41_reencode(_p(codes), _p(scale_bits), _p(min_bits), codes.size,
                                group, bits, _p(out))
    if rc:
        raise ValueError("re-encode refused (group % 32 != 0, bits > 4 or code overflow)")
    return out


def matvec(qtype: int, w: np.ndarray, rows: int, cols: int, x: np.ndarray) -> np.ndarray:
    w = np.ascontiguousarray(w, dtype=np.uint8)
    x = np.ascontiguousarray(x, dtype=np.float32)
    y = np.empty(rows, dtype=np.float64)
    rc = lib().orc_matvec(qtype, _p(w), rows, cols, _p(x), _p(y))
    if rc:
        raise ValueError(f"orc_matvec rc={rc}")
    return y


def route(logits: np.ndarray, k: int):
    logits = np.ascontiguousarray(logits, dtype=np.float32)
    T, E = logits.shape
    ids = np.empty((T, k), dtype=np.int32)
    w = np.empty((T, k), dtype=np.float64)
    lib().orc_route(_p(logits), T, E, k, _p(ids), _p(w))
    return ids, w


def group(ids: np.ndarray, n_expert: int):
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    T, k = ids.shape
    counts = np.empty(n_expert, dtype=np.int32)
    offsets = np.empty(n_expert + 1, dtype=np.int32)
    pairs = np.empty(T * k, dtype=np.int32)
    lib().orc_group(_p(ids), T, k, n_expert, _p(counts), _p(offsets), _p(pairs))
    return counts, offsets, pairs


def expert_ffn(layer: Layer, e: int, x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float64)
    o = np.empty(layer.s.n_embd, dtype=np.float64)
    rc = lib().orc_expert_ffn(ctypes.byref(layer.s), e, _p(x), _p(o))
    if rc:
        raise ValueError("bad layer types")
    return o


def moe(layer: Layer, x: np.ndarray, logits: np.ndarray, n_threads: int = 0) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    logits = np.ascontiguousarray(logits, dtype=np.float32)
    T = x.shape[0]
    y = np.empty((T, layer.s.n_embd), dtype=np.float64)
    rc = lib().orc_moe(ctypes.byref(layer.s), _p(x), _p(logits), T, _p(y), n_threads)
    if rc:
        raise ValueError("bad layer types")
    return y


def expert_swiglu(layer: Layer, e: int, x: np.ndarray) -> np.ndarray:
    """The expert's SwiGLU row silu(W1 x) * (W3 x), fp64 [n_ff]."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    h = np.empty(layer.s.n_ff, dtype=np.float64)
    if lib().orc_expert_swiglu(ctypes.byref(layer.s), e, _p(x), _p(h)):
        raise ValueError("bad layer types")
    return h


def moe_imatrix(layer: Layer, x: np.ndarray, logits: np.ndarray, n_threads: int = 0):
    """[P1] imatrix statistics of one layer call on MoE input rows x:
    (imat_in [E][n_embd], imat_down [E][n_ff]), fp64, expert-major."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    logits = np.ascontiguousarray(logits, dtype=np.float32)
    E = layer.s.n_expert
    a = np.zeros((E, layer.s.n_embd), dtype=np.float64)
    b = np.zeros((E, layer.s.n_ff), dtype=np.float64)
    if lib().orc_moe_imatrix(ctypes.byref(layer.s), _p(x), _p(logits), x.shape[0], _p(a), _p(b),
                             n_threads):
        raise ValueError("bad layer types")
    return a, b


def rmsnorm(x: np.ndarray, eps: float = 1e-6) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.float64)
    lib().orc_rmsnorm(_p(x), x.size, eps, _p(out))
    return out


def stack(layers, x: np.ndarray, logits: np.ndarray, prefill_bf16: bool,
          eps: float = 1e-6, n_threads: int = 0, dirs: np.ndarray | None = None,
          steer_scale: float = 0.0) -> np.ndarray:
    """x: [T][D] fp32 residual stream; logits: [L][T][E]; dirs (optional):
    layer-major steering directions [L][D] ([P3]).  Returns the new x."""
    arr = (_Layer * len(layers))(*[l.s for l in layers])
    x = np.array(x, dtype=np.float32, copy=True, order="C")
    logits = np.ascontiguousarray(logits, dtype=np.float32)
    if dirs is not None:
        dirs = np.ascontiguousarray(dirs, dtype=np.float32)
        assert dirs.shape == (len(layers), x.shape[1])
    rc = lib().orc_stack(arr, len(layers), int(prefill_bf16), _p(x), _p(logits), x.shape[0],
                         eps, n_threads, None if dirs is None else _p(dirs), float(steer_scale))
    if rc:
        raise ValueError("bad layer types")
    return x


def steer(dir_: np.ndarray, scale: float, y: np.ndarray, residual: np.ndarray | None = None) -> np.ndarray:
    """[P3] out_r (+)= y_r - scale * dir * (dir . y_r), fp64, one rounding."""
    y = np.ascontiguousarray(y, dtype=np.float32)
    dir_ = np.ascontiguousarray(dir_, dtype=np.float32)
    rows, n = y.reshape(-1, y.shape[-1]).shape
    out = np.empty_like(y)
    res = None if residual is None else np.ascontiguousarray(residual, dtype=np.float32)
    lib().orc_steer(_p(dir_), float(scale), _p(y), rows, n, None if res is None else _p(res), _p(out))
    return out


def steer_f64(dir_: np.ndarray, scale: float, y: np.ndarray) -> np.ndarray:
    """[P3] y_r - scale * dir * (dir . y_r) on fp64 rows, no rounding."""
    y = np.array(y, dtype=np.float64, copy=True, order="C")
    dir_ = np.ascontiguousarray(dir_, dtype=np.float32)
    rows, n = y.reshape(-1, y.shape[-1]).shape
    lib().orc_steer_f64(_p(dir_), float(scale), _p(y), rows, n)
    return y


def f16_rne(x: np.ndarray) -> np.ndarray:
    """[P4] f32 -> binary16 bits (see ds4q_oracle.h for the rounding reading)."""
    x = np.ascontiguousarray(x, dtype=np.float32).ravel()
    L = lib()
    return np.array([L.orc_f16_rne(float(v)) for v in x], dtype=np.uint16)


def e4m3_rne(x: np.ndarray) -> np.ndarray:
    """[P4] f32 -> OCP E4M3 bits, round to nearest even, saturating."""
    x = np.ascontiguousarray(x, dtype=np.float32).ravel()
    L = lib()
    return np.array([L.orc_e4m3_rne(float(v)) for v in x], dtype=np.uint8)


def e4m3_value(bits) -> np.ndarray:
    L = lib()
    return np.array([L.orc_e4m3_value(int(b)) for b in np.asarray(bits).ravel()], dtype=np.float64)
