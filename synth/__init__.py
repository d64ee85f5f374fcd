"""Seeded synthetic inputs for the routed-MoE expert path.

This module is shared by the test oracle and by the GPU library's callers
(tests, bench).  It holds *no* arithmetic of the method: it never decodes a
block, never computes a dot product, never routes.  It only draws bytes and
numbers from a counter-based generator and places them where the input
formats say they live.

Generator
---------
SplitMix64 (G. Steele, D. Lea, C. Flood, "Fast splittable pseudorandom number
generators", OOPSLA 2014), used counter-style: word ``i`` of stream ``key`` is
``mix(key + (i + 1) * 0x9E3779B97F4A7C15)`` where ``mix`` is SplitMix64's
output function.  A HIP twin of the same function lives in
``synth/csrc/synth_gen.hip`` so that multi-GB weight stacks can be drawn on the
device; tests check that both produce the same bytes.

Recipes (all seeded)
--------------------
* Q2_K block (84 B): bytes 0..79 (16 scale/min nibble bytes + 64 code bytes)
  are uniform random bytes, i.e. scale and min nibbles U{0..15} and 2-bit
  codes U{0..3}; the two fp16 fields at bytes 80 and 82 (``d``, ``dmin``) are
  drawn from |N(0, 0.01)|.  Block ``b`` of a stream consumes words
  ``11b .. 11b+10``: their 88 little-endian bytes give bytes 0..79 directly,
  bytes 80..81 and 82..83 are 16-bit indices into the |N(0, 0.01)| fp16
  quantile table, bytes 84..87 are unused.
* Q4_1 block (20 B): ``d`` (bytes 0..1) from |N(0, 0.01)|, ``m`` (bytes 2..3)
  from -7.5 * |N(0, 0.01)| (an independent draw: the block offset is the
  group minimum, so that d*q + m is centred near zero like a real group of
  weights), 16 code bytes (bytes 4..19) uniform, i.e. nibbles U{0..15}.
  Block ``b`` consumes words ``3b .. 3b+2``.
* fp16 draws use 65536-entry quantile tables (value at the midpoint of each of
  65536 equal-probability cells, rounded to fp16), so host and device produce
  identical bits without evaluating transcendental functions on the device.
* Activations and router logits: N(0, 1) by Box-Muller in float64, rounded to
  float32 (and, for bf16 activations, from float32 to bf16 round-to-nearest-
  even).  Zipf-skewed logits: ``-s * ln(rank(e)) + Gumbel(0, 1)`` with a seeded
  permutation ``rank`` of 1..E, so that top-k is a Zipf(s) sample without
  replacement (the Gumbel-top-k trick).
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "GAMMA", "splitmix64", "stream_key", "words", "uniform01", "normal_f32",
    "f16_tables", "q2k_blocks", "q41_blocks", "expert_tensor_blocks",
    "x_f32", "x_bf16", "logits_normal", "logits_zipf", "bf16_bits_from_f32",
    "Q2K_BLOCK_BYTES", "Q41_BLOCK_BYTES", "Q2K_WORDS_PER_BLOCK",
    "Q41_WORDS_PER_BLOCK", "TENSOR_TAG", "layer_key",
]

M64 = (1 << 64) - 1
GAMMA = 0x9E3779B97F4A7C15
_C1 = 0xBF58476D1CE4E5B9
_C2 = 0x94D049BB133111EB

Q2K_BLOCK_BYTES = 84
Q41_BLOCK_BYTES = 20
Q2K_WORDS_PER_BLOCK = 11
Q41_WORDS_PER_BLOCK = 3

# Tensor tags follow the routed-expert roles: w1 = gate, w2 = down, w3 = up.
TENSOR_TAG = {"gate": 1, "down": 2, "up": 3}


def _mix_scalar(z: int) -> int:
    z &= M64
    z = ((z ^ (z >> 30)) * _C1) & M64
    z = ((z ^ (z >> 27)) * _C2) & M64
    return z ^ (z >> 31)


def splitmix64(key: int, idx) -> np.ndarray:
    """Counter-based SplitMix64: word ``idx`` (uint64 array) of stream ``key``."""
    idx = np.asarray(idx, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = np.uint64(key & M64) + (idx + np.uint64(1)) * np.uint64(GAMMA)
        z = (z ^ (z >> np.uint64(30))) * np.uint64(_C1)
        z = (z ^ (z >> np.uint64(27))) * np.uint64(_C2)
        z = z ^ (z >> np.uint64(31))
    return z


def stream_key(*tags: int) -> int:
    """Fold integer tags into one 64-bit stream key."""
    h = 0x243F6A8885A308D3
    for t in tags:
        h = _mix_scalar(h ^ (int(t) & M64))
        h = _mix_scalar(h + GAMMA)
    return h


def layer_key(seed: int, layer: int, tensor: str, expert: int) -> int:
    """Stream key of one expert matrix (``tensor`` in gate/up/down)."""
    return stream_key(seed, 0x5741, layer, TENSOR_TAG[tensor], expert)


def words(key: int, start: int, count: int) -> np.ndarray:
    return splitmix64(key, np.arange(start, start + count, dtype=np.uint64))


def uniform01(key: int, n: int, start: int = 0) -> np.ndarray:
    """U(0,1) float64 from the top 53 bits, open at both ends."""
    w = words(key, start, n)
    return ((w >> np.uint64(11)).astype(np.float64) + 0.5) * (2.0 ** -53)


def normal_f32(key: int, n: int) -> np.ndarray:
    """N(0,1) by Box-Muller (cosine branch), computed in float64, rounded to f32."""
    u = uniform01(key, 2 * n).reshape(n, 2)
    z = np.sqrt(-2.0 * np.log(u[:, 0])) * np.cos(2.0 * np.pi * u[:, 1])
    return z.astype(np.float32)


_TABLES: dict = {}


def f16_tables(sigma: float = 0.01):
    """(half_normal, q41_min) fp16 quantile tables as uint16[65536] bit patterns:
    |N(0, sigma)| and -7.5 * |N(0, sigma)|.

    Entry ``u`` is the distribution's quantile at the midpoint of cell ``u``
    of 65536 equal-probability cells, rounded to fp16 (RNE)."""
    key = float(sigma)
    if key not in _TABLES:
        from scipy.special import ndtri
        u = (np.arange(65536, dtype=np.float64) + 0.5) / 65536.0
        half = sigma * ndtri(0.5 + 0.5 * u)
        _TABLES[key] = (half.astype(np.float16).view(np.uint16).copy(),
                        (-7.5 * half).astype(np.float16).view(np.uint16).copy())
    return _TABLES[key]


def q2k_blocks(key: int, n_blocks: int, start_block: int = 0) -> np.ndarray:
    """``n_blocks`` Q2_K blocks (uint8 [n, 84]) of stream ``key``."""
    half, _ = f16_tables()
    w = words(key, start_block * Q2K_WORDS_PER_BLOCK, n_blocks * Q2K_WORDS_PER_BLOCK)
    raw = w.astype("<u8").view(np.uint8).reshape(n_blocks, 88)
    out = np.empty((n_blocks, Q2K_BLOCK_BYTES), dtype=np.uint8)
    out[:, :80] = raw[:, :80]
    idx = raw[:, 80:84].copy().view("<u2")          # [n, 2] indices
    f = half[idx]                                    # [n, 2] fp16 bits
    out[:, 80:84] = f.astype("<u2").view(np.uint8).reshape(n_blocks, 4)
    return out


def q41_blocks(key: int, n_blocks: int, start_block: int = 0) -> np.ndarray:
    """``n_blocks`` Q4_1 blocks (uint8 [n, 20]) of stream ``key``."""
    half, mtab = f16_tables()
    w = words(key, start_block * Q41_WORDS_PER_BLOCK, n_blocks * Q41_WORDS_PER_BLOCK)
    raw = w.astype("<u8").view(np.uint8).reshape(n_blocks, 24)
    out = np.empty((n_blocks, Q41_BLOCK_BYTES), dtype=np.uint8)
    idx = raw[:, 0:4].copy().view("<u2")
    dm = np.stack([half[idx[:, 0]], mtab[idx[:, 1]]], axis=1)
    out[:, 0:4] = dm.astype("<u2").view(np.uint8).reshape(n_blocks, 4)
    out[:, 4:20] = raw[:, 4:20]
    return out


def expert_tensor_blocks(qtype: str, key: int, rows: int, cols: int) -> np.ndarray:
    """Blocks of one [rows][cols] matrix, row-major, blocks along cols."""
    if qtype == "q2_k":
        assert cols % 256 == 0
        return q2k_blocks(key, rows * (cols // 256)).reshape(rows, -1)
    if qtype == "q4_1":
        assert cols % 32 == 0
        return q41_blocks(key, rows * (cols // 32)).reshape(rows, -1)
    raise ValueError(qtype)


def bf16_bits_from_f32(a: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns, round-to-nearest-even (input recipe only)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    nan = np.isnan(np.asarray(a, dtype=np.float32))
    r = ((u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16))
    r = r.astype(np.uint16)
    r[nan] = 0x7FC0
    return r


def x_f32(key: int, T: int, D: int) -> np.ndarray:
    return normal_f32(key, T * D).reshape(T, D)


def x_bf16(key: int, T: int, D: int) -> np.ndarray:
    """bf16 activations as uint16 bit patterns, RNE(float32 N(0,1))."""
    return bf16_bits_from_f32(x_f32(key, T, D))


def logits_normal(key: int, T: int, E: int) -> np.ndarray:
    return normal_f32(key, T * E).reshape(T, E)


def logits_zipf(key: int, T: int, E: int, s: float = 1.1) -> np.ndarray:
    """Zipf(s)-skewed router logits via Gumbel-top-k (Kool, van Hoof & Welling 2019)."""
    perm = np.argsort(uniform01(stream_key(key, 0x7A), E), kind="stable")
    rank = np.empty(E, dtype=np.int64)
    rank[perm] = np.arange(1, E + 1)
    u = uniform01(stream_key(key, 0x6B), T * E).reshape(T, E)
    g = -np.log(-np.log(u))
    return (-s * np.log(rank.astype(np.float64))[None, :] + g).astype(np.float32)


# ---------------------------------------------------------------- device twin

_dev_lib = None
_DEV_LIB_PATH = __import__("os").path.join(__import__("os").path.dirname(__file__), "libds4q_synth.so")


def build_device(force: bool = True) -> str:
    """Compile the HIP twin of the block generators (gfx950)."""
    import os
    import subprocess
    if force or not os.path.exists(_DEV_LIB_PATH):
        src = os.path.join(os.path.dirname(__file__), "csrc", "synth_gen.hip")
        hipcc = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")
        cmd = [hipcc, "-O3", "-std=c++17", "-fPIC", "-shared", "--offload-arch=gfx950",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-o", _DEV_LIB_PATH + ".tmp", src]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(r.stderr)
        os.replace(_DEV_LIB_PATH + ".tmp", _DEV_LIB_PATH)
    return _DEV_LIB_PATH


def _device_lib():
    global _dev_lib
    if _dev_lib is None:
        import ctypes
        import os
        if not os.path.exists(_DEV_LIB_PATH):
            raise ImportError(f"{_DEV_LIB_PATH} is not built")
        L = ctypes.CDLL(_DEV_LIB_PATH)
        P, i64 = ctypes.c_void_p, ctypes.c_int64
        L.synth_q2k_fill.restype = ctypes.c_int
        L.synth_q2k_fill.argtypes = [P, P, i64, i64, P, P]
        L.synth_q41_fill.restype = ctypes.c_int
        L.synth_q41_fill.argtypes = [P, P, i64, i64, P, P, P]
        _dev_lib = L
    return _dev_lib


_dev_tables: dict = {}


def device_fill(qtype: str, dst, keys, blocks_per_tensor: int):
    """Fill ``len(keys)`` consecutive tensors of ``blocks_per_tensor`` blocks in
    the uint8 CUDA tensor ``dst`` (on its device, current stream) with the
    same bytes q2k_blocks / q41_blocks draw for those stream keys."""
    import torch
    dev = dst.device
    if dev not in _dev_tables:
        half, mtab = f16_tables()
        _dev_tables[dev] = (torch.from_numpy(half.view(np.int16).copy()).to(dev),
                            torch.from_numpy(mtab.view(np.int16).copy()).to(dev))
    half_t, mtab_t = _dev_tables[dev]
    bb = Q2K_BLOCK_BYTES if qtype == "q2_k" else Q41_BLOCK_BYTES
    n = len(keys)
    assert dst.dtype == torch.uint8 and dst.is_contiguous()
    assert dst.numel() >= n * blocks_per_tensor * bb
    assert dst.data_ptr() % 4 == 0
    k = torch.tensor(np.array([int(v) for v in keys], dtype=np.uint64).view(np.int64), device=dev)
    s = torch.cuda.current_stream(dev).cuda_stream
    L = _device_lib()
    if qtype == "q2_k":
        rc = L.synth_q2k_fill(dst.data_ptr(), k.data_ptr(), n, blocks_per_tensor, half_t.data_ptr(), s)
    else:
        rc = L.synth_q41_fill(dst.data_ptr(), k.data_ptr(), n, blocks_per_tensor, half_t.data_ptr(),
                              mtab_t.data_ptr(), s)
    if rc != 0:
        raise RuntimeError(f"synth device fill failed: hip error {rc}")
    return k            # keep alive until the stream has consumed it
