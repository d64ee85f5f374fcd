"""GPU parity of directional steering ("【#8】ds4.c 해독하기", directional
steering section) and the activation wire formats ("【#6】ds4.c 분석하기",
distributed-transport passage) through the C ABI against the oracle.

Codec: bit-exact (every f16 and E4M3 code decoded; encoding of exact ties at
every binary16 and E4M3 midpoint, the saturation and subnormal ranges,
specials, random bit patterns, ragged lengths and the 4096 x 4096 pipeline
hop).  Steering: fp32 arithmetic against the fp64 oracle with the bound of
an fp32 dot product: |err_i| <= 2^-22 (|ref_i| + |y_i| + |res_i|)
+ |scale dir_i| n 2^-24 sum_j |dir_j y_j|.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import SynthLayer

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _log(msg):
    print(msg, flush=True)


# ---------------------------------------------------------------- codec

def _encode(ds4q, x: np.ndarray, bits: int) -> np.ndarray:
    n = x.size
    src = torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(DEV)
    dst = torch.empty(max(16, n * bits // 8), dtype=torch.uint8, device=DEV)
    ds4q.ds4q_act_encode(src, n, bits, dst)
    torch.cuda.synchronize()
    out = dst.cpu().numpy()[: n * bits // 8]
    return out.view(np.uint16) if bits == 16 else (out.view(np.float32) if bits == 32 else out)


def _decode(ds4q, codes: np.ndarray, bits: int) -> np.ndarray:
    n = codes.size
    src = torch.from_numpy(np.ascontiguousarray(codes).view(np.uint8).copy()).to(DEV)
    dst = torch.empty(n, dtype=torch.float32, device=DEV)
    ds4q.ds4q_act_decode(src, n, bits, dst)
    torch.cuda.synchronize()
    return dst.cpu().numpy()


def _f16_ties():
    h = np.arange(0x0000, 0x7C00, dtype=np.uint16)        # every finite non-negative code
    lo = h.view(np.float16).astype(np.float64)
    hi = (h + 1).view(np.float16).astype(np.float64)
    mids = ((lo + hi) / 2).astype(np.float32)              # exact: binary16 midpoints fit f32
    return np.concatenate([mids, -mids])


def _f16_cases():
    rng = np.random.default_rng(11)
    bits = rng.integers(0, 2 ** 32, 200_000, dtype=np.uint64).astype(np.uint32)
    specials = np.array([0.0, -0.0, 65504.0, 65519.99, 65520.0, -65520.0, 1e30, np.inf, -np.inf,
                         np.nan, -np.nan, 2.0 ** -24, 2.0 ** -25, 2.0 ** -26, 1e-45], np.float32)
    return np.concatenate([specials, _f16_ties(), bits.view(np.float32),
                           rng.standard_normal(50_000).astype(np.float32)])


def test_f16_encode_bit_exact(gpu):
    ds4q = gpu
    x = _f16_cases()
    _log(f"f16 encode: {x.size} values")
    assert np.array_equal(_encode(ds4q, x, 16), oracle.f16_rne(x))


def test_f16_decode_all_codes(gpu):
    ds4q = gpu
    codes = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = _decode(ds4q, codes, 16)
    ref = codes.view(np.float16).astype(np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def _e4m3_cases():
    rng = np.random.default_rng(12)
    v = oracle.e4m3_value(np.arange(0x7F))                   # non-negative finite codes
    mids = ((v[1:] + v[:-1]) / 2).astype(np.float32)
    near = np.concatenate([np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(1e9))])
    specials = np.array([0.0, -0.0, 448.0, 455.99, 456.0, 463.99, 464.0, 479.0, 480.0, 1e5, -1e5,
                         np.inf, -np.inf, np.nan, 2.0 ** -9, 2.0 ** -10, 3 * 2.0 ** -11, 2.0 ** -6,
                         2.0 ** -6 - 2.0 ** -10, 1e-30, 1e-45], np.float32)
    rnd = (rng.standard_normal(100_000) * 10.0 ** rng.integers(-4, 3, 100_000)).astype(np.float32)
    return np.concatenate([specials, mids, -mids, near, v.astype(np.float32), rnd])


def test_e4m3_encode_bit_exact(gpu):
    ds4q = gpu
    x = _e4m3_cases()
    _log(f"e4m3 encode: {x.size} values")
    assert np.array_equal(_encode(ds4q, x, 8), oracle.e4m3_rne(x))


def test_e4m3_decode_all_codes(gpu):
    ds4q = gpu
    codes = np.arange(256, dtype=np.uint32).astype(np.uint8)
    got = _decode(ds4q, codes, 8)
    ref = oracle.e4m3_value(codes).astype(np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))


@pytest.mark.parametrize("n", [1, 7, 9, 15, 17, 33, 1_000_003])
@pytest.mark.parametrize("bits", [16, 8, 32])
def test_codec_ragged_round_trip(gpu, n, bits):
    ds4q = gpu
    rng = np.random.default_rng(n)
    x = (rng.standard_normal(n) * 3).astype(np.float32)
    codes = _encode(ds4q, x, bits)
    if bits == 32:
        assert np.array_equal(codes.view(np.uint32), x.view(np.uint32))
        return
    sample = np.unique(np.linspace(0, n - 1, min(n, 4000)).astype(int))
    ref = oracle.f16_rne(x[sample]) if bits == 16 else oracle.e4m3_rne(x[sample])
    assert np.array_equal(codes[sample], ref)
    back = _decode(ds4q, codes, bits)
    assert np.array_equal(back.view(np.uint32), _decode_ref(codes, bits).view(np.uint32))


def _decode_ref(codes, bits):
    if bits == 16:
        return codes.view(np.float16).astype(np.float32)
    table = oracle.e4m3_value(np.arange(256)).astype(np.float32)
    return table[codes]


def test_codec_pipeline_hop(gpu):
    """The activation hop of a 4096-token chunk (4096 x 4096 f32): both
    widths, sampled rows against the oracle, and the round-trip error bound
    (half an ulp of the wire format)."""
    ds4q = gpu
    T, D = 4096, 4096
    x = synth.x_f32(synth.stream_key(21), T, D) * np.float32(4.0)
    rows = np.array([0, 1, 2047, 4095])
    for bits in (16, 8):
        codes = _encode(ds4q, x, bits).reshape(T, -1)
        ref = oracle.f16_rne(x[rows]) if bits == 16 else oracle.e4m3_rne(x[rows])
        assert np.array_equal(codes[rows].ravel(), ref)
        back = _decode(ds4q, codes.ravel(), bits).reshape(T, D)
        ax = np.abs(x)
        if bits == 16:
            assert np.all(np.abs(back - x) <= np.maximum(ax * 2.0 ** -11, 2.0 ** -25))
        else:
            ok = ax <= 448
            assert np.all(np.abs(back - x)[ok] <= np.maximum(ax[ok] * 2.0 ** -4, 2.0 ** -10))


# ---------------------------------------------------------------- steering

def _steer_gpu(ds4q, dir_, scale, y, out0=None, accumulate=False, in_place=False):
    R, n = y.shape
    d = torch.from_numpy(dir_).to(DEV)
    yd = torch.from_numpy(y).to(DEV)
    if in_place:
        od = yd
    else:
        od = torch.from_numpy(out0).to(DEV) if out0 is not None else torch.empty_like(yd)
    ds4q.ds4q_steer(d, scale, yd, R, n, od, ds4q.F_ACCUMULATE if accumulate else 0)
    torch.cuda.synchronize()
    return od.cpu().numpy()


def _steer_bound(dir_, scale, y, ref, res=None):
    n = y.shape[1]
    dots = np.abs(y.astype(np.float64)) @ np.abs(dir_.astype(np.float64))
    b = 2.0 ** -22 * (np.abs(ref) + np.abs(y) + (0 if res is None else np.abs(res)))
    return b + abs(scale) * np.abs(dir_)[None, :] * (n * 2.0 ** -24 * dots)[:, None] + 1e-30


@pytest.mark.parametrize("n,rows", [(4096, 1), (4096, 37), (256, 5), (4, 3), (1028, 9)])
@pytest.mark.parametrize("scale", [0.0, 1.0, -2.5])
def test_steer_parity(gpu, n, rows, scale):
    ds4q = gpu
    rng = np.random.default_rng(n * 100 + rows)
    d = rng.standard_normal(n)
    d = (d / np.linalg.norm(d)).astype(np.float32)
    y = (rng.standard_normal((rows, n)) * 3).astype(np.float32)
    ref = oracle.steer(d, scale, y)
    got = _steer_gpu(ds4q, d, scale, y)
    assert np.all(np.abs(got.astype(np.float64) - ref) <= _steer_bound(d, scale, y, ref))
    if scale == 0.0:
        assert np.array_equal(got, y)
    got_ip = _steer_gpu(ds4q, d, scale, y, in_place=True)
    assert np.array_equal(got_ip, got)
    res = rng.standard_normal((rows, n)).astype(np.float32)
    ref_a = oracle.steer(d, scale, y, residual=res)
    got_a = _steer_gpu(ds4q, d, scale, y, out0=res, accumulate=True)
    assert np.all(np.abs(got_a.astype(np.float64) - ref_a) <= _steer_bound(d, scale, y, ref_a, res))


def test_steer_on_moe_output_into_residual(gpu):
    """The steering epilogue as the pages place it: on the FFN (MoE) output of
    a layer, added to the residual stream: x <- x + steer(MoE(rmsnorm(x)))."""
    ds4q = gpu
    T, D, F, E, k = 8, 1024, 512, 16, 6
    lay = SynthLayer(ds4q, DEV, D, F, E, k, 10, seed=950)
    rng = np.random.default_rng(950)
    x = synth.x_f32(synth.stream_key(95), T, D)
    lg = synth.logits_normal(synth.stream_key(96), T, E)
    d = rng.standard_normal(D)
    d = (d / np.linalg.norm(d)).astype(np.float32)
    lay.L.flags = ds4q.F_RMSNORM_INPUT
    xd = torch.from_numpy(x).to(DEV)
    yd = torch.empty(T, D, device=DEV)
    ws = torch.empty(ds4q.ds4q_moe_workspace_size(lay.L, T, 0), dtype=torch.uint8, device=DEV)
    ds4q.ds4q_moe_decode(lay.L, xd, torch.from_numpy(lg).to(DEV), T, yd, None, ws)
    ds4q.ds4q_steer(torch.from_numpy(d).to(DEV), 0.75, yd, T, D, xd, ds4q.F_ACCUMULATE)
    torch.cuda.synchronize()
    got = xd.cpu().numpy()
    n = np.stack([oracle.rmsnorm(x[t]) for t in range(T)]).astype(np.float32)
    moe = lay.oracle_moe(n, lg, n_threads=16).astype(np.float32)
    ref = oracle.steer(d, 0.75, moe, residual=x)
    # the MoE part carries the decode tolerance; the steering adds its own bound
    err = np.abs(got.astype(np.float64) - ref).max(axis=1) / np.abs(moe).max(axis=1)
    assert np.all(err <= 2e-3), err
