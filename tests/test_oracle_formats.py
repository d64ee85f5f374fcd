"""Pins of the oracle's block formats against what the pages and the
mathematics fix (CPU only).

Q2_K: "【#2】ds4.c 해독하기", block-layout table (scales @0, qs @16, d @80,
dmin @82, 84 B) and the printed packing of the first three bit pairs.
Q4_1: ThakiCloud "...GGUF Q4_1 재부호화", Q4_1 block section (fp16 d, fp16 m,
qs[16]; low nibble = value j, high nibble = value j+16; y = d*q + m) and the
read-back section (re-encoded values bit-identical, max abs error 0.0).
"""
import json
import os
import struct

import numpy as np
import pytest
import torch

import oracle
import synth

GOLD = os.path.join(os.path.dirname(__file__), "golden")
F16_ONE, F16_HALF, F16_QUARTER = 0x3C00, 0x3800, 0x3400


# ---------------------------------------------------------------- scalars

def test_f16_decode_matches_numpy_for_all_bit_patterns():
    bits = np.arange(65536, dtype=np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([oracle.f16_value(int(b)) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


def test_bf16_rne_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(20000).astype(np.float32),
        (rng.standard_normal(2000) * 1e30).astype(np.float32),
        np.array([0.0, -0.0, np.inf, -np.inf, 3.4028235e38, 1e-45, -1e-40], dtype=np.float32),
        # exact ties: low 16 bits = 0x8000, both parities of bit 16
        np.array([0x3F808000, 0x3F818000, 0xBF808000, 0x7F7F8000], dtype=np.uint32).view(np.float32),
    ])
    got = oracle.bf16_rne(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, ref)
    nanbits = oracle.bf16_rne(np.array([np.nan], dtype=np.float32))[0]
    assert (nanbits & 0x7F80) == 0x7F80 and (nanbits & 0x7F) != 0


# ---------------------------------------------------------------- Q2_K

def _blank_q2k(d=F16_ONE, dmin=0):
    b = np.zeros(84, dtype=np.uint8)
    b[80:82] = np.frombuffer(struct.pack("<H", d), np.uint8)
    b[82:84] = np.frombuffer(struct.pack("<H", dmin), np.uint8)
    return b


def test_q2k_field_offsets():
    # d @80 scales every value, dmin @82 shifts every value, scales @0..15 hold
    # one byte per 16-value sub-block, qs @16..79 hold the codes.
    b = _blank_q2k(d=F16_ONE, dmin=F16_ONE)
    b[0:16] = 0x11                      # scale nibble 1, min nibble 1 everywhere
    b[16:80] = 0xFF                     # every code = 3
    v = oracle.q2k_decode_block(b)
    assert np.all(v == 2.0)             # 1*1*3 - 1*1
    b2 = b.copy(); b2[80:82] = np.frombuffer(struct.pack("<H", F16_HALF), np.uint8)
    assert np.all(oracle.q2k_decode_block(b2) == 0.5)
    b3 = b.copy(); b3[82:84] = 0
    assert np.all(oracle.q2k_decode_block(b3) == 3.0)
    for s in range(16):                 # sub-block s is values 16s..16s+15
        b4 = b.copy(); b4[s] = 0x12     # scale 2, min 1 in sub-block s only
        v4 = oracle.q2k_decode_block(b4)
        assert np.all(v4[16 * s:16 * s + 16] == 5.0)
        assert np.all(np.delete(v4, np.arange(16 * s, 16 * s + 16)) == 2.0)


@pytest.mark.parametrize("half", [0, 128])
@pytest.mark.parametrize("pair", [0, 1, 2])
def test_q2k_printed_packing(half, pair):
    # Printed expression: qs[j/4 + l] = L[j+l] | L[j+l+32] << 2 | L[j+l+64] << 4 ...
    # A single code at bit offset 2*pair of byte j/4 + l is value j + l + 32*pair.
    for l in range(32):
        b = _blank_q2k()
        b[0:16] = 0x01                  # scale 1, min 0
        b[16 + half // 4 + l] = 3 << (2 * pair)
        v = oracle.q2k_decode_block(b)
        want = np.zeros(256, dtype=np.float32)
        want[half + l + 32 * pair] = 3.0
        assert np.array_equal(v, want)


def test_q2k_fourth_pair_reading():
    # The page elides the fourth term; reading: L[j+l+96] << 6.  Not pinned by
    # the pages (recorded as a reading), but the four pairs must tile all 256
    # values exactly once.
    seen = np.zeros(256, dtype=int)
    for byte in range(64):
        for pair in range(4):
            b = _blank_q2k(); b[0:16] = 0x01
            b[16 + byte] = 1 << (2 * pair)
            seen += (oracle.q2k_decode_block(b) != 0)
    assert np.all(seen == 1)


def test_q2k_byte_count_invariants():
    assert 16 + 64 + 2 + 2 == 84
    # 2.625 bits per weight; one 2048x4096 matrix = 32768 blocks = 2,752,512 B
    assert 84 * 8 / 256 == 2.625
    assert 2048 * (4096 // 256) * 84 == 2_752_512
    assert 256 * 3 * 2_752_512 == 2_113_929_216           # one layer of experts


def _int_reference_q2k(blk):
    """Exact value via integers: d and dmin are integer multiples of 2^-24, so
    D*sc*q - M*mn is an exact integer; one rounding to fp32 follows."""
    d = np.frombuffer(blk[80:82].tobytes(), "<f2")[0]
    dm = np.frombuffer(blk[82:84].tobytes(), "<f2")[0]
    D = int(round(float(d) * 2 ** 24))
    M = int(round(float(dm) * 2 ** 24))
    assert D == float(d) * 2 ** 24 and M == float(dm) * 2 ** 24
    out = np.empty(256, dtype=np.float32)
    for e in range(256):
        h, k, l = e >> 7, (e >> 5) & 3, e & 31
        q = (int(blk[16 + 32 * h + l]) >> (2 * k)) & 3
        s = e >> 4
        sc, mn = int(blk[s]) & 15, int(blk[s]) >> 4
        n = D * sc * q - M * mn
        if n:
            out[e] = np.float32(float(n)) * np.float32(2.0 ** -24)
        else:
            # IEEE: t1 - t2 is -0 only when t1 = -0 and t2 = +0 (both zero);
            # a zero product carries the sign of the fp16 factor.
            t1_zero, t2_zero = D * sc * q == 0, M * mn == 0
            neg = t1_zero and t2_zero and np.signbit(d) and not np.signbit(dm)
            out[e] = np.float32(-0.0) if neg else np.float32(0.0)
    return out


def test_q2k_exact_integer_cross_check():
    blks = synth.q2k_blocks(synth.stream_key(11), 200)
    # include sign-flipped and subnormal fp16 fields
    blks[:20, 81] |= 0x80
    blks[20:40, 80:84] = np.frombuffer(struct.pack("<HH", 0x0001, 0x03FF), np.uint8)
    for blk in blks:
        got = oracle.q2k_decode_block(blk)
        ref = _int_reference_q2k(blk)
        assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


def test_q2k_golden_block():
    g = json.load(open(os.path.join(GOLD, "q2k_hand_block.json")))
    blk = np.frombuffer(bytes.fromhex(g["block_hex"]), dtype=np.uint8).copy()
    assert blk.size == 84
    got = oracle.q2k_decode_block(blk)
    assert np.array_equal(got, np.array(g["values"], dtype=np.float32))


def test_q2k_nan_inf_propagate():
    b = _blank_q2k(d=0x7E00)            # d = NaN
    b[0:16] = 0x01; b[16:80] = 0x55
    assert np.all(np.isnan(oracle.q2k_decode_block(b)))
    b = _blank_q2k(d=0x7C00)            # d = +Inf; code 0 gives Inf*0 = NaN
    b[0:16] = 0x01
    v = oracle.q2k_decode_block(b)
    assert np.all(np.isnan(v))


def test_q2k_encode_decode_roundtrip():
    rng = np.random.default_rng(5)
    for _ in range(50):
        sc = rng.integers(0, 16, 16, dtype=np.uint8)
        mn = rng.integers(0, 16, 16, dtype=np.uint8)
        q = rng.integers(0, 4, 256, dtype=np.uint8)
        d, dm = (int(v) for v in rng.integers(0, 0x7C00, 2))
        blk = oracle.q2k_encode_block(sc, mn, q, d, dm)
        v = oracle.q2k_decode_block(blk)
        want = (np.float64(np.uint16(d).view(np.float16)) * sc.repeat(16) * q
                - np.float64(np.uint16(dm).view(np.float16)) * mn.repeat(16)).astype(np.float32)
        assert np.array_equal(v, want)
        assert np.array_equal(oracle.q2k_encode_block(sc, mn, q, d, dm), blk)


# ---------------------------------------------------------------- Q4_1

def test_q41_nibble_sentinel_golden():
    g = json.load(open(os.path.join(GOLD, "q41_nibble_sentinel.json")))
    blk = np.frombuffer(bytes.fromhex(g["block_hex"]), dtype=np.uint8).copy()
    assert blk.size == 20
    got = oracle.q41_decode_block(blk)
    assert np.array_equal(got, np.array(g["values"], dtype=np.float32))


def test_q41_field_offsets():
    b = np.zeros(20, dtype=np.uint8)
    b[0:2] = np.frombuffer(struct.pack("<H", F16_HALF), np.uint8)      # d = 0.5
    b[2:4] = np.frombuffer(struct.pack("<H", 0xBC00), np.uint8)        # m = -1
    b[4:20] = 0x42                       # low nibble 2 (values 0..15), high 4 (16..31)
    v = oracle.q41_decode_block(b)
    assert np.all(v[:16] == 0.0) and np.all(v[16:] == 1.0)


def _p5_source(rng, n_values, group, bits):
    codes = rng.integers(0, 1 << bits, n_values, dtype=np.uint8)
    ng = n_values // group
    scale = (np.abs(rng.standard_normal(ng)) * 0.02).astype(np.float16)
    mins = (rng.standard_normal(ng) * 0.05).astype(np.float16)
    return codes, scale, mins


@pytest.mark.parametrize("bits,group", [(3, 32), (4, 64), (3, 64), (4, 32)])
def test_q41_lossless_reencode_readback(bits, group):
    # ThakiCloud read-back: re-encoded tensors reproduce code*scale + min with
    # identical fp32 bit patterns (max abs error 0.0).
    rng = np.random.default_rng(bits * 100 + group)
    codes, scale, mins = _p5_source(rng, 64 * 512, group, bits)
    q41 = oracle.q41_reencode(codes, scale.view(np.uint16), mins.view(np.uint16), group, bits)
    assert q41.size == codes.size // 32 * 20
    back = oracle.dequant_f32(oracle.Q4_1, q41, 64, 512).ravel()
    src = (codes.astype(np.float32) * np.repeat(scale.astype(np.float32), group)
           + np.repeat(mins.astype(np.float32), group))
    assert np.array_equal(back.view(np.uint32), src.view(np.uint32))
    assert np.max(np.abs(back - src)) == 0.0


def test_q41_reencode_large_matrix():
    rng = np.random.default_rng(77)
    codes, scale, mins = _p5_source(rng, 256 * 4096, 64, 4)
    q41 = oracle.q41_reencode(codes, scale.view(np.uint16), mins.view(np.uint16), 64, 4)
    back = oracle.dequant_f32(oracle.Q4_1, q41, 256, 4096).ravel()
    src = (codes.astype(np.float32) * np.repeat(scale.astype(np.float32), 64)
           + np.repeat(mins.astype(np.float32), 64))
    assert np.array_equal(back.view(np.uint32), src.view(np.uint32))


@pytest.mark.parametrize("bits,group", [(5, 32), (4, 48), (2, 16)])
def test_q41_reencode_refuses_without_fallback(bits, group):
    rng = np.random.default_rng(1)
    codes = rng.integers(0, min(1 << bits, 16), 96 * 2, dtype=np.uint8)
    ng = codes.size // group
    with pytest.raises(ValueError):
        oracle.q41_reencode(codes, np.zeros(ng, np.uint16), np.zeros(ng, np.uint16), group, bits)


def test_q41_reencode_refuses_code_overflow():
    codes = np.full(64, 9, dtype=np.uint8)          # 9 does not fit 3 bits
    with pytest.raises(ValueError):
        oracle.q41_reencode(codes, np.zeros(2, np.uint16), np.zeros(2, np.uint16), 32, 3)


def test_bits_group_not_inferable_from_bytes():
    # With n_groups known from the scale table, n_groups * group * bits ==
    # packed_bytes * 8 fixes only the product group*bits: (bits 4, group 64)
    # and (bits 2, group 128) give the same byte count, so the API always takes
    # the type explicitly and never infers it from a size.
    n_groups = 64
    assert n_groups * 64 * 4 == n_groups * 128 * 2


def test_q41_encode_decode_roundtrip():
    rng = np.random.default_rng(9)
    for _ in range(100):
        q = rng.integers(0, 16, 32, dtype=np.uint8)
        d, m = (int(v) for v in rng.integers(0, 0x7C00, 2))
        m |= int(rng.integers(0, 2)) << 15
        blk = oracle.q41_encode_block(q, d, m)
        v = oracle.q41_decode_block(blk)
        want = (np.float64(np.uint16(d).view(np.float16)) * q
                + np.float64(np.uint16(m).view(np.float16))).astype(np.float32)
        assert np.array_equal(v, want)


def test_dequant_tensor_layout_and_bf16():
    rows, cols = 3, 512
    w = synth.expert_tensor_blocks("q2_k", synth.stream_key(21), rows, cols)
    f = oracle.dequant_f32(oracle.Q2_K, w, rows, cols)
    for r in range(rows):
        for b in range(cols // 256):
            assert np.array_equal(f[r, 256 * b:256 * b + 256], oracle.q2k_decode_block(w[r, 84 * b:84 * b + 84]))
    bf = oracle.dequant_bf16(oracle.Q2_K, w, rows, cols)
    ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(bf, ref)
    with pytest.raises(ValueError):
        oracle.dequant_f32(oracle.Q2_K, w, rows, 300)
