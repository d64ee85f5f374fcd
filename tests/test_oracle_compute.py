"""Pins of the oracle's compute steps (CPU only): brute force on tiny
shapes, closed forms, library routines and invariants.

Routing: "ds4.c 해독하기 1/8", DS4_SHAPE_FLASH passage (256 routed experts,
6 used per token).  Expert FFN: "【#2】ds4.c 해독하기" (w1 = gate, w2 = down,
w3 = up; the down input is the routed SwiGLU row after the routing weight).
"""
import struct

import numpy as np
import pytest
from scipy.special import softmax

import oracle
import synth

Q2, Q4 = oracle.Q2_K, oracle.Q4_1


def _f16bits(v):
    return int(np.float16(v).view(np.uint16))


def const_q2k_matrix(rows, cols, row_values):
    """Q2_K matrix whose row r is the constant row_values[r] (exactly): every
    scale nibble 0, min nibble 1, dmin = -c, so value = -dmin*1 = c."""
    nb = cols // 256
    out = np.zeros((rows, nb, 84), dtype=np.uint8)
    out[:, :, 0:16] = 0x10
    for r in range(rows):
        out[r, :, 82:84] = np.frombuffer(struct.pack("<H", _f16bits(-row_values[r])), np.uint8)
    return out.reshape(rows, nb * 84)


def const_q41_matrix(rows, cols, row_values):
    nb = cols // 32
    out = np.zeros((rows, nb, 20), dtype=np.uint8)
    for r in range(rows):
        out[r, :, 2:4] = np.frombuffer(struct.pack("<H", _f16bits(row_values[r])), np.uint8)
    return out.reshape(rows, nb * 20)


# ---------------------------------------------------------------- matvec

@pytest.mark.parametrize("qt,qname", [(Q2, "q2_k"), (Q4, "q4_1")])
@pytest.mark.parametrize("rows,cols", [(1, 256), (3, 256), (1, 512), (3, 512)])
def test_matvec_brute_force(qt, qname, rows, cols):
    w = synth.expert_tensor_blocks(qname, synth.stream_key(rows, cols, qt), rows, cols)
    x = synth.x_f32(synth.stream_key(9, cols), 1, cols)[0]
    dense = oracle.dequant_f32(qt, w, rows, cols).astype(np.float64)
    ref = dense @ x.astype(np.float64)          # library matmul, any summation order
    got = oracle.matvec(qt, w, rows, cols, x)
    assert np.allclose(got, ref, rtol=1e-12, atol=1e-12 * np.abs(dense).sum())


@pytest.mark.parametrize("qt,qname", [(Q2, "q2_k"), (Q4, "q4_1")])
def test_matvec_one_hot_extracts_column(qt, qname):
    rows, cols = 5, 512
    w = synth.expert_tensor_blocks(qname, synth.stream_key(3, qt), rows, cols)
    dense = oracle.dequant_f32(qt, w, rows, cols)
    for c in (0, 1, 17, 255, 256, 300, 511):
        x = np.zeros(cols, dtype=np.float32); x[c] = 1.0
        assert np.array_equal(oracle.matvec(qt, w, rows, cols, x), dense[:, c].astype(np.float64))


def test_matvec_zero_codes_closed_form():
    # All codes 0: y_r = -sum_s dmin*mn_s * sum_{c in s} x_c.
    rows, cols = 2, 512
    w = synth.expert_tensor_blocks("q2_k", synth.stream_key(44), rows, cols).reshape(rows, 2, 84).copy()
    w[:, :, 16:80] = 0
    x = synth.x_f32(synth.stream_key(45), 1, cols)[0].astype(np.float64)
    ref = np.zeros(rows)
    for r in range(rows):
        for b in range(2):
            dmin = float(w[r, b, 82:84].copy().view("<f2")[0])
            for s in range(16):
                mn = int(w[r, b, s]) >> 4
                ref[r] -= dmin * mn * x[256 * b + 16 * s: 256 * b + 16 * s + 16].sum()
    got = oracle.matvec(Q2, w.reshape(rows, -1), rows, cols, x.astype(np.float32))
    assert np.allclose(got, ref, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------- routing

def _brute_route(logits, k):
    T, E = logits.shape
    ids = np.empty((T, k), np.int32); w = np.empty((T, k))
    for t in range(T):
        order = np.lexsort((np.arange(E), -logits[t].astype(np.float64)))   # logit desc, index asc
        ids[t] = order[:k]
        w[t] = softmax(logits[t, order[:k]].astype(np.float64))
    return ids, w


def test_route_matches_brute_force():
    lg = synth.logits_normal(synth.stream_key(50), 300, 256)
    ids, w = oracle.route(lg, 6)
    bi, bw = _brute_route(lg, 6)
    assert np.array_equal(ids, bi)
    assert np.allclose(w, bw, rtol=1e-14, atol=0)
    assert np.allclose(w.sum(1), 1.0, atol=1e-15)
    assert np.all(np.diff(w, axis=1) <= 0)            # weights follow the logit order


def test_route_ties_lower_index_first():
    lg = np.zeros((3, 256), np.float32)
    ids, w = oracle.route(lg, 6)                      # all equal
    assert np.array_equal(ids, np.tile(np.arange(6), (3, 1)))
    assert np.allclose(w, 1 / 6, atol=1e-15)
    lg = synth.logits_normal(synth.stream_key(51), 4, 256)
    lg[:, [200, 10, 99]] = 9.0                         # three-way tie at the top
    lg[:, [250, 3]] = 8.0
    lg[:, 77] = 7.5
    ids, _ = oracle.route(lg, 6)
    assert np.array_equal(ids, np.tile([10, 99, 200, 3, 250, 77], (4, 1)))
    lg2 = lg.copy(); lg2[:, 77] = 8.0                  # tie at the 6/7 boundary
    ids2, _ = oracle.route(lg2, 6)
    assert np.array_equal(ids2, np.tile([10, 99, 200, 3, 77, 250], (4, 1)))


def test_route_one_dominant_logit():
    lg = synth.logits_normal(synth.stream_key(52), 2, 256)
    lg[:, 123] = 1000.0
    ids, w = oracle.route(lg, 6)
    assert np.all(ids[:, 0] == 123)
    assert np.allclose(w[:, 0], 1.0, atol=1e-300) and np.all(w[:, 1:] < 1e-300)


# ---------------------------------------------------------------- grouping

@pytest.mark.parametrize("T", [1, 7, 64, 4096])
def test_group_matches_stable_sort(T):
    lg = synth.logits_normal(synth.stream_key(60, T), T, 256)
    ids, _ = oracle.route(lg, 6)
    counts, offsets, pairs = oracle.group(ids, 256)
    flat = ids.ravel()
    assert np.array_equal(counts, np.bincount(flat, minlength=256))
    assert offsets[0] == 0 and np.array_equal(np.diff(offsets), counts)
    assert np.array_equal(pairs, np.argsort(flat, kind="stable"))
    assert np.array_equal(flat[pairs], np.repeat(np.arange(256), counts))


# ---------------------------------------------------------------- expert FFN, MoE

def _silu(z):
    return z / (1.0 + np.exp(-z))


def test_silu_textbook_limits():
    assert _silu(0.0) == 0.0
    assert abs(_silu(30.0) - 30.0) < 1e-11 and abs(_silu(-40.0)) < 1e-15


def tiny_layer(qt, D, F, E, k, gate_c, up_c, down_rows):
    """Layer whose expert e has constant gate gate_c[e], constant up up_c[e] and
    down row i equal to down_rows[e][i]."""
    mk = const_q2k_matrix if qt == Q2 else const_q41_matrix
    gate = np.stack([mk(F, D, [gate_c[e]] * F) for e in range(E)])
    up = np.stack([mk(F, D, [up_c[e]] * F) for e in range(E)])
    down = np.stack([mk(D, F, down_rows[e]) for e in range(E)])
    return oracle.Layer(D, F, E, k, qt, gate, up, down)


@pytest.mark.parametrize("qt", [Q2, Q4])
def test_expert_ffn_closed_form(qt):
    # gate = a, up = b (constants), down row i = c_i:
    # g = a*S, u = b*S with S = sum(x); h = silu(g)*u for every row;
    # o_i = c_i * F * h.  a != b catches a gate/up swap, distinct c_i catch a
    # transposed down.
    D, F, E = 512, 256, 2
    c = [np.float16(0.25 * ((i % 7) - 3)).item() for i in range(D)]
    L = tiny_layer(qt, D, F, E, 1, [0.5, 0.125], [-0.25, 2.0], [c, c])
    x = synth.x_f32(synth.stream_key(70), 1, D)[0].astype(np.float64) * 0.01
    for e, (a, b) in enumerate([(0.5, -0.25), (0.125, 2.0)]):
        S = x.sum()
        h = _silu(a * S) * (b * S)
        ref = np.array(c) * F * h
        got = oracle.expert_ffn(L, e, x)
        assert np.allclose(got, ref, rtol=1e-12, atol=1e-14)


def test_moe_constant_experts_closed_form():
    D, F, E, k = 256, 256, 16, 6
    rng = np.random.default_rng(3)
    gate_c = [float(np.float16(v)) for v in rng.uniform(-0.5, 0.5, E)]
    up_c = [float(np.float16(v)) for v in rng.uniform(-0.5, 0.5, E)]
    down_c = [float(np.float16(v)) for v in rng.uniform(-0.5, 0.5, E)]
    L = tiny_layer(Q2, D, F, E, k, gate_c, up_c, [[down_c[e]] * D for e in range(E)])
    T = 5
    x = synth.x_f32(synth.stream_key(71), T, D) * 0.05
    lg = synth.logits_normal(synth.stream_key(72), T, E)
    ids, w = _brute_route(lg, k)
    y = oracle.moe(L, x, lg)
    for t in range(T):
        S = x[t].astype(np.float64).sum()
        ref = sum(w[t, j] * down_c[ids[t, j]] * F * _silu(gate_c[ids[t, j]] * S) * up_c[ids[t, j]] * S
                  for j in range(k))
        assert np.allclose(y[t], ref, rtol=1e-11, atol=1e-13)


def _random_layer(qname, D, F, E, k, seed):
    qt = Q2 if qname == "q2_k" else Q4
    g = np.stack([synth.expert_tensor_blocks(qname, synth.layer_key(seed, 0, "gate", e), F, D) for e in range(E)])
    u = np.stack([synth.expert_tensor_blocks(qname, synth.layer_key(seed, 0, "up", e), F, D) for e in range(E)])
    d = np.stack([synth.expert_tensor_blocks(qname, synth.layer_key(seed, 0, "down", e), D, F) for e in range(E)])
    return oracle.Layer(D, F, E, k, qt, g, u, d), (g, u, d)


def test_moe_identical_experts_and_relabelling():
    D, F, E, k, T = 256, 256, 12, 6, 4
    L, (g, u, d) = _random_layer("q2_k", D, F, E, k, 80)
    x = synth.x_f32(synth.stream_key(81), T, D)
    lg = synth.logits_normal(synth.stream_key(82), T, E)
    # identical experts: output = that expert's FFN, whatever the routing
    same = oracle.Layer(D, F, E, k, Q2, np.repeat(g[:1], E, 0), np.repeat(u[:1], E, 0), np.repeat(d[:1], E, 0))
    y = oracle.moe(same, x, lg)
    for t in range(T):
        assert np.allclose(y[t], oracle.expert_ffn(L, 0, x[t].astype(np.float64)), rtol=1e-12, atol=1e-9)
    # relabelling experts together with their logits leaves y unchanged
    perm = np.random.default_rng(1).permutation(E)
    Lp = oracle.Layer(D, F, E, k, Q2, g[perm], u[perm], d[perm])
    yp = oracle.moe(Lp, x, lg[:, perm])
    assert np.allclose(yp, oracle.moe(L, x, lg), rtol=1e-12, atol=1e-9)


def test_moe_token_separability_and_dominant_expert():
    D, F, E, k, T = 256, 256, 10, 6, 6
    L, _ = _random_layer("q4_1", D, F, E, k, 90)
    x = synth.x_f32(synth.stream_key(91), T, D)
    lg = synth.logits_normal(synth.stream_key(92), T, E)
    y = oracle.moe(L, x, lg, n_threads=3)
    for t in range(T):
        assert np.array_equal(oracle.moe(L, x[t:t + 1], lg[t:t + 1], n_threads=1)[0], y[t])
    lg2 = lg.copy(); lg2[:, 4] = 500.0
    y2 = oracle.moe(L, x, lg2)
    for t in range(T):
        assert np.allclose(y2[t], oracle.expert_ffn(L, 4, x[t].astype(np.float64)), rtol=1e-12, atol=1e-9)


# ---------------------------------------------------------------- imatrix
# "【#2】ds4.c 해독하기", imatrix passage: per routed expert and input column,
# sum of squares of the gate/up input (the MoE input row) and of the down
# input (the routed SwiGLU row after the routing weight), expert-major.

def test_imatrix_constant_experts_closed_form():
    """gate = a_e, up = b_e constants: h = silu(a_e S) * b_e S in every row,
    so imat_down[e][j] = sum over e's pairs of (p * h)^2 for every j, and
    imat_in[e] = sum over e's tokens of x^2.  Distinct a_e, b_e per expert pin
    the expert-major layout; p inside the square pins where the weight goes."""
    D, F, E, k, T = 256, 256, 16, 6, 7
    rng = np.random.default_rng(31)
    gate_c = [float(np.float16(v)) for v in rng.uniform(-0.5, 0.5, E)]
    up_c = [float(np.float16(v)) for v in rng.uniform(-0.5, 0.5, E)]
    L = tiny_layer(Q2, D, F, E, k, gate_c, up_c, [[0.0] * D for _ in range(E)])
    x = synth.x_f32(synth.stream_key(32), T, D) * 0.05
    lg = synth.logits_normal(synth.stream_key(33), T, E)
    ids, w = _brute_route(lg, k)
    a, b = oracle.moe_imatrix(L, x, lg)
    ref_a = np.zeros((E, D))
    ref_b = np.zeros((E, F))
    for t in range(T):
        S = x[t].astype(np.float64).sum()
        for j in range(k):
            e = ids[t, j]
            ref_a[e] += x[t].astype(np.float64) ** 2
            ref_b[e] += (w[t, j] * _silu(gate_c[e] * S) * up_c[e] * S) ** 2
    assert np.allclose(a, ref_a, rtol=1e-13, atol=0)
    assert np.allclose(b, ref_b, rtol=1e-11, atol=1e-300)
    assert np.all(b[np.setdiff1d(np.arange(E), ids)] == 0)


@pytest.mark.parametrize("qname", ["q2_k", "q4_1"])
def test_imatrix_brute_force_dequant_numpy(qname):
    """A random layer: the SwiGLU rows recomputed with numpy from the
    dequantised matrices, the statistics summed by hand; every token lands in
    exactly k experts, so the input statistic summed over experts is k times
    the column energy of x."""
    D, F, E, k, T = 256, 256, 8, 3, 5
    L, (g, u, d) = _random_layer(qname, D, F, E, k, 34)
    qt = Q2 if qname == "q2_k" else Q4
    x = synth.x_f32(synth.stream_key(35), T, D)
    lg = synth.logits_normal(synth.stream_key(36), T, E)
    ids, w = _brute_route(lg, k)
    a, b = oracle.moe_imatrix(L, x, lg)
    ref_a = np.zeros((E, D))
    ref_b = np.zeros((E, F))
    for t in range(T):
        xt = x[t].astype(np.float64)
        for j in range(k):
            e = ids[t, j]
            G = oracle.dequant_f32(qt, g[e], F, D).astype(np.float64)
            U = oracle.dequant_f32(qt, u[e], F, D).astype(np.float64)
            gv, uv = G @ xt, U @ xt
            ref_a[e] += xt ** 2
            ref_b[e] += (w[t, j] * gv / (1.0 + np.exp(-gv)) * uv) ** 2
    assert np.allclose(a, ref_a, rtol=1e-13)
    assert np.allclose(b, ref_b, rtol=1e-9, atol=1e-12 * ref_b.max())
    assert np.allclose(a.sum(axis=0), k * (x.astype(np.float64) ** 2).sum(axis=0), rtol=1e-13)
    # the SwiGLU row helper itself against numpy
    h = oracle.expert_swiglu(L, int(ids[0, 0]), x[0])
    G = oracle.dequant_f32(qt, g[ids[0, 0]], F, D).astype(np.float64)
    U = oracle.dequant_f32(qt, u[ids[0, 0]], F, D).astype(np.float64)
    gv, uv = G @ x[0].astype(np.float64), U @ x[0].astype(np.float64)
    assert np.allclose(h, gv / (1.0 + np.exp(-gv)) * uv, rtol=1e-12, atol=1e-15)


# ---------------------------------------------------------------- stack

def test_rmsnorm_closed_form():
    x = np.full(64, -3.0, np.float32)
    n = oracle.rmsnorm(x, eps=1e-6)
    assert np.allclose(n, -3.0 / np.sqrt(9.0 + 1e-6), rtol=1e-15)
    x = synth.x_f32(synth.stream_key(100), 1, 4096)[0]
    n = oracle.rmsnorm(x, eps=0.0)
    assert abs(np.mean(n ** 2) - 1.0) < 1e-12


def test_stack_zero_weights_is_identity_and_one_layer_composes():
    D, F, E, k, T = 256, 256, 8, 6, 3
    L, (g, u, d) = _random_layer("q2_k", D, F, E, k, 110)
    zero = oracle.Layer(D, F, E, k, Q2, np.zeros_like(g), np.zeros_like(u), np.zeros_like(d))
    x = synth.x_f32(synth.stream_key(111), T, D)
    lg = synth.logits_normal(synth.stream_key(112), 2 * T, E).reshape(2, T, E)
    assert np.array_equal(oracle.stack([zero, zero], x, lg, prefill_bf16=False), x)
    # one layer = x + MoE(rmsnorm(x)) from the separately pinned parts
    n = np.stack([oracle.rmsnorm(x[t]) for t in range(T)]).astype(np.float32)
    ref = (x.astype(np.float64) + oracle.moe(L, n, lg[0])).astype(np.float32)
    assert np.array_equal(oracle.stack([L], x, lg[:1], prefill_bf16=False), ref)
    # prefill variant rounds the normalised input to bf16 first
    nb = (oracle.bf16_rne(n).astype(np.uint32) << 16).view(np.float32)
    refb = (x.astype(np.float64) + oracle.moe(L, nb, lg[0])).astype(np.float32)
    assert np.array_equal(oracle.stack([L], x, lg[:1], prefill_bf16=True), refb)


def _two_layers(qname, D, F, E, k, seed):
    """Two layers with their own weights (distinct seeds per layer)."""
    qt = Q2 if qname == "q2_k" else Q4
    out = []
    for l in range(2):
        t = [np.stack([synth.expert_tensor_blocks(qname, synth.layer_key(seed, l, n, e), r, c)
                       for e in range(E)])
             for n, r, c in (("gate", F, D), ("up", F, D), ("down", D, F))]
        out.append(oracle.Layer(D, F, E, k, qt, *t))
    return out


@pytest.mark.parametrize("prefill_bf16", [False, True])
def test_stack_two_layers_compose_with_their_own_logits_and_weights(prefill_bf16):
    """x2 = x1 + MoE_1(n(x1)) with x1 = x0 + MoE_0(n(x0)), built by hand from
    the separately pinned rmsnorm and moe; layer l reads logits[l] and its own
    weights ("ds4.c 해독하기 1/8": one routed-expert set and router per layer)."""
    D, F, E, k, T = 256, 256, 8, 3, 3
    layers = _two_layers("q2_k", D, F, E, k, 120)
    x0 = synth.x_f32(synth.stream_key(121), T, D)
    lg = synth.logits_normal(synth.stream_key(122), 2 * T, E).reshape(2, T, E)
    # the two layers route differently, so a stride mistake changes the result
    assert not np.array_equal(oracle.route(lg[0], k)[0], oracle.route(lg[1], k)[0])

    def layer(L, x, lgl):
        n = np.stack([oracle.rmsnorm(x[t]) for t in range(T)]).astype(np.float32)
        if prefill_bf16:
            n = (oracle.bf16_rne(n).astype(np.uint32) << 16).view(np.float32)
        return (x.astype(np.float64) + oracle.moe(L, n, lgl)).astype(np.float32)

    x1 = layer(layers[0], x0, lg[0])
    x2 = layer(layers[1], x1, lg[1])
    got = oracle.stack(layers, x0, lg, prefill_bf16=prefill_bf16)
    assert np.array_equal(got, x2)
    # the same stack with layer 0's logits for both layers is a different model
    wrong = layer(layers[1], x1, lg[0])
    assert not np.array_equal(got, wrong)


def test_stack_steering_uses_each_layers_own_direction_row():
    """Steering ("【#8】ds4.c 해독하기", directional-steering section): layer l
    projects row l of the layer-major table out of its MoE output before the
    residual add.  Row 0 = 0 (no change on layer 0), row 1 = basis vector e_c
    at scale 1: layer 1's output loses exactly its coordinate c, so x2[c]
    stays where layer 0 put it and every other coordinate equals the
    unsteered stack bit for bit."""
    D, F, E, k, T, c = 256, 256, 8, 3, 2, 17
    layers = _two_layers("q4_1", D, F, E, k, 130)
    x0 = synth.x_f32(synth.stream_key(131), T, D)
    lg = synth.logits_normal(synth.stream_key(132), 2 * T, E).reshape(2, T, E)
    dirs = np.zeros((2, D), np.float32)
    dirs[1, c] = 1.0
    x1 = oracle.stack(layers[:1], x0, lg[:1], prefill_bf16=False)
    plain = oracle.stack(layers, x0, lg, prefill_bf16=False)
    steered = oracle.stack(layers, x0, lg, prefill_bf16=False, dirs=dirs, steer_scale=1.0)
    assert np.array_equal(steered[:, c], x1[:, c])
    assert not np.array_equal(plain[:, c], x1[:, c])   # layer 1 does move coordinate c
    rest = np.arange(D) != c
    assert np.array_equal(steered[:, rest], plain[:, rest])
    # layer 0's row is the one applied to layer 0: a basis row there (and none
    # on layer 1) removes coordinate c from layer 0's output only
    dirs0 = np.zeros((2, D), np.float32)
    dirs0[0, c] = 1.0
    s0 = oracle.stack(layers[:1], x0, lg[:1], prefill_bf16=False, dirs=dirs0[:1], steer_scale=1.0)
    assert np.array_equal(s0[:, c], x0[:, c])
    # scale -1 doubles layer 1's coordinate c instead (the sign of the scale)
    amp = oracle.stack(layers, x0, lg, prefill_bf16=False, dirs=dirs, steer_scale=-1.0)
    y1c = plain[:, c].astype(np.float64) - x1[:, c].astype(np.float64)
    assert np.allclose(amp[:, c].astype(np.float64) - x1[:, c], 2.0 * y1c, rtol=1e-5,
                       atol=1e-6 * np.abs(x1[:, c]).max())
