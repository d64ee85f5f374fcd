"""GPU parity of the imatrix statistics ("【#2】ds4.c 해독하기", imatrix passage:
per routed expert and input column, sum of squares of the gate/up input and
of the routed SwiGLU row after the routing weight, expert-major) through the
C ABI against the oracle's statistics of the same call.

Every path is covered: one token (Q2_K int8 kernels, whose gate/up launch
keeps the inverse RMS to itself; Q4_1 and mixed vector kernels), 2..64
tokens (grouped int8 kernels on m-tiles; vector kernels on active experts),
prefill (bf16 and f32 inputs, uniform and Zipf routing, where one expert
spans many m-tiles), and the layer stack.  Bars, per expert over its columns
(max |err| / max |ref|): the input statistic squares the same values on both
sides (fp32 sums against fp64: 1e-5; prefill from f32 rounds the normalised
row to bf16 on both sides, where a one-ulp difference of the fp32 product
can move a rounding: 4e-3, twice bf16's half-ulp); the down statistic
squares SwiGLU rows that carry the path's own error, so twice the layer's bar
(4e-3 decode, 2e-2 prefill).  A second call adds exactly the same amounts
(2x bit for bit from zero); experts no pair reached stay exactly zero.
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


def _bf16(a):
    return (oracle.bf16_rne(a).astype(np.uint32) << 16).view(np.float32)


def _expert_err(got, ref):
    got = np.asarray(got, np.float64)
    den = np.maximum(np.abs(ref).max(axis=1), 1e-30)
    live = np.abs(ref).max(axis=1) > 0
    assert np.all(got[~live] == 0), "an expert no pair reached has a statistic"
    return (np.abs(got - ref).max(axis=1)[live] / den[live]).max() if live.any() else 0.0


def _stats(ds4q, lay):
    a = torch.zeros(lay.E, lay.D, device=DEV)
    b = torch.zeros(lay.E, lay.F, device=DEV)
    lay.L.set_imatrix(a, b)
    return a, b


DECODE_CASES = [(10, 10, 1), (3, 3, 1), (10, 3, 1), (10, 10, 2), (10, 10, 5), (10, 10, 64),
                (3, 3, 3), (3, 10, 7)]


@pytest.mark.parametrize("qt,qtd,T", DECODE_CASES)
@pytest.mark.parametrize("norm", [True, False])
def test_imatrix_decode(gpu, qt, qtd, T, norm):
    ds4q = gpu
    D, F, E, k = 1024, 512, 16, 6
    seed = 2000 + 10 * qt + qtd + T
    _log(f"imatrix decode qt={qt}/{qtd} T={T} norm={norm}")
    lay = SynthLayer(ds4q, DEV, D, F, E, k, qt, seed=seed, qtype_down=qtd)
    x = synth.x_f32(synth.stream_key(seed, 1), T, D) * np.float32(3.0)
    lg = synth.logits_normal(synth.stream_key(seed, 2), T, E)
    a, b = _stats(ds4q, lay)
    lay.L.flags = ds4q.F_RMSNORM_INPUT if norm else 0
    ws = torch.empty(ds4q.ds4q_moe_workspace_size(lay.L, T, 0), dtype=torch.uint8, device=DEV)
    y = torch.empty(T, D, device=DEV)
    xd, lgd = torch.from_numpy(x).to(DEV), torch.from_numpy(lg).to(DEV)
    ds4q.ds4q_moe_decode(lay.L, xd, lgd, T, y, None, ws)
    torch.cuda.synchronize()
    a1, b1 = a.cpu().numpy(), b.cpu().numpy()
    n = np.stack([oracle.rmsnorm(x[t]) for t in range(T)]).astype(np.float32) if norm else x
    ids, _ = oracle.route(lg, k)
    for e in np.unique(ids):
        lay.host_expert(int(e))
    ra, rb = oracle.moe_imatrix(lay.orc, n, lg, n_threads=16)
    ea, eb = _expert_err(a1, ra), _expert_err(b1, rb)
    _log(f"  input stat err {ea:.2e}, down stat err {eb:.2e}")
    assert ea <= 1e-5 and eb <= 4e-3
    # a second call adds the same amounts: 2x, bit for bit
    ds4q.ds4q_moe_decode(lay.L, xd, lgd, T, y, None, ws)
    torch.cuda.synchronize()
    assert np.array_equal(a.cpu().numpy(), 2 * a1) and np.array_equal(b.cpu().numpy(), 2 * b1)


@pytest.mark.parametrize("qt,x_type,zipf", [(10, "bf16", False), (10, "f32", False), (10, "f32", True),
                                            (3, "bf16", True), (3, "f32", False)])
def test_imatrix_prefill(gpu, qt, x_type, zipf):
    ds4q = gpu
    D, F, E, k, T = 2048, 1024, 32, 6, 700
    seed = 2100 + qt + (1 if zipf else 0) + (2 if x_type == "f32" else 0)
    _log(f"imatrix prefill qt={qt} x={x_type} zipf={zipf}")
    lay = SynthLayer(ds4q, DEV, D, F, E, k, qt, seed=seed)
    for e in range(E):
        lay.host_expert(e)
    x = synth.x_f32(synth.stream_key(seed, 1), T, D)
    lg = (synth.logits_zipf(synth.stream_key(seed, 2), T, E) if zipf
          else synth.logits_normal(synth.stream_key(seed, 2), T, E))
    a, b = _stats(ds4q, lay)
    if x_type == "bf16":
        xin = _bf16(x)
        xd = torch.from_numpy(oracle.bf16_rne(x).view(np.int16)).to(DEV)
        tid = ds4q.TYPE_BF16
        lay.L.flags = 0
        n = xin
    else:
        xd = torch.from_numpy(x).to(DEV)
        tid = ds4q.TYPE_F32
        lay.L.flags = ds4q.F_RMSNORM_INPUT
        n = _bf16(np.stack([oracle.rmsnorm(x[t]) for t in range(T)]).astype(np.float32))
    ws = torch.empty(ds4q.ds4q_moe_workspace_size(lay.L, T, 1), dtype=torch.uint8, device=DEV)
    y = torch.empty(T, D, device=DEV)
    ds4q.ds4q_moe_prefill(lay.L, xd, tid, torch.from_numpy(lg).to(DEV), T, y, None, ws)
    torch.cuda.synchronize()
    ra, rb = oracle.moe_imatrix(lay.orc, n, lg, n_threads=16)
    ea, eb = _expert_err(a.cpu().numpy(), ra), _expert_err(b.cpu().numpy(), rb)
    ids, _ = oracle.route(lg, k)
    _log(f"  max pairs per expert {np.bincount(ids.ravel(), minlength=E).max()}; "
         f"input stat err {ea:.2e}, down stat err {eb:.2e}")
    assert ea <= (1e-5 if x_type == "bf16" else 4e-3)
    assert eb <= 2e-2


@pytest.mark.parametrize("mode,T", [(0, 1), (0, 5), (1, 200)])
def test_imatrix_stack(gpu, mode, T):
    """Per-layer statistics through ds4q_moe_stack equal those of the
    layer-by-layer calls bit for bit, and each layer's against the oracle on
    the layer's own GPU input."""
    ds4q = gpu
    NL, D, F, E, k = 4, 1024, 512, 16, 6
    seed = 2200 + 10 * mode + T
    lays = [SynthLayer(ds4q, DEV, D, F, E, k, 10 if l % 2 == 0 else 3, seed=seed, layer=l)
            for l in range(NL)]
    for lay in lays:
        for e in range(E):
            lay.host_expert(e)
    x0 = synth.x_f32(synth.stream_key(seed, 1), T, D)
    lg = np.stack([synth.logits_normal(synth.stream_key(seed, 2, l), T, E) for l in range(NL)])
    lg_d = torch.from_numpy(lg).to(DEV)
    st = [_stats(ds4q, lay) for lay in lays]
    wsb = max(ds4q.ds4q_moe_workspace_size(l.L, T, mode) for l in lays)
    ws = torch.empty(wsb, dtype=torch.uint8, device=DEV)
    xs = torch.from_numpy(x0).to(DEV)
    ds4q.ds4q_moe_stack([l.L for l in lays], mode, xs, lg_d, T, ws)
    torch.cuda.synchronize()
    st_stack = [(a.cpu().numpy().copy(), b.cpu().numpy().copy()) for a, b in st]
    for a, b in st:
        a.zero_()
        b.zero_()
    x = torch.from_numpy(x0).to(DEV)
    y = torch.empty(T, D, device=DEV)
    for l, lay in enumerate(lays):
        lay.L.flags = ds4q.F_RMSNORM_INPUT
        xin = x.cpu().numpy()
        if mode == 0:
            ds4q.ds4q_moe_decode(lay.L, x, lg_d[l], T, y, None, ws)
        else:
            ds4q.ds4q_moe_prefill(lay.L, x, ds4q.TYPE_F32, lg_d[l], T, y, None, ws)
        torch.cuda.synchronize()
        a, b = st[l]
        assert np.array_equal(a.cpu().numpy(), st_stack[l][0])
        assert np.array_equal(b.cpu().numpy(), st_stack[l][1])
        n = np.stack([oracle.rmsnorm(xin[t]) for t in range(T)]).astype(np.float32)
        if mode == 1:
            n = _bf16(n)
        ra, rb = oracle.moe_imatrix(lay.orc, n, lg[l], n_threads=16)
        ea, eb = _expert_err(st_stack[l][0], ra), _expert_err(st_stack[l][1], rb)
        _log(f"  layer {l}: input stat err {ea:.2e}, down stat err {eb:.2e}")
        assert ea <= (1e-5 if mode == 0 else 4e-3)
        assert eb <= (4e-3 if mode == 0 else 2e-2)
        x += y
