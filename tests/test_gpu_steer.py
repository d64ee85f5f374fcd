"""GPU parity of the directional-steering epilogue on the MoE output
("【#8】ds4.c 해독하기", directional-steering section: each layer projects its
own direction out of its FFN output, y - scale * dir * (dir . y)) through the
C ABI against the oracle.

Every path that writes a layer's output is covered: one token on Q2_K (int8
matrix cores; the last down workgroup to arrive steers the row), one token
on Q4_1 and mixed types (vector kernels, the same tail), 2..64 tokens
(grouped int8 and vector kernels; steering inside the row-per-workgroup
combine), the prefill chunk, and the layer stack with a layer-major
direction table.  Bar: the layer's own tolerance on the steered output
(2e-3 decode, 1e-2 prefill, per token row, max-norm relative to the row's
largest steered value).  Repeated calls check that the tail's arrival
counter starts from zero every time.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import report, SynthLayer

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _log(msg):
    print(msg, flush=True)


def _unit(seed, n):
    d = np.random.default_rng(seed).standard_normal(n)
    return (d / np.linalg.norm(d)).astype(np.float32)


def _row_err(got, ref, scale_ref):
    """max_i |got - ref| / max_i |scale_ref| per row (floored)."""
    got = np.asarray(got, np.float64)
    den = np.maximum(np.abs(scale_ref).max(axis=1), 1e-30)
    return (np.abs(got - ref).max(axis=1) / den).max()


def _bf16(a):
    return (oracle.bf16_rne(a).astype(np.uint32) << 16).view(np.float32)


# (qt gate/up, qt down, T): every decode path
DECODE_CASES = [(10, 10, 1), (3, 3, 1), (10, 3, 1), (10, 10, 2), (10, 10, 5), (10, 10, 64),
                (3, 3, 3), (3, 10, 7)]


@pytest.mark.parametrize("qt,qtd,T", DECODE_CASES)
@pytest.mark.parametrize("scale", [1.0, -0.5])
def test_steered_decode(gpu, qt, qtd, T, scale):
    ds4q = gpu
    D, F, E, k = 1024, 512, 16, 6
    seed = 1000 + 10 * qt + qtd + T
    _log(f"steered decode qt={qt}/{qtd} T={T} scale={scale}")
    lay = SynthLayer(ds4q, DEV, D, F, E, k, qt, seed=seed, qtype_down=qtd)
    x = synth.x_f32(synth.stream_key(seed, 1), T, D)
    lg = synth.logits_normal(synth.stream_key(seed, 2), T, E)
    d = _unit(seed, D)
    dd = torch.from_numpy(d).to(DEV)
    lay.L.set_steering(dd, scale)
    lay.L.flags = ds4q.F_RMSNORM_INPUT
    xd = torch.from_numpy(x).to(DEV)
    lgd = torch.from_numpy(lg).to(DEV)
    ws = torch.empty(ds4q.ds4q_moe_workspace_size(lay.L, T, 0), dtype=torch.uint8, device=DEV)
    y = torch.empty(T, D, device=DEV)
    outs = []
    for _ in range(3):  # the arrival counter must start from zero on every call
        ds4q.ds4q_moe_decode(lay.L, xd, lgd, T, y, None, ws)
        torch.cuda.synchronize()
        outs.append(y.cpu().numpy())
    for o in outs[1:]:
        assert np.array_equal(o.view(np.uint32), outs[0].view(np.uint32))
    n = np.stack([oracle.rmsnorm(x[t]) for t in range(T)]).astype(np.float32)
    moe = lay.oracle_moe(n, lg, n_threads=16)
    ref = oracle.steer_f64(d, scale, moe)
    err = _row_err(outs[0], ref, ref)
    _log(f"  rel err {err:.2e}")
    assert err <= 2e-3
    # the projection really happened: the steered output's component along dir
    # is (1 - scale) times the unsteered one
    comp = outs[0].astype(np.float64) @ d.astype(np.float64)
    want = (1.0 - scale) * (moe @ d.astype(np.float64))
    assert np.all(np.abs(comp - want) <= 2e-3 * np.abs(ref).max(axis=1) * np.sqrt(D))

    # in place onto the residual stream: x <- x + steer(MoE(rmsnorm(x)))
    lay.L.flags = ds4q.F_RMSNORM_INPUT | ds4q.F_ACCUMULATE
    ds4q.ds4q_moe_decode(lay.L, xd, lgd, T, xd, None, ws)
    torch.cuda.synchronize()
    err_acc = _row_err(xd.cpu().numpy(), x.astype(np.float64) + ref, ref)
    assert err_acc <= 2e-3, err_acc


@pytest.mark.parametrize("qt,T", [(10, 1), (3, 1), (10, 5)])
def test_steer_scale_zero_matches_unsteered(gpu, qt, T):
    ds4q = gpu
    D, F, E, k = 512, 256, 8, 6
    lay = SynthLayer(ds4q, DEV, D, F, E, k, qt, seed=1200 + qt + T)
    x = torch.from_numpy(synth.x_f32(synth.stream_key(1201, T), T, D)).to(DEV)
    lg = torch.from_numpy(synth.logits_normal(synth.stream_key(1202, T), T, E)).to(DEV)
    ws = torch.empty(ds4q.ds4q_moe_workspace_size(lay.L, T, 0), dtype=torch.uint8, device=DEV)
    y0 = torch.empty(T, D, device=DEV)
    y1 = torch.empty(T, D, device=DEV)
    ds4q.ds4q_moe_decode(lay.L, x, lg, T, y0, None, ws)
    lay.L.set_steering(torch.from_numpy(_unit(3, D)).to(DEV), 0.0)
    ds4q.ds4q_moe_decode(lay.L, x, lg, T, y1, None, ws)
    torch.cuda.synchronize()
    assert np.array_equal(y0.cpu().numpy(), y1.cpu().numpy())


def test_steered_decode_phases_repeat_down(gpu):
    """The one-token phases: ROUTE, GATEUP, then DOWN twice (without
    accumulation) gives the single call's bits both times."""
    ds4q = gpu
    D, F, E, k, T = 4096, 2048, 256, 6, 1
    lay = SynthLayer(ds4q, DEV, D, F, E, k, 10, seed=1300)
    lay.L.set_steering(torch.from_numpy(_unit(1301, D)).to(DEV), 0.8)
    x = torch.from_numpy(synth.x_f32(synth.stream_key(1302), T, D)).to(DEV)
    lg = torch.from_numpy(synth.logits_normal(synth.stream_key(1303), T, E)).to(DEV)
    ws = torch.empty(ds4q.ds4q_moe_workspace_size(lay.L, T, 0), dtype=torch.uint8, device=DEV)
    y = torch.empty(T, D, device=DEV)
    ds4q.ds4q_moe_decode(lay.L, x, lg, T, y, None, ws)
    torch.cuda.synchronize()
    ref = y.cpu().numpy().copy()
    yp = torch.empty(T, D, device=DEV)
    ds4q.ds4q_moe_decode_phases(lay.L, x, lg, T, yp, None, ws, ds4q.PHASE_ROUTE | ds4q.PHASE_GATEUP)
    for _ in range(2):
        ds4q.ds4q_moe_decode_phases(lay.L, x, lg, T, yp, None, ws, ds4q.PHASE_DOWN)
        torch.cuda.synchronize()
        assert np.array_equal(yp.cpu().numpy().view(np.uint32), ref.view(np.uint32))


def test_steered_decode_flash_shape(gpu):
    """The headline shape (4096 / 2048, 256 experts, top-6), one token."""
    ds4q = gpu
    D, F, E, k = 4096, 2048, 256, 6
    for T in (1, 8):
        lay = SynthLayer(ds4q, DEV, D, F, E, k, 10, seed=1400 + T)
        x = synth.x_f32(synth.stream_key(1401, T), T, D)
        lg = synth.logits_normal(synth.stream_key(1402, T), T, E)
        d = _unit(1403, D)
        lay.L.set_steering(torch.from_numpy(d).to(DEV), 1.0)
        ws = torch.empty(ds4q.ds4q_moe_workspace_size(lay.L, T, 0), dtype=torch.uint8, device=DEV)
        y = torch.empty(T, D, device=DEV)
        ds4q.ds4q_moe_decode(lay.L, torch.from_numpy(x).to(DEV), torch.from_numpy(lg).to(DEV), T, y,
                             None, ws)
        torch.cuda.synchronize()
        ref = oracle.steer_f64(d, 1.0, lay.oracle_moe(x, lg, n_threads=16))
        err = _row_err(y.cpu().numpy(), ref, ref)
        _log(f"flash shape T={T}: rel err {err:.2e}")
        assert err <= 2e-3


@pytest.mark.parametrize("qt", [10, 3])
def test_steered_prefill(gpu, qt):
    ds4q = gpu
    D, F, E, k, T = 4096, 2048, 32, 6, 256
    seed = 1500 + qt
    lay = SynthLayer(ds4q, DEV, D, F, E, k, qt, seed=seed)
    x = synth.x_f32(synth.stream_key(seed, 1), T, D)
    lg = synth.logits_normal(synth.stream_key(seed, 2), T, E)
    d = _unit(seed, D)
    lay.L.set_steering(torch.from_numpy(d).to(DEV), 1.5)
    lay.L.flags = ds4q.F_RMSNORM_INPUT
    ws = torch.empty(ds4q.ds4q_moe_workspace_size(lay.L, T, 1), dtype=torch.uint8, device=DEV)
    y = torch.empty(T, D, device=DEV)
    ds4q.ds4q_moe_prefill(lay.L, torch.from_numpy(x).to(DEV), ds4q.TYPE_F32,
                          torch.from_numpy(lg).to(DEV), T, y, None, ws)
    torch.cuda.synchronize()
    rows = np.linspace(0, T - 1, 24).astype(int)
    n = _bf16(np.stack([oracle.rmsnorm(x[t]) for t in rows]).astype(np.float32))
    ref = oracle.steer_f64(d, 1.5, lay.oracle_moe(n, lg[rows], n_threads=16))
    err = _row_err(y.cpu().numpy()[rows], ref, ref)
    _log(f"steered prefill qt={qt}: rel err {err:.2e}")
    assert err <= 1e-2


@pytest.mark.parametrize("mode,T", [(0, 1), (0, 4), (1, 160)])
def test_steered_stack_layer_major_table(gpu, mode, T):
    """ds4q_moe_stack with layer l steered by row l of a layer-major
    [n_layers][n_embd] table: bit-identical to the layer-by-layer calls;
    each layer's steered output on the GPU's own layer input against the
    oracle (teacher-forced, the layer's bar); decode also end to end against
    the oracle's steered stack (prefill drift through bf16 layer inputs is
    reported only, as for the unsteered stack)."""
    ds4q = gpu
    NL, D, F, E, k = 6, 1024, 512, 16, 6
    seed = 1600 + 10 * mode + T
    _log(f"steered stack mode={mode} T={T}")
    lays = [SynthLayer(ds4q, DEV, D, F, E, k, 10 if l % 3 else 3, seed=seed, layer=l) for l in range(NL)]
    for lay in lays:
        for e in range(E):
            lay.host_expert(e)
    dirs = np.stack([_unit(seed + l, D) for l in range(NL)])
    dirs_d = torch.from_numpy(dirs).to(DEV)
    scale = 0.9
    for l, lay in enumerate(lays):
        lay.L.set_steering(dirs_d[l], scale)
    x0 = synth.x_f32(synth.stream_key(seed, 1), T, D)
    lg = np.stack([synth.logits_normal(synth.stream_key(seed, 2, l), T, E) for l in range(NL)])
    lg_d = torch.from_numpy(lg).to(DEV)
    wsb = max(ds4q.ds4q_moe_workspace_size(l.L, T, mode) for l in lays)
    ws = torch.empty(wsb, dtype=torch.uint8, device=DEV)
    xs = torch.from_numpy(x0).to(DEV)
    ds4q.ds4q_moe_stack([l.L for l in lays], mode, xs, lg_d, T, ws)
    torch.cuda.synchronize()
    x_stack = xs.cpu().numpy()
    # layer by layer, each layer checked on its own GPU input
    x = torch.from_numpy(x0).to(DEV)
    y = torch.empty(T, D, device=DEV)
    rows = np.arange(T) if mode == 0 else np.linspace(0, T - 1, 12).astype(int)
    for l, lay in enumerate(lays):
        lay.L.flags = ds4q.F_RMSNORM_INPUT
        if mode == 0:
            ds4q.ds4q_moe_decode(lay.L, x, lg_d[l], T, y, None, ws)
        else:
            ds4q.ds4q_moe_prefill(lay.L, x, ds4q.TYPE_F32, lg_d[l], T, y, None, ws)
        torch.cuda.synchronize()
        xin = x.cpu().numpy()
        n = np.stack([oracle.rmsnorm(xin[t]) for t in rows]).astype(np.float32)
        if mode == 1:
            n = _bf16(n)
        ref = oracle.steer_f64(dirs[l], scale, lay.oracle_moe(n, lg[l][rows], n_threads=16))
        err = _row_err(y.cpu().numpy()[rows], ref, ref)
        _log(f"  layer {l}: teacher-forced rel err {err:.2e}")
        assert err <= (2e-3 if mode == 0 else 1e-2), (l, err)
        x += y
    torch.cuda.synchronize()
    assert np.array_equal(x_stack.view(np.uint32), x.cpu().numpy().view(np.uint32))
    ref = oracle.stack([l.orc for l in lays], x0, lg, prefill_bf16=mode == 1, n_threads=16,
                       dirs=dirs, steer_scale=scale)
    upd = ref.astype(np.float64) - x0
    err = _row_err(x_stack.astype(np.float64) - x0, upd, upd)
    _log(f"  end-to-end rel err of the accumulated update {err:.2e}")
    if mode == 0:
        assert err <= 2e-2


@pytest.mark.parametrize("steered", [True, False])
def test_prefill_eight_slots_full_width(gpu, steered):
    """Eight routed slots at n_embd = 4096: the combine kernels' straight-line
    path for that slot count, with and without steering."""
    ds4q = gpu
    D, F, E, k, T = 4096, 256, 16, 8, 72
    seed = 1600 + int(steered)
    lay = SynthLayer(ds4q, DEV, D, F, E, k, 10, seed=seed)
    x = synth.x_f32(synth.stream_key(seed, 1), T, D)
    lg = synth.logits_normal(synth.stream_key(seed, 2), T, E)
    d = _unit(seed, D)
    if steered:
        lay.L.set_steering(torch.from_numpy(d).to(DEV), 0.75)
    ws = torch.empty(ds4q.ds4q_moe_workspace_size(lay.L, T, 1), dtype=torch.uint8, device=DEV)
    y = torch.empty(T, D, device=DEV)
    ds4q.ds4q_moe_prefill(lay.L, torch.from_numpy(x).to(DEV), ds4q.TYPE_F32,
                          torch.from_numpy(lg).to(DEV), T, y, None, ws)
    torch.cuda.synchronize()
    n = _bf16(x)
    ref = lay.oracle_moe(n, lg, n_threads=16)
    if steered:
        ref = oracle.steer_f64(d, 0.75, ref)
    err = _row_err(y.cpu().numpy(), ref, ref)
    _log(f"prefill k=8 steered={steered}: rel err {err:.2e}")
    assert err <= 1e-2
