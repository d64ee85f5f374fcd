"""GPU parity of the decode path through the C ABI against the oracle:
device generator, dequant (bit-exact), matvec, routing (bit-exact ids and
grouping), decode MoE layer (normwise <= 2e-3)."""
import struct

import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import BAR_DECODE, PATH_MATVEC, SynthLayer, decode_path_bound, normwise_err, report

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
TOL_FP32 = BAR_DECODE


def _check(err, T, qt=10, qtd=None):
    """The workload's bar, and the bound of the path the call takes."""
    assert err <= TOL_FP32
    assert err <= decode_path_bound(T, qt, qt if qtd is None else qtd)


def _log(msg):
    print(msg, flush=True)


# ---------------------------------------------------------------- generator twin

@pytest.mark.parametrize("qname,bb,per", [("q2_k", 84, 256), ("q4_1", 20, 32)])
def test_device_generator_matches_host(gpu, qname, bb, per):
    keys = [synth.layer_key(77, 3, "gate", e) for e in (0, 1, 255)]
    nblk = 2048 * 4096 // per // 16
    t = torch.empty(len(keys) * nblk * bb, dtype=torch.uint8, device=DEV)
    synth.device_fill(qname, t, keys, nblk)
    torch.cuda.synchronize()
    got = t.cpu().numpy().reshape(len(keys), -1)
    gen = synth.q2k_blocks if qname == "q2_k" else synth.q41_blocks
    for i, kk in enumerate(keys):
        assert np.array_equal(got[i], gen(kk, nblk).ravel())


# ---------------------------------------------------------------- dequant

def _special_q2k_blocks(n):
    b = synth.q2k_blocks(synth.stream_key(5, 5), n)
    fields = [0x7E00, 0x7C00, 0xFC00, 0x0001, 0x03FF, 0x8000, 0x0000, 0xBC00]
    for i in range(n):
        d, dm = fields[i % len(fields)], fields[(i // len(fields)) % len(fields)]
        b[i, 80:84] = np.frombuffer(struct.pack("<HH", d, dm), np.uint8)
    return b


def _compare_f32_bits(got, ref):
    gn, rn = np.isnan(got), np.isnan(ref)
    assert np.array_equal(gn, rn)
    assert np.array_equal(got[~gn].view(np.uint32), ref[~rn].view(np.uint32))


@pytest.mark.parametrize("qt", [10, 3])
@pytest.mark.parametrize("rows,cols", [(2048, 4096), (3, 256), (7, 512), (1, 4096)])
def test_dequant_bitexact(gpu, qt, rows, cols):
    ds4q = gpu
    _log(f"dequant qt={qt} rows={rows} cols={cols}")
    qname = "q2_k" if qt == 10 else "q4_1"
    w = synth.expert_tensor_blocks(qname, synth.stream_key(6, qt, rows, cols), rows, cols)
    if rows <= 8 and qt == 10:
        w = _special_q2k_blocks(rows * cols // 256).reshape(rows, -1)
    wd = torch.from_numpy(w.ravel().copy()).to(DEV)
    f = torch.empty(rows, cols, dtype=torch.float32, device=DEV)
    b = torch.empty(rows, cols, dtype=torch.int16, device=DEV)
    ds4q.ds4q_dequant(qt, wd, rows, cols, ds4q.TYPE_F32, f)
    ds4q.ds4q_dequant(qt, wd, rows, cols, ds4q.TYPE_BF16, b)
    torch.cuda.synchronize()
    ref = oracle.dequant_f32(qt, w, rows, cols)
    _compare_f32_bits(f.cpu().numpy(), ref)
    refb = oracle.dequant_bf16(qt, w, rows, cols)
    gb = b.cpu().numpy().view(np.uint16)
    nan = np.isnan(ref)
    assert np.array_equal(gb[~nan], refb[~nan])
    assert np.all((gb[nan] & 0x7F80) == 0x7F80) and np.all((gb[nan] & 0x7F) != 0)


def test_dequant_q41_special_fields(gpu):
    ds4q = gpu
    w = synth.q41_blocks(synth.stream_key(8), 64)
    fields = [0x7E00, 0x7C00, 0xFC00, 0x0001, 0x03FF, 0x8000, 0x0000, 0xBC00]
    for i in range(64):
        w[i, 0:4] = np.frombuffer(struct.pack("<HH", fields[i % 8], fields[i // 8]), np.uint8)
    wd = torch.from_numpy(w.ravel().copy()).to(DEV)
    f = torch.empty(2, 1024, dtype=torch.float32, device=DEV)
    ds4q.ds4q_dequant(3, wd, 2, 1024, ds4q.TYPE_F32, f)
    torch.cuda.synchronize()
    _compare_f32_bits(f.cpu().numpy(), oracle.dequant_f32(3, w, 2, 1024))


def test_dequant_empty_is_noop(gpu):
    ds4q = gpu
    ds4q.ds4q_dequant(10, 0, 0, 256, ds4q.TYPE_F32, 0)


# ---------------------------------------------------------------- matvec

@pytest.mark.parametrize("qt", [10, 3])
@pytest.mark.parametrize("rows,cols,T", [(2048, 4096, 1), (2048, 4096, 3), (5, 256, 1),
                                         (37, 512, 2), (130, 2048, 1), (64, 1024, 1)])
def test_matvec_parity(gpu, qt, rows, cols, T):
    ds4q = gpu
    _log(f"matvec qt={qt} rows={rows} cols={cols} T={T}")
    qname = "q2_k" if qt == 10 else "q4_1"
    w = synth.expert_tensor_blocks(qname, synth.stream_key(7, qt, rows, cols), rows, cols)
    x = synth.x_f32(synth.stream_key(8, cols, T), T, cols)
    y = torch.full((T, rows), float("nan"), dtype=torch.float32, device=DEV)
    ds4q.ds4q_matvec(qt, torch.from_numpy(w.ravel().copy()).to(DEV), rows, cols,
                     torch.from_numpy(x).to(DEV), T, y)
    torch.cuda.synchronize()
    ref = np.stack([oracle.matvec(qt, w, rows, cols, x[t]) for t in range(T)])
    err = report(normwise_err(y.cpu().numpy(), ref))
    assert err <= TOL_FP32 and err <= PATH_MATVEC


# ---------------------------------------------------------------- routing

def _route_gpu(ds4q, lg, k):
    T, E = lg.shape
    ids = torch.empty(T, k, dtype=torch.int32, device=DEV)
    w = torch.empty(T, k, dtype=torch.float32, device=DEV)
    cnt = torch.empty(E, dtype=torch.int32, device=DEV)
    off = torch.empty(E + 1, dtype=torch.int32, device=DEV)
    pairs = torch.empty(T * k, dtype=torch.int32, device=DEV)
    out = ds4q.RouteOut.from_tensors(ids, w, cnt, off, pairs)
    ws = torch.empty(ds4q.ds4q_route_workspace_size(T, E, k), dtype=torch.uint8, device=DEV)
    ds4q.ds4q_route(torch.from_numpy(lg).to(DEV), T, E, k, out, ws)
    torch.cuda.synchronize()
    return [a.cpu().numpy() for a in (ids, w, cnt, off, pairs)]


@pytest.mark.parametrize("T,kind", [(1, "n"), (7, "n"), (64, "n"), (4096, "n"), (4096, "zipf")])
def test_route_parity(gpu, T, kind):
    ds4q = gpu
    E, k = 256, 6
    gen = synth.logits_normal if kind == "n" else synth.logits_zipf
    lg = gen(synth.stream_key(9, T), T, E)
    ids, w, cnt, off, pairs = _route_gpu(ds4q, lg, k)
    rids, rw = oracle.route(lg, k)
    assert np.array_equal(ids, rids)
    assert np.max(np.abs(w - rw)) <= 1e-6
    rc, ro, rp = oracle.group(rids, E)
    assert np.array_equal(cnt, rc) and np.array_equal(off, ro) and np.array_equal(pairs, rp)


def test_route_ties_and_signed_zero(gpu):
    ds4q = gpu
    lg = synth.logits_normal(synth.stream_key(10), 8, 256)
    lg[0] = 0.0
    lg[1, [200, 10, 99]] = 9.0
    lg[2, :] = -0.0
    lg[2, 3] = 0.0                       # +0 and -0 compare equal: index order decides
    lg[3, [5, 6, 7, 8, 9, 10, 11]] = 3.5  # tie across the 6/7 boundary
    ids, w, cnt, off, pairs = _route_gpu(ds4q, lg, 6)
    rids, rw = oracle.route(lg, 6)
    assert np.array_equal(ids, rids)
    assert np.max(np.abs(w - rw)) <= 1e-6
    rc, ro, rp = oracle.group(rids, 256)
    assert np.array_equal(pairs, rp)


@pytest.mark.parametrize("E,k", [(16, 1), (16, 8), (1024, 6), (8, 8)])
def test_route_shapes(gpu, E, k):
    ds4q = gpu
    lg = synth.logits_normal(synth.stream_key(11, E, k), 33, E)
    ids, w, cnt, off, pairs = _route_gpu(ds4q, lg, k)
    rids, rw = oracle.route(lg, k)
    assert np.array_equal(ids, rids)
    rc, ro, rp = oracle.group(rids, E)
    assert np.array_equal(pairs, rp) and np.array_equal(off, ro)


@pytest.mark.parametrize("T,k", [(4999, 7), (4096, 8), (4097, 6)])
def test_route_many_pairs(gpu, T, k):
    """More pairs than one grouping round of 24,576 takes (the later rounds
    reload their ids), and pair counts that are not a multiple of 4."""
    ds4q = gpu
    E = 256
    lg = synth.logits_zipf(synth.stream_key(12, T, k), T, E)
    ids, w, cnt, off, pairs = _route_gpu(ds4q, lg, k)
    rids, rw = oracle.route(lg, k)
    assert np.array_equal(ids, rids)
    rc, ro, rp = oracle.group(rids, E)
    assert np.array_equal(cnt, rc) and np.array_equal(off, ro) and np.array_equal(pairs, rp)


# ---------------------------------------------------------------- decode MoE

def _decode(ds4q, lay, x, lg, flags=0, y0=None, in_place=False):
    T = x.shape[0]
    lay.L.flags = flags
    xd = torch.from_numpy(x).to(DEV)
    if in_place:
        y = xd
    else:
        y = torch.from_numpy(y0).to(DEV) if y0 is not None else torch.empty(T, lay.D, device=DEV)
    ws = torch.empty(ds4q.ds4q_moe_workspace_size(lay.L, T, 0), dtype=torch.uint8, device=DEV)
    ids = torch.empty(T, lay.k, dtype=torch.int32, device=DEV)
    ds4q.ds4q_moe_decode(lay.L, xd, torch.from_numpy(lg).to(DEV), T, y,
                         ds4q.RouteOut.from_tensors(topk_ids=ids), ws)
    torch.cuda.synchronize()
    return y.cpu().numpy(), ids.cpu().numpy()


@pytest.mark.parametrize("qt,qtd", [(10, 10), (3, 3), (10, 3), (3, 10)])
@pytest.mark.parametrize("T", [1, 2, 5, 64])
def test_decode_small(gpu, qt, qtd, T):
    ds4q = gpu
    _log(f"decode small qt={qt} qtd={qtd} T={T}")
    lay = SynthLayer(ds4q, DEV, 512, 256, 16, 6, qt, seed=100 + T, qtype_down=qtd)
    x = synth.x_f32(synth.stream_key(12, T), T, 512)
    lg = synth.logits_normal(synth.stream_key(13, T), T, 16)
    y, ids = _decode(ds4q, lay, x, lg)
    assert np.array_equal(ids, oracle.route(lg, 6)[0])
    _check(report(normwise_err(y, lay.oracle_moe(x, lg))), T, qt, qtd)


@pytest.mark.parametrize("qt", [10, 3])
@pytest.mark.parametrize("T", [1, 3])
@pytest.mark.parametrize("D,F", [(256, 4096), (4096, 256), (1024, 512), (2048, 1024), (512, 2048)])
def test_decode_shapes(gpu, D, F, T, qt):
    """Every count of 256-value blocks per row (1..16) on both sides of the
    layer, for both formats (the grouped kernels have one instance each)."""
    ds4q = gpu
    _log(f"decode shapes D={D} F={F} T={T} qt={qt}")
    lay = SynthLayer(ds4q, DEV, D, F, 8, 2, qt, seed=200 + D)
    x = synth.x_f32(synth.stream_key(14, D), T, D)
    lg = synth.logits_normal(synth.stream_key(15, D), T, 8)
    y, _ = _decode(ds4q, lay, x, lg)
    _check(report(normwise_err(y, lay.oracle_moe(x, lg))), T, qt)


@pytest.mark.parametrize("T", [1, 4])
def test_decode_flags_residual_rmsnorm(gpu, T):
    ds4q = gpu
    lay = SynthLayer(ds4q, DEV, 512, 256, 16, 6, 10, seed=300)
    x = synth.x_f32(synth.stream_key(16, T), T, 512) * 3.0
    lg = synth.logits_normal(synth.stream_key(17, T), T, 16)
    n = np.stack([oracle.rmsnorm(x[t]) for t in range(T)]).astype(np.float32)
    ref = lay.oracle_moe(n, lg)
    y0 = synth.x_f32(synth.stream_key(18, T), T, 512)
    y, _ = _decode(ds4q, lay, x, lg, flags=ds4q.F_RMSNORM_INPUT | ds4q.F_ACCUMULATE, y0=y0)
    _check(report(normwise_err(y - y0, ref)), T)
    y2, _ = _decode(ds4q, lay, x, lg, flags=ds4q.F_RMSNORM_INPUT | ds4q.F_ACCUMULATE, in_place=True)
    _check(report(normwise_err(y2 - x, ref)), T)


@pytest.mark.parametrize("k", [1, 6, 8])
def test_decode_full_layer_one_token(gpu, k):
    """One-layer decode, 1 token, DeepSeek-V4-Flash expert shape (Q2_K), with
    the smallest, the model's and the largest routed-slot count the ABI takes
    (the gate/up grid has k rows of workgroups; the down workgroup has
    2 * 64 * k threads)."""
    ds4q = gpu
    _log(f"decode full T=1 k={k}")
    lay = SynthLayer(ds4q, DEV, 4096, 2048, 256, k, 10, seed=400)
    x = synth.x_f32(synth.stream_key(19), 1, 4096)
    lg = synth.logits_normal(synth.stream_key(20), 1, 256)
    y, ids = _decode(ds4q, lay, x, lg)
    assert np.array_equal(ids, oracle.route(lg, k)[0])
    _check(report(normwise_err(y, lay.oracle_moe(x, lg, n_threads=16))), 1)


@pytest.mark.parametrize("qt", [10, 3])
def test_decode_full_layer_64_tokens(gpu, qt):
    """One-layer batched decode, 64 tokens, full shape; every token row is
    checked against the oracle."""
    ds4q = gpu
    _log(f"decode full T=64 qt={qt}")
    lay = SynthLayer(ds4q, DEV, 4096, 2048, 256, 6, qt, seed=500 + qt)
    x = synth.x_f32(synth.stream_key(21), 64, 4096)
    lg = synth.logits_normal(synth.stream_key(22), 64, 256)
    y, ids = _decode(ds4q, lay, x, lg)
    assert np.array_equal(ids, oracle.route(lg, 6)[0])
    ref = lay.oracle_moe(x, lg, n_threads=16)
    _check(report(normwise_err(y, ref)), 64, qt)


@pytest.mark.parametrize("qt,qtd", [(10, 10), (3, 3), (3, 10)])
@pytest.mark.parametrize("T", [9, 64])
def test_decode_experts_over_several_tiles(gpu, T, qt, qtd):
    """Every expert routed every token (E = k = 8): experts hold T pairs, i.e.
    several m-tiles of the grouped decode (4 pairs each, the last one partial)."""
    ds4q = gpu
    _log(f"decode several tiles per expert T={T} qt={qt} qtd={qtd}")
    lay = SynthLayer(ds4q, DEV, 512, 256, 8, 8, qt, seed=700 + T, qtype_down=qtd)
    x = synth.x_f32(synth.stream_key(40, T), T, 512)
    lg = synth.logits_normal(synth.stream_key(41, T), T, 8)
    y, ids = _decode(ds4q, lay, x, lg)
    assert np.array_equal(ids, oracle.route(lg, 8)[0])
    _check(report(normwise_err(y, lay.oracle_moe(x, lg))), T, qt, qtd)


@pytest.mark.parametrize("qt", [10, 3])
def test_decode_64_tokens_zipf(gpu, qt):
    """64 tokens with Zipf(1.1)-skewed routing, full shape: the popular experts
    hold tens of pairs (several tiles each); every token row vs the oracle."""
    ds4q = gpu
    _log(f"decode full T=64 zipf qt={qt}")
    lay = SynthLayer(ds4q, DEV, 4096, 2048, 256, 6, qt, seed=710)
    x = synth.x_f32(synth.stream_key(42), 64, 4096)
    lg = synth.logits_zipf(synth.stream_key(43), 64, 256)
    y, ids = _decode(ds4q, lay, x, lg)
    assert np.array_equal(ids, oracle.route(lg, 6)[0])
    counts = np.bincount(ids.ravel(), minlength=256)
    assert counts.max() > 8  # the case this test is for
    ref = lay.oracle_moe(x, lg, n_threads=16)
    _check(report(normwise_err(y, ref)), 64, qt)


@pytest.mark.parametrize("qt,T", [(10, 1), (10, 3), (3, 1)])
def test_decode_phases_compose(gpu, qt, T):
    """ROUTE, GATEUP and DOWN run as separate calls on one workspace give the
    bits of a single ds4q_moe_decode call; repeating GATEUP + DOWN alone is
    idempotent (the form the per-kernel timing uses)."""
    ds4q = gpu
    _log(f"decode phases qt={qt} T={T}")
    lay = SynthLayer(ds4q, DEV, 4096, 2048, 256, 6, qt, seed=600 + T)
    x = torch.from_numpy(synth.x_f32(synth.stream_key(23, T), T, 4096)).to(DEV)
    lg = torch.from_numpy(synth.logits_normal(synth.stream_key(24, T), T, 256)).to(DEV)
    ws = torch.empty(ds4q.ds4q_moe_workspace_size(lay.L, T, 0), dtype=torch.uint8, device=DEV)
    y_ref = torch.empty(T, 4096, dtype=torch.float32, device=DEV)
    ds4q.ds4q_moe_decode(lay.L, x, lg, T, y_ref, None, ws)
    ws.zero_()
    y = torch.full((T, 4096), float("nan"), dtype=torch.float32, device=DEV)
    for ph in (ds4q.PHASE_ROUTE, ds4q.PHASE_GATEUP, ds4q.PHASE_DOWN):
        ds4q.ds4q_moe_decode_phases(lay.L, x, lg, T, y, None, ws, ph)
    torch.cuda.synchronize()
    a, b = y_ref.cpu().numpy(), y.cpu().numpy()
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    for _ in range(2):
        ds4q.ds4q_moe_decode_phases(lay.L, x, lg, T, y, None, ws, ds4q.PHASE_GATEUP)
        ds4q.ds4q_moe_decode_phases(lay.L, x, lg, T, y, None, ws, ds4q.PHASE_DOWN)
    torch.cuda.synchronize()
    assert np.array_equal(a.view(np.uint32), y.cpu().numpy().view(np.uint32))


@pytest.mark.parametrize("E", [256, 200, 512])
def test_decode_one_token_route_ties(gpu, E):
    """The one-token Q2_K path routes inside its gate/up kernel: tied logits
    (equal values, +0 against -0, a tie across the k boundary) must pick the
    same experts in the same slot order as the oracle, for E up to 256 (four
    logits per lane) and above (the general top-k)."""
    ds4q = gpu
    lay = SynthLayer(ds4q, DEV, 512, 256, E, 6, 10, seed=700 + E)
    base = synth.logits_normal(synth.stream_key(25, E), 5, E)
    base[0] = 0.0
    base[1, [E - 1, 10, 99]] = 9.0
    base[2, :] = -0.0
    base[2, 3] = 0.0
    base[3, [5, 6, 7, 8, 9, 10, 11]] = 3.5
    base[4, [E - 2, E - 1, 0]] = 7.0
    for t in range(5):
        _log(f"one-token ties E={E} row {t}")
        x = synth.x_f32(synth.stream_key(26, t), 1, 512)
        y, ids = _decode(ds4q, lay, x, base[t:t + 1])
        assert np.array_equal(ids, oracle.route(base[t:t + 1], 6)[0]), t
        _check(report(normwise_err(y, lay.oracle_moe(x, base[t:t + 1]))), 1)
