"""The allocation-free decode entry point (ds4q_moe_decode_static, for
callers that cannot allocate device memory) against ds4q_moe_decode on the
same inputs: identical bits, on consecutive calls where the second is
smaller than the first (the static scratch keeps the first call's contents),
for each kernel family of the decode path."""
import numpy as np
import pytest
import torch

import synth
from helpers import SynthLayer

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _run(ds4q, lay, x, lg, static, flags=0):
    T = x.shape[0]
    lay.L.flags = flags
    xd, lgd = torch.from_numpy(x).to(DEV), torch.from_numpy(lg).to(DEV)
    y = torch.full((T, lay.D), float("nan"), dtype=torch.float32, device=DEV)
    ids = torch.full((T, lay.k), -1, dtype=torch.int32, device=DEV)
    w = torch.full((T, lay.k), float("nan"), dtype=torch.float32, device=DEV)
    route = ds4q.RouteOut.from_tensors(topk_ids=ids, topk_w=w)
    if static:
        ds4q.ds4q_moe_decode_static(lay.L, xd, lgd, T, y, route)
    else:
        ws = torch.empty(ds4q.ds4q_moe_workspace_size(lay.L, T, 0), dtype=torch.uint8, device=DEV)
        ds4q.ds4q_moe_decode(lay.L, xd, lgd, T, y, route, ws)
    torch.cuda.synchronize()
    return [a.cpu().numpy() for a in (y, ids, w)]


def _same(a, b):
    for u, v in zip(a, b):
        assert u.dtype == v.dtype and u.shape == v.shape
        assert np.array_equal(u.view(np.uint32), v.view(np.uint32))


@pytest.mark.parametrize("qt,qtd", [(10, 10), (3, 3), (10, 3)])
def test_decode_static_matches_workspace_call(gpu, qt, qtd):
    ds4q = gpu
    print(f"decode_static qt={qt} qtd={qtd}", flush=True)
    lay = SynthLayer(ds4q, DEV, 4096, 2048, 256, 6, qt, seed=900 + qt, qtype_down=qtd)
    for T in (64, 5, 1):   # each call smaller than the one before
        x = synth.x_f32(synth.stream_key(90, T), T, 4096)
        lg = synth.logits_normal(synth.stream_key(91, T), T, 256)
        flags = ds4q.F_RMSNORM_INPUT if T == 5 else 0
        ref = _run(ds4q, lay, x, lg, False, flags)
        got = _run(ds4q, lay, x, lg, True, flags)
        _same(got, ref)
        # twice in a row on the same inputs: the same bits again
        _same(_run(ds4q, lay, x, lg, True, flags), ref)


def test_decode_static_largest_shape(gpu):
    """The largest decode call the ABI accepts fits the static scratch."""
    ds4q = gpu
    lay = SynthLayer(ds4q, DEV, 4096, 4096, 1024, 8, 10, seed=910)
    x = synth.x_f32(synth.stream_key(92), 64, 4096)
    lg = synth.logits_normal(synth.stream_key(93), 64, 1024)
    _same(_run(ds4q, lay, x, lg, True), _run(ds4q, lay, x, lg, False))
    x2, lg2 = x[:3].copy(), lg[:3].copy()
    _same(_run(ds4q, lay, x2, lg2, True), _run(ds4q, lay, x2, lg2, False))
