"""GPU parity of the 43-layer routed-expert stack (DeepSeek-V4-Flash depth:
43 layers x 256 experts, top-6, 4096/2048) held resident in HBM: Q2_K
(90.9 GB), Q4_1 (173.1 GB) and mixed (Q2_K layers 0-36, Q4_1 layers 37-42,
the placement of the pages' mixed GGUF with the two block types built here:
102.4 GB), decode of one token and a 4096-token prefill chunk.
x <- x + MoE_l(rmsnorm(x)) per layer.

Checks:
* ds4q_moe_stack equals the layer-by-layer composition through
  ds4q_moe_decode / ds4q_moe_prefill bit for bit (same kernels);
* teacher-forced per layer: each sampled layer's MoE output on the GPU's own
  layer input matches the oracle (2e-3 decode, 1e-2 prefill, per token row);
* end to end: the final residual stream against the oracle's own 43-layer
  run (decode) is reported and bounded loosely (drift accumulates).
"""
import gc

import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import PATH_LIMBS3, report, SynthLayer, normwise_err

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
L_FLASH, D, F, E, K = 43, 4096, 2048, 256, 6


def _log(msg):
    print(msg, flush=True)


MIXED_FIRST_Q41 = 37  # mixed stack: layers 37..42 are Q4_1


def _qtype(qt, l):
    if qt == "mixed":
        return 3 if l >= MIXED_FIRST_Q41 else 10
    return qt


def _layers(ds4q, qt, seed):
    return [SynthLayer(ds4q, DEV, D, F, E, K, _qtype(qt, l), seed=seed, layer=l) for l in range(L_FLASH)]


def _free():
    gc.collect()
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _stack_case(ds4q, qt, mode, T, check_layers, seed):
    _log(f"stack qt={qt} mode={mode} T={T}: generating {L_FLASH} layers on the device")
    lays = _layers(ds4q, qt, seed)
    torch.cuda.synchronize()
    x0 = synth.x_f32(synth.stream_key(seed, 1), T, D)
    lg = np.stack([synth.logits_normal(synth.stream_key(seed, 2, l), T, E) for l in range(L_FLASH)])
    lg_d = torch.from_numpy(lg).to(DEV)
    # the stack needs the largest of its layers' workspaces (the types differ in a mixed stack)
    wsb = max(ds4q.ds4q_moe_workspace_size(l.L, T, mode) for l in lays)
    ws = torch.empty(wsb, dtype=torch.uint8, device=DEV)

    # 1. the stack entry point
    xs = torch.from_numpy(x0).to(DEV)
    ds4q.ds4q_moe_stack([l.L for l in lays], mode, xs, lg_d, T, ws)
    torch.cuda.synchronize()
    x_stack = xs.cpu().numpy()
    _log("stack call done")

    # 2. layer by layer, keeping each layer's input and output
    x = torch.from_numpy(x0).to(DEV)
    y = torch.empty(T, D, dtype=torch.float32, device=DEV)
    errs = []
    for l, lay in enumerate(lays):
        lay.L.flags = ds4q.F_RMSNORM_INPUT
        if mode == 0:
            ds4q.ds4q_moe_decode(lay.L, x, lg_d[l], T, y, None, ws)
        else:
            ds4q.ds4q_moe_prefill(lay.L, x, ds4q.TYPE_F32, lg_d[l], T, y, None, ws)
        if l in check_layers:
            torch.cuda.synchronize()
            xin = x.cpu().numpy()
            yl = y.cpu().numpy()
            rows = np.arange(T) if mode == 0 else np.linspace(0, T - 1, 4).astype(int)
            n = np.stack([oracle.rmsnorm(xin[t]) for t in rows]).astype(np.float32)
            if mode == 1:
                n = (oracle.bf16_rne(n).astype(np.uint32) << 16).view(np.float32)
            ref = lay.oracle_moe(n, lg[l][rows], n_threads=16)
            errs.append((l, normwise_err(yl[rows], ref)))
            _log(f"layer {l}: teacher-forced rel err {errs[-1][1]:.2e}")
        x += y
    torch.cuda.synchronize()
    x_lbl = x.cpu().numpy()
    return lays, x0, lg, x_stack, x_lbl, errs


def _seed(base, qt):
    return base + (qt if isinstance(qt, int) else 20)


@pytest.mark.parametrize("qt", [10, 3, "mixed"])
def test_stack_decode_one_token(gpu, qt):
    ds4q = gpu
    lays, x0, lg, x_stack, x_lbl, errs = _stack_case(ds4q, qt, 0, 1, set(range(L_FLASH)), _seed(700, qt))
    assert np.array_equal(x_stack.view(np.uint32), x_lbl.view(np.uint32))
    for l, e in errs:
        assert e <= 2e-3 and e <= PATH_LIMBS3, (l, e)   # one token: the three-limb path
    # end to end against the oracle's own 43-layer run
    ref = oracle.stack([l.orc for l in lays], x0, lg, prefill_bf16=False, n_threads=1)
    drift = normwise_err(x_stack, ref.astype(np.float64))
    _log(f"end-to-end drift after {L_FLASH} layers: {drift:.2e}")
    assert drift <= 1e-2
    del lays
    _free()


@pytest.mark.parametrize("qt", [10, 3, "mixed"])
def test_stack_prefill_chunk(gpu, qt):
    ds4q = gpu
    check = {0, 21, 42} if qt != "mixed" else {0, 21, MIXED_FIRST_Q41 - 1, MIXED_FIRST_Q41, 42}
    lays, x0, lg, x_stack, x_lbl, errs = _stack_case(ds4q, qt, 1, 4096, check, _seed(800, qt))
    assert np.array_equal(x_stack.view(np.uint32), x_lbl.view(np.uint32))
    for l, e in errs:
        assert e <= 1e-2, (l, e)
    assert np.all(np.isfinite(x_stack))
    del lays
    _free()
