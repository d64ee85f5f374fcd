"""Shared helpers of the GPU parity tests: seeded layers generated on the
device (synth's HIP twin) with lazily generated host copies of the experts
the oracle needs, and the normwise error measure."""
from __future__ import annotations

import numpy as np

import oracle
import synth

QTYPE_NAME = {10: "q2_k", 3: "q4_1"}


# Denominator floor of the relative measures: far below any magnitude fp32
# arithmetic resolves (a SwiGLU row can underflow exactly to zero in fp32 while
# the fp64 value is ~1e-76).
REL_FLOOR = 1e-30


def normwise_err_tensor(y, ref):
    """Tensor-wide: max |y - ref| / max |ref| over all elements.  Used for the
    bf16 prefill path at shapes smaller than the DeepSeek-V4-Flash expert
    shape, where per-row cancellation lets even an exactly rounded bf16
    pipeline exceed 1e-2 on single rows (1.32e-2 measured by emulation at
    512 x 256, against 4.2e-3 at 4096 x 2048)."""
    y = np.asarray(y, dtype=np.float64).reshape(ref.shape)
    return float(np.max(np.abs(y - ref)) / max(np.max(np.abs(ref)), REL_FLOOR))


def normwise_err(y, ref):
    """Per token row: max_i |y_i - ref_i| / max_i |ref_i|; returns the max over rows."""
    y = np.asarray(y, dtype=np.float64).reshape(ref.shape)
    den = np.maximum(np.max(np.abs(ref), axis=-1, keepdims=True), REL_FLOOR)
    return float(np.max(np.max(np.abs(y - ref), axis=-1, keepdims=True) / den))


class SynthLayer:
    """One routed-MoE layer: device weights + on-demand host experts."""

    def __init__(self, ds4q, dev, D, F, E, k, qtype, seed, layer=0, qtype_down=None, flags=0,
                 eps=1e-6, fill_device=True):
        import torch
        self.D, self.F, self.E, self.k = D, F, E, k
        self.qt, self.qtd = qtype, qtype if qtype_down is None else qtype_down
        self.seed, self.layer = seed, layer
        self.shape = {"gate": (F, D, self.qt), "up": (F, D, self.qt), "down": (D, F, self.qtd)}
        self.dev_t = {}
        for name, (rows, cols, qt) in self.shape.items():
            nbytes = E * rows * ds4q.row_bytes(qt, cols)
            t = torch.empty(nbytes, dtype=torch.uint8, device=dev)
            if fill_device:
                keys = [synth.layer_key(seed, layer, name, e) for e in range(E)]
                synth.device_fill(QTYPE_NAME[qt], t, keys, rows * cols // ds4q.QK[qt])
            self.dev_t[name] = t
        self.L = ds4q.MoeLayer.from_tensors(self.dev_t["gate"], self.dev_t["up"], self.dev_t["down"],
                                            D, F, E, k, self.qt, self.qt, self.qtd, flags, eps)
        # host buffers: calloc'd (untouched pages cost nothing), experts filled on demand
        self.host = {n: np.zeros((E, r * (c // (256 if qt == 10 else 32)) * (84 if qt == 10 else 20)),
                                 dtype=np.uint8) for n, (r, c, qt) in self.shape.items()}
        self.filled = set()
        self.orc = oracle.Layer(D, F, E, k, self.qt, self.host["gate"], self.host["up"],
                                self.host["down"], type_up=self.qt, type_down=self.qtd)

    def host_expert(self, e):
        if e in self.filled:
            return
        for name, (rows, cols, qt) in self.shape.items():
            blk = synth.expert_tensor_blocks(QTYPE_NAME[qt], synth.layer_key(self.seed, self.layer, name, e),
                                             rows, cols)
            self.host[name][e] = blk.ravel()
        self.filled.add(e)

    def oracle_moe(self, x, logits, n_threads=0):
        ids, _ = oracle.route(logits, self.k)
        for e in np.unique(ids):
            self.host_expert(int(e))
        return oracle.moe(self.orc, x, logits, n_threads=n_threads)
