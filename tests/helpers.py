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
    """Tensor-wide: max |y - ref| / max |ref| over all elements (reported
    beside the per-row measure at the small prefill shapes)."""
    y = np.asarray(y, dtype=np.float64).reshape(ref.shape)
    return float(np.max(np.abs(y - ref)) / max(np.max(np.abs(ref)), REL_FLOOR))


# The workload's bars (max relative error per token row, normwise): fp32
# decode paths 2e-3, bf16 prefill 1e-2.
BAR_DECODE = 2e-3
BAR_PREFILL = 1e-2
# Each decode path's own bound, a few times above what its arithmetic was
# measured to reach on the GPU (so that a lost limb or digit fails), far below
# the bar: every decode path takes its activations as three int8 digits per
# value (one token; 2..64 tokens, grouped on Q2_K weights or per expert with
# Q4_1 / mixed formats), measured up to 4.9e-6; the fp32 vector matvec up to
# 2.1e-7.
PATH_LIMBS3 = 1e-5
PATH_MATVEC = 2e-6


def decode_path_bound(T, qt, qtd):
    """The measured-error bound of the decode path a call takes."""
    return PATH_LIMBS3


def report(err, name=""):
    """Print a measured error with the running test's id (grep-able as ERR)."""
    import os
    test = os.environ.get("PYTEST_CURRENT_TEST", "?").split(" ")[0]
    print(f"ERR {test} {name} {err:.3e}", flush=True)
    return err


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


def tile_cover_tokens(ids, n_expert, tile_m, group=16):
    """A set of tokens whose pairs put a checked pair in every 16-pair group of
    every m-tile (each expert's pairs, sorted by (expert, token, slot), cut into
    tiles of tile_m from the expert's first pair, as the grouped GEMMs cut
    them) and at every position of a tile that occurs.  Greedy set cover;
    returns sorted token indices."""
    T, k = ids.shape
    _, offsets, pairs = oracle.group(ids, n_expert)
    pos_of = np.empty(T * k, np.int64)
    pos_of[pairs] = np.arange(T * k)
    expert = np.searchsorted(offsets, pos_of, side="right") - 1
    local = pos_of - offsets[expert]
    tile = np.zeros(T * k, np.int64)
    # global tile index: tiles of earlier experts, then this expert's
    tiles_per = (np.diff(offsets) + tile_m - 1) // tile_m
    tile_base = np.concatenate([[0], np.cumsum(tiles_per)])
    tile = tile_base[expert] + local // tile_m
    n_cells_a = int(tile_base[-1]) * (tile_m // group)
    cell_a = tile * (tile_m // group) + (local % tile_m) // group
    cell_b = n_cells_a + local % tile_m
    cells = np.stack([cell_a, cell_b], 1).reshape(T, 2 * k)   # pair p = t*k + j
    need = np.zeros(n_cells_a + tile_m, bool)
    need[cells.ravel()] = True
    chosen = []
    while need.any():
        score = need[cells].sum(axis=1)
        t = int(np.argmax(score))
        chosen.append(t)
        need[cells[t]] = False
    return np.array(sorted(chosen))
