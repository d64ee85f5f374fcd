#!/usr/bin/env python3
"""Benchmark of the routed-MoE expert path on Q2_K weights, one MI355X.

Headline workload: one MoE layer decode of one token in the DeepSeek-V4-Flash
routed-expert shape (256 experts, top-6, gate/up 4096->2048, SwiGLU, down
2048->4096), weights Q2_K, activations fp32.  A step is one full layer call
(routing, gate/up + SwiGLU, down + weighted combine) through the C ABI.
Steps cycle over --layers distinct seeded weight sets (2.11 GB each; the
default 43 is the Flash depth, 91 GB in total, far beyond the 256 MB MALL),
each with its own seeded router logits and activations, so weight bytes come
from HBM.  Steps are replayed from a HIP graph that holds one step per layer.

Also measured in the same run: the 4096-token prefill chunk (bf16, uniform
routing), one token through the 43-layer stack (Q2_K; mixed: Q2_K
layers 0-36 with Q4_1 layers 37-42; and Q2_K with every layer's MoE output
steered by its own row of a [43][4096] direction table), and the
activation-hop codec and standalone directional steering on 4096 x 4096 f32
as secondary figures, the dominant kernels' durations from HIP
events the library records around its own launches, and the CPU oracle on a
bounded sample of the same decode workload.

Prints one JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE expert tokens/s + achieved HBM GB/s (decode); TFLOP/s (4096-tok prefill)"
HBM_PEAK_GBPS = 8000.0
MFMA_F16_PEAK_TFLOPS = 2500.0   # dense fp16 / bf16 MFMA, MI355X

D, F, E, K = 4096, 2048, 256, 6
Q2K_ROW_D = D // 256 * 84       # bytes of one gate/up row (1344)
Q2K_ROW_F = F // 256 * 84       # bytes of one down row (672)
PAIR_FLOPS = 2 * 2 * D * F + 2 * F * D

# Arithmetic each workload computes in (what the kernels multiply, not a
# precision claim).
DTYPE_T1 = "i8x3limb+f32"          # one token: three int8 limbs per activation
DTYPE_I8X3 = "i8x3digit+i8min"     # 2..64-token Q2_K decode: three int8 digits per
                                   # activation, min term exact on int8 matrix cores
DTYPE_I8X3_Q41 = "i8x3digit+f32offset"  # 2..64-token Q4_1 decode: the same digits, the
                                        # offset term from fp32 sums of 32 inputs
DTYPE_F16 = "f16"                  # prefill: fp16 weights (each Q2_K weight rounded once
                                   # from its exact fp32 value, each Q4_1 weight d*q + m by
                                   # one fp16 fma) and fp16 inputs (bf16 values scaled by a
                                   # power of two), fp32 accumulation


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# Algorithmic bytes of one gate/up launch at one token: the six experts'
# gate and up rows, the input vector and the SwiGLU rows written.
GATEUP_BYTES = K * 2 * F * Q2K_ROW_D + D * 4 + K * F * 4
# Algorithmic HBM bytes of one prefill gate/up launch at 4096 tokens, uniform
# routing (every expert one m-tile): all experts' gate and up rows once, the
# fp16 input rows once, the bf16 SwiGLU rows written once.
PREFILL_GATEUP_BYTES = E * 2 * F * Q2K_ROW_D + 4096 * D * 2 + 4096 * K * F * 2
COUNTER_FILE = os.path.join(ROOT, "profiles", "decode_q2k_1tok_hbm_counters.txt")
KERNEL_SOURCES = ("bit_quantized_moe_q2_amd/csrc/decode_mfma.hip",
                  "bit_quantized_moe_q2_amd/csrc/mfma_t1.h",
                  "bit_quantized_moe_q2_amd/csrc/common.h")
PREFILL_COUNTER_FILE = os.path.join(ROOT, "profiles", "prefill_q2k_4096tok_hbm_counters.txt")
PREFILL_SOURCES = ("bit_quantized_moe_q2_amd/csrc/prefill_f16.hip",
                   "bit_quantized_moe_q2_amd/csrc/i8_ops.h",
                   "bit_quantized_moe_q2_amd/csrc/common.h")


def kernel_source_hash(sources=None):
    h = hashlib.sha256()
    for rel in sources or KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def counter_traffic(kernel, path=None, sources=None):
    """HBM bytes per launch of `kernel` from a committed FETCH_SIZE /
    WRITE_SIZE summary (default: the one-token decode's), each scaled by its
    plain-copy calibration factor; None when there is no summary or the
    kernel sources have changed since the counters were taken."""
    try:
        with open(path or COUNTER_FILE) as f:
            rows = [json.loads(ln.split(":", 1)[1]) for ln in f if ln.startswith("traffic_json:")]
    except OSError:
        return None
    for r in rows:
        if r.get("kernel") == kernel and r.get("src_sha256") == kernel_source_hash(sources):
            return int(round((r["fetch_kib"] * r["fetch_factor"] + r["write_kib"] * r["write_factor"])
                             * 1024))
    return None


def decode_bytes(T_pairs, T):
    """Algorithmic HBM bytes of one decode step (T tokens, T_pairs pairs over
    distinct experts counted once each in the grouped path)."""
    gateup_w = T_pairs * 2 * F * Q2K_ROW_D
    down_w = T_pairs * D * Q2K_ROW_F
    acts = T * D * 4 * 2 + T * E * 4          # x read, y write, logits read
    return gateup_w + down_w + acts


def host_cpu():
    """The host's CPU model, logical CPU count and the CPUs this process may use."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    model = ln.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except AttributeError:
        usable = os.cpu_count()
    return {"cpu_model": model, "nproc": os.cpu_count(), "cpus_usable": usable}


def oracle_configs():
    """The CPU oracle (fp64 C, built -O2 without fast-math) timed on each
    workload: the single 2048 x 4096 matvec, one-layer decode of 1 and of 64
    tokens on one core; the 4096-token prefill chunk in full with OpenMP over
    tokens on every usable core (each output element still summed by one
    thread); one token through the 43-layer Q2_K stack on one core (one token
    has no token parallelism); the 43-layer prefill chunk on 8 sampled tokens
    (one thread each), extrapolated linearly (4096 / threads rounds) to 4096 tokens (tokens are
    independent given the logits).  Expert weights are generated on the host
    first (not timed)."""
    import numpy as np

    import oracle
    import synth

    seed = 20260601
    cpu = host_cpu()
    threads = max(1, min(16, cpu["cpus_usable"] or 1))
    out = {"kind": "oracle", **cpu, "threads_parallel": threads, "workloads": {}}
    shapes = (("gate", F, D), ("up", F, D), ("down", D, F))

    def host_layer(l, experts):
        host = {n: np.zeros((E, r * c // 256 * 84), dtype=np.uint8) for n, r, c in shapes}
        for e in experts:
            for n, r, c in shapes:
                host[n][e] = synth.expert_tensor_blocks("q2_k", synth.layer_key(seed, l, n, int(e)), r, c).ravel()
        return oracle.Layer(D, F, E, K, oracle.Q2_K, host["gate"], host["up"], host["down"])

    def rec(name, seconds, work, unit, note):
        out["workloads"][name] = {"seconds": round(seconds, 3), "value": round(work / seconds, 4),
                                  "unit": unit, "note": note}
        log(f"oracle {name}: {seconds:.2f} s, {work / seconds:.4g} {unit}")

    # single matvec (one core)
    w = synth.expert_tensor_blocks("q2_k", synth.layer_key(seed, 0, "gate", 0), F, D)
    xv = synth.x_f32(synth.stream_key(seed, 10), 1, D)[0]
    t0 = time.perf_counter()
    reps = 5
    for _ in range(reps):
        oracle.matvec(oracle.Q2_K, w, F, D, xv)
    rec("matvec_q2_k_2048x4096", (time.perf_counter() - t0) / reps, 1.0, "matvecs/s", "1 core")
    # one-layer decode, 1 and 64 tokens (one core)
    for T, key in ((1, 2), (64, 12)):
        lg = synth.logits_normal(synth.stream_key(seed, key, 0), T, E)
        x = synth.x_f32(synth.stream_key(seed, key - 1, 0), T, D)
        L = host_layer(0, np.unique(oracle.route(lg, K)[0]))
        t0 = time.perf_counter()
        oracle.moe(L, x, lg, n_threads=1)
        rec(f"decode_{T}tok_q2_k", time.perf_counter() - t0, T, "tokens/s", "1 core")
    # 4096-token chunk, in full (all usable cores)
    Tp = 4096
    lg = synth.logits_normal(synth.stream_key(seed, 4), Tp, E)
    xb = synth.x_bf16(synth.stream_key(seed, 3), Tp, D)
    xf = (xb.astype(np.uint32) << 16).view(np.float32)
    L = host_layer(0, np.arange(E))
    t0 = time.perf_counter()
    oracle.moe(L, xf, lg, n_threads=threads)
    rec("prefill_4096tok_q2_k_uniform", time.perf_counter() - t0, Tp, "tokens/s",
        f"in full, OpenMP over tokens on {threads} threads")
    del L
    # 43-layer stack: one decode token (one core), 16 prefill tokens
    lgs = np.stack([synth.logits_normal(synth.stream_key(seed, 5, l), 1, E) for l in range(43)])
    lays = [host_layer(l, np.unique(oracle.route(lgs[l], K)[0])) for l in range(43)]
    x1 = synth.x_f32(synth.stream_key(seed, 6), 1, D)
    t0 = time.perf_counter()
    oracle.stack(lays, x1, lgs, prefill_bf16=False, n_threads=1)
    rec("stack43_decode_1tok_q2_k", time.perf_counter() - t0, 1, "tokens/s", "1 core, in full")
    S = 8
    lgp = np.stack([synth.logits_normal(synth.stream_key(seed, 14, l), S, E) for l in range(43)])
    lays = [host_layer(l, np.unique(oracle.route(lgp[l], K)[0])) for l in range(43)]
    xp = synth.x_f32(synth.stream_key(seed, 15), S, D)
    t0 = time.perf_counter()
    oracle.stack(lays, xp, lgp, prefill_bf16=True, n_threads=S)
    dt = time.perf_counter() - t0
    rec("stack43_prefill_4096tok_q2_k", dt * Tp / threads, Tp, "tokens/s",
        f"{S} sampled tokens, one thread each ({dt:.1f} s); the {Tp}-token chunk extrapolated to "
        f"{threads} threads as {Tp}/{threads} such rounds")
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=4300)
    ap.add_argument("--warmup", type=int, default=430)
    ap.add_argument("--layers", type=int, default=43,
                    help="distinct weight sets cycled (43 = DeepSeek-V4-Flash depth, 91 GB of Q2_K)")
    ap.add_argument("--prefill-steps", type=int, default=20)
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-stack", action="store_true")
    ap.add_argument("--no-aux", action="store_true", help="skip the codec and steering figures")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the other workloads (matvec/dequant, 64-token decode, Zipf and Q4_1 "
                         "prefill, 43-layer prefill)")
    ap.add_argument("--stack-tokens", type=int, default=50,
                    help="tokens timed through each 43-layer stack")
    ap.add_argument("--cpu-sample", type=int, default=1024,
                    help="decode tokens the oracle runs (about 15 s on 16 host threads)")
    ap.add_argument("--oracle-configs", action="store_true",
                    help="only time the CPU oracle on each workload (single matvec, 1- and "
                         "64-token decode on one core; the 4096-token chunk on all cores; the "
                         "43-layer stack) and print those figures; no GPU work")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="also run plain device copies of this size (counter calibration)")
    args = ap.parse_args()
    if args.steps < 1 or args.warmup < 0 or args.layers < 1:
        ap.error("--steps and --layers must be positive, --warmup non-negative")
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path (a GPU would "
              "hold its share of the experts, with tokens exchanged all-to-all); run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    if args.oracle_configs:
        print(json.dumps(oracle_configs()), flush=True)
        return

    import numpy as np
    import torch

    import bit_quantized_moe_q2_amd as ds4q
    import synth

    ds4q.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    seed = 20260601
    NL = args.layers

    # ------------------------------------------------------------ weights
    log(f"generating {NL} layers of Q2_K experts on the device ...")
    layers, keep = [], []
    for l in range(NL):
        t = {}
        for name, rows, cols in (("gate", F, D), ("up", F, D), ("down", D, F)):
            buf = torch.empty(E * rows * cols // 256 * 84, dtype=torch.uint8, device=dev)
            keep.append(synth.device_fill("q2_k", buf, [synth.layer_key(seed, l, name, e) for e in range(E)],
                                          rows * cols // 256))
            t[name] = buf
        layers.append(ds4q.MoeLayer.from_tensors(t["gate"], t["up"], t["down"], D, F, E, K,
                                                 ds4q.TYPE_Q2_K))
    torch.cuda.synchronize()

    # ------------------------------------------------------------ decode inputs
    xs = torch.from_numpy(np.stack([synth.x_f32(synth.stream_key(seed, 1, l), 1, D) for l in range(NL)])).to(dev)
    lgs = torch.from_numpy(np.stack([synth.logits_normal(synth.stream_key(seed, 2, l), 1, E)
                                     for l in range(NL)])).to(dev)
    ys = torch.empty(NL, 1, D, dtype=torch.float32, device=dev)
    # one workspace per layer, so that a graph of one phase over all layers
    # finds each layer's routing and activations where its full step left them
    ws_bytes = ds4q.ds4q_moe_workspace_size(layers[0], 1, 0)
    ws_dec = [torch.empty(ws_bytes, dtype=torch.uint8, device=dev) for _ in range(NL)]

    def decode_step(l):
        ds4q.ds4q_moe_decode(layers[l], xs[l], lgs[l], 1, ys[l], None, ws_dec[l])

    def decode_phase(l, ph):
        ds4q.ds4q_moe_decode_phases(layers[l], xs[l], lgs[l], 1, ys[l], None, ws_dec[l], ph)

    for l in range(NL):
        decode_step(l)
    torch.cuda.synchronize()

    def capture(fn):
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr):
            fn()
        torch.cuda.synchronize()
        return gr

    # a graph of NL steps (one per layer) plus one for the remainder, so that
    # exactly --steps steps are timed
    g = capture(lambda: [decode_step(l) for l in range(NL)])

    def run_steps(n):
        for _ in range(n // NL):
            g.replay()
        if n % NL:
            capture_rem(n % NL).replay()

    rem_graphs = {}

    def capture_rem(r, tail=False):
        key = (r, tail)
        if key not in rem_graphs:
            ls = range(NL - r, NL) if tail else range(r)
            rem_graphs[key] = capture(lambda: [decode_step(l) for l in ls])
        return rem_graphs[key]

    if args.steps % NL:
        capture_rem(args.steps % NL)
    # warm-up: the LAST --warmup layers of the cycle (whole cycles first), so
    # the timed steps start on layer 0, whose weights the warm-up did not
    # just read (the 256 MB memory-side cache holds about five layers' experts)
    if args.warmup % NL:
        capture_rem(args.warmup % NL, tail=True).replay()
    for _ in range(args.warmup // NL):
        g.replay()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    run_steps(args.steps)
    ev1.record()
    torch.cuda.synchronize()
    dec_ms = ev0.elapsed_time(ev1)
    steps_done = args.steps
    reps = max(1, args.steps // NL)
    ms_per_step = dec_ms / steps_done
    tok_s = steps_done / (dec_ms / 1e3)
    step_bytes = decode_bytes(K, 1)
    log(f"decode: {ms_per_step * 1e3:.2f} us/step, {tok_s:.0f} tok/s, "
        f"{step_bytes / (ms_per_step / 1e3) / 1e9:.0f} GB/s algorithmic")

    # Per-kernel durations: a graph of one kernel launch per layer (the same
    # launches as in the step graph, on the same stream), replayed between
    # two events; launch gaps inside a graph are far below a microsecond.
    # (one token on Q2_K: the gate/up launch also routes; the routing phase
    # launches nothing of its own)
    phases = (("decode_gateup", ds4q.PHASE_GATEUP), ("decode_down", ds4q.PHASE_DOWN))
    k_us = {}
    k_reps = max(1, min(reps, 40))
    for name, ph in phases:
        gk = capture(lambda ph=ph: [decode_phase(l, ph) for l in range(NL)])
        for _ in range(2):
            gk.replay()
        torch.cuda.synchronize()
        ev0.record()
        for _ in range(k_reps):
            gk.replay()
        ev1.record()
        torch.cuda.synchronize()
        k_us[name] = ev0.elapsed_time(ev1) * 1e3 / (k_reps * NL)
        del gk
    g.replay()                      # leave every layer's outputs consistent
    torch.cuda.synchronize()
    gu_us, dn_us = k_us["decode_gateup"], k_us["decode_down"]
    gu_bytes = GATEUP_BYTES
    dn_bytes = K * D * Q2K_ROW_F + K * F * 4 + D * 4
    gu_gbps = gu_bytes / (gu_us / 1e6) / 1e9
    log(f"kernels: gateup {gu_us:.2f} us "
        f"({gu_gbps:.0f} GB/s), down {dn_us:.2f} us ({dn_bytes / (dn_us / 1e6) / 1e9:.0f} GB/s)")
    traffic = counter_traffic("decode_gateup")

    result = {
        "metric": METRIC,
        "value": round(tok_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps_done,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        # the arithmetic of the one-token path: int8 matrix cores on the exact
        # integer weights against three int8 limbs of each activation (about
        # 24 bits), int32 sums, fp32 scales, min term and accumulation
        "dtype": DTYPE_T1,
        "data": "synthetic (seeded Q2_K blocks: codes U{0..3}, scale/min nibbles U{0..15}, "
                "d/dmin |N(0,0.01)|; x, logits N(0,1))",
        "config": {"workload": "moe_layer_decode_1tok", "weights": "q2_k", "n_expert": E,
                   "top_k": K, "n_embd": D, "n_ff": F, "tokens": 1,
                   "weight_sets_cycled": NL, "graph_replay": True},
        "hbm_gbps_step": round(step_bytes / (ms_per_step / 1e3) / 1e9, 1),
        "roofline": {"bound": "hbm", "kernel": "decode_gateup", "achieved": round(gu_gbps, 1),
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(gu_gbps / HBM_PEAK_GBPS, 4),
                     "traffic": traffic, "bytes_per_launch": gu_bytes,
                     "avg_launch_us": round(gu_us, 3)},
        "kernels_us": {k: round(v, 3) for k, v in k_us.items()},
    }

    # ------------------------------------------------------------ prefill (secondary)
    if not args.no_prefill:
        T = 4096
        xb = torch.from_numpy(synth.x_bf16(synth.stream_key(seed, 3), T, D).view(np.int16)).to(dev)
        lgp = torch.from_numpy(synth.logits_normal(synth.stream_key(seed, 4), T, E)).to(dev)
        yp = torch.empty(T, D, dtype=torch.float32, device=dev)
        ws_p = torch.empty(ds4q.ds4q_moe_workspace_size(layers[0], T, 1), dtype=torch.uint8, device=dev)

        def prefill_step():
            ds4q.ds4q_moe_prefill(layers[0], xb, ds4q.TYPE_BF16, lgp, T, yp, None, ws_p)

        prefill_step()
        torch.cuda.synchronize()
        gp = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gp):
            prefill_step()
        for _ in range(3):
            gp.replay()
        torch.cuda.synchronize()
        ev0.record()
        for _ in range(args.prefill_steps):
            gp.replay()
        ev1.record()
        torch.cuda.synchronize()
        p_ms = ev0.elapsed_time(ev1) / args.prefill_steps
        flops = T * K * PAIR_FLOPS
        ds4q.ds4q_timing_enable(True)
        for _ in range(5):
            prefill_step()
        torch.cuda.synchronize()
        pt = ds4q.ds4q_timing_read()
        ds4q.ds4q_timing_enable(False)
        g1_ms = pt["prefill_gateup"][0] / pt["prefill_gateup"][1]
        g1_tf = T * K * 2 * 2 * D * F / (g1_ms / 1e3) / 1e12
        # the same chunk with the layer's output steered (fused into the combine)
        dp = torch.from_numpy(synth.x_f32(synth.stream_key(seed, 9, 0), 1, D)[0]).to(dev)
        dp /= torch.linalg.vector_norm(dp)
        Lsp = ds4q.MoeLayer.from_buffer_copy(layers[0])
        Lsp.steer_dir, Lsp.steer_scale = dp.data_ptr(), 1.0
        ds4q.ds4q_timing_enable(True)
        for _ in range(5):
            ds4q.ds4q_moe_prefill(Lsp, xb, ds4q.TYPE_BF16, lgp, T, yp, None, ws_p)
        torch.cuda.synchronize()
        pts = ds4q.ds4q_timing_read()
        ds4q.ds4q_timing_enable(False)
        comb_us = pt["combine"][0] / pt["combine"][1] * 1e3
        comb_steer_us = pts["combine"][0] / pts["combine"][1] * 1e3
        # the same chunk collecting the imatrix statistics (input and down)
        st_in = torch.zeros(E, D, device=dev)
        st_dn = torch.zeros(E, F, device=dev)
        Lim = ds4q.MoeLayer.from_buffer_copy(layers[0])
        Lim.imatrix_in, Lim.imatrix_down = st_in.data_ptr(), st_dn.data_ptr()
        ws_im = torch.empty(ds4q.ds4q_moe_workspace_size(Lim, T, 1), dtype=torch.uint8, device=dev)
        ds4q.ds4q_moe_prefill(Lim, xb, ds4q.TYPE_BF16, lgp, T, yp, None, ws_im)
        torch.cuda.synchronize()
        ds4q.ds4q_timing_enable(True)
        for _ in range(5):
            ds4q.ds4q_moe_prefill(Lim, xb, ds4q.TYPE_BF16, lgp, T, yp, None, ws_im)
        torch.cuda.synchronize()
        pti = ds4q.ds4q_timing_read()
        ds4q.ds4q_timing_enable(False)
        im_us = pti["imatrix"][0] / pti["imatrix"][1] * 1e3
        P = T * K
        # live m-tiles of this routing (up to 128 sorted pairs of one expert each)
        cnt = np.bincount(np.argsort(-lgp.cpu().numpy(), axis=1, kind="stable")[:, :K].ravel(), minlength=E)
        n_tiles = int(((cnt + 127) // 128).sum())
        # bf16 input rows and SwiGLU rows read once per pair, partial rows
        # written and read back, the statistics read and written
        im_bytes = P * (D + F) * 2 + n_tiles * (D + F) * 4 * 2 + E * (D + F) * 4 * 2
        del ws_im
        log(f"prefill: {p_ms:.3f} ms/chunk, {flops / (p_ms / 1e3) / 1e12:.1f} TFLOP/s; "
            f"gateup {g1_ms:.3f} ms ({g1_tf:.1f} TFLOP/s)")
        result["prefill"] = {
            "workload": "moe_layer_prefill_4096tok_bf16_uniform", "dtype": DTYPE_F16,
            "ms_per_chunk": round(p_ms, 4),
            "tflops": round(flops / (p_ms / 1e3) / 1e12, 2),
            "tokens_per_s": round(T / (p_ms / 1e3), 1),
            # algorithmic GEMM flops per second of the gate/up GEMM against the
            # dense fp16 peak (one fp16 MAC per algorithmic MAC)
            "roofline": {"bound": "mfma", "kernel": "prefill_gateup", "achieved": round(g1_tf, 2),
                         "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(g1_tf / MFMA_F16_PEAK_TFLOPS, 4),
                         "traffic": counter_traffic("prefill_gateup", PREFILL_COUNTER_FILE, PREFILL_SOURCES),
                         "bytes_algorithmic": PREFILL_GATEUP_BYTES},
            "kernels_us": {k: round(v[0] / v[1] * 1e3, 2) for k, v in pt.items()},
            # combine of the 4096 x 6 expert rows, plain and with the steering
            # epilogue (row dot product + projection in the same launch)
            "combine_us": round(comb_us, 2), "combine_steered_us": round(comb_steer_us, 2),
            # imatrix statistics hook on the same chunk (bytes are an upper
            # bound: the partial rows of live tiles only are written)
            "imatrix_us": round(im_us, 2), "imatrix_bytes": im_bytes,
            "imatrix_gbps": round(im_bytes / (im_us / 1e6) / 1e9, 1),
        }
        log(f"prefill imatrix hook: {im_us:.1f} us, {im_bytes / (im_us / 1e6) / 1e9:.0f} GB/s")
        log(f"prefill combine: {comb_us:.1f} us, steered {comb_steer_us:.1f} us")

    # ------------------------------------------------------------ stack (secondary)
    q41 = []
    if not args.no_stack and NL == 43:
        # mixed stack: the first 37 Q2_K layers above plus 6 Q4_1 layers
        log("generating 6 layers of Q4_1 experts for the mixed stack ...")
        for l in range(37, 43):
            t = {}
            for name, rows, cols in (("gate", F, D), ("up", F, D), ("down", D, F)):
                buf = torch.empty(E * rows * cols // 32 * 20, dtype=torch.uint8, device=dev)
                keep.append(synth.device_fill("q4_1", buf, [synth.layer_key(seed + 1, l, name, e)
                                                             for e in range(E)], rows * cols // 32))
                t[name] = buf
            q41.append(ds4q.MoeLayer.from_tensors(t["gate"], t["up"], t["down"], D, F, E, K,
                                                  ds4q.TYPE_Q4_1))
        torch.cuda.synchronize()
        lgs_st = torch.from_numpy(np.stack([synth.logits_normal(synth.stream_key(seed, 5, l), 1, E)
                                            for l in range(NL)])).to(dev)
        x_st = torch.from_numpy(synth.x_f32(synth.stream_key(seed, 6), 1, D)).to(dev)
        x_run = torch.empty_like(x_st)
        # steered Q2_K stack: layer l's MoE output loses row l of a layer-major
        # [43][4096] table of unit directions (scale 1)
        dirs = torch.from_numpy(np.stack([synth.x_f32(synth.stream_key(seed, 9, l), 1, D)[0]
                                          for l in range(NL)])).to(dev)
        dirs /= torch.linalg.vector_norm(dirs, dim=1, keepdim=True)
        steered = []
        for l, L in enumerate(layers):
            Ls = ds4q.MoeLayer.from_buffer_copy(L)
            Ls.steer_dir, Ls.steer_scale = dirs[l].data_ptr(), 1.0
            steered.append(Ls)
        result["stack_decode"] = {}
        for name, lays in (("q2_k", layers), ("mixed", layers[:37] + q41), ("q2_k_steered", steered)):
            ws_st = torch.empty(max(ds4q.ds4q_moe_workspace_size(L, 1, 0) for L in lays),
                                dtype=torch.uint8, device=dev)

            def stack_token():
                x_run.copy_(x_st)
                ds4q.ds4q_moe_stack(lays, 0, x_run, lgs_st, 1, ws_st)

            stack_token()
            torch.cuda.synchronize()
            gs = capture(stack_token)
            gs.replay()
            torch.cuda.synchronize()
            ev0.record()
            for _ in range(args.stack_tokens):
                gs.replay()
            ev1.record()
            torch.cuda.synchronize()
            t_ms = ev0.elapsed_time(ev1) / args.stack_tokens
            wbytes = sum(K * (2 * F * ds4q.row_bytes(L.type_gate, D) + D * ds4q.row_bytes(L.type_down, F))
                         for L in lays)
            log(f"stack {name}: {t_ms * 1e3:.1f} us/token through {len(lays)} layers, "
                f"{wbytes / (t_ms / 1e3) / 1e9:.0f} GB/s")
            result["stack_decode"][name] = {
                "workload": f"stack43_decode_1tok_{name}", "us_per_token": round(t_ms * 1e3, 2),
                "tokens_per_s": round(1e3 / t_ms, 1), "weight_bytes_per_token": wbytes,
                "hbm_gbps": round(wbytes / (t_ms / 1e3) / 1e9, 1)}
            if name == "q2_k_steered":
                base_us = result["stack_decode"]["q2_k"]["us_per_token"]
                result["stack_decode"][name]["steer_us_per_layer"] = round((t_ms * 1e3 - base_us) / NL, 3)
            del gs, ws_st

    # ------------------------------------------------------------ other workloads (secondary)
    if not args.no_configs and NL == 43:
        cf = {}
        evs = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

        def graph_time(fn, reps):
            """ms per replay of a graph of fn (after one eager call)."""
            fn()
            torch.cuda.synchronize()
            gr = capture(fn)
            gr.replay()
            torch.cuda.synchronize()
            evs[0].record()
            for _ in range(reps):
                gr.replay()
            evs[1].record()
            torch.cuda.synchronize()
            return evs[0].elapsed_time(evs[1]) / reps

        # single matrices (2048 x 4096): each expert's gate tensor is one, so
        # 128 distinct ones rotate through the graphs (352 MB of Q2_K, beyond
        # the 256 MB MALL; outputs of the dequant rotate over 268 MB)
        NM = 128
        mats = {"q2_k": (ds4q.TYPE_Q2_K, layers[0].gate, 2048 * 4096 // 256 * 84)}
        if q41:
            mats["q4_1"] = (ds4q.TYPE_Q4_1, q41[0].gate, 2048 * 4096 // 32 * 20)
        xv = torch.from_numpy(synth.x_f32(synth.stream_key(seed, 10), 1, D)).to(dev)
        yv = torch.empty(NM, F, device=dev)
        deq = [torch.empty(F * D, device=dev) for _ in range(8)]
        # the least a kernel costs in such a graph: NM one-element fills
        tiny = torch.zeros(NM, device=dev)
        floor_us = graph_time(lambda: [tiny[i:i + 1].fill_(1.0) for i in range(NM)], 20) / NM * 1e3
        cf["launch_floor_graph"] = {"us": round(floor_us, 3),
                                    "what": "one-element fill kernel per graph node, same graph shape"}
        for qn, (qt, base, mb) in mats.items():
            ms = graph_time(lambda: [ds4q.ds4q_matvec(qt, base + i * mb, F, D, xv, 1, yv[i]) for i in range(NM)], 20) / NM
            b = mb + D * 4 + F * 4
            cf[f"matvec_{qn}_2048x4096"] = {"us": round(ms * 1e3, 3), "bytes": b,
                                            "gbps": round(b / (ms / 1e3) / 1e9, 1),
                                            "launch_floor_us": round(floor_us, 3),
                                            "us_above_floor": round(ms * 1e3 - floor_us, 3)}
            ms = graph_time(lambda: [ds4q.ds4q_dequant(qt, base + i * mb, F, D, ds4q.TYPE_F32, deq[i % 8])
                                     for i in range(NM)], 10) / NM
            b = mb + F * D * 4
            cf[f"dequant_{qn}_f32_2048x4096"] = {"us": round(ms * 1e3, 3), "bytes": b,
                                                 "gbps": round(b / (ms / 1e3) / 1e9, 1)}
        # the write side alone: a fill of the same f32 output per graph node
        ms = graph_time(lambda: [deq[i % 8].fill_(1.0) for i in range(NM)], 10) / NM
        b = F * D * 4
        cf["fill_f32_2048x4096"] = {"us": round(ms * 1e3, 3), "bytes": b, "gbps": round(b / (ms / 1e3) / 1e9, 1),
                                    "what": "torch fill of one dequant output, same graph shape"}
        del deq, yv, tiny

        # one layer decode of 64 tokens, cycling over the 43 layers
        T64 = 64
        x64 = torch.from_numpy(np.stack([synth.x_f32(synth.stream_key(seed, 11, l), T64, D) for l in range(NL)])).to(dev)
        lg64n = np.stack([synth.logits_normal(synth.stream_key(seed, 12, l), T64, E) for l in range(NL)])
        lg64 = torch.from_numpy(lg64n).to(dev)
        y64 = torch.empty(NL, T64, D, device=dev)
        wsb64 = ds4q.ds4q_moe_workspace_size(layers[0], T64, 0)
        ws64 = [torch.empty(wsb64, dtype=torch.uint8, device=dev) for _ in range(NL)]
        ms = graph_time(lambda: [ds4q.ds4q_moe_decode(layers[l], x64[l], lg64[l], T64, y64[l], None, ws64[l])
                                 for l in range(NL)], 5) / NL
        touched = np.mean([len(np.unique(np.argsort(-lg64n[l], axis=1, kind="stable")[:, :K])) for l in range(NL)])
        b = touched * 3 * 2048 * 4096 // 256 * 84
        cf["decode_64tok_q2_k"] = {"dtype": DTYPE_I8X3,
                                   "us_per_layer": round(ms * 1e3, 2), "tokens_per_s": round(T64 / (ms / 1e3), 1),
                                   "experts_touched": round(float(touched), 1), "weight_bytes": int(b),
                                   "gbps": round(b / (ms / 1e3) / 1e9, 1)}
        if q41:
            # the same on the Q4_1 layers (the mixed stack's last six)
            nq = len(q41)
            ms = graph_time(lambda: [ds4q.ds4q_moe_decode(q41[l], x64[l], lg64[l], T64, y64[l], None, ws64[l])
                                     for l in range(nq)], 5) / nq
            touched = np.mean([len(np.unique(np.argsort(-lg64n[l], axis=1, kind="stable")[:, :K])) for l in range(nq)])
            b = touched * 3 * 2048 * 4096 // 32 * 20
            cf["decode_64tok_q4_1"] = {"dtype": DTYPE_I8X3_Q41,
                                       "us_per_layer": round(ms * 1e3, 2), "tokens_per_s": round(T64 / (ms / 1e3), 1),
                                       "experts_touched": round(float(touched), 1), "weight_bytes": int(b),
                                       "gbps": round(b / (ms / 1e3) / 1e9, 1)}
        del x64, lg64, y64, ws64

        # 4096-token prefill chunks: Zipf(1.1) routing, and Q4_1 weights
        if not args.no_prefill:
            Tp = 4096
            xbz = torch.from_numpy(synth.x_bf16(synth.stream_key(seed, 3), Tp, D).view(np.int16)).to(dev)
            lgz = torch.from_numpy(synth.logits_zipf(synth.stream_key(seed, 13), Tp, E)).to(dev)
            ypz = torch.empty(Tp, D, device=dev)
            wsz = torch.empty(ds4q.ds4q_moe_workspace_size(layers[0], Tp, 1), dtype=torch.uint8, device=dev)
            ms = graph_time(lambda: ds4q.ds4q_moe_prefill(layers[0], xbz, ds4q.TYPE_BF16, lgz, Tp, ypz, None, wsz), 10)
            cf["prefill_4096tok_q2_k_zipf"] = {"dtype": DTYPE_F16, "ms": round(ms, 4),
                                               "tflops": round(Tp * K * PAIR_FLOPS / (ms / 1e3) / 1e12, 1)}
            if q41:
                lgu = torch.from_numpy(synth.logits_normal(synth.stream_key(seed, 4), Tp, E)).to(dev)
                wsq = torch.empty(ds4q.ds4q_moe_workspace_size(q41[0], Tp, 1), dtype=torch.uint8, device=dev)
                ms = graph_time(lambda: ds4q.ds4q_moe_prefill(q41[0], xbz, ds4q.TYPE_BF16, lgu, Tp, ypz, None, wsq), 10)
                cf["prefill_4096tok_q4_1_uniform"] = {"dtype": DTYPE_F16, "ms": round(ms, 4),
                                                      "tflops": round(Tp * K * PAIR_FLOPS / (ms / 1e3) / 1e12, 1)}
                del wsq, lgu
            del wsz, lgz

            # one 4096-token chunk through the 43-layer stack (RMS norm, bf16
            # layer inputs, residual), Q2_K and mixed
            lgs_p = torch.from_numpy(np.stack([synth.logits_normal(synth.stream_key(seed, 14, l), Tp, E)
                                               for l in range(NL)])).to(dev)
            x0p = torch.from_numpy(synth.x_f32(synth.stream_key(seed, 15), Tp, D)).to(dev)
            xrun = torch.empty_like(x0p)
            for name, lays in (("q2_k", layers), ("mixed", layers[:37] + q41)):
                if len(lays) != NL:
                    continue
                wsp = torch.empty(max(ds4q.ds4q_moe_workspace_size(L, Tp, 1) for L in lays), dtype=torch.uint8,
                                  device=dev)

                def run_stack():
                    xrun.copy_(x0p)
                    ds4q.ds4q_moe_stack(lays, 1, xrun, lgs_p, Tp, wsp)

                run_stack()
                torch.cuda.synchronize()
                evs[0].record()
                for _ in range(2):
                    run_stack()
                evs[1].record()
                torch.cuda.synchronize()
                ms = evs[0].elapsed_time(evs[1]) / 2
                cf[f"stack43_prefill_4096tok_{name}"] = {
                    "ms_per_chunk": round(ms, 2), "tokens_per_s": round(Tp / (ms / 1e3), 1),
                    "tflops": round(NL * Tp * K * PAIR_FLOPS / (ms / 1e3) / 1e12, 1)}
                del wsp
            del lgs_p, x0p, xrun, xbz, ypz
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        result["configs"] = cf
        log("other workloads: " + json.dumps(cf))

    # ------------------------------------------------------------ codec and steering (secondary)
    if not args.no_aux:
        T_h = 4096
        n = T_h * D
        xh = torch.from_numpy(synth.x_f32(synth.stream_key(seed, 7), T_h, D)).to(dev)
        wire = torch.empty(n * 2, dtype=torch.uint8, device=dev)
        back = torch.empty(T_h, D, dtype=torch.float32, device=dev)
        res_h = torch.empty(T_h, D, dtype=torch.float32, device=dev)
        dvec = torch.from_numpy(synth.x_f32(synth.stream_key(seed, 8), 1, D)).to(dev)
        dvec /= torch.linalg.vector_norm(dvec)

        def timed(fn, reps=20):
            fn()
            torch.cuda.synchronize()
            gx = capture(fn)
            gx.replay()
            torch.cuda.synchronize()
            ev0.record()
            for _ in range(reps):
                gx.replay()
            ev1.record()
            torch.cuda.synchronize()
            return ev0.elapsed_time(ev1) / reps * 1e3  # us

        aux = {}
        for bits in (16, 8):
            us = timed(lambda b=bits: ds4q.ds4q_act_encode(xh, n, b, wire))
            nb = n * 4 + n * bits // 8
            aux[f"encode_f32_to_{'f16' if bits == 16 else 'e4m3'}"] = {
                "us": round(us, 2), "gbps": round(nb / (us / 1e6) / 1e9, 1)}
            us = timed(lambda b=bits: ds4q.ds4q_act_decode(wire, n, b, back))
            aux[f"decode_{'f16' if bits == 16 else 'e4m3'}_to_f32"] = {
                "us": round(us, 2), "gbps": round(nb / (us / 1e6) / 1e9, 1)}
        us = timed(lambda: ds4q.ds4q_steer(dvec, 0.5, back, T_h, D, res_h, ds4q.F_ACCUMULATE))
        nb = n * 4 * 3 + D * 4
        aux["steer_accumulate"] = {"us": round(us, 2), "gbps": round(nb / (us / 1e6) / 1e9, 1)}
        log("aux (4096 x 4096 f32 hop / rows): " + ", ".join(f"{k} {v['us']} us {v['gbps']} GB/s"
                                                             for k, v in aux.items()))
        result["aux_4096x4096"] = {"workload": "activation hop codec and steering, 4096 x 4096 f32",
                                   "peak_gbps": HBM_PEAK_GBPS, **aux}
        del xh, wire, back, res_h

    if args.calib_copy_mib:
        n = args.calib_copy_mib * (1 << 20) // 4
        a = torch.empty(n, dtype=torch.float32, device=dev).fill_(1.0)
        b = torch.empty_like(a)
        for _ in range(4):
            b.copy_(a)
        torch.cuda.synchronize()
        result["calib_copy_bytes"] = n * 4

    # ------------------------------------------------------------ Q4_1 stack (secondary)
    # the 43-layer stack on Q4_1 weights (173 GB): after the Q2_K layers are
    # freed, one token and one 4096-token chunk through it
    if not args.no_stack and not args.no_configs and NL == 43:
        import gc
        for lst in (layers, q41, keep):
            lst.clear()
        steered = lays = L = Ls = None
        gc.collect()
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        q41_bytes = 43 * 3 * E * (D * F // 32 * 20)
        free_b, _ = torch.cuda.mem_get_info()
        if free_b < q41_bytes + (16 << 30):
            log(f"Q4_1 stack skipped: {free_b / 1e9:.1f} GB free")
        else:
            log("generating 43 layers of Q4_1 experts (173 GB) ...")
            stack41 = []
            for l in range(NL):
                t = {}
                for name, rows, cols in (("gate", F, D), ("up", F, D), ("down", D, F)):
                    buf = torch.empty(E * rows * cols // 32 * 20, dtype=torch.uint8, device=dev)
                    synth.device_fill("q4_1", buf, [synth.layer_key(seed + 2, l, name, e) for e in range(E)],
                                      rows * cols // 32)
                    t[name] = buf
                stack41.append(ds4q.MoeLayer.from_tensors(t["gate"], t["up"], t["down"], D, F, E, K,
                                                          ds4q.TYPE_Q4_1))
            torch.cuda.synchronize()
            # one token (same inputs as the Q2_K stack)
            ws41 = torch.empty(ds4q.ds4q_moe_workspace_size(stack41[0], 1, 0), dtype=torch.uint8, device=dev)

            def stack41_token():
                x_run.copy_(x_st)
                ds4q.ds4q_moe_stack(stack41, 0, x_run, lgs_st, 1, ws41)

            stack41_token()
            torch.cuda.synchronize()
            g41 = capture(stack41_token)
            g41.replay()
            torch.cuda.synchronize()
            ev0.record()
            for _ in range(args.stack_tokens):
                g41.replay()
            ev1.record()
            torch.cuda.synchronize()
            t_ms = ev0.elapsed_time(ev1) / args.stack_tokens
            wbytes = NL * K * 3 * (F * ds4q.row_bytes(ds4q.TYPE_Q4_1, D))
            log(f"stack q4_1: {t_ms * 1e3:.1f} us/token through {NL} layers, "
                f"{wbytes / (t_ms / 1e3) / 1e9:.0f} GB/s")
            result["stack_decode"]["q4_1"] = {
                "workload": "stack43_decode_1tok_q4_1", "us_per_token": round(t_ms * 1e3, 2),
                "tokens_per_s": round(1e3 / t_ms, 1), "weight_bytes_per_token": wbytes,
                "hbm_gbps": round(wbytes / (t_ms / 1e3) / 1e9, 1)}
            del g41, ws41
            # one 4096-token chunk
            Tp = 4096
            lgs_p = torch.from_numpy(np.stack([synth.logits_normal(synth.stream_key(seed, 14, l), Tp, E)
                                               for l in range(NL)])).to(dev)
            x0p = torch.from_numpy(synth.x_f32(synth.stream_key(seed, 15), Tp, D)).to(dev)
            xrun = torch.empty_like(x0p)
            wsp = torch.empty(ds4q.ds4q_moe_workspace_size(stack41[0], Tp, 1), dtype=torch.uint8, device=dev)

            def run_stack41():
                xrun.copy_(x0p)
                ds4q.ds4q_moe_stack(stack41, 1, xrun, lgs_p, Tp, wsp)

            run_stack41()
            torch.cuda.synchronize()
            ev0.record()
            for _ in range(2):
                run_stack41()
            ev1.record()
            torch.cuda.synchronize()
            ms = ev0.elapsed_time(ev1) / 2
            result["configs"]["stack43_prefill_4096tok_q4_1"] = {
                "ms_per_chunk": round(ms, 2), "tokens_per_s": round(Tp / (ms / 1e3), 1),
                "tflops": round(NL * Tp * K * PAIR_FLOPS / (ms / 1e3) / 1e12, 1)}
            log(f"stack q4_1 prefill: {ms:.2f} ms per 4096-token chunk")
            del wsp, lgs_p, x0p, xrun, stack41
            torch.cuda.synchronize()
            torch.cuda.empty_cache()

    # ------------------------------------------------------------ CPU oracle baseline
    if not args.no_cpu_baseline:
        import oracle
        S = args.cpu_sample
        threads = min(16, os.cpu_count() or 1)
        x = np.stack([synth.x_f32(synth.stream_key(seed, 5, i), 1, D)[0] for i in range(S)])
        lg = np.stack([synth.logits_normal(synth.stream_key(seed, 6, i), 1, E)[0] for i in range(S)])
        ids, _ = oracle.route(lg, K)
        host = {n: np.zeros((E, (F if n != "down" else D) * (D if n != "down" else F) // 256 * 84),
                            dtype=np.uint8) for n in ("gate", "up", "down")}
        for e in np.unique(ids):
            for n, rows, cols in (("gate", F, D), ("up", F, D), ("down", D, F)):
                host[n][e] = synth.expert_tensor_blocks("q2_k", synth.layer_key(seed, 0, n, int(e)),
                                                        rows, cols).ravel()
        orc = oracle.Layer(D, F, E, K, oracle.Q2_K, host["gate"], host["up"], host["down"])
        t0 = time.perf_counter()
        oracle.moe(orc, x, lg, n_threads=threads)
        dt = time.perf_counter() - t0
        result["cpu_baseline"] = {"value": round(S / dt, 3), "unit": "tokens/s", "cores": threads,
                                  "kind": "oracle",
                                  "sample": f"{S} decode tokens through layer-0 weights (fp64 C oracle, "
                                            f"OpenMP over tokens), {dt:.1f} s wall",
                                  **host_cpu()}
        log(f"cpu oracle: {S / dt:.2f} tok/s on {threads} threads")

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
