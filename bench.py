#!/usr/bin/env python3
"""Throughput of the HARP rotated low-bit linear on one MI355X.

Headline (the step ``--steps``/``--warmup`` time): the Llama-2-7B-shaped
decode linear, 4096 -> 4096, batch M = 1, 2-bit group-64 weights, b = 4096
butterflies on both sides, as 192 layers in four stacks of 48 dependent
layers (each layer's input is the previous layer's bf16 output), one
``harp_linear_chain`` launch per stack.  The stack's footprint (1.09 GB) exceeds four times the
256 MB last-level cache, so every weight byte comes from HBM.  All inputs are
resident in HBM before timing starts; the step is captured once in a HIP
graph and replayed.

value = algorithmic bytes of every layer in a step / step time  (GB/s).
Algorithmic bytes per layer = packed weights + fp16 scales/zeros + float32
(cos, sin) pairs of both sides + sign bits + the bf16 input and output rows
(nothing counted for the intermediates).

Also on the same line: the roofline of the dominant kernel (its algorithmic
bytes per launch over its average launch duration, timed with HIP events on
the stream it runs on), the same workload as independent single-layer
``harp_linear_fused`` calls with their per-kernel durations, every other
configuration of the workload set (the Llama-2-7B MLP pair at M = 1 and 16,
the Qwen3-8B-shaped prefill at M = 512, the Llama-70B-shaped slice at M = 1
and 32 with 2/3/4-bit grids), each over its own >= 1 GiB working set, the
int8-angle, mixed-radix and offline-preparation legs, and the float64 oracle
timed on the host cores.

Working sets: every cell builds four distinct seeded instances with the
synthetic generators and fills the rest of its >= 1 GiB with device copies
of them at distinct addresses (identical contents cost the same HBM traffic
and keep host-side generation short).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0            # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 matrix cores, TFLOP/s
WORKING_SET_BYTES = 1 << 30
CHAIN_LAYERS_PER_LAUNCH = 48
DISTINCT = 4                     # seeded instances per cell; the rest are copies

# HBM traffic per launch from two rocprofv3 counter passes (FETCH_SIZE and
# WRITE_SIZE, each scaled by what the counter reads for a 256 MiB device
# copy); None for a kernel changed since its counters were taken.
TRAFFIC_BYTES = {
    "chain_kernel_4096_2bit_M1_48layers": 319692307,   # FETCH 153916.5 KiB, WRITE 4416.3 KiB
    "rotate_in_deq_gemv_2bit": 7006101,                # FETCH 3413.5 KiB, WRITE 16.0 KiB
    "rotate_out_b4096": 590755,                        # FETCH 280.5 KiB, WRITE 16.0 KiB
}


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def side_bytes(d, b, pair_bytes=8):
    """One side's parameters: (cos, sin) pairs (8 bytes, or one int8 code
    plus the two float32 step values) and the sign bits."""
    L = b.bit_length() - 1
    steps = 4 if pair_bytes == 1 else 0
    return pair_bytes * (d // 2) * L + steps + d // 8


def weight_bytes(N, K, bits):
    return N * K * bits // 8 + N * (K // 64) * 4


def alg_bytes(M, N, K, bits, b_v, b_u, x_bytes=2, y_bytes=4, pair_bytes=8):
    return (weight_bytes(N, K, bits) + side_bytes(K, b_v, pair_bytes)
            + side_bytes(N, b_u, pair_bytes) + x_bytes * M * K + y_bytes * M * N)


def gemv_bytes(M, N, K, bits):
    """The product kernel alone: weights, scales/zeros, float32 x~ in, y' out."""
    return weight_bytes(N, K, bits) + 4 * M * K + 4 * M * N


def rotgemv_bytes(M, N, K, bits, b, pair_bytes=8):
    """Input rotation + product in one kernel: weights, scales/zeros, the
    input side's angles and signs, bf16 x in, float32 y' out."""
    return weight_bytes(N, K, bits) + side_bytes(K, b, pair_bytes) + 2 * M * K + 4 * M * N


def rotate_bytes(M, d, b, in_bytes, out_bytes, pair_bytes=8):
    return side_bytes(d, b, pair_bytes) + in_bytes * M * d + out_bytes * M * d


def time_graph(torch, fn, reps, warmup=3):
    """Capture fn() once in a graph; return (ms per replay, graph)."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for _ in range(2):
            fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(reps):
        g.replay()
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / reps, g


class Layer:
    """Device buffers of one layer instance: both sides, the packed weight,
    and per batch size M an input x [M][K] and an output y [M][N]."""

    def __init__(self, V, W, U, xs, ys):
        self.V, self.W, self.U, self.xs, self.ys = V, W, U, xs, ys


def _dev(torch, a):
    import numpy as np
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint32:
        a = a.view(np.int32)
    elif a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).cuda()


def _rotation(torch, H, r, copy=False):
    c = (lambda t: t.clone()) if copy else (lambda t: t)
    if isinstance(r, H.Rotation):
        if r.cs is None:
            return H.Rotation(None, c(r.sign_bits), r.dim, r.block,
                              phi_codes=c(r.phi_codes), phi_step=r.phi_step)
        return H.Rotation(c(r.cs), c(r.sign_bits), r.dim, r.block)
    if r.cs is None:
        return H.Rotation(None, _dev(torch, r.sign_bits), r.dim, r.block,
                          phi_codes=_dev(torch, r.phi_codes), phi_step=r.phi_step)
    return H.Rotation(_dev(torch, r.cs), _dev(torch, r.sign_bits), r.dim, r.block)


def build_layers(torch, H, cfg_name, lin_idx, bits, Ms, count, y_dtype, angles="f32"):
    """count layer instances of one linear of a config: DISTINCT seeded ones
    from the generators, the rest device copies of them."""
    from synth import workloads as S
    cfg = S.CONFIGS[cfg_name]
    lin = cfg.linears[lin_idx]
    base = []
    for i in range(min(DISTINCT, count)):
        li = S.layer_inputs(cfg, lin_idx, bits, Ms[0], inst=i, angles=angles)
        out = S.outlier_channels(lin.K, S.rng_for(cfg.cid, S.T_OUTLIER, lin_idx, i)) \
            if cfg.outliers else None
        xs = {}
        for M in Ms:
            xa = li.x if M == Ms[0] else S.activations(
                M, lin.K, S.rng_for(cfg.cid, S.T_X, lin_idx, i * 1000 + M), cfg.x_dtype, out)
            xs[M] = _dev(torch, xa).view(torch.bfloat16)
        W = H.QWeight(_dev(torch, li.W.words), _dev(torch, li.W.scale), _dev(torch, li.W.zero),
                      lin.N, lin.K, bits)
        base.append((_rotation(torch, H, li.V), W, _rotation(torch, H, li.U), xs))
    layers = []
    for i in range(count):
        V, W, U, xs = base[i % len(base)]
        if i >= len(base):
            V, U = _rotation(torch, H, V, copy=True), _rotation(torch, H, U, copy=True)
            W = H.QWeight(W.qweight.clone(), W.scale.clone(), W.zero.clone(), W.N, W.K, W.bits)
            xs = {M: x.clone() for M, x in xs.items()}
        ys = {M: torch.empty((M, lin.N), dtype=y_dtype, device="cuda") for M in Ms}
        layers.append(Layer(V, W, U, xs, ys))
    torch.cuda.synchronize()
    return lin, layers


def count_for(per_instance):
    return max(DISTINCT, -(-WORKING_SET_BYTES // per_instance))


def fused_cell(torch, H, lin, layers, M, bits, reps=5):
    """Independent harp_linear_fused calls over the cell's instances."""
    ws = torch.zeros(max(256, H.harp_linear_workspace_bytes(M, lin.N, lin.K)),
                     dtype=torch.uint8, device="cuda")
    ms, _ = time_graph(torch, lambda: [H.harp_linear_fused(L.V, L.W, L.U, L.xs[M], L.ys[M], ws)
                                       for L in layers], reps)
    us = ms * 1e3 / len(layers)
    nb = alg_bytes(M, lin.N, lin.K, bits, lin.b_v, lin.b_u)
    out = {"us_per_linear": round(us, 3), "GB_s": round(nb / (us * 1e-6) / 1e9, 1),
           "frac_hbm": round(nb / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
           "TFLOPs": round(2.0 * M * lin.N * lin.K / (us * 1e-6) / 1e12, 2),
           "bytes_per_call": nb, "instances": len(layers)}
    del ws
    return out


def product_cell(torch, H, lin, layers, reps=5):
    """The one-row product alone over the cell's instances, on one float32
    x~: harp_deq_gemv_ws with its workspace (the FP4 x FP8 matrix-core
    product where it applies) and without (the vector-ALU product)."""
    xt = torch.randn((1, lin.K), dtype=torch.float32, device="cuda")
    yp = torch.empty((1, lin.N), dtype=torch.float32, device="cuda")
    nb = gemv_bytes(1, lin.N, lin.K, layers[0].W.bits)
    out = {"alg_bytes": nb, "instances": len(layers)}
    wsb = H.harp_deq_gemv_workspace_bytes(1, lin.N, lin.K)
    ws = torch.zeros(max(256, wsb), dtype=torch.uint8, device="cuda")
    for name, w in (("fp4", ws if wsb else None), ("vector", None)):
        ms, _ = time_graph(torch, lambda: [H.harp_deq_gemv_ws(L.W, xt, yp, w) for L in layers],
                           reps)
        us = ms * 1e3 / len(layers)
        out[f"{name}_us"] = round(us, 3)
        out[f"{name}_GB_s"] = round(nb / (us * 1e-6) / 1e9, 1)
        out[f"{name}_frac_hbm"] = round(nb / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)
    del ws, xt, yp
    return out


def chain_cell(torch, H, lin, layers, M):
    """The layers as stacks of 48 dependent layers, one harp_linear_chain
    launch each: a stack's first layer reads the cell's input x, each next
    one the previous layer's bf16 output.  (With the configs' N(0, 0.02^2)
    weights and no normalisation between layers, activations grow about
    2.7x per layer, so a stack is kept to 48 layers to stay finite.)
    Returns (workspace, stacks, step function)."""
    ws = torch.zeros(H.harp_linear_chain_workspace_bytes(lin.K), dtype=torch.uint8,
                     device="cuda")
    segs = [layers[i:i + CHAIN_LAYERS_PER_LAUNCH]
            for i in range(0, len(layers), CHAIN_LAYERS_PER_LAUNCH)]
    x0 = layers[0].xs[M]

    def step():
        for seg in segs:
            H.harp_linear_chain([(L.V, L.W, L.U, L.ys[M]) for L in seg], x0, ws)

    return ws, segs, step


def cpu_baseline(li, budget_s=12.0):
    """The float64 oracle (unchanged) on the host cores, same layer inputs."""
    import numpy as np
    from oracle import harp_oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    lin, w = li.lin, li.W
    x64 = O.bf16_bits_to_f64(li.x)
    args = (w.words, w.scale.view(np.float16), w.zero.view(np.float16), li.bits,
            li.V.cs, li.V.sign_bits, lin.b_v, li.U.cs, li.U.sign_bits, lin.b_u)
    O.linear(x64, *args)                       # warm
    n, t0 = 0, time.perf_counter()
    while True:
        O.linear(x64, *args)
        n += 1
        el = time.perf_counter() - t0
        if el >= budget_s or n >= 200:
            break
    per = el / n
    b = alg_bytes(li.M, lin.N, lin.K, li.bits, lin.b_v, lin.b_u, y_bytes=2)
    return {"value": round(b / per / 1e9, 4), "unit": "GB/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{n} full oracle linears (unpack, dequant, F_V, matvec, F_U^T) of "
                      f"one 4096x4096 2-bit M=1 layer, {per * 1e3:.1f} ms each, float64 "
                      f"numpy; GB/s over the same per-layer bytes as the headline"}


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--layers", type=int, default=192,
                    help="headline stack depth (a multiple of 32 keeps launches equal)")
    ap.add_argument("--only-headline", action="store_true",
                    help="time the headline stack only (profiling runs)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle baseline")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the other configurations of the workload set")
    ap.add_argument("--configs", default="l7b_mlp,l70b_slice,q8b_prefill",
                    help="comma-separated configurations to run (profiling runs)")
    ap.add_argument("--no-legs", action="store_true",
                    help="skip the int8-angle, mixed-radix and offline-preparation legs")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a plain 256 MiB device copy (the known-size "
                         "reference for the HBM byte counters)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the hot path is a single-GPU kernel "
              "set (the multi-GPU sharding is a design note, not built); run with "
              "--gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    import rotated_bit_amd as H

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)

    # ---------------- headline: the 4096-wide decode stack -----------------
    M, N, K, bits, bv, bu = 1, 4096, 4096, 2, 4096, 4096
    per_layer = alg_bytes(M, N, K, bits, bv, bu, y_bytes=2)
    count = args.layers
    log(f"building {count} layers of 4096x4096 2-bit ({count * per_layer / 1e9:.2f} GB)")
    t0 = time.time()
    lin, layers = build_layers(torch, H, "l7b_decode", 0, bits, (M,), count, torch.bfloat16)
    log(f"  built in {time.time() - t0:.1f} s")
    ws, segs, step = chain_cell(torch, H, lin, layers, M)

    step()
    torch.cuda.synchronize()
    ref = [layers[0].ys[M].clone(), layers[-1].ys[M].clone()]
    _, g = time_graph(torch, step, reps=1, warmup=0)
    for _ in range(args.warmup):
        g.replay()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(args.steps):
        g.replay()
    end.record()
    torch.cuda.synchronize()
    ms_step = start.elapsed_time(end) / args.steps
    for r, L in zip(ref, (layers[0], layers[-1])):
        if not torch.equal(r.view(torch.int16), L.ys[M].view(torch.int16)):
            raise RuntimeError("graph replay differs from eager result")
        if not torch.isfinite(L.ys[M]).all():
            raise RuntimeError("non-finite layer output")
    err = int(ws[4:8].view(torch.int32).item())
    if err:
        raise RuntimeError("a wait inside the chain ran out")
    value = count * per_layer / (ms_step * 1e-3) / 1e9
    us_layer = ms_step * 1e3 / count
    log(f"step: {count} dependent layers in {len(segs)} launches, {ms_step:.3f} ms "
        f"({us_layer:.2f} us per layer, {value:.1f} GB/s)")
    # the step is the chain kernel alone (one launch per 48 layers, nothing
    # else in the graph): its average launch duration is the step time over
    # the launches, timed by the events above on the replay stream
    launch_us = ms_step * 1e3 / len(segs)
    launch_bytes = CHAIN_LAYERS_PER_LAUNCH * per_layer
    dom = "chain_kernel_4096_2bit_M1_48layers"
    achieved = launch_bytes / (launch_us * 1e-6) / 1e9
    roofline = {"bound": "hbm", "kernel": dom, "achieved": round(achieved, 1),
                "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": TRAFFIC_BYTES.get(dom),
                "alg_bytes_per_launch": launch_bytes,
                "us_per_launch": round(launch_us, 2)}

    if args.calibrate_copy:
        src = torch.empty(64 << 20, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log("calibration: 3 x 256 MiB device copies done")
        del src, dst

    headline_cfg = {"workload": "l7b_decode: 4096x4096 2-bit group-64, M=1, b=4096 both "
                                "sides, stacks of 48 dependent layers (harp_linear_chain)",
                    "layers_per_step": count, "launches_per_step": len(segs),
                    "bytes_per_layer": per_layer, "us_per_layer": round(us_layer, 3),
                    "graph": True}

    # the same layers as independent single-layer calls (fused linear)
    fused = None
    kern = {}
    if not args.only_headline:
        for L in layers:
            L.ys[M] = torch.empty((M, N), dtype=torch.float32, device="cuda")
        fused = fused_cell(torch, H, lin, layers, M, bits, reps=max(3, args.steps // 10))
        fused["speedup_chain_vs_fused"] = round(fused["us_per_linear"] / us_layer, 3)
        xt32 = torch.empty((M, K), dtype=torch.float32, device="cuda")
        yp = torch.empty((M, N), dtype=torch.float32, device="cuda")
        reps = max(3, args.steps // 10)
        ms_rg, _ = time_graph(torch, lambda: [H.harp_rotate_in_deq_gemv(L.V, L.W, L.xs[M], yp)
                                              for L in layers], reps)
        ms_ro, _ = time_graph(torch, lambda: [H.harp_rotate_out(L.U, yp, L.ys[M])
                                              for L in layers], reps)
        ms_ri, _ = time_graph(torch, lambda: [H.harp_rotate_in(L.V, L.xs[M], xt32)
                                              for L in layers], reps)
        ms_gv, _ = time_graph(torch, lambda: [H.harp_deq_gemv(L.W, xt32, yp) for L in layers],
                              reps)
        for name, msk, nbytes, launches in (
                ("rotate_in_deq_gemv_2bit", ms_rg, rotgemv_bytes(M, N, K, bits, bv), 1),
                ("rotate_out_b4096", ms_ro, rotate_bytes(M, N, bu, 4, 4), 1),
                ("rotate_in_b4096", ms_ri, rotate_bytes(M, K, bv, 2, 4), 2),
                ("deq_gemv_2bit", ms_gv, gemv_bytes(M, N, K, bits), 1)):
            us = msk * 1e3 / count
            kern[name] = {("us_per_launch" if launches == 1 else "us_per_call"): round(us, 3),
                          "launches_per_call": launches, "alg_bytes": nbytes,
                          "GB_s": round(nbytes / (us * 1e-6) / 1e9, 1),
                          "traffic": TRAFFIC_BYTES.get(name)}
        fused["kernels"] = kern
        log("fused per call: " + json.dumps(fused))
        del xt32, yp
    del layers, ws, g
    torch.cuda.empty_cache()

    # ---------------- the other configurations ------------------------------
    configs = {}
    if not args.no_configs and not args.only_headline:
        wanted = set(args.configs.split(","))
        # Llama-2-7B MLP pair, M = 1 and 16
        mlp = {}
        for li_idx, name in (((0, "up_4096x11008"), (1, "down_11008x4096"))
                             if "l7b_mlp" in wanted else ()):
            from synth import workloads as S
            ln = S.CONFIGS["l7b_mlp"].linears[li_idx]
            cnt = count_for(alg_bytes(16, ln.N, ln.K, 2, ln.b_v, ln.b_u))
            ln, ls = build_layers(torch, H, "l7b_mlp", li_idx, 2, (1, 16), cnt, torch.float32)
            mlp[name] = {f"M{m}": fused_cell(torch, H, ln, ls, m, 2) for m in (1, 16)}
            del ls
            torch.cuda.empty_cache()
        if mlp:
            configs["l7b_mlp_2bit"] = mlp
        log("l7b_mlp: " + json.dumps(mlp))

        # Llama-70B-shaped slice, M = 1 and 32, 2/3/4 bits; the 8192-wide
        # attention projection also as a dependent stack at M = 1
        l70 = {}
        from synth import workloads as S
        for li_idx, name in (((0, "attn_8192x8192"), (1, "up_8192x28672"),
                              (2, "down_28672x8192")) if "l70b_slice" in wanted else ()):
            for b in (2, 3, 4):
                ln = S.CONFIGS["l70b_slice"].linears[li_idx]
                cnt = count_for(alg_bytes(32, ln.N, ln.K, b, ln.b_v, ln.b_u))
                if li_idx == 0:
                    cnt = -(-cnt // CHAIN_LAYERS_PER_LAUNCH) * CHAIN_LAYERS_PER_LAUNCH
                ln, ls = build_layers(torch, H, "l70b_slice", li_idx, b, (1, 32), cnt,
                                      torch.float32)
                cell = {f"M{m}": fused_cell(torch, H, ln, ls, m, b) for m in (1, 32)}
                if li_idx > 0 and b == 2:
                    cell["product_M1"] = product_cell(torch, H, ln, ls)
                if li_idx == 0:
                    for L in ls:
                        L.ys[1] = torch.empty((1, ln.N), dtype=torch.bfloat16, device="cuda")
                    cws, csegs, cstep = chain_cell(torch, H, ln, ls, 1)
                    ms_c, _ = time_graph(torch, cstep, 5)
                    if int(cws[4:8].view(torch.int32).item()):
                        raise RuntimeError("a wait inside the 8192-wide chain ran out")
                    nb = alg_bytes(1, ln.N, ln.K, b, ln.b_v, ln.b_u, y_bytes=2)
                    us = ms_c * 1e3 / len(ls)
                    cell["chain_M1"] = {"us_per_layer": round(us, 3),
                                        "GB_s": round(nb / (us * 1e-6) / 1e9, 1),
                                        "frac_hbm": round(nb / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                                        "layers": len(ls), "launches": len(csegs)}
                    del cws
                l70[f"{name}_{b}bit"] = cell
                log(f"l70b {name} {b}-bit: " + json.dumps(cell))
                del ls
                torch.cuda.empty_cache()
        if l70:
            configs["l70b_slice"] = l70

        # Qwen3-8B-shaped prefill, M = 512, 2 and 4 bits: the GEMM alone (on
        # the rotated bf16 x~) and the whole fused linear
        pre = {}
        for li_idx, lnm in enumerate(("attn_4096x4096", "up_4096x12288", "down_12288x4096")
                                     if "q8b_prefill" in wanted else ()):
            for b in (2, 4):
                ln = S.CONFIGS["q8b_prefill"].linears[li_idx]
                Mp = 512
                cnt = count_for(alg_bytes(Mp, ln.N, ln.K, b, ln.b_v, ln.b_u))
                ln, ls = build_layers(torch, H, "q8b_prefill", li_idx, b, (Mp,), cnt,
                                      torch.float32)
                flops = 2.0 * Mp * ln.N * ln.K
                xt16 = [torch.empty((Mp, ln.K), dtype=torch.bfloat16, device="cuda")
                        for _ in ls]
                for L, xt in zip(ls, xt16):
                    H.harp_rotate_in(L.V, L.xs[Mp], xt)
                gb = H.harp_deq_gemm_workspace_bytes(Mp, ln.N, ln.K)
                gws = torch.zeros(gb, dtype=torch.uint8, device="cuda") if gb else None
                ms_gm, _ = time_graph(torch, lambda: [H.harp_deq_gemm(L.W, xt, L.ys[Mp], gws)
                                                      for L, xt in zip(ls, xt16)], 5)
                us_gm = ms_gm * 1e3 / len(ls)
                cell = fused_cell(torch, H, ln, ls, Mp, b)
                tf_gm = flops / (us_gm * 1e-6) / 1e12
                cell.update({"deq_gemm_us": round(us_gm, 2),
                             "deq_gemm_TFLOPs": round(tf_gm, 1),
                             "deq_gemm_frac_mfma": round(tf_gm / MFMA_BF16_PEAK_TFLOPS, 4),
                             "fused_frac_mfma": round(cell["TFLOPs"] / MFMA_BF16_PEAK_TFLOPS, 4)})
                pre[f"{lnm}_{b}bit"] = cell
                log(f"q8b prefill {lnm} {b}-bit: " + json.dumps(cell))
                del ls, xt16, gws
                torch.cuda.empty_cache()
        if pre:
            configs["q8b_prefill_M512"] = pre

    # ---------------- legs ---------------------------------------------------
    legs = {}
    if not args.no_legs and not args.only_headline:
        import numpy as np
        from synth import workloads as S
        # the headline workload with int8-stored angles, per call
        per8 = alg_bytes(M, N, K, bits, bv, bu, pair_bytes=1)
        ln, ls = build_layers(torch, H, "l7b_decode", 0, bits, (M,), count_for(per8),
                              torch.float32, angles="int8")
        q8 = fused_cell(torch, H, ln, ls, M, bits)
        q8["bytes_per_call"] = per8
        q8["GB_s"] = round(per8 / (q8["us_per_linear"] * 1e-6) / 1e9, 1)
        q8["frac_hbm"] = round(q8["GB_s"] / HBM_PEAK_GBS, 4)
        legs["int8_angles_l7b_decode_fused"] = q8
        log("int8 angles: " + json.dumps(q8))
        del ls
        torch.cuda.empty_cache()

        # mixed radix: blocks expanded inside libharp from learnable
        # parameters (orthogonal: Givens / Cayley times the fixed mixer)
        mixed = {"workload": "full-width mixed-radix sides, blocks from harp_mixed_expand "
                             "(parameters N(0, 0.1^2)), rotations alone and the 5120-wide "
                             "2-bit linear"}

        def expand(radices, seed):
            ms_ = S.mixed_rotation(radices, np.random.default_rng(seed))
            blocks = H.harp_mixed_expand(radices, ms_.params, ms_.gaussians)
            return torch.from_numpy(blocks).cuda(), _dev(torch, ms_.sign_bits)

        for radices in ((8, 8, 8, 5, 2), (8, 8, 4, 43), (8, 8, 8, 8, 3), (8, 8, 8, 8, 7)):
            dim = int(np.prod(radices))
            nblk = sum(dim * b for b in radices)
            base = [expand(radices, s) for s in range(DISTINCT)]
            entry = {}
            for side, Mm, idt, odt in (("in", 1, torch.bfloat16, torch.float32),
                                       ("in", 512, torch.bfloat16, torch.float32),
                                       ("in", 512, torch.bfloat16, torch.bfloat16),
                                       ("out", 1, torch.float32, torch.float32),
                                       ("out", 512, torch.float32, torch.float32)):
                ib, ob = (2 if idt == torch.bfloat16 else 4), (2 if odt == torch.bfloat16 else 4)
                nb = 4 * nblk + dim // 8 + (ib + ob) * Mm * dim
                cnt = count_for(nb)
                Rs = [H.MixedRotation(base[i % DISTINCT][0].clone(),
                                      base[i % DISTINCT][1].clone(), radices) for i in range(cnt)]
                xs = [torch.randn((Mm, dim), device="cuda").to(idt) for _ in range(cnt)]
                outs = [torch.empty((Mm, dim), device="cuda", dtype=odt) for _ in range(cnt)]
                fn = H.harp_rotate_in_mixed if side == "in" else H.harp_rotate_out_mixed
                mws = None
                if odt == torch.bfloat16:
                    mws = torch.empty(H.harp_rotate_mixed_workspace_bytes(dim, Mm, odt),
                                      dtype=torch.uint8, device="cuda")
                ms_m, _ = time_graph(torch, lambda: [fn(R, a, o, mws)
                                                     for R, a, o in zip(Rs, xs, outs)], 3)
                us = ms_m * 1e3 / cnt
                key = f"{side}_M{Mm}" + ("_bf16" if odt == torch.bfloat16 else "")
                entry[f"{key}_us"] = round(us, 2)
                entry[f"{key}_GB_s"] = round(nb / (us * 1e-6) / 1e9, 1)
                del Rs, xs, outs, mws
                torch.cuda.empty_cache()
            mixed["x".join(str(b) for b in radices)] = entry
        radices, mb = (8, 8, 8, 5, 2), 2
        d = int(np.prod(radices))
        nblk = sum(d * b for b in radices)
        base = [expand(radices, s) for s in range(2 * DISTINCT)]
        lin5 = {}
        for Mm in (1, 16):
            nb = weight_bytes(d, d, mb) + 2 * (4 * nblk + d // 8) + 2 * Mm * d + 4 * Mm * d
            cnt = count_for(nb)
            rng = np.random.default_rng(5)
            qw = S.qweight(d, d, mb, rng)
            Wb = H.QWeight(_dev(torch, qw.words), _dev(torch, qw.scale), _dev(torch, qw.zero),
                           d, d, mb)
            inst = []
            for i in range(cnt):
                V = H.MixedRotation(base[(2 * i) % len(base)][0].clone(),
                                    base[(2 * i) % len(base)][1].clone(), radices)
                U = H.MixedRotation(base[(2 * i + 1) % len(base)][0].clone(),
                                    base[(2 * i + 1) % len(base)][1].clone(), radices)
                W = H.QWeight(Wb.qweight.clone(), Wb.scale.clone(), Wb.zero.clone(), d, d, mb)
                x = torch.randn((Mm, d), device="cuda").to(torch.bfloat16)
                inst.append((V, W, U, x, torch.empty((Mm, d), device="cuda")))
            mws = torch.zeros(H.harp_linear_mixed_workspace_bytes(Mm, d, d), dtype=torch.uint8,
                              device="cuda")
            ms_m, _ = time_graph(torch, lambda: [H.harp_linear_fused_mixed(*i, mws)
                                                 for i in inst], 3)
            us = ms_m * 1e3 / cnt
            lin5[f"M{Mm}_us"] = round(us, 2)
            lin5[f"M{Mm}_GB_s"] = round(nb / (us * 1e-6) / 1e9, 1)
            del inst, mws, Wb
            torch.cuda.empty_cache()
        mixed["linear_5120x5120_2bit"] = lin5
        legs["mixed_radix"] = mixed
        log("mixed radix: " + json.dumps(mixed))

        # offline preparation: W' = F_U W F_V^T, then quantize and pack (2-bit)
        prep = {"workload": "dense float32 W 4096x4096 (b=4096 both sides) and 8192x28672 "
                            "(b_V=256, b_U=8192): harp_rotate_weight, harp_quantize_pack 2-bit"}
        for (Np, Kp, bup, bvp) in ((4096, 4096, 4096, 4096), (8192, 28672, 8192, 256)):
            rV = S.rotation(Kp, bvp, np.random.default_rng(1))
            rU = S.rotation(Np, bup, np.random.default_rng(2))
            V = _rotation(torch, H, rV)
            U = _rotation(torch, H, rU)
            W = torch.randn((Np, Kp), device="cuda") * 0.02
            Wp = torch.empty_like(W)
            pws = torch.empty(H.harp_rotate_weight_workspace_bytes(Np, Kp), dtype=torch.uint8,
                              device="cuda")
            qw = torch.empty((Np, Kp * 2 // 32), dtype=torch.int32, device="cuda")
            sc = torch.empty((Np, Kp // 64), dtype=torch.int16, device="cuda")
            zr = torch.empty((Np, Kp // 64), dtype=torch.int16, device="cuda")
            ms_r, _ = time_graph(torch, lambda: H.harp_rotate_weight(V, U, W, Wp, pws), 5)
            ms_q, _ = time_graph(torch, lambda: H.harp_quantize_pack(Wp, 2, qw, sc, zr), 5)
            nrot = 8 * Np * Kp + 8 * (Kp // 2 * (bvp.bit_length() - 1)
                                      + Np // 2 * (bup.bit_length() - 1))
            nq = 4 * Np * Kp + Np * Kp // 4 + Np * (Kp // 64) * 4
            prep[f"{Np}x{Kp}"] = {
                "rotate_weight_us": round(ms_r * 1e3, 1),
                "rotate_weight_GB_s": round(nrot / (ms_r * 1e-3) / 1e9, 1),
                "quantize_pack_us": round(ms_q * 1e3, 1),
                "quantize_pack_GB_s": round(nq / (ms_q * 1e-3) / 1e9, 1)}
            del W, Wp, pws, qw, sc, zr
            torch.cuda.empty_cache()
        legs["offline_prep"] = prep
        log("offline prep: " + json.dumps(prep))

    cpu = None
    if not args.no_cpu:
        from synth import workloads as S
        li0 = S.layer_inputs(S.CONFIGS["l7b_decode"], 0, 2, 1, inst=0)
        cpu = cpu_baseline(li0)
        log("cpu_baseline: " + json.dumps(cpu))

    tok_s = value * 1e9 / 2.135e9   # Llama-2-7B quantized-linear bytes per token
    out = {
        "metric": "rotated 2-bit linear: GB/s & % HBM peak (decode M=1), % MFMA peak (M=512)",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": headline_cfg,
        "frac_hbm": round(value / HBM_PEAK_GBS, 4),
        "tok_s_equiv_llama2_7b_linears": round(tok_s, 1),
        "roofline": roofline,
        "fused_per_call": fused,
        "configs": configs,
        "legs": legs,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
