#!/usr/bin/env python3
"""Throughput of the HARP rotated 2-bit linear on one MI355X.

Default workload: the Llama-2-7B-shaped decode linear, 4096 -> 4096, batch
M = 1, 2-bit group-64 weights, b = 4096 butterflies on both sides, one
``harp_linear_fused`` call per layer.  One step is one pass over a chain of
distinct layer instances whose combined footprint exceeds 1 GiB (four times
the 256 MB last-level cache), captured once in a HIP graph and replayed.
All inputs are resident in HBM before timing starts.

value = algorithmic bytes of every call in a step / step time  (GB/s).
Algorithmic bytes per call = packed weights + fp16 scales/zeros + float32
(cos, sin) pairs + sign bits + bf16 x + float32 y (nothing counted for the
intermediates).

Also reported on the same line: the roofline of the dominant kernel (its
algorithmic bytes / its average launch duration, measured with HIP events on
the stream it runs on), per-kernel launch durations, the M = 512 prefill
matrix-core figure, and the float64 oracle timed on the host cores.
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

# Memory traffic per launch of the decode-chain kernels, from two rocprofv3
# counter passes (FETCH_SIZE x 2.000, WRITE_SIZE x 1.000, the factors a
# 256 MiB device copy gives) on the current kernels; set an entry to None
# when its kernel changes until the counters are taken again.
TRAFFIC_BYTES = {
    "rotate_in_deq_gemv_2bit": 7009280,
    "rotate_out_b4096": 590848,
}
MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 matrix cores, TFLOP/s
WORKING_SET_BYTES = 1 << 30


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def alg_bytes(M, N, K, bits, b_v, b_u, x_bytes=2, y_bytes=4, pair_bytes=8):
    """pair_bytes: 8 for float32 (cos, sin) pairs, 1 for int8-stored angles
    (plus the two float32 steps)."""
    Lv, Lu = b_v.bit_length() - 1, b_u.bit_length() - 1
    steps = 8 if pair_bytes == 1 else 0
    return (N * K * bits // 8 + N * (K // 64) * 4
            + pair_bytes * (K // 2 * Lv + N // 2 * Lu) + steps
            + (K + N) // 8 + x_bytes * M * K + y_bytes * M * N)


def gemv_bytes(M, N, K, bits):
    """The product kernel alone: weights, scales/zeros, float32 x~ in, y' out."""
    return N * K * bits // 8 + N * (K // 64) * 4 + 4 * M * K + 4 * M * N


def rotgemv_bytes(M, N, K, bits, b, pair_bytes=8):
    """Input rotation + product in one kernel: weights, scales/zeros, the
    input side's angles and signs, bf16 x in, float32 y' out."""
    L = b.bit_length() - 1
    steps = 4 if pair_bytes == 1 else 0
    return (N * K * bits // 8 + N * (K // 64) * 4 + pair_bytes * (K // 2) * L + steps
            + K // 8 + 2 * M * K + 4 * M * N)


def rotate_bytes(M, d, b, in_bytes, out_bytes, pair_bytes=8):
    L = b.bit_length() - 1
    steps = 4 if pair_bytes == 1 else 0
    return pair_bytes * (d // 2) * L + steps + d // 8 + in_bytes * M * d + out_bytes * M * d


class Instance:
    """Device buffers of one layer instance (from the seeded generators)."""

    def __init__(self, li, torch, H, y_dtype):
        import numpy as np

        def dev(a):
            a = np.ascontiguousarray(a)
            if a.dtype == np.uint32:
                a = a.view(np.int32)
            elif a.dtype == np.uint16:
                a = a.view(np.int16)
            return torch.from_numpy(a).cuda()

        lin = li.lin
        self.li = li
        def rot(r):
            if r.cs is None:
                return H.Rotation(None, dev(r.sign_bits), r.dim, r.block,
                                  phi_codes=dev(r.phi_codes), phi_step=r.phi_step)
            return H.Rotation(dev(r.cs), dev(r.sign_bits), r.dim, r.block)

        self.V = rot(li.V)
        self.U = rot(li.U)
        self.W = H.QWeight(dev(li.W.words), dev(li.W.scale), dev(li.W.zero),
                           lin.N, lin.K, li.bits)
        self.x = dev(li.x).view(torch.bfloat16)
        self.y = torch.empty((li.M, lin.N), dtype=y_dtype, device="cuda")
        # zero-filled: the GEMM arrival counters in its tail must start at 0
        self.ws = torch.zeros(max(256, H.harp_linear_workspace_bytes(li.M, lin.N, lin.K)),
                              dtype=torch.uint8, device="cuda")
        gb = H.harp_deq_gemm_workspace_bytes(li.M, lin.N, lin.K)
        self.gws = torch.zeros(gb, dtype=torch.uint8, device="cuda") if gb else None
        self.xt32 = torch.empty((li.M, lin.K), dtype=torch.float32, device="cuda")
        self.xt16 = torch.empty((li.M, lin.K), dtype=torch.bfloat16, device="cuda")
        self.yp = torch.empty((li.M, lin.N), dtype=torch.float32, device="cuda")


def make_instances(cfg_name, lin_idx, bits, M, count, torch, H, angles="f32"):
    from synth import workloads as S
    cfg = S.CONFIGS[cfg_name]
    return [Instance(S.layer_inputs(cfg, lin_idx, bits, M, inst=i, angles=angles),
                     torch, H, torch.float32)
            for i in range(count)]


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
    b = alg_bytes(li.M, lin.N, lin.K, li.bits, lin.b_v, lin.b_u)
    return {"value": round(b / per / 1e9, 4), "unit": "GB/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{n} full oracle linears (unpack, dequant, F_V, matvec, F_U^T) "
                      f"of instance 0, {per * 1e3:.1f} ms each, float64 numpy"}


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--instances", type=int, default=0, help="layer instances (0: >= 1 GiB)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle baseline")
    ap.add_argument("--no-prefill", action="store_true", help="skip the M=512 figure")
    ap.add_argument("--no-int8", action="store_true",
                    help="skip the decode leg with int8-stored angles")
    ap.add_argument("--no-batched", action="store_true",
                    help="skip the M=16 batched-decode leg")
    ap.add_argument("--no-prep", action="store_true",
                    help="skip the offline-preparation leg")
    ap.add_argument("--no-mixed", action="store_true",
                    help="skip the mixed-radix rotation leg")
    ap.add_argument("--eager", action="store_true", help="time eager launches, no graph")
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

    M, N, K, bits, bv, bu = 1, 4096, 4096, 2, 4096, 4096
    per_call = alg_bytes(M, N, K, bits, bv, bu)
    count = args.instances or -(-WORKING_SET_BYTES // per_call)
    log(f"building {count} layer instances of 4096x4096 2-bit (>= 1 GiB)")
    t0 = time.time()
    inst = make_instances("l7b_decode", 0, bits, M, count, torch, H)
    torch.cuda.synchronize()
    log(f"  built in {time.time() - t0:.1f} s")

    def step():
        for it in inst:
            H.harp_linear_fused(it.V, it.W, it.U, it.x, it.y, it.ws)

    # eager reference result for the graph check
    step()
    torch.cuda.synchronize()
    ref = [inst[0].y.clone(), inst[-1].y.clone()]

    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    if args.eager:
        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()
        start.record()
        for _ in range(args.steps):
            step()
        end.record()
        torch.cuda.synchronize()
        ms = start.elapsed_time(end) / args.steps
    else:
        # capture once, replay: warmup W, then exactly K timed replays
        _, g = time_graph(torch, step, reps=1, warmup=0)
        for _ in range(args.warmup):
            g.replay()
        torch.cuda.synchronize()
        start.record()
        for _ in range(args.steps):
            g.replay()
        end.record()
        torch.cuda.synchronize()
        ms = start.elapsed_time(end) / args.steps
        for r, it in zip(ref, (inst[0], inst[-1])):
            if not torch.equal(r, it.y):
                raise RuntimeError("graph replay differs from eager result")
    log(f"step: {count} fused linears in {ms:.3f} ms "
        f"({ms * 1e3 / count:.2f} us per linear)")
    value = count * per_call / (ms * 1e-3) / 1e9
    ms_step = ms   # the timed step; the legs below time their own work

    if args.calibrate_copy:
        src = torch.empty(64 << 20, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log("calibration: 3 x 256 MiB device copies done")
        del src, dst

    # Per-kernel launch durations: each kernel alone, a graph of `count`
    # launches on the capture stream, timed with events around the replays.
    # The fused decode call launches rotate_in_deq_gemv then rotate_out; the
    # stand-alone rotate_in and deq_gemv are listed for reference.
    kern = {}
    reps = max(3, args.steps // 10)
    ms_rg, _ = time_graph(torch, lambda: [H.harp_rotate_in_deq_gemv(i.V, i.W, i.x, i.yp)
                                          for i in inst], reps)
    ms_ro, _ = time_graph(torch, lambda: [H.harp_rotate_out(i.U, i.yp, i.y) for i in inst], reps)
    ms_ri, _ = time_graph(torch, lambda: [H.harp_rotate_in(i.V, i.x, i.xt32) for i in inst], reps)
    ms_gv, _ = time_graph(torch, lambda: [H.harp_deq_gemv(i.W, i.xt32, i.yp) for i in inst], reps)
    # (the stand-alone rotate_in of a few rows into float32 at b = 4096 is two
    # launches: sub-blocks, then the last three stages)
    for name, msk, nbytes, in_path, launches in (
            ("rotate_in_deq_gemv_2bit", ms_rg, rotgemv_bytes(M, N, K, bits, bv), True, 1),
            ("rotate_out_b4096", ms_ro, rotate_bytes(M, N, bu, 4, 4), True, 1),
            ("rotate_in_b4096", ms_ri, rotate_bytes(M, K, bv, 2, 4), False, 2),
            ("deq_gemv_2bit", ms_gv, gemv_bytes(M, N, K, bits), False, 1)):
        us = msk * 1e3 / count
        kern[name] = {("us_per_launch" if launches == 1 else "us_per_call"): round(us, 3),
                      "launches_per_call": launches, "alg_bytes": nbytes,
                      "GB_s": round(nbytes / (us * 1e-6) / 1e9, 1), "in_fused_path": in_path}
    log("kernels: " + json.dumps(kern))
    dom = max((k for k in kern if kern[k]["in_fused_path"]),
              key=lambda k: kern[k]["us_per_launch"])
    achieved = kern[dom]["GB_s"]
    roofline = {"bound": "hbm", "kernel": dom, "achieved": achieved,
                "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": TRAFFIC_BYTES.get(dom)}

    # the same decode workload with int8-stored angles
    del inst
    torch.cuda.empty_cache()
    q8 = None
    if not args.no_int8:
        per8 = alg_bytes(M, N, K, bits, bv, bu, pair_bytes=1)
        count8 = args.instances or -(-WORKING_SET_BYTES // per8)
        inst8 = make_instances("l7b_decode", 0, bits, M, count8, torch, H, angles="int8")
        ms8, _ = time_graph(torch, lambda: [H.harp_linear_fused(i.V, i.W, i.U, i.x, i.y, i.ws)
                                            for i in inst8], max(3, args.steps // 4))
        ms8_rg, _ = time_graph(torch, lambda: [H.harp_rotate_in_deq_gemv(i.V, i.W, i.x, i.yp)
                                               for i in inst8], reps)
        ms8_ro, _ = time_graph(torch, lambda: [H.harp_rotate_out(i.U, i.yp, i.y) for i in inst8], reps)
        us8 = ms8 * 1e3 / count8
        q8 = {"workload": "l7b_decode with int8-stored angles (one byte per pair)",
              "instances_per_step": count8, "bytes_per_call": per8,
              "us_per_linear": round(us8, 3),
              "GB_s": round(per8 / (us8 * 1e-6) / 1e9, 2),
              "speedup_vs_f32_pairs": round((ms_step * 1e3 / count) / us8, 3),
              "kernels": {}}
        for name, msk, nbytes in (
                ("rotate_in_deq_gemv_2bit_int8", ms8_rg, rotgemv_bytes(M, N, K, bits, bv, 1)),
                ("rotate_out_b4096_int8", ms8_ro, rotate_bytes(M, N, bu, 4, 4, 1))):
            us = msk * 1e3 / count8
            q8["kernels"][name] = {"us_per_launch": round(us, 3), "alg_bytes": nbytes,
                                   "GB_s": round(nbytes / (us * 1e-6) / 1e9, 1)}
        log("int8 angles: " + json.dumps(q8))
        del inst8
        torch.cuda.empty_cache()

    # batched decode: the Llama-2-7B MLP pair at M = 16 (small-batch
    # matrix-core product)
    batched = None
    if not args.no_batched:
        batched = {"workload": "l7b_mlp: 4096->11008 (b_U=256) and 11008->4096 (b_V=256), "
                               "2-bit, M=16, harp_linear_fused", "linears": {}}
        for li_idx, name in ((0, "up_4096x11008"), (1, "down_11008x4096")):
            bi = make_instances("l7b_mlp", li_idx, 2, 16, 16, torch, H)
            lin = bi[0].li.lin
            for it in bi:
                H.harp_rotate_in(it.V, it.x, it.xt16)
            msf, _ = time_graph(torch, lambda: [H.harp_linear_fused(i.V, i.W, i.U, i.x, i.y, i.ws)
                                                for i in bi], 10)
            msg, _ = time_graph(torch, lambda: [H.harp_deq_gemm(i.W, i.xt16, i.yp) for i in bi], 10)
            usf, usg = msf * 1e3 / len(bi), msg * 1e3 / len(bi)
            nb = alg_bytes(16, lin.N, lin.K, 2, lin.b_v, lin.b_u)
            wb = lin.N * lin.K * 2 // 8 + lin.N * (lin.K // 64) * 4
            batched["linears"][name] = {
                "fused_us": round(usf, 2), "fused_GB_s": round(nb / (usf * 1e-6) / 1e9, 1),
                "deq_gemm_us": round(usg, 2),
                "deq_gemm_TFLOPs": round(2.0 * 16 * lin.N * lin.K / (usg * 1e-6) / 1e12, 1),
                "deq_gemm_weight_GB_s": round(wb / (usg * 1e-6) / 1e9, 1)}
            del bi
            torch.cuda.empty_cache()
        log("batched decode: " + json.dumps(batched))

    # mixed-radix rotation (full-width schedules instead of block-diagonal 256)
    mixed = None
    if not args.no_mixed:
        import numpy as np
        mixed = {"workload": "harp_rotate_in_mixed (bf16 x -> float32 x~, or bf16 x~ for the "
                             "matrix-core product, with its float32 workspace) and "
                             "harp_rotate_out_mixed (float32 -> float32), "
                             "random orthogonal blocks (float32) per stage and group"}
        for radices in ((8, 8, 8, 5, 2), (8, 8, 4, 43), (8, 8, 8, 8, 3), (8, 8, 8, 8, 7)):
            dim = int(np.prod(radices))
            nblk = sum(dim * b for b in radices)
            R = H.MixedRotation(torch.randn(nblk, device="cuda") * 0.1,
                                torch.zeros((dim + 31) // 32, dtype=torch.int32, device="cuda"),
                                radices)
            entry = {}
            legs = [("in", 1, torch.bfloat16, torch.float32),
                    ("in", 512, torch.bfloat16, torch.float32),
                    ("in", 512, torch.bfloat16, torch.bfloat16),
                    ("out", 1, torch.float32, torch.float32),
                    ("out", 512, torch.float32, torch.float32)]
            for side, M, idt, odt in legs:
                xs = [torch.randn((M, dim), device="cuda").to(idt) for _ in range(8)]
                outs = [torch.empty((M, dim), device="cuda", dtype=odt) for _ in range(8)]
                fn = H.harp_rotate_in_mixed if side == "in" else H.harp_rotate_out_mixed
                ws = None
                if odt == torch.bfloat16:   # float32 stages in a workspace, bf16 last stage
                    ws = torch.empty(H.harp_rotate_mixed_workspace_bytes(dim, M, odt),
                                     dtype=torch.uint8, device="cuda")
                ms_m, _ = time_graph(torch, lambda: [fn(R, a, o, ws) for a, o in zip(xs, outs)], 5)
                us = ms_m * 1e3 / 8
                nb = 4 * nblk + dim // 8 + (xs[0].element_size() + outs[0].element_size()) * M * dim
                key = f"{side}_M{M}" + ("_bf16" if odt == torch.bfloat16 else "")
                entry[f"{key}_us"] = round(us, 2)
                entry[f"{key}_GB_s"] = round(nb / (us * 1e-6) / 1e9, 1)
                del xs, outs
            mixed["x".join(str(b) for b in radices)] = entry
            del R
            torch.cuda.empty_cache()
        # the whole linear on a 5120-wide layer (8x8x8x5x2 on both sides), 2-bit
        radices, bits = (8, 8, 8, 5, 2), 2
        d = int(np.prod(radices))
        nblk = sum(d * b for b in radices)
        lin = {}
        for M in (1, 16):
            inst = []
            for _ in range(32):
                V = H.MixedRotation(torch.randn(nblk, device="cuda") * 0.1,
                                    torch.zeros((d + 31) // 32, dtype=torch.int32, device="cuda"),
                                    radices)
                U = H.MixedRotation(torch.randn(nblk, device="cuda") * 0.1,
                                    torch.zeros((d + 31) // 32, dtype=torch.int32, device="cuda"),
                                    radices)
                words = torch.randint(-2**31, 2**31 - 1, (d, d * bits // 32), dtype=torch.int32,
                                      device="cuda")
                sc = torch.full((d, d // 64), 0.01, dtype=torch.float16, device="cuda").view(torch.int16)
                zr = torch.full((d, d // 64), 1.0, dtype=torch.float16, device="cuda").view(torch.int16)
                W = H.QWeight(words, sc, zr, d, d, bits)
                x = torch.randn((M, d), device="cuda").to(torch.bfloat16)
                y = torch.empty((M, d), device="cuda")
                ws = torch.zeros(H.harp_linear_mixed_workspace_bytes(M, d, d), dtype=torch.uint8,
                                 device="cuda")
                inst.append((V, W, U, x, y, ws))
            ms_m, _ = time_graph(torch, lambda: [H.harp_linear_fused_mixed(*i) for i in inst], 5)
            us = ms_m * 1e3 / len(inst)
            nb = d * d * bits // 8 + d * (d // 64) * 4 + 2 * (4 * nblk + d // 8) + 2 * M * d + 4 * M * d
            lin[f"M{M}_us"] = round(us, 2)
            lin[f"M{M}_GB_s"] = round(nb / (us * 1e-6) / 1e9, 1)
            del inst
            torch.cuda.empty_cache()
        mixed["linear_5120x5120_2bit"] = lin
        log("mixed radix: " + json.dumps(mixed))

    # offline preparation: W' = F_U W F_V^T, then quantize and pack (2-bit)
    prep = None
    if not args.no_prep:
        import numpy as np
        from synth import workloads as S
        prep = {"workload": "dense float32 W 4096x4096 (b=4096 both sides) and 8192x28672 "
                            "(b_V=256, b_U=8192): harp_rotate_weight, harp_quantize_pack 2-bit"}
        for (N, K, bu, bv) in ((4096, 4096, 4096, 4096), (8192, 28672, 8192, 256)):
            rV = S.rotation(K, bv, np.random.default_rng(1))
            rU = S.rotation(N, bu, np.random.default_rng(2))
            dv = lambda a: torch.from_numpy(np.ascontiguousarray(a.view(np.int32) if a.dtype == np.uint32 else a)).cuda()
            V = H.Rotation(dv(rV.cs), dv(rV.sign_bits), K, bv)
            U = H.Rotation(dv(rU.cs), dv(rU.sign_bits), N, bu)
            W = torch.randn((N, K), device="cuda") * 0.02
            Wp = torch.empty_like(W)
            ws = torch.empty(H.harp_rotate_weight_workspace_bytes(N, K), dtype=torch.uint8,
                             device="cuda")
            qw = torch.empty((N, K * 2 // 32), dtype=torch.int32, device="cuda")
            sc = torch.empty((N, K // 64), dtype=torch.int16, device="cuda")
            zr = torch.empty((N, K // 64), dtype=torch.int16, device="cuda")
            ms_r, _ = time_graph(torch, lambda: H.harp_rotate_weight(V, U, W, Wp, ws), 5)
            ms_q, _ = time_graph(torch, lambda: H.harp_quantize_pack(Wp, 2, qw, sc, zr), 5)
            nrot = 8 * N * K + 8 * (K // 2 * (bv.bit_length() - 1) + N // 2 * (bu.bit_length() - 1))
            nq = 4 * N * K + N * K // 4 + N * (K // 64) * 4
            prep[f"{N}x{K}"] = {
                "rotate_weight_us": round(ms_r * 1e3, 1),
                "rotate_weight_GB_s": round(nrot / (ms_r * 1e-3) / 1e9, 1),
                "quantize_pack_us": round(ms_q * 1e3, 1),
                "quantize_pack_GB_s": round(nq / (ms_q * 1e-3) / 1e9, 1)}
            del W, Wp, ws, qw, sc, zr
            torch.cuda.empty_cache()
        log("offline prep: " + json.dumps(prep))

    # prefill: M = 512 on the matrix cores, the three linears of the
    # Qwen3-8B-shaped prefill config at 2 and 4 bits; the top-level keys are
    # the 4096 x 4096 2-bit case
    prefill = None
    if not args.no_prefill:
        from synth import workloads as S
        pcfg = S.CONFIGS["q8b_prefill"]
        shapes = {}
        for li_idx, lin in enumerate(pcfg.linears):
            for bits in (2, 4):
                n_pre = 8 if lin.N * lin.K <= 4096 * 4096 else 4
                pre = make_instances("q8b_prefill", li_idx, bits, 512, n_pre, torch, H)
                flops = 2.0 * 512 * lin.N * lin.K
                for it in pre:
                    H.harp_rotate_in(it.V, it.x, it.xt16)
                ms_gm, _ = time_graph(
                    torch, lambda: [H.harp_deq_gemm(i.W, i.xt16, i.yp, i.gws) for i in pre], 10)
                ms_fu, _ = time_graph(
                    torch, lambda: [H.harp_linear_fused(i.V, i.W, i.U, i.x, i.y, i.ws)
                                    for i in pre], 10)
                us_gm, us_fu = ms_gm * 1e3 / len(pre), ms_fu * 1e3 / len(pre)
                tf_gm = flops / (us_gm * 1e-6) / 1e12
                ctx = {}
                if li_idx == 0 and bits == 2:
                    # context, not our path: the vendor library's plain bf16
                    # GEMM on the same x~ with the weights dequantized first
                    wb = [torch.empty((lin.N, lin.K), dtype=torch.bfloat16, device="cuda")
                          for _ in pre]
                    for i, w in zip(pre, wb):
                        H.harp_dequant(i.W, w)
                    ms_lib, _ = time_graph(
                        torch, lambda: [torch.matmul(i.xt16, w.t()) for i, w in zip(pre, wb)], 10)
                    us_lib = ms_lib * 1e3 / len(pre)
                    ctx = {"context_library_bf16_gemm_us": round(us_lib, 2),
                           "context_library_frac_mfma": round(
                               flops / (us_lib * 1e-6) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)}
                    del wb
                shapes[f"{lin.K}x{lin.N}_{bits}bit"] = {
                    "K": lin.K, "N": lin.N, "bits": bits, "b_V": lin.b_v, "b_U": lin.b_u,
                    "deq_gemm_us": round(us_gm, 2),
                    "deq_gemm_TFLOPs": round(tf_gm, 1),
                    "deq_gemm_frac_mfma": round(tf_gm / MFMA_BF16_PEAK_TFLOPS, 4),
                    "fused_us": round(us_fu, 2),
                    "fused_frac_mfma": round(flops / (us_fu * 1e-6) / 1e12
                                             / MFMA_BF16_PEAK_TFLOPS, 4), **ctx}
                del pre
                torch.cuda.empty_cache()
        head = shapes["4096x4096_2bit"]
        prefill = {"workload": "4096x4096 2-bit M=512",
                   "deq_gemm_us": head["deq_gemm_us"],
                   "deq_gemm_TFLOPs": head["deq_gemm_TFLOPs"],
                   "deq_gemm_frac_mfma": head["deq_gemm_frac_mfma"],
                   "fused_us": head["fused_us"],
                   "fused_frac_mfma": head["fused_frac_mfma"],
                   "context_library_bf16_gemm_us": head.get("context_library_bf16_gemm_us"),
                   "context_library_frac_mfma": head.get("context_library_frac_mfma"),
                   "peak_TFLOPs": MFMA_BF16_PEAK_TFLOPS,
                   "shapes": shapes}
        log("prefill: " + json.dumps(prefill))

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
        "config": {"workload": "l7b_decode: 4096x4096 2-bit group-64, M=1, b=4096 both "
                               "sides, harp_linear_fused",
                   "instances_per_step": count, "bytes_per_call": per_call,
                   "graph": not args.eager},
        "frac_hbm": round(value / HBM_PEAK_GBS, 4),
        "tok_s_equiv_llama2_7b_linears": round(tok_s, 1),
        "roofline": roofline,
        "kernels": kern,
        "int8_angles": q8,
        "batched_decode": batched,
        "mixed_radix": mixed,
        "offline_prep": prep,
        "prefill": prefill,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
