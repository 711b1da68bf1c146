"""Bench: achieved HBM GB/s (% of peak) and equivalent decode tok/s of the
block-float quantized GEMV on one MI355X.

Headline workload (one "step"): one decode token, batch 1, through a 64-layer
stack of the dense 30B-class MXFP4 layer -- per layer the fused gate/up GEMV
(51200 x 5120), the down GEMV (5120 x 25600) and the QKV GEMV (7168 x 5120).
Every layer reads its own copy of the weights (64 x 228.4 MB = 14.6 GB
resident in HBM), so the 256 MB last-level cache cannot serve them; the
weight contents are seeded synthetic data (E2M1 codes uniform, E8M0 exponents
uniform in [118, 130], bf16 N(0,1) activations), identical in every layer.

value = weight bytes read per step / step time (GB/s).  The same JSON line
carries: the roofline of the dominant kernel (the gate/up GEMV) measured with
HIP events around each of its launches in an instrumented pass, the batch-4
step, the MoE GEMV (128-expert bank, top-8, 1/2/4 tokens), the MXFP8 / NVFP4
format sweep, the prefill GEMM's MFMA-peak fraction, a plain copy kernel for
reference, and the CPU oracle timed on one layer (cpu_baseline).
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
PEAK_BF16_TFLOPS = 2500.0
LAYERS = 64
MOE_LAYERS = 48


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=30)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--layers", type=int, default=LAYERS)
    p.add_argument("--skip-cpu-baseline", action="store_true")
    p.add_argument("--skip-extras", action="store_true", help="headline step and roofline only")
    p.add_argument("--only", default="", help="comma list of parts: dense,moe,formats,gemm,copy,cpu")
    return p.parse_args()


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: this build measures one GPU only; --gpus {args.gpus} is not supported "
              "(the multi-GPU sharding is a design note, not an implementation).", file=sys.stderr)
        sys.exit(2)

    import torch

    import block_float_quantized_mxq_amd as mxq
    import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    parts = set(args.only.split(",")) if args.only else {"dense", "moe", "formats", "gemm", "copy", "cpu"}
    if args.skip_extras:
        parts &= {"dense", "cpu"}
    if args.skip_cpu_baseline:
        parts.discard("cpu")

    def u8(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    def bf(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    def log(*a):
        print("[bench]", *a, file=sys.stderr, flush=True)

    # ---------------- dense decode layer stack ----------------
    shapes = synth.DENSE_SHAPES
    order = ["gate_up", "down", "qkv"]
    host = {w: synth.dense_layer(w, 4, seed=0) for w in order}
    wbytes = {w: mxq.weight_bytes(mxq.MXFP4, *shapes[w]) for w in order}
    layer_bytes = sum(wbytes.values())
    log(f"uploading {args.layers} layers x {layer_bytes / 1e6:.1f} MB")
    base = {w: (u8(host[w]["codes"]), u8(host[w]["scales"])) for w in order}
    layers = []
    for _ in range(args.layers):
        layers.append({w: (base[w][0].clone(), base[w][1].clone()) for w in order})
    del base
    xs = {b: {w: bf(host[w]["x"][:b]) for w in order} for b in (1, 4)}
    ys = {b: {w: torch.empty((b, shapes[w][0]), dtype=torch.float32, device=dev) for w in order} for b in (1, 4)}
    torch.cuda.synchronize()

    def step(b, instrument=None):
        for L in layers:
            for w in order:
                c, s = L[w]
                if instrument is not None:
                    instrument[w][0].append(torch.cuda.Event(enable_timing=True))
                    instrument[w][0][-1].record(stream)
                mxq.gemv(mxq.MXFP4, c, s, xs[b][w], out=ys[b][w])
                if instrument is not None:
                    instrument[w][1].append(torch.cuda.Event(enable_timing=True))
                    instrument[w][1][-1].record(stream)

    def timed_steps(b):
        for _ in range(args.warmup):
            step(b)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(args.steps):
            step(b)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.steps  # ms per step

    def per_kernel(b, nsteps):
        ins = {w: ([], []) for w in order}
        for _ in range(nsteps):
            step(b, ins)
        torch.cuda.synchronize()
        out = {}
        for w in order:
            d = np.array([a.elapsed_time(z) for a, z in zip(*ins[w])]) * 1e-3  # seconds
            out[w] = dict(us_mean=float(d.mean() * 1e6), us_p50=float(np.median(d) * 1e6),
                          gbs=float(wbytes[w] / d.mean() / 1e9), launches=int(d.size))
            out[w]["pct_peak"] = 100.0 * out[w]["gbs"] / PEAK_HBM_GBS
        return out

    result = {}
    if "dense" in parts:
        ms1 = timed_steps(1)
        kern1 = per_kernel(1, max(2, args.steps // 3))
        ms4 = timed_steps(4)
        kern4 = per_kernel(4, max(2, args.steps // 3))
        step_bytes = layer_bytes * args.layers
        gbs1 = step_bytes / (ms1 * 1e-3) / 1e9
        gbs4 = step_bytes / (ms4 * 1e-3) / 1e9
        result["dense"] = dict(ms1=ms1, gbs1=gbs1, ms4=ms4, gbs4=gbs4, kern1=kern1, kern4=kern4,
                               step_bytes=step_bytes)
        log(f"dense B=1: {ms1:.3f} ms/step, {gbs1:.0f} GB/s ({100 * gbs1 / PEAK_HBM_GBS:.1f}%); "
            f"B=4: {ms4:.3f} ms/step, {gbs4:.0f} GB/s")
        for w in order:
            log(f"  {w}: B1 {kern1[w]['us_mean']:.2f} us {kern1[w]['gbs']:.0f} GB/s | "
                f"B4 {kern4[w]['us_mean']:.2f} us {kern4[w]['gbs']:.0f} GB/s")
    del layers
    torch.cuda.empty_cache()

    extras = {}
    # ---------------- MoE expert-indexed GEMV ----------------
    if "moe" in parts:
        moe = {}
        copies = 4
        for which in ("gate_up", "down"):
            case = synth.moe_layer(which, 1, seed=0)
            banks = [(u8(case["codes"]), u8(case["scales"])) for _ in range(copies)]
            n, k = case["n"], case["k"]
            per_expert = mxq.weight_bytes(mxq.MXFP4, n, k)
            for T in (1, 2, 4):
                _, _, sx, si, _ = synth.streams(100 + T)
                nsets = 64
                idsets = [synth.moe_ids(si, T, 8, 128) for _ in range(nsets)]
                ids_dev = [torch.from_numpy(i).to(dev) for i in idsets]
                active = [len(np.unique(i)) * per_expert for i in idsets]
                x = bf(synth.bf16_normal(sx, (T, 8, k) if which == "down" else (T, k)))
                y = torch.empty((T, 8, n), dtype=torch.float32, device=dev)
                per_slot = 1 if which == "down" else 0
                for i in range(8):
                    mxq.moe_gemv(1, *banks[i % copies], ids_dev[i % nsets], x, per_slot, out=y)
                torch.cuda.synchronize()
                reps = 256
                ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
                tot0, tot1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                tot0.record(stream)
                for i in range(reps):
                    ev[i][0].record(stream)
                    mxq.moe_gemv(1, *banks[i % copies], ids_dev[i % nsets], x, per_slot, out=y)
                    ev[i][1].record(stream)
                tot1.record(stream)
                torch.cuda.synchronize()
                d = np.array([a.elapsed_time(z) for a, z in ev]) * 1e-3
                byts = np.array([active[i % nsets] for i in range(reps)], dtype=np.float64)
                moe[f"{which}_T{T}"] = dict(us_mean=float(d.mean() * 1e6), active_mb_mean=float(byts.mean() / 1e6),
                                            gbs=float(byts.sum() / d.sum() / 1e9),
                                            gbs_incl_gaps=float(byts.sum() / (tot0.elapsed_time(tot1) * 1e-3) / 1e9))
                moe[f"{which}_T{T}"]["pct_peak"] = 100 * moe[f"{which}_T{T}"]["gbs"] / PEAK_HBM_GBS
                log(f"moe {which} T={T}: {d.mean() * 1e6:.2f} us, {moe[f'{which}_T{T}']['gbs']:.0f} GB/s")
            del banks
            torch.cuda.empty_cache()
        for T in (1, 2, 4):
            t_layer = (moe[f"gate_up_T{T}"]["us_mean"] + moe[f"down_T{T}"]["us_mean"]) * 1e-6
            moe[f"equiv_tok_s_T{T}"] = T / (MOE_LAYERS * t_layer)
        extras["moe"] = moe

    # ---------------- format sweep at the down shape ----------------
    if "formats" in parts:
        fm = {}
        for fmt, name, copies in ((mxq.MXFP4, "mxfp4", 16), (mxq.MXFP8, "mxfp8", 8), (mxq.NVFP4, "nvfp4", 16)):
            case = synth.format_sweep(fmt, seed=0)
            w = [(u8(case["codes"]), u8(case["scales"])) for _ in range(copies)]
            g = None if case["g"] is None else torch.from_numpy(case["g"]).to(dev)
            x = bf(case["x"])
            y = torch.empty((1, case["n"]), dtype=torch.float32, device=dev)
            for i in range(copies):
                mxq.gemv(fmt, *w[i], x, g, out=y)
            torch.cuda.synchronize()
            reps = 64
            ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
            for i in range(reps):
                ev[i][0].record(stream)
                mxq.gemv(fmt, *w[i % copies], x, g, out=y)
                ev[i][1].record(stream)
            torch.cuda.synchronize()
            d = np.array([a.elapsed_time(z) for a, z in ev]) * 1e-3
            byts = mxq.weight_bytes(fmt, case["n"], case["k"])
            fm[name] = dict(us_mean=float(d.mean() * 1e6), gbs=float(byts / d.mean() / 1e9), weight_bytes=byts)
            fm[name]["pct_peak"] = 100 * fm[name]["gbs"] / PEAK_HBM_GBS
            log(f"format {name}: {d.mean() * 1e6:.2f} us, {fm[name]['gbs']:.0f} GB/s")
            del w
            torch.cuda.empty_cache()
        extras["formats_down_shape_b1"] = fm

    # ---------------- prefill GEMM ----------------
    if "gemm" in parts:
        c = synth.prefill(seed=0)
        codes, scales, X = u8(c["codes"]), u8(c["scales"]), bf(c["x"])
        Y = torch.empty((c["m"], c["n"]), dtype=torch.bfloat16, device=dev)
        for _ in range(2):
            mxq.gemm(1, codes, scales, X, out=Y)
        torch.cuda.synchronize()
        reps = 10
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for i in range(reps):
            ev[i][0].record(stream)
            mxq.gemm(1, codes, scales, X, out=Y)
            ev[i][1].record(stream)
        torch.cuda.synchronize()
        d = np.array([a.elapsed_time(z) for a, z in ev]) * 1e-3
        flops = 2.0 * c["m"] * c["n"] * c["k"]
        tf = flops / d.mean() / 1e12
        extras["prefill_gemm"] = dict(ms_mean=float(d.mean() * 1e3), tflops=float(tf),
                                      mfma_peak_frac=float(tf / PEAK_BF16_TFLOPS), mfma="bf16 32x32x16",
                                      tok_s=float(c["m"] / d.mean()))
        log(f"gemm: {d.mean() * 1e3:.3f} ms, {tf:.1f} TFLOP/s ({100 * tf / PEAK_BF16_TFLOPS:.1f}% of bf16 peak)")
        del codes, scales, X, Y
        torch.cuda.empty_cache()

    # ---------------- plain copy kernel for reference ----------------
    if "copy" in parts:
        nb = 1 << 30
        src = torch.empty(nb, dtype=torch.uint8, device=dev)
        dst = torch.empty(nb, dtype=torch.uint8, device=dev)
        src.fill_(1)
        for _ in range(2):
            dst.copy_(src)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(10):
            dst.copy_(src)
        e1.record(stream)
        torch.cuda.synchronize()
        t = e0.elapsed_time(e1) * 1e-3 / 10
        extras["copy_1GiB"] = dict(read_plus_write_gbs=float(2 * nb / t / 1e9), us=float(t * 1e6))
        log(f"copy: {2 * nb / t / 1e9:.0f} GB/s read+write")
        del src, dst

    # ---------------- CPU oracle baseline ----------------
    cpu = None
    if "cpu" in parts:
        import oracle

        threads = oracle.num_threads()
        t0 = time.perf_counter()
        for w in order:
            h = host[w]
            oracle.gemv(mxq.MXFP4, h["codes"], h["scales"], None, h["x"][:1], h["n"], h["k"])
        t = time.perf_counter() - t0
        cpu = dict(value=float(layer_bytes / t / 1e9), unit="GB/s", cores=int(threads), kind="oracle",
                   sample="one 30B-class MXFP4 layer at batch 1 (gate/up 51200x5120, down 5120x25600, "
                          f"QKV 7168x5120; {layer_bytes} weight bytes), fp64 accumulation, {t:.2f} s",
                   cpu_model=platform.processor() or platform.machine())
        log(f"cpu oracle: {t:.2f} s for one layer on {threads} threads")

    d = result.get("dense")
    line = {
        "metric": "achieved HBM GB/s (% of peak) + equiv decode tok/s, MXFP4 GEMV/MoE",
        "value": round(d["gbs1"], 1) if d else None,
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(d["ms1"], 4) if d else None,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "mxfp4 weights, bf16 activations, fp32 accumulate",
        "data": "synthetic (seeded: E2M1 codes uniform, E8M0 exponents U[118,130], bf16 N(0,1))",
        "config": {"workload": f"dense 30B-class MXFP4 decode, batch 1, {args.layers} layers x "
                               "(gate/up 51200x5120 + down 5120x25600 + QKV 7168x5120)",
                   "layers": args.layers, "batch": 1, "weight_bytes_per_step": d["step_bytes"] if d else None},
    }
    if d:
        line["pct_of_peak"] = round(100 * d["gbs1"] / PEAK_HBM_GBS, 2)
        line["equiv_decode_tok_s"] = round(1.0 / (d["ms1"] * 1e-3), 1)
        line["batch4"] = dict(ms_per_step=round(d["ms4"], 4), gbs=round(d["gbs4"], 1),
                              pct_of_peak=round(100 * d["gbs4"] / PEAK_HBM_GBS, 2),
                              equiv_decode_tok_s=round(4.0 / (d["ms4"] * 1e-3), 1))
        k1 = d["kern1"]["gate_up"]
        line["roofline"] = dict(bound="hbm", achieved=round(k1["gbs"], 1), peak=PEAK_HBM_GBS, unit="GB/s",
                                frac=round(k1["gbs"] / PEAK_HBM_GBS, 4), traffic=None,
                                kernel="gemv_kernel<MXFP4> gate/up 51200x5120 B=1",
                                algorithmic_bytes_per_launch=wbytes["gate_up"], us_per_launch=round(k1["us_mean"], 3))
        line["kernels_b1"] = {w: {kk: round(v, 3) for kk, v in d["kern1"][w].items()} for w in order}
        line["kernels_b4"] = {w: {kk: round(v, 3) for kk, v in d["kern4"][w].items()} for w in order}
    line["cpu_baseline"] = cpu
    line.update(extras)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
