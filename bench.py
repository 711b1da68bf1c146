"""Bench: achieved HBM GB/s (% of peak) and equivalent decode tok/s of the
block-float quantized GEMV on one MI355X.

Headline workload (one "step"): one decode token, batch 1, through a 64-layer
stack of the dense 30B-class MXFP4 layer -- per layer the fused gate/up GEMV
(51200 x 5120), the down GEMV (5120 x 25600) and the QKV GEMV (7168 x 5120).
Every layer reads its own copy of the weights (64 x 228.4 MB = 14.6 GB
resident in HBM), so the 256 MB last-level cache cannot serve them; the
weights are seeded synthetic data (E2M1 codes uniform, E8M0 exponents uniform
in [118, 130], bf16 N(0,1) activations), identical in every layer.  The step's
192 launches are captured once in a HIP graph and replayed, so the host's
per-call cost is not part of the measurement.

value = weight bytes read per step / step time (GB/s).  The same JSON line
carries: the roofline of the dominant kernel (the gate/up GEMV: a graph of
back-to-back launches over the 64 distinct copies, timed with HIP events on
the launch stream), the batch-4 step, the MoE GEMV (128-expert bank, top-8,
1/2/4 tokens), the fused MoE decode block (routing, gate/up, SwiGLU, down and
the weighted combine, same bank), the expert-batched MoE prefill GEMM (a
512-token prompt through the same bank), the block-float quantizer on a
51200 x 5120 bf16 matrix, the MXFP8 / NVFP4 format sweep, the prefill GEMM's MFMA-peak
fraction, a plain copy kernel for reference, and the CPU oracle timed on a
bounded sample (cpu_baseline).

--profile-kernel NAME runs one kernel eagerly a few times (no graph, no
timing) so that rocprofv3 can attribute counters to it:
gate_up | down | qkv | copy.
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import platform
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
PEAK_BF16_TFLOPS = 2500.0
LAYERS = 64
MOE_LAYERS = 48
TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "gemv_mxfp4_gate_up_51200x5120_b1_traffic.md")


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--layers", type=int, default=LAYERS)
    p.add_argument("--only", default="", help="comma list of parts: dense,moe,moe_block,formats,gemm,moe_gemm,quantize,copy,cpu")
    p.add_argument("--profile-kernel", default="", help="run one kernel eagerly for rocprofv3")
    return p.parse_args()


def kernel_sources_sha():
    """Hash of the HIP sources: a stored traffic figure is valid only for these."""
    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(ROOT, "block_float_quantized_mxq_amd", "csrc", "*"))):
        with open(f, "rb") as fh:
            h.update(os.path.basename(f).encode())
            h.update(fh.read())
    return h.hexdigest()


def stored_traffic():
    """HBM bytes per gate/up launch from the committed rocprofv3 summary, if it
    was taken on the current kernel sources (else None)."""
    if not os.path.exists(TRAFFIC_PROFILE):
        return None
    text = open(TRAFFIC_PROFILE).read()
    m_sha = re.search(r"source_sha256:\s*([0-9a-f]{64})", text)
    m_val = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m_sha or not m_val or m_sha.group(1) != kernel_sources_sha():
        return None
    return float(m_val.group(1))


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: this build measures one GPU only; --gpus {args.gpus} is not supported "
              "(sharding over several GPUs is a design note, not an implementation).", file=sys.stderr)
        sys.exit(2)

    import torch

    import block_float_quantized_mxq_amd as mxq
    import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    all_parts = {"dense", "moe", "moe_block", "formats", "gemm", "moe_gemm", "quantize", "copy", "cpu"}
    parts = set(args.only.split(",")) if args.only else all_parts

    def u8(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    def bf(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    def log(*a):
        print("[bench]", *a, file=sys.stderr, flush=True)

    def timed_graph(fn, replays):
        """Capture fn() once, replay `replays` times; ms per replay (HIP events on the launch stream)."""
        fn()  # eager warm-up (loads code objects)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn()
        g.replay()
        torch.cuda.synchronize()
        stream = torch.cuda.current_stream()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(replays):
            g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / replays
        del g
        return ms

    # ---------------- dense decode layer stack ----------------
    shapes = synth.DENSE_SHAPES
    order = ["gate_up", "down", "qkv"]
    need_dense = bool(parts & {"dense", "cpu"}) or args.profile_kernel in order
    host = {w: synth.dense_layer(w, 4, seed=0) for w in order} if need_dense else {}
    wbytes = {w: mxq.weight_bytes(mxq.MXFP4, *shapes[w]) for w in order}
    layer_bytes = sum(wbytes.values())

    if args.profile_kernel:
        name = args.profile_kernel
        if name == "copy":
            nb = 1 << 30
            src = torch.full((nb,), 1, dtype=torch.uint8, device=dev)
            dst = torch.empty_like(src)
            for _ in range(5):
                dst.copy_(src)
        else:
            c0, s0 = u8(host[name]["codes"]), u8(host[name]["scales"])
            W = [(c0.clone(), s0.clone()) for _ in range(8)]
            x = bf(host[name]["x"][:1])
            y = torch.empty((1, shapes[name][0]), dtype=torch.float32, device=dev)
            for i in range(16):
                mxq.gemv(mxq.MXFP4, *W[i % 8], x, out=y)
        torch.cuda.synchronize()
        print(json.dumps({"profiled": name}), flush=True)
        return

    result = {}
    if "dense" in parts:
        log(f"uploading {args.layers} layers x {layer_bytes / 1e6:.1f} MB")
        base = {w: (u8(host[w]["codes"]), u8(host[w]["scales"])) for w in order}
        layers = [{w: (base[w][0].clone(), base[w][1].clone()) for w in order} for _ in range(args.layers)]
        del base
        xs = {b: {w: bf(host[w]["x"][:b]) for w in order} for b in (1, 4)}
        ys = {b: {w: torch.empty((b, shapes[w][0]), dtype=torch.float32, device=dev) for w in order} for b in (1, 4)}
        torch.cuda.synchronize()

        def step(b):
            for L in layers:
                for w in order:
                    mxq.gemv(mxq.MXFP4, *L[w], xs[b][w], out=ys[b][w])

        def one_kernel(b, w):
            def fn():
                for L in layers:
                    mxq.gemv(mxq.MXFP4, *L[w], xs[b][w], out=ys[b][w])
            return fn

        dense = {"step_bytes": layer_bytes * args.layers}
        for b in (1, 4):
            # the graph is replayed warmup + steps times; only the last `steps` are timed
            timed_graph(lambda: step(b), max(1, args.warmup))
            ms = timed_graph(lambda: step(b), args.steps)
            dense[f"ms{b}"] = ms
            dense[f"gbs{b}"] = dense["step_bytes"] / (ms * 1e-3) / 1e9
            kern = {}
            for w in order:
                kms = timed_graph(one_kernel(b, w), max(2, args.steps // 4)) / args.layers
                kern[w] = dict(us=kms * 1e3, gbs=wbytes[w] / (kms * 1e-3) / 1e9)
                kern[w]["pct_peak"] = 100.0 * kern[w]["gbs"] / PEAK_HBM_GBS
            dense[f"kern{b}"] = kern
            log(f"dense B={b}: {ms:.3f} ms/step, {dense[f'gbs{b}']:.0f} GB/s "
                f"({100 * dense[f'gbs{b}'] / PEAK_HBM_GBS:.1f}%); " +
                ", ".join(f"{w} {kern[w]['us']:.2f} us {kern[w]['gbs']:.0f} GB/s" for w in order))
        # the captured step must reproduce the eager result bit for bit
        step(1)
        torch.cuda.synchronize()
        eager = ys[1]["gate_up"].clone()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step(1)
        for _ in range(3):
            ys[1]["gate_up"].zero_()
            g.replay()
            torch.cuda.synchronize()
            if not torch.equal(ys[1]["gate_up"], eager):
                raise RuntimeError("graph replay differs from the eager result")
        del g, layers
        torch.cuda.empty_cache()
        result["dense"] = dense

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
                nsets = 32
                idsets = [synth.moe_ids(si, T, 8, 128) for _ in range(nsets)]
                ids_dev = [torch.from_numpy(i).to(dev) for i in idsets]
                active = np.array([len(np.unique(i)) * per_expert for i in idsets], dtype=np.float64)
                x = bf(synth.bf16_normal(sx, (T, 8, k) if which == "down" else (T, k)))
                y = torch.empty((T, 8, n), dtype=torch.float32, device=dev)
                per_slot = 1 if which == "down" else 0

                def fn():
                    for i in range(nsets):
                        mxq.moe_gemv(1, *banks[i % copies], ids_dev[i], x, per_slot, out=y)

                ms = timed_graph(fn, 8)
                us = ms * 1e3 / nsets
                r = dict(us=us, active_mb=float(active.mean() / 1e6), gbs=float(active.mean() / (us * 1e-6) / 1e9))
                r["pct_peak"] = 100 * r["gbs"] / PEAK_HBM_GBS
                moe[f"{which}_T{T}"] = r
                log(f"moe {which} T={T}: {us:.2f} us, {r['active_mb']:.1f} MB active, {r['gbs']:.0f} GB/s")
            del banks
            torch.cuda.empty_cache()
        for T in (1, 2, 4):
            t_layer = (moe[f"gate_up_T{T}"]["us"] + moe[f"down_T{T}"]["us"]) * 1e-6
            moe[f"layer_T{T}"] = dict(
                us=t_layer * 1e6,
                gbs=(moe[f"gate_up_T{T}"]["active_mb"] + moe[f"down_T{T}"]["active_mb"]) * 1e6 / t_layer / 1e9,
                equiv_tok_s=T / (MOE_LAYERS * t_layer))
        extras["moe"] = {k: {kk: round(v, 3) for kk, v in d.items()} for k, d in moe.items()}

    # ---------------- MoE decode block: routing -> gate/up -> SwiGLU -> down -> combine ----------------
    if "moe_block" in parts:
        mb = {}
        copies = 4
        gu_case = synth.moe_layer("gate_up", 1, seed=0)
        dn_case = synth.moe_layer("down", 1, seed=0)
        gu = [(u8(gu_case["codes"]), u8(gu_case["scales"])) for _ in range(copies)]
        dn = [(u8(dn_case["codes"]), u8(dn_case["scales"])) for _ in range(copies)]
        per_expert = mxq.weight_bytes(mxq.MXFP4, 1536, 2048) + mxq.weight_bytes(mxq.MXFP4, 2048, 768)
        for T in (1, 2, 4):
            _, _, sx, si, _ = synth.streams(200 + T)
            nsets = 32
            logits = [torch.from_numpy(synth.router_logits(si, T, 128)).to(dev) for _ in range(nsets)]
            x = bf(synth.bf16_normal(sx, (T, 2048)))
            ids = torch.empty((T, 8), dtype=torch.int32, device=dev)
            wts = torch.empty((T, 8), dtype=torch.float32, device=dev)
            h = torch.empty((T, 8, 1536), dtype=torch.float32, device=dev)
            y = torch.empty((T, 2048), dtype=torch.float32, device=dev)
            active = []
            for lg in logits:  # union of routed experts per set (for the byte count only)
                i, _ = mxq.moe_route(lg, 8, True)
                active.append(len(np.unique(i.cpu().numpy())) * per_expert)
            active = float(np.mean(active))

            def fn():
                for i in range(nsets):
                    mxq.moe_route(logits[i], 8, True, ids=ids, weights=wts)
                    mxq.moe_block(1, *gu[i % copies], *dn[i % copies], ids, wts, x, h=h, out=y)

            us = timed_graph(fn, 8) * 1e3 / nsets
            mb[f"T{T}"] = dict(us=round(us, 3), active_mb=round(active / 1e6, 3), gbs=round(active / (us * 1e-6) / 1e9, 1),
                               pct_peak=round(100 * active / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 2),
                               equiv_tok_s=round(T / (MOE_LAYERS * us * 1e-6), 1))
            log(f"moe block T={T}: {us:.2f} us (route + gate/up + SwiGLU/down/combine), {active / 1e6:.1f} MB active, "
                f"{mb[f'T{T}']['gbs']:.0f} GB/s")
        del gu, dn
        torch.cuda.empty_cache()
        extras["moe_block"] = mb

    # ---------------- format sweep at the down shape ----------------
    if "formats" in parts:
        fm = {}
        for fmt, name in ((mxq.MXFP4, "mxfp4"), (mxq.MXFP8, "mxfp8"), (mxq.NVFP4, "nvfp4")):
            case = synth.format_sweep(fmt, seed=0)
            byts = mxq.weight_bytes(fmt, case["n"], case["k"])
            copies = max(2, int(np.ceil(1.2e9 / byts)))
            c0, s0 = u8(case["codes"]), u8(case["scales"])
            w = [(c0.clone(), s0.clone()) for _ in range(copies)]
            g = None if case["g"] is None else torch.from_numpy(case["g"]).to(dev)
            x = bf(case["x"])
            y = torch.empty((1, case["n"]), dtype=torch.float32, device=dev)

            def fn():
                for i in range(copies):
                    mxq.gemv(fmt, *w[i], x, g, out=y)

            us = timed_graph(fn, 4) * 1e3 / copies
            fm[name] = dict(us=round(us, 3), gbs=round(byts / us / 1e3, 1), weight_bytes=byts,
                            pct_peak=round(100 * byts / us / 1e3 / PEAK_HBM_GBS, 2))
            log(f"format {name}: {us:.2f} us, {fm[name]['gbs']:.0f} GB/s")
            del w, c0, s0
            torch.cuda.empty_cache()
        extras["formats_down_shape_b1"] = fm

    # ---------------- prefill GEMM ----------------
    if "gemm" in parts:
        c = synth.prefill(seed=0)
        codes, scales, X = u8(c["codes"]), u8(c["scales"]), bf(c["x"])
        Y = torch.empty((c["m"], c["n"]), dtype=torch.bfloat16, device=dev)
        ms = timed_graph(lambda: mxq.gemm(1, codes, scales, X, out=Y), 10)
        flops = 2.0 * c["m"] * c["n"] * c["k"]
        tf = flops / (ms * 1e-3) / 1e12
        extras["prefill_gemm"] = dict(ms=round(ms, 4), tflops=round(tf, 1), mfma_peak_frac=round(tf / PEAK_BF16_TFLOPS, 4),
                                      mfma="bf16 32x32x16, bf16 peak 2500 TFLOP/s",
                                      prefill_tok_s=round(c["m"] / (ms * 1e-3), 1))
        log(f"gemm: {ms:.3f} ms, {tf:.1f} TFLOP/s ({100 * tf / PEAK_BF16_TFLOPS:.1f}% of bf16 peak)")
        del codes, scales, X, Y
        torch.cuda.empty_cache()

    # ---------------- expert-batched MoE prefill GEMM ----------------
    if "moe_gemm" in parts:
        mg = {}
        P = 512  # prompt tokens
        for which in ("gate_up", "down"):
            case = synth.moe_layer(which, 1, seed=0)
            codes, scales = u8(case["codes"]), u8(case["scales"])
            n, k = case["n"], case["k"]
            _, _, sx, si, _ = synth.streams(300)
            ids = torch.from_numpy(synth.moe_ids(si, P, 8, 128)).to(dev)
            per = 1 if which == "down" else 0
            x = bf(synth.bf16_normal(sx, (P, 8, k) if per else (P, k)))
            y = torch.empty((P, 8, n), dtype=torch.bfloat16, device=dev)
            ws = torch.empty((128 + 1 + P * 8,), dtype=torch.int32, device=dev)
            ms = timed_graph(lambda: mxq.moe_gemm(1, codes, scales, ids, x, per, out=y, workspace=ws), 10)
            flops = 2.0 * P * 8 * n * k
            tf = flops / (ms * 1e-3) / 1e12
            mg[which] = dict(us=round(ms * 1e3, 2), tflops=round(tf, 1), mfma_peak_frac=round(tf / PEAK_BF16_TFLOPS, 4))
            log(f"moe gemm {which} {P} tokens x top-8: {ms * 1e3:.1f} us, {tf:.1f} TFLOP/s")
            del codes, scales
            torch.cuda.empty_cache()
        t_layer = (mg["gate_up"]["us"] + mg["down"]["us"]) * 1e-6
        mg["layer"] = dict(us=round(t_layer * 1e6, 2), prefill_tok_s=round(P / (MOE_LAYERS * t_layer), 1),
                           note=f"{P}-token prompt, expert FFN of {MOE_LAYERS} layers (gate/up + down GEMMs only)")
        extras["moe_prefill_gemm"] = mg

    # ---------------- block-float quantizer ----------------
    if "quantize" in parts:
        qz = {}
        rows, k = 51200, 5120
        xq = torch.randn(rows, k, device=dev, generator=torch.Generator(device=dev).manual_seed(0)).to(torch.bfloat16)
        gq = torch.tensor([1.0 / 2688.0], dtype=torch.float32, device=dev)
        for fmt, name in ((mxq.MXFP4, "mxfp4"), (mxq.MXFP8, "mxfp8"), (mxq.NVFP4, "nvfp4")):
            cq, sq = mxq.quantize(fmt, xq, gq if fmt == mxq.NVFP4 else None)
            ms = timed_graph(lambda: mxq.quantize(fmt, xq, gq if fmt == mxq.NVFP4 else None, codes=cq, scales=sq), 10)
            byts = rows * k * 2 + mxq.weight_bytes(fmt, rows, k)
            qz[name] = dict(us=round(ms * 1e3, 2), gbs=round(byts / (ms * 1e-3) / 1e9, 1),
                            pct_peak=round(100 * byts / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 2), bytes=byts)
            log(f"quantize {name} {rows}x{k}: {ms * 1e3:.1f} us, {qz[name]['gbs']:.0f} GB/s (bf16 in + codes/scales out)")
        del xq
        torch.cuda.empty_cache()
        extras["quantize_51200x5120"] = qz

    # ---------------- plain copy kernel for reference ----------------
    if "copy" in parts:
        nb = 1 << 30
        src = torch.full((nb,), 1, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        ms = timed_graph(lambda: dst.copy_(src), 10)
        extras["copy_1GiB"] = dict(read_plus_write_gbs=round(2 * nb / (ms * 1e-3) / 1e9, 1), us=round(ms * 1e3, 2))
        log(f"copy: {2 * nb / (ms * 1e-3) / 1e9:.0f} GB/s read+write")
        del src, dst

    # ---------------- CPU oracle baseline ----------------
    cpu = None
    if "cpu" in parts:
        import oracle

        threads = oracle.num_threads()
        passes, t_all = 0, 0.0
        while t_all < 10.0 and passes < 50:
            t0 = time.perf_counter()
            for w in order:
                h = host[w]
                oracle.gemv(mxq.MXFP4, h["codes"], h["scales"], None, h["x"][:1], h["n"], h["k"])
            t_all += time.perf_counter() - t0
            passes += 1
        cpu = dict(value=round(layer_bytes * passes / t_all / 1e9, 4), unit="GB/s", cores=int(threads), kind="oracle",
                   sample=f"{passes} passes of the CPU oracle over one 30B-class MXFP4 layer at batch 1 "
                          f"(gate/up 51200x5120, down 5120x25600, QKV 7168x5120; {layer_bytes} weight bytes each), "
                          f"fp64 accumulation, {t_all:.1f} s",
                   cpu=platform.processor() or platform.machine())
        log(f"cpu oracle: {passes} layer passes in {t_all:.2f} s on {threads} threads")

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
        "dtype": "f32",
        "data": "synthetic (seeded: E2M1 codes uniform, E8M0 exponents U[118,130], bf16 N(0,1) activations)",
        "config": {"workload": f"dense 30B-class MXFP4 decode step, batch 1: {args.layers} layers x "
                               "(gate/up 51200x5120 + down 5120x25600 + QKV 7168x5120 GEMV)",
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
                                frac=round(k1["gbs"] / PEAK_HBM_GBS, 4), traffic=stored_traffic(),
                                kernel="gemv_rows_kernel, MXFP4 gate/up 51200x5120, batch 1",
                                algorithmic_bytes_per_launch=wbytes["gate_up"], us_per_launch=round(k1["us"], 3))
        line["kernels_b1"] = {w: {kk: round(v, 3) for kk, v in d["kern1"][w].items()} for w in order}
        line["kernels_b4"] = {w: {kk: round(v, 3) for kk, v in d["kern4"][w].items()} for w in order}
    line["cpu_baseline"] = cpu
    line.update(extras)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
