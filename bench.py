#!/usr/bin/env python3
"""Benchmark of the GGUF quantized matmul hot path on one MI355X.

Workload (one "step" = one pass of the whole path over one batch): the
HBM-resident scale-up, 8 stacked layers of W 14336x4096 (N(0,0.02), seeded),
each quantized to Q8_0 and to Q4_K (~499 MB and ~264 MB of blocks), activations
x 512x4096 N(0,1).  Per step, for both formats and both modes (a: f32
activations, b: quantized activations):
  * decode: M = 1 and M = 8 (the GEMV kernel), rotating over the 8 layers;
  * prefill: M = 512 (the GEMM kernel), rotating over the 8 layers.

value = effective weight GB/s of the decode phase (weight bytes streamed /
decode time), the headline metric's first part; the prefill TOPS (useful
2*M*N*K per second) is reported beside it.  Every timing comes from HIP events
recorded on the stream the kernels run on, with inputs resident in HBM.

CPU baseline: the CPU oracle (plain C, f64/int64) timed on the decode phase
of the same step (M = 1 and 8, both formats and modes, all 8 layers) on the
host's threads, reported in the same unit.

Context, outside the step and the value: the dequantize-all form (weights
decoded to f32 once, then the library f32 GEMM), timed on the same layers and
M, as the page "同一个 GGUF，CPU 和 Metal 生成的文字不一样" (section 修法)
compares it with the quantized forms; and the decode (M = 1 and 8, both
modes) of the same layers in the other formats of the pages' files (Q4_0,
Q5_0, Q6_K: the page "自己量化" quantizes to Q4_0 and falls back to Q5_0, the
downloaded file holds Q6K tensors).
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "quantized GEMV effective weight GB/s (% of 8 TB/s) + prefill GEMM TOPS (% MFMA peak)"
PEAK_HBM_GBS = 8000.0
PEAK_F16_TFLOPS = 2500.0
PEAK_I8_TOPS = 5000.0
N, K, LAYERS, M_PREFILL = 14336, 4096, 8, 512
DECODE_M = (1, 8)


def parse():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-layers", type=int, default=LAYERS, help="layers in the CPU-baseline sample")
    p.add_argument("--no-dequant", action="store_true", help="skip the dequantize-all context rows")
    p.add_argument("--no-other-formats", action="store_true", help="skip the Q4_0/Q5_0/Q6_K decode context rows")
    p.add_argument("--workload", default="c5", choices=["c1", "c2", "c3", "c4", "c5", "c6"],
                   help="c5 (default): the step above.  c1-c4: the pages' smaller workloads as context lines "
                        "(q_proj GEMV, lm_head GEMV warm and cold, ffn_down Q4_K at M=1 and 37, the 30-layer "
                        "SmolLM2 prefill at M=307 on a stream and as a HIP graph).  c6: the step's layers in "
                        "the other formats of the pages' files (Q4_0, Q5_0, Q6_K)")
    p.add_argument("--only", default="", help="restrict the step to one part, e.g. gemv:q8_0:b:1 or gemm:q4_k:a "
                                              "(for profiling one kernel); 'copy' times a plain 512 MiB device copy "
                                              "instead (the calibration for the HBM byte counters)")
    return p.parse_args()


CSRC = os.path.join(ROOT, "block_quantized_matmul_gguf_amd", "csrc")


def kernel_sources(main):
    """The source file `main` (under csrc/) and every csrc header it includes, directly or not."""
    seen, todo = set(), [main]
    while todo:
        name = todo.pop()
        if name in seen or not os.path.isfile(os.path.join(CSRC, name)):
            continue
        seen.add(name)
        with open(os.path.join(CSRC, name)) as f:
            for line in f:
                line = line.strip()
                if line.startswith("#include \""):
                    todo.append(line.split("\"")[1])
    return sorted(seen)


def kernel_source_hash(main):
    """Hash of the sources that build the kernels of `main` (its text and its headers')."""
    h = hashlib.sha256()
    for name in kernel_sources(main):
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def traffic_from_profile(key):
    """HBM bytes per launch from the committed counter summary, if it was taken
    on the current sources of that kernel (each entry names its source file and
    the hash of it and its headers); else None."""
    path = os.path.join(ROOT, "profiles", "counters.json")
    try:
        with open(path) as f:
            data = json.load(f)
    except (OSError, ValueError):
        return None
    entry = data.get("kernels", {}).get(key)
    if not entry or not entry.get("source") or entry.get("source_hash") != kernel_source_hash(entry["source"]):
        return None
    return entry.get("hbm_bytes_per_launch")


def cpu_baseline(layers, min_seconds=10.0, threads=None):
    """The oracle on the decode phase of the step (M = 1 and 8, both formats,
    both modes) over the first `layers` layers, on `threads` host threads (all
    by default); the phase is repeated until at least `min_seconds` of oracle
    time have been measured."""
    import oracle
    import synth

    want = threads or int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    threads = oracle.set_threads(min(want, os.cpu_count() or 1))
    x = synth.acts_f32(5100, M_PREFILL, K)
    wqs = []
    for layer in range(layers):
        w = synth.weights_f32(5000 + layer, N, K)
        wqs.append([(fmt, oracle.quantize(fmt, w)) for fmt in (oracle.Q8_0, oracle.Q4_K)])
        del w
    total_bytes, total_s, reps = 0, 0.0, 0
    while total_s < min_seconds and reps < 64:
        for per_layer in wqs:
            for fmt, wq in per_layer:
                for fn in (oracle.matmul_a, oracle.matmul_b):
                    for m in DECODE_M:
                        t0 = time.perf_counter()
                        fn(fmt, wq, N, K, x[:m])
                        total_s += time.perf_counter() - t0
                        total_bytes += wq.nbytes
        reps += 1
    return {
        "value": round(total_bytes / total_s / 1e9, 3),
        "unit": "GB/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"decode phase of the step on {layers} of {LAYERS} layers (M=1 and M=8, Q8_0 and Q4_K, "
                  f"modes a and b, N=14336 K=4096), repeated {reps} times: {total_bytes / 1e9:.2f} GB of weight "
                  f"blocks in {total_s:.1f} s",
    }


def timed_rows(qmm, torch, runs, stream, args):
    """[(label, fn)] -> per-call microseconds from HIP events on the launch
    stream, each fn one launch-group of `n` calls: fn() returns n."""
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    out = []
    for label, fn in runs:
        for _ in range(max(1, args.warmup)):
            fn()
        torch.cuda.synchronize()
        ev[0].record(stream)
        calls = 0
        for _ in range(args.steps):
            calls += fn()
        ev[1].record(stream)
        torch.cuda.synchronize()
        out.append((label, ev[0].elapsed_time(ev[1]) * 1000.0 / calls))
    return out


def q4k_sixteen_layers(qmm, torch, synth, wq8, modes, xs, ys, stream, args):
    """Decode (M = 1 and 8, both modes) over 16 stacked 14336x4096 Q4_K layers
    (528 MB of blocks, twice the Infinity Cache): the step's 8 layers plus 8
    more seeded the same way, rotated per launch so the weights stream from
    HBM.  Outside the step and its value."""
    dev = xs[1].device
    layers = list(wq8)
    for layer in range(LAYERS, 2 * LAYERS):
        wf = torch.from_numpy(synth.weights_f32(5000 + layer, N, K)).to(dev)
        layers.append(qmm.quantize_weights(qmm.Q4_K, wf))
        del wf
    b = layers[0].numel()
    rows = []
    for md, mcode in modes.items():
        with qmm.Plan(qmm.Q4_K, N, K, max(DECODE_M), mcode) as plan:
            def fn(m):
                def run():
                    for w in layers:
                        plan.run(w, xs[m], ys[m], stream)
                    return len(layers)
                return run
            for (label, us) in timed_rows(qmm, torch, [(m, fn(m)) for m in DECODE_M], stream, args):
                rows.append({"mode": md, "M": label, "us_per_launch": round(us, 3),
                             "weight_GBps": round(b / (us * 1e-6) / 1e9, 1),
                             "frac_hbm": round(b / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)})
    del layers
    torch.cuda.synchronize()
    return {"layers": 2 * LAYERS, "bytes": b * 2 * LAYERS, "rows": rows}


def one_gpu_share(qmm, torch, wq, fmts, modes, xs, ys, stream, args, shards=8):
    """The kernel on one GPU's share of the scale-up when its output rows are
    split over 8 GPUs: N = 14336/8 = 1792, K = 4096.  The 8 row shards of each
    of the step's 8 layers (64 shards, the whole 499 / 264 MB) are rotated per
    launch, so the weights stream from HBM.  Decode M = 1 and 8, prefill
    M = 512, both formats and modes.  Outside the step and its value."""
    ns = N // shards
    rows = []
    for f, code in fmts.items():
        rb = wq[f][0].numel() // N
        views = [w[i * ns:(i + 1) * ns] for w in wq[f] for i in range(shards)]  # [ns, row bytes] row shards
        b = ns * rb
        ysh = {m: ys[m][:, :ns].contiguous() for m in ys}
        for md, mcode in modes.items():
            with qmm.Plan(code, ns, K, M_PREFILL, mcode) as plan:
                def fn(m):
                    def run():
                        sel = views if m <= 8 else views[::shards]  # prefill: one shard per layer
                        for w in sel:
                            plan.run(w, xs[m], ysh[m], stream)
                        return len(sel)
                    return run
                for (m, us) in timed_rows(qmm, torch, [(m, fn(m)) for m in DECODE_M + (M_PREFILL,)], stream, args):
                    r = {"fmt": f, "mode": md, "M": m, "us_per_launch": round(us, 3)}
                    if m <= 8:
                        r["weight_GBps"] = round(b / (us * 1e-6) / 1e9, 1)
                        r["frac_hbm"] = round(b / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)
                    else:
                        r["TOPS"] = round(2.0 * m * ns * K / (us * 1e-6) / 1e12, 1)
                    rows.append(r)
    return {"N": ns, "K": K, "shards_rotated": len(wq["q8_0"]) * shards, "rows": rows}


def other_formats_decode(qmm, torch, wq, others, modes, xs, ys, stream, args):
    """Decode (M = 1 and 8) of the same 8 layers in Q4_0, Q5_0 and Q6_K (the
    other formats of the pages' files), both modes, layers rotated (HBM
    streams), HIP events on the launch stream; per launch = group time /
    launches.  Context beside the step, not part of its value."""
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    rows = []
    for f, code in others.items():
        b = wq[f][0].numel()
        for md, mcode in modes.items():
            with qmm.Plan(code, N, K, max(DECODE_M), mcode) as plan:
                for m in DECODE_M:
                    for _ in range(max(1, args.warmup)):
                        for l in range(LAYERS):
                            plan.run(wq[f][l], xs[m], ys[m], stream)
                    torch.cuda.synchronize()
                    ev[0].record(stream)
                    for _ in range(args.steps):
                        for l in range(LAYERS):
                            plan.run(wq[f][l], xs[m], ys[m], stream)
                    ev[1].record(stream)
                    torch.cuda.synchronize()
                    us = ev[0].elapsed_time(ev[1]) * 1000.0 / (args.steps * LAYERS)
                    rows.append({"fmt": f, "mode": md, "M": m, "us_per_launch": round(us, 3),
                                 "weight_GBps": round(b / (us * 1e-6) / 1e9, 1),
                                 "frac_hbm": round(b / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)})
    return {"layer_bytes": {f: wq[f][0].numel() for f in others}, "rows": rows}


def dequant_context(qmm, torch, wq, xs, ys, fmts, stream, args):
    """The dequantize-all form on the step's layers: the one-time decode of
    each layer to f32, then y = x . W^T with the f32 weights for M = 1, 8 and
    512 (HIP events on the launch stream, per launch = group time / layers)."""
    out = {}
    for f, code in fmts.items():
        plan = qmm.Plan(code, N, K, M_PREFILL, qmm.MODE_DEQUANT)
        wf = [torch.empty((N, K), dtype=torch.float32, device=xs[1].device) for _ in range(LAYERS)]
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]

        def timed(fn):
            for _ in range(max(1, args.warmup)):
                fn()
            torch.cuda.synchronize()
            ev[0].record(stream)
            for _ in range(args.steps):
                fn()
            ev[1].record(stream)
            torch.cuda.synchronize()
            return ev[0].elapsed_time(ev[1]) * 1000.0 / (args.steps * LAYERS)

        row = {"dequantize_us_per_layer": round(timed(lambda: [qmm.dequantize_weights(code, wq[f][l], N, K, wf[l], stream)
                                                               for l in range(LAYERS)]), 2)}
        f32_bytes = N * K * 4
        for m in DECODE_M + (M_PREFILL,):
            us = timed(lambda: [plan.run_dequantized(wf[l], xs[m], ys[m], stream) for l in range(LAYERS)])
            r = {"us_per_launch": round(us, 3)}
            if m in DECODE_M:
                r["f32_weight_GBps"] = round(f32_bytes / (us * 1e-6) / 1e9, 1)
            else:
                r["TFLOPS"] = round(2.0 * m * N * K / (us * 1e-6) / 1e12, 1)
            row[f"M={m}"] = r
        out[f] = row
        plan.close()
        del wf
        torch.cuda.synchronize()
    return out


def small_workload(args, qmm, torch, synth, stream):
    """One JSON line for c1-c4: per-launch times from HIP events on the launch
    stream (no weight rotation: these shapes live in the L2 or Infinity Cache,
    as the line says), c2 also cold (a 512 MiB write between launches), c4 the
    whole 211-projection prefill pass on a stream and replayed as a HIP graph
    (every replay checked bit-for-bit against the stream pass first)."""
    import numpy as np
    dev = torch.device("cuda:0")
    modes = {"a": qmm.MODE_F32ACT, "b": qmm.MODE_QACT}
    fmt_code = {"q8_0": qmm.Q8_0, "q4_k": qmm.Q4_K, "q5_0": qmm.Q5_0}
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]

    def timed(fn, reps):
        for _ in range(max(3, args.warmup)):
            fn()
        torch.cuda.synchronize()
        ev[0].record(stream)
        for _ in range(reps):
            fn()
        ev[1].record(stream)
        torch.cuda.synchronize()
        return ev[0].elapsed_time(ev[1]) * 1000.0 / reps  # us

    def weights(prob, fmt):
        return qmm.quantize_weights(fmt_code[fmt], torch.from_numpy(prob.weights()).to(dev))

    rows = []
    wl = args.workload
    if wl in ("c1", "c2", "c3"):
        probs = {"c1": [("q8_0", synth.c1_q_proj())], "c2": [("q8_0", synth.c2_lm_head())],
                 "c3": [("q4_k", synth.c3_ffn_down(1)), ("q4_k", synth.c3_ffn_down(37))]}[wl]
        flush = torch.empty(128 * 2 ** 20, dtype=torch.float32, device=dev) if wl == "c2" else None
        for fmt, prob in probs:
            w = weights(prob, fmt)
            x = torch.from_numpy(prob.acts()).to(dev)
            y = torch.empty((prob.m, prob.n), dtype=torch.float32, device=dev)
            for md, mcode in modes.items():
                with qmm.Plan(fmt_code[fmt], prob.n, prob.k, prob.m, mcode) as plan:
                    us = timed(lambda: plan.run(w, x, y, stream), 1000 if prob.m <= 8 else 200)
                    r = {"problem": prob.name, "fmt": fmt, "mode": md, "M": prob.m, "us_per_launch": round(us, 3),
                         "weight_GBps": round(w.numel() / (us * 1e-6) / 1e9, 1)}
                    if prob.m > 8:
                        r["TOPS"] = round(2.0 * prob.m * prob.n * prob.k / (us * 1e-6) / 1e12, 2)
                    if flush is not None:  # cold: the weights evicted by a 512 MiB write before each launch
                        cold = []
                        for _ in range(30):
                            flush.fill_(1.0)
                            ev[0].record(stream)
                            plan.run(w, x, y, stream)
                            ev[1].record(stream)
                            torch.cuda.synchronize()
                            cold.append(ev[0].elapsed_time(ev[1]) * 1000.0)
                        cu = float(np.median(cold))
                        r["cold_us_per_launch"] = round(cu, 3)
                        r["cold_weight_GBps"] = round(w.numel() / (cu * 1e-6) / 1e9, 1)
                    rows.append(r)
        resid = {"c1": "L2-resident (352 KB of blocks)", "c2": "warm: Infinity-Cache/L2-resident (30 MB); cold: "
                 "after a 512 MiB write", "c3": "L2-resident (498 KB of blocks); M=37 takes the prefill kernel"}[wl]
        out = {"workload": wl, "note": resid, "rows": rows}
    else:  # c4
        probs = synth.c4_prefill()
        xp = [torch.from_numpy(p.acts()).to(dev) for p in probs]
        yp = [torch.empty((p.m, p.n), dtype=torch.float32, device=dev) for p in probs]
        # the decode step of the same model: every projection at M = 1 (the first token's row)
        xd = [t[:1].contiguous() for t in xp]
        yd = [torch.empty((1, p.n), dtype=torch.float32, device=dev) for p in probs]
        # the page's own Q4K file: K-quants only where K divides by 256 (ffn_down),
        # every other matrix Q5_0 (page "自己量化", section 3. 量化)
        passes = {"q8_0": ["q8_0"] * len(probs),
                  "down_q4_k": ["q4_k" if p.name.split()[0].endswith(".down") else "q8_0" for p in probs],
                  "q4k_file": ["q4_k" if p.name.split()[0].endswith(".down") else "q5_0" for p in probs]}
        wcache = {}
        out = {"workload": "c4", "problems": len(probs), "M_prefill": probs[0].m, "M_decode": 1, "passes": {}}
        total_flop = sum(2.0 * p.m * p.n * p.k for p in probs)
        for pname, fmts in passes.items():
            w = []
            for p, f in zip(probs, fmts):
                if (p.name, f) not in wcache:
                    wcache[(p.name, f)] = weights(p, f)
                w.append(wcache[(p.name, f)])
            for (md, mcode), phase in [(mm, ph) for mm in modes.items() for ph in ("prefill", "decode")]:
                x, y = (xp, yp) if phase == "prefill" else (xd, yd)
                plans = {}
                for p, f in zip(probs, fmts):
                    key = (f, p.n, p.k)
                    if key not in plans:
                        plans[key] = qmm.Plan(fmt_code[f], p.n, p.k, p.m, mcode)

                def one_pass():
                    for i, (p, f) in enumerate(zip(probs, fmts)):
                        plans[(f, p.n, p.k)].run(w[i], x[i], y[i], stream)

                us = timed(one_pass, 10)
                ref = [t.clone() for t in y]
                # the same pass captured once as a HIP graph, each replay checked against the stream pass
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g):
                    cap = torch.cuda.current_stream()
                    for i, (p, f) in enumerate(zip(probs, fmts)):
                        plans[(f, p.n, p.k)].run(w[i], x[i], y[i], cap)
                for rep in range(3):
                    for t in y:
                        t.zero_()
                    torch.cuda.synchronize()
                    g.replay()
                    torch.cuda.synchronize()
                    assert all(torch.equal(a, b) for a, b in zip(y, ref)), f"graph replay {rep} differs"
                gus = timed(g.replay, 10)
                flop = total_flop if phase == "prefill" else total_flop / probs[0].m
                out["passes"][f"{phase}:{pname}:{md}"] = {
                    "ms_per_pass_stream": round(us / 1000.0, 3), "ms_per_pass_graph": round(gus / 1000.0, 3),
                    "TOPS_stream": round(flop / (us * 1e-6) / 1e12, 3),
                    "TOPS_graph": round(flop / (gus * 1e-6) / 1e12, 3),
                    "launches": len(probs)}
                del g
                if True:
                    # the same pass with each layer's q/k/v and gate/up as one grouped run on
                    # one activation matrix (that of q, or gate), the others as before
                    groups = []
                    for base in range(0, len(probs) - 1, 7):  # q k v o gate up down
                        groups += [[base, base + 1, base + 2], [base + 3], [base + 4, base + 5], [base + 6]]
                    groups.append([len(probs) - 1])

                    def grouped_pass(st):
                        for grp in groups:
                            if len(grp) == 1:
                                i = grp[0]
                                plans[(fmts[i], probs[i].n, probs[i].k)].run(w[i], x[i], y[i], st)
                            else:
                                qmm.run_group([plans[(fmts[i], probs[i].n, probs[i].k)] for i in grp],
                                              [w[i] for i in grp], x[grp[0]], [y[i] for i in grp], st)

                    us = timed(lambda: grouped_pass(stream), 10)
                    ref = [t.clone() for t in y]
                    g = torch.cuda.CUDAGraph()
                    with torch.cuda.graph(g):
                        grouped_pass(torch.cuda.current_stream())
                    for rep in range(3):
                        for t in y:
                            t.zero_()
                        torch.cuda.synchronize()
                        g.replay()
                        torch.cuda.synchronize()
                        assert all(torch.equal(a, b) for a, b in zip(y, ref)), f"grouped graph replay {rep} differs"
                    gus = timed(g.replay, 10)
                    out["passes"][f"{phase}_grouped:{pname}:{md}"] = {
                        "ms_per_pass_stream": round(us / 1000.0, 3), "ms_per_pass_graph": round(gus / 1000.0, 3),
                        "TOPS_stream": round(flop / (us * 1e-6) / 1e12, 3),
                        "TOPS_graph": round(flop / (gus * 1e-6) / 1e12, 3),
                        "launches": len(groups)}
                    del g
                for pl in plans.values():
                    pl.close()
        out["GFLOP_per_prefill_pass"] = round(total_flop / 1e9, 2)
    print(json.dumps(out))


def formats_workload(args, qmm, torch, synth, stream):
    """c6: the step's 8 layers of 14336x4096 weights (the same seeds) in Q4_0,
    Q5_0 and Q6_K, quantized by the library, rotated per launch (264, 323 and
    385 MB: HBM-resident), both modes, M = 1 and 8 (decode) and 512 (prefill:
    Q4_0/Q5_0 rewrite the weights as Q8_0 blocks and take the Q8_0 kernels,
    Q6_K runs on the f16 prefill kernel).  Per-launch times from HIP events on
    the launch stream.  --only fmt:mode:M (e.g. q6_k:a:512) keeps one row."""
    dev = torch.device("cuda:0")
    fmts = {"q4_0": qmm.Q4_0, "q5_0": qmm.Q5_0, "q6_k": qmm.Q6_K}
    modes = {"a": qmm.MODE_F32ACT, "b": qmm.MODE_QACT}
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    x = torch.from_numpy(synth.acts_f32(5100, M_PREFILL, K)).to(dev)
    xs = {m: x[:m].contiguous() for m in DECODE_M + (M_PREFILL,)}
    ys = {m: torch.empty((m, N), dtype=torch.float32, device=dev) for m in DECODE_M + (M_PREFILL,)}
    rows = []
    only = args.only.split(":") if args.only else []

    def wanted(*key):
        return all(str(v) == p for v, p in zip(key, only))

    for f, code in fmts.items():
        if not wanted(f):
            continue
        wq = []
        for layer in range(LAYERS):
            wf = torch.from_numpy(synth.weights_f32(5000 + layer, N, K)).to(dev)
            wq.append(qmm.quantize_weights(code, wf))
            del wf
        b = wq[0].numel()
        for md, mcode in modes.items():
            if not wanted(f, md):
                continue
            with qmm.Plan(code, N, K, M_PREFILL, mcode) as plan:
                for m in DECODE_M + (M_PREFILL,):
                    if not wanted(f, md, m):
                        continue
                    reps = args.steps if m <= 8 else max(2, args.steps // 4)
                    for _ in range(max(1, args.warmup)):
                        for l in range(LAYERS):
                            plan.run(wq[l], xs[m], ys[m], stream)
                    torch.cuda.synchronize()
                    ev[0].record(stream)
                    for _ in range(reps):
                        for l in range(LAYERS):
                            plan.run(wq[l], xs[m], ys[m], stream)
                    ev[1].record(stream)
                    torch.cuda.synchronize()
                    us = ev[0].elapsed_time(ev[1]) * 1000.0 / (reps * LAYERS)
                    r = {"fmt": f, "mode": md, "M": m, "us_per_launch": round(us, 3),
                         "weight_GBps": round(b / (us * 1e-6) / 1e9, 1)}
                    if m <= 8:
                        r["frac_hbm"] = round(b / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)
                    else:
                        r["TOPS"] = round(2.0 * m * N * K / (us * 1e-6) / 1e12, 1)
                    rows.append(r)
        del wq
        torch.cuda.synchronize()
    print(json.dumps({"workload": "c6", "note": "8 layers of 14336x4096 rotated per launch (HBM-resident); weight "
                      "bytes per layer: Q4_0 33.0 MB, Q5_0 40.4 MB, Q6_K 48.2 MB", "rows": rows}))


def copy_calibration(torch, dev, stream, args):
    """A plain elementwise copy of 512 MiB of f32 (read 512 MiB, write
    512 MiB): the known-size kernel against which the FETCH_SIZE and WRITE_SIZE
    counters are scaled, and the streaming ceiling of the device."""
    nbytes = 512 * 2 ** 20
    src = torch.randn(nbytes // 4, device=dev)
    dst = torch.empty_like(src)
    for _ in range(args.warmup):
        torch.neg(src, out=dst)
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for _ in range(args.steps):
        torch.neg(src, out=dst)
    end.record(stream)
    torch.cuda.synchronize()
    us = start.elapsed_time(end) * 1000.0 / args.steps
    print(json.dumps({"copy_bytes_read": nbytes, "copy_bytes_written": nbytes, "us_per_copy": round(us, 2),
                      "GBps_read_plus_write": round(2 * nbytes / (us * 1e-6) / 1e9, 1)}))


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU; --gpus {args.gpus} is not supported "
              "(the path shards over N across GPUs by design but no multi-GPU run is built)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import block_quantized_matmul_gguf_amd as qmm
    import synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    if args.only == "copy":
        copy_calibration(torch, dev, stream, args)
        return
    if args.workload == "c6":
        formats_workload(args, qmm, torch, synth, stream)
        return
    if args.workload != "c5":
        small_workload(args, qmm, torch, synth, stream)
        return
    fmts = {"q8_0": qmm.Q8_0, "q4_k": qmm.Q4_K}
    modes = {"a": qmm.MODE_F32ACT, "b": qmm.MODE_QACT}

    # the other formats of the pages' files, decode only, outside the step and its value
    others = {} if (args.only or args.no_other_formats) else {"q4_0": qmm.Q4_0, "q5_0": qmm.Q5_0, "q6_k": qmm.Q6_K}

    # ---- inputs: quantized on the GPU by the library's weight quantizer ----
    t_setup = time.perf_counter()
    wq = {f: [] for f in list(fmts) + list(others)}
    for layer in range(LAYERS):
        wf = torch.from_numpy(synth.weights_f32(5000 + layer, N, K)).to(dev)
        for f, code in list(fmts.items()) + list(others.items()):
            wq[f].append(qmm.quantize_weights(code, wf))
        del wf
    x = torch.from_numpy(synth.acts_f32(5100, M_PREFILL, K)).to(dev)
    xs = {m: x[:m].contiguous() for m in DECODE_M + (M_PREFILL,)}
    ys = {m: torch.empty((m, N), dtype=torch.float32, device=dev) for m in DECODE_M + (M_PREFILL,)}
    plans = {(f, md): qmm.Plan(code, N, K, M_PREFILL, mcode) for f, code in fmts.items() for md, mcode in modes.items()}
    torch.cuda.synchronize()
    setup_s = time.perf_counter() - t_setup
    layer_bytes = {f: wq[f][0].numel() for f in fmts}

    groups = []  # (kind, fmt, mode, M)
    for f in fmts:
        for md in modes:
            for m in DECODE_M:
                groups.append(("gemv", f, md, m))
    for f in fmts:
        for md in modes:
            groups.append(("gemm", f, md, M_PREFILL))
    if args.only:
        parts = args.only.split(":")
        groups = [g for g in groups if all(str(v) == p for v, p in zip(g, parts))]
        assert groups, f"--only {args.only} matches nothing"

    def run_group(g):
        kind, f, md, m = g
        p = plans[(f, md)]
        for layer in range(LAYERS):
            p.run(wq[f][layer], xs[m], ys[m], stream)

    def step(evs=None):
        for i, g in enumerate(groups):
            if evs is not None:
                evs[i][0].record(stream)
            run_group(g)
            if evs is not None:
                evs[i][1].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    evs = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in groups]
           for _ in range(args.steps)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record(stream)
    for s in range(args.steps):
        step(evs[s])
    end.record(stream)
    torch.cuda.synchronize()
    wall_s = time.perf_counter() - t0
    total_ms = start.elapsed_time(end)

    group_ms = [sum(evs[s][i][0].elapsed_time(evs[s][i][1]) for s in range(args.steps)) / args.steps
                for i in range(len(groups))]
    detail = []
    gemv_ms = gemv_bytes = gemm_ms = gemm_flops = 0.0
    for g, ms in zip(groups, group_ms):
        kind, f, md, m = g
        us = ms * 1000.0 / LAYERS
        row = {"kernel": kind, "fmt": f, "mode": md, "M": m, "us_per_launch": round(us, 3)}
        if kind == "gemv":
            b = layer_bytes[f]
            row["weight_GBps"] = round(b / (us * 1e-6) / 1e9, 1)
            row["frac_hbm"] = round(row["weight_GBps"] / PEAK_HBM_GBS, 4)
            gemv_ms += ms
            gemv_bytes += b * LAYERS
        else:
            fl = 2.0 * m * N * K
            row["TOPS"] = round(fl / (us * 1e-6) / 1e12, 1)
            row["frac_f16_peak"] = round(row["TOPS"] / PEAK_F16_TFLOPS, 4)
            row["frac_int8_peak"] = round(row["TOPS"] / PEAK_I8_TOPS, 4)
            gemm_ms += ms
            gemm_flops += fl * LAYERS
        detail.append(row)

    def pick(kind, f, md, m):
        for g, r in zip(groups, detail):
            if g == (kind, f, md, m):
                return r
        return None

    out = {
        "metric": METRIC,
        "value": round(gemv_bytes / (gemv_ms * 1e-3) / 1e9, 1) if gemv_ms else None,
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(total_ms / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8/f16 MFMA, f32 accumulate",
        "data": "synthetic",
        "config": {
            "workload": "HBM-resident scale-up: 8 layers of 14336x4096 GGUF weights (Q8_0 499 MB, Q4_K 264 MB), "
                        "modes a and b, decode M=1 and 8, prefill M=512, layers rotated",
            "N": N, "K": K, "layers": LAYERS, "formats": list(fmts), "modes": list(modes),
            "decode_M": list(DECODE_M), "prefill_M": M_PREFILL,
            "only": args.only or None,
        },
    }
    if gemm_ms:
        out["prefill"] = {"TOPS": round(gemm_flops / (gemm_ms * 1e-3) / 1e12, 1),
                          "frac_f16_peak": round(gemm_flops / (gemm_ms * 1e-3) / 1e12 / PEAK_F16_TFLOPS, 4),
                          "frac_int8_peak": round(gemm_flops / (gemm_ms * 1e-3) / 1e12 / PEAK_I8_TOPS, 4)}
    def gemv_roof(r):
        b = layer_bytes[r["fmt"]]
        return {
            "kernel": f"{'gemv_row_kernel' if r['M'] == 1 else 'gemv_kernel'} {r['fmt']} mode {r['mode']} M={r['M']}",
            "bound": "hbm", "achieved": r["weight_GBps"], "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": r["frac_hbm"], "algorithmic_bytes_per_launch": b,
            "traffic": traffic_from_profile(f"gemv:{r['fmt']}:{r['mode']}:{r['M']}"),
        }

    def gemm_roof(r):
        # mode (a) runs on the f16 matrix cores (hi/lo split), mode (b) on the int8 ones
        int8 = r["mode"] == "b"
        return {
            # one run = the activation preparation launch + the prefill kernel, timed together
            "kernel": (f"{'quantize_' + ('q8_0' if r['fmt'] == 'q8_0' else 'q8k') + '_kernel + gemm_q_kernel' if int8 else 'gemm_prep_kernel + gemm_kernel'}"
                       f" {r['fmt']} mode {r['mode']} M={r['M']} (one run)"),
            "bound": "mfma", "achieved": r["TOPS"], "peak": PEAK_I8_TOPS if int8 else PEAK_F16_TFLOPS,
            "unit": "TOP/s" if int8 else "TFLOP/s",
            "frac": r["frac_int8_peak"] if int8 else r["frac_f16_peak"],
            "algorithmic_ops_per_launch": 2 * r["M"] * N * K,
            "traffic": traffic_from_profile(f"gemm:{r['fmt']}:{r['mode']}:{r['M']}"),
        }

    # the step's dominant kernel: the launch group with the most time per step
    if detail:
        i_dom = max(range(len(detail)), key=lambda i: group_ms[i])
        d = detail[i_dom]
        out["roofline"] = gemv_roof(d) if d["kernel"] == "gemv" else gemm_roof(d)
        out["roofline"]["share_of_step"] = round(group_ms[i_dom] / sum(group_ms), 4)
    r = pick("gemv", "q8_0", "b", 1)
    if r is not None:  # the headline decode kernel: Q8_0 weights, quantized activations, one token
        out["roofline_gemv"] = gemv_roof(r)
    for md in modes:
        rg = pick("gemm", "q8_0", md, M_PREFILL)
        if rg is not None:
            out[f"roofline_gemm_{md}"] = gemm_roof(rg)
    out["detail"] = detail
    if others:
        out["other_formats"] = other_formats_decode(qmm, torch, wq, others, modes, xs, ys, stream, args)
    if not args.only:
        out["one_gpu_share"] = one_gpu_share(qmm, torch, wq, fmts, modes, xs, ys, stream, args)
        out["q4_k_16_layers"] = q4k_sixteen_layers(qmm, torch, synth, wq["q4_k"], modes, xs, ys, stream, args)
    if not args.only and not args.no_dequant:
        out["dequantize_all"] = dequant_context(qmm, torch, wq, xs, ys, fmts, stream, args)
    out["wall_s_timed"] = round(wall_s, 3)
    out["setup_s"] = round(setup_s, 1)
    out["weights_fit_infinity_cache_256MB"] = {f: layer_bytes[f] * LAYERS <= 256 * 2 ** 20 for f in fmts}
    if not args.no_cpu_baseline and not args.only:
        out["cpu_baseline"] = cpu_baseline(args.cpu_layers)
        out["cpu_baseline_1thread"] = cpu_baseline(1, min_seconds=3.0, threads=1)
    for p in plans.values():
        p.close()
    print(json.dumps(out))


if __name__ == "__main__":
    main()
