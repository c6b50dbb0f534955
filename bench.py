"""Benchmark of the sampled-softmax cross-entropy step on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload stage01] [--dtype e4m3]

A step is one call of sampled_ce_forward_backward: candidate build, row gather,
logits GEMM, fused CE forward/backward, dX and dW GEMMs, dense scatter, over one
microbatch of synthetic inputs already resident in HBM. --dtype e4m3 times
sampled_ce_forward_backward_fp8 on the same microbatch instead (the lm_head as an
e4m3 cache with one scale, x quantised per call, e4m3 products). Prints ONE JSON line:
tokens/s of the whole step, the roofline fraction of its dominant kernel (timed
live with HIP events the library records on the call's stream), the same library
at P = V for the speedup of the sampled path, and the CPU oracle on a bounded
sample of the same workload.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "tokens/s sampled-CE fwd+bwd (V=50304,d=768,P=10240/14336/24576); % roofline"
PEAK_HBM_GBS = 8000.0
PEAK_TFLOPS = {"bf16": 2500.0, "f32": 157.3, "e4m3": 5000.0}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def stage_work(w, P_eff, e4m3=False):
    """Algorithmic work of one launch of each stage: (kind, amount)."""
    es = 2 if w.dtype == "bf16" else 4
    ldz = (P_eff + 7) // 8 * 8
    flops = 2.0 * w.T * P_eff * w.d
    # read Z once, write dZ once (e4m3 step: read bf16 Z, write the e4m3 gradient), plus
    # labels and the row loss
    ce_bytes = (w.T * ldz * 3.0 if e4m3 else 2.0 * w.T * ldz * es) + w.T * 12
    return {
        "logits": ("mfma", flops),
        "dx": ("mfma", flops),
        "dw": ("mfma", flops),
        "ce": ("hbm", ce_bytes),
        # read the fp32 candidate-row gradient once, write the candidate rows of dense dW
        # (the rows outside C are cleared in the candidates stage)
        "scatter": ("hbm", P_eff * w.d * (4.0 + (2 if e4m3 else es))),
        # sum the fp32 k-split partials of dX into dX (bytes of a 2-way split)
        "dx_reduce": ("hbm", 2 * w.T * w.d * 4.0 + w.T * w.d * es),
    }


def source_sha():
    """Hash of the kernel sources (every HIP file but the host-side ABI layer); recorded
    counter traffic is valid only for the same hash."""
    import glob
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "sampled_softmax_cross_amd", "csrc")
    files = glob.glob(os.path.join(csrc, "*.hip")) + glob.glob(os.path.join(csrc, "*.h"))
    for f in sorted(x for x in files if os.path.basename(x) != "api.hip"):
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def recorded_traffic(workload, stage, e4m3=False):
    """HBM bytes per launch (calibrated FETCH_SIZE + WRITE_SIZE) recorded under profiles/
    for this workload, operand type and stage, or None when absent or taken from other
    kernel sources."""
    name = f"{workload}_e4m3" if e4m3 else workload
    path = os.path.join(ROOT, "profiles", f"{name}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_sha") != source_sha() or stage not in rec.get("stages", {}):
        return None
    s = rec["stages"][stage]
    return int(s["fetch_bytes"] + s["write_bytes"])


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default="stage01")
    ap.add_argument("--dtype", choices=["auto", "e4m3"], default="auto",
                    help="auto: the workload's own precision (bf16 or f32); e4m3: the e4m3 "
                         "operand step on the same bf16 microbatch")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-full-compare", action="store_true")
    ap.add_argument("--no-achievable", action="store_true",
                    help="skip the measured reference peaks (device copy, library GEMM)")
    ap.add_argument("--cpu-sample-tokens", type=int, default=16384)
    ap.add_argument("--micro", choices=["softmax", "gather"], default=None,
                    help="instead of the step: time one building block on its own over the "
                         "secondary workloads (one JSON line per shape)")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="also run one device copy of this many MiB (a known-size reference "
                         "for HBM traffic counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}): the sampled-CE "
              "step has no cross-GPU exchange inside it, so one GPU's share of a data-parallel "
              "batch is the unit measured here", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from sampled_softmax_cross_amd import binding, synth

    if args.micro:
        micro(args.micro)
        return
    w = synth.workload(args.workload)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    log(f"[bench] workload {w.name}: T={w.T} d={w.d} V={w.V} P={w.P} {w.dtype}")
    x, W = synth.make_weights(w)
    y, p = synth.make_labels(w, 0)

    def to_dev(a):
        if w.dtype == "bf16":
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(a).to(dev)

    e4m3 = args.dtype == "e4m3"
    if e4m3 and w.dtype != "bf16":
        raise SystemExit("--dtype e4m3 needs a bf16 workload")
    xd, Wd = to_dev(x), to_dev(W)
    yd = torch.from_numpy(y).to(dev)
    pd = torch.from_numpy(p).to(dev) if p is not None else None
    off = w.offset
    outs = {}
    if e4m3:
        W8, w_scale = synth.e4m3_cache(W)
        W8d = torch.from_numpy(W8).to(dev)
        log(f"[bench] e4m3 products: lm_head cache scale {w_scale:.4g}")

    def step(P):
        if e4m3:
            return binding.forward_backward_fp8(xd, W8d, w_scale, yd, pd, P, w.stride, off,
                                                outputs=outs.get(P))
        return binding.forward_backward(xd, Wd, yd, pd, P, w.stride, off, outputs=outs.get(P))

    def timed(P, steps, warmup):
        outs[P] = step(P)  # allocate outputs and workspace once
        for _ in range(warmup):
            step(P)
        torch.cuda.synchronize()
        s = torch.cuda.Event(enable_timing=True)
        e = torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        s.record()
        for _ in range(steps):
            step(P)
        e.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        return s.elapsed_time(e) / steps, wall

    ms, wall = timed(w.P, args.steps, args.warmup)

    def graph_ms(P, reps):
        """The same call captured once in a HIP graph and replayed (the launches of
        the step without host-side launch overhead)."""
        code = binding.SCE_E4M3 if e4m3 else binding.dtype_code(xd.dtype)
        ws = binding.workspace(binding.workspace_size(w.T, w.d, w.V, P, code), dev)
        o = outs[P]
        if e4m3:
            call = lambda: binding.forward_backward_fp8(xd, W8d, w_scale, yd, pd, P, w.stride, off,
                                                        outputs=o, ws=ws)
        else:
            call = lambda: binding.forward_backward(xd, Wd, yd, pd, P, w.stride, off, outputs=o,
                                                    ws=ws)
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            call()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            call()
        gms = _time_ms(g.replay, reps=reps, warmup=3)
        del g
        return gms

    gms = graph_ms(w.P, max(20, min(args.steps, 200)))
    log(f"[bench] as a replayed HIP graph: {gms:.4f} ms/step ({w.T / gms * 1e3 / 1e6:.2f} M tokens/s)")
    aux = outs[w.P]["aux"].cpu().tolist()
    if aux[3] != 0:
        raise RuntimeError(f"device status {aux[3]} in the benchmark step")
    log(f"[bench] {ms:.4f} ms/step ({w.T / ms * 1e3 / 1e6:.2f} M tokens/s); wall {wall:.3f} s")

    # per-stage times from HIP events recorded by the library on the call's stream
    binding.profile_enable(True)
    nprof = max(10, min(args.steps, 50))
    for _ in range(nprof):
        step(w.P)
    binding.profile_enable(False)
    stage_ms, ncalls = binding.profile_collect()
    stage_ms = {k: v / ncalls for k, v in stage_ms.items()}
    P_eff = w.P if w.P else w.V
    work = stage_work(w, P_eff, e4m3)
    ptype = "e4m3" if e4m3 else w.dtype
    stages = {}
    for k, t in stage_ms.items():
        entry = {"ms": round(t, 5)}
        if k in work and t > 0.01:
            kind, amount = work[k]
            if kind == "mfma":
                ach = amount / (t * 1e-3) / 1e12
                entry.update(tflops=round(ach, 2), frac=round(ach / PEAK_TFLOPS[ptype], 4))
            else:
                ach = amount / (t * 1e-3) / 1e9
                entry.update(gbs=round(ach, 1), frac=round(ach / PEAK_HBM_GBS, 4))
        stages[k] = entry
    log("[bench] stages: " + json.dumps(stages))
    dom = max((k for k in work if k in stage_ms), key=lambda k: stage_ms[k])
    kind, amount = work[dom]
    if kind == "mfma":
        achieved = amount / (stage_ms[dom] * 1e-3) / 1e12
        roof = {"kernel": dom, "bound": "mfma", "achieved": round(achieved, 2),
                "peak": PEAK_TFLOPS[ptype], "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_TFLOPS[ptype], 4),
                "traffic": recorded_traffic(w.name, dom, e4m3)}
    else:
        achieved = amount / (stage_ms[dom] * 1e-3) / 1e9
        roof = {"kernel": dom, "bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
                "traffic": recorded_traffic(w.name, dom, e4m3)}

    if args.calibrate_copy_mib:
        src = torch.empty(args.calibrate_copy_mib << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        src.fill_(1)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    achievable = None if args.no_achievable else measured_peaks(torch, dev, ptype)
    if achievable:
        ref = achievable["gemm_tflops"] if kind == "mfma" else achievable["copy_gbs"]
        achievable["dominant_frac"] = round(roof["achieved"] / ref, 4)
        log(f"[bench] achievable on this GPU: {achievable}")

    full_cmp = None
    if not args.no_full_compare and w.P > 0:
        ms_v, _ = timed(w.V, max(5, args.steps // 5), 2)
        full_cmp = {"P": w.V, "ms_per_step": round(ms_v, 4), "speedup": round(ms_v / ms, 3)}
        log(f"[bench] same library at P=V: {ms_v:.4f} ms/step -> sampled speedup {ms_v / ms:.2f}x")
        del outs[w.V]
        torch.cuda.empty_cache()

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, x, W, y, p, args.cpu_sample_tokens, e4m3)
        log(f"[bench] cpu oracle: {cpu}")

    line = {
        "metric": METRIC,
        "value": round(w.T / (ms * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ptype,
        "data": "synthetic",
        "config": {"workload": w.name, "T": w.T, "d": w.d, "V": w.V, "P": w.P,
                   "stride": w.stride, "offset": off, "targets": f"zipf({w.zipf_s})",
                   "prefix_targets": w.prefix,
                   **({"operands": "e4m3 x and lm_head, bf16 logits"} if e4m3 else {})},
        "roofline": roof,
        "achievable": achievable,
        "graph_replay": {"ms_per_step": round(gms, 5), "value": round(w.T / (gms * 1e-3), 1)},
        "stages": stages,
        "full_softmax_same_library": full_cmp,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def measured_peaks(torch, dev, ptype):
    """Reference rates measured on this GPU beside the published peaks: a 1 GiB
    device-to-device copy (bytes read + written per second) and the vendor library's
    dense product at 8192^3 in the step's product type (hipBLASLt through torch;
    e4m3 through torch._scaled_mm with unit scales, f32 through torch.matmul)."""
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    src.fill_(1)
    copy_ms = _time_ms(lambda: dst.copy_(src), reps=20, warmup=3)
    del src, dst
    m = 8192
    if ptype == "e4m3":
        a = torch.randn(m, m, device=dev).to(torch.float8_e4m3fn)
        b = torch.randn(m, m, device=dev).to(torch.float8_e4m3fn).t()  # k-contiguous columns
        one = torch.tensor(1.0, device=dev)
        fn = lambda: torch._scaled_mm(a, b, scale_a=one, scale_b=one, out_dtype=torch.bfloat16)
    else:
        dt = torch.bfloat16 if ptype == "bf16" else torch.float32
        a = torch.randn(m, m, device=dev, dtype=dt)
        b = torch.randn(m, m, device=dev, dtype=dt)
        fn = lambda: torch.matmul(a, b)
    gemm_ms = _time_ms(fn, reps=10, warmup=3)
    del a, b
    torch.cuda.empty_cache()
    return {"copy_gbs": round(2.0 * n / (copy_ms * 1e-3) / 1e9, 1),
            "gemm_tflops": round(2.0 * m ** 3 / (gemm_ms * 1e-3) / 1e12, 1),
            "gemm": f"{m}^3 {ptype}, vendor library"}


def _time_ms(fn, reps=50, warmup=10):
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        fn()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / reps


def micro(kind):
    """Building blocks over the pages' secondary workloads.

    softmax: the fused row CE forward/backward (read a row, write its gradient) over
    M = 4096 rows and N = 256 .. 12672 columns ("Learning Triton one kernel at a time:
    softmax", its benchmark sweep; bandwidth counted as 2 * M * N * element bytes),
    fp32 and bf16, next to PyTorch's softmax forward on the same tensor.
    gather: the row gather (index select) of bf16 rows of 4096 for the index counts of
    torchtitan PR #1083's benchmark script ([1024, 512], [4096, 4096], [8192, 8192]
    rows and indices), bandwidth as read + write, next to torch.index_select.
    """
    import numpy as np
    import torch

    from sampled_softmax_cross_amd import binding
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    gen = torch.Generator(device=dev).manual_seed(0)
    import ctypes
    lib = binding.load_library()
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    P_ = ctypes.c_void_p
    if kind == "softmax":
        M = 4096
        loss = torch.empty(1, dtype=torch.float32, device=dev)
        nbytes = ctypes.c_size_t(0)
        lib.sce_ce_rows_workspace_size(M, ctypes.byref(nbytes))
        ws = torch.empty(nbytes.value, dtype=torch.uint8, device=dev)
        for dt, es in ((torch.float32, 4), (torch.bfloat16, 2)):
            for N in (256, 512, 1024, 2048, 3072, 4096, 6144, 8192, 10240, 12672):
                Z = torch.randn(M, N, generator=gen, device=dev).to(dt)
                tp = torch.randint(0, N, (M,), generator=gen, device=dev, dtype=torch.int32)
                Zs = Z.clone()
                # the C entry point with its arguments prepared once (no Python work per call)
                args = (P_(Z.data_ptr()), N, M, N, binding.dtype_code(dt), P_(tp.data_ptr()), None,
                        P_(loss.data_ptr()), None, None, None, P_(ws.data_ptr()), ws.numel(), stream)
                ms = _time_ms(lambda: lib.sce_ce_rows(*args))
                ms_t = _time_ms(lambda: torch.softmax(Zs, dim=1))
                gbs = 2.0 * M * N * es / (ms * 1e-3) / 1e9
                print(json.dumps({"micro": "softmax_ce_rows", "M": M, "N": N,
                                  "dtype": "bf16" if es == 2 else "f32", "us": round(ms * 1e3, 2),
                                  "GB/s": round(gbs, 1), "frac_hbm": round(gbs / 8000.0, 4),
                                  "torch_softmax_us": round(ms_t * 1e3, 2)}), flush=True)
    else:
        d = 4096
        for rows, n in ((1024, 512), (4096, 4096), (8192, 8192)):
            W = torch.randn(rows, d, generator=gen, device=dev).to(torch.bfloat16)
            idx = torch.randint(0, rows, (n,), generator=gen, device=dev, dtype=torch.int32)
            out = torch.empty(n, d, dtype=torch.bfloat16, device=dev)
            idx64 = idx.long()
            args = (P_(W.data_ptr()), rows, d, P_(idx.data_ptr()), n, binding.SCE_BF16,
                    P_(out.data_ptr()), d, None, stream)
            ms = _time_ms(lambda: lib.sce_gather_rows(*args))
            ms_t = _time_ms(lambda: torch.index_select(W, 0, idx64, out=out))
            byts = 2.0 * n * d * 2
            print(json.dumps({"micro": "gather_rows", "rows": rows, "d": d, "indices": n,
                              "dtype": "bf16", "us": round(ms * 1e3, 2),
                              "TB/s": round(byts / (ms * 1e-3) / 1e12, 3),
                              "frac_hbm": round(byts / (ms * 1e-3) / 8e12, 4),
                              "torch_index_select_us": round(ms_t * 1e3, 2)}), flush=True)


def cpu_baseline(w, x, W, y, p, sample_tokens, e4m3=False):
    """The float64 CPU oracle, as it stands, on the first `sample_tokens` tokens of the
    same microbatch: candidate build + dense loss and gradients (the e4m3 oracle for the
    e4m3 step)."""
    from threadpoolctl import threadpool_info

    from oracle import build_candidates, ce, fp8
    from sampled_softmax_cross_amd import synth

    Ts = min(sample_tokens, w.T)
    xs = synth.to_f64(x[:Ts], w.dtype)
    Wf = synth.to_f64(W, w.dtype)
    ys = y[:Ts]
    ps = None if p is None else p[:Ts]
    if e4m3:
        W8, w_scale = synth.e4m3_cache(W)
    t0 = time.perf_counter()
    cand = build_candidates(w.V, w.P, w.stride, w.offset, ys, ps)
    C = None if w.P == 0 else cand["C"]
    ppos = cand["prefix_pos"] if ps is not None else None
    if e4m3:
        fp8.forward_backward(xs, W8, w_scale, C, cand["target_pos"], ppos)
    else:
        ce.forward_backward(xs, Wf, C, cand["target_pos"], ppos)
    dt = time.perf_counter() - t0
    threads = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    return {"value": round(Ts / dt, 1), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "seconds": round(dt, 2),
            "sample": f"first {Ts} of {w.T} tokens of the {w.name} microbatch (same P, V, d, "
                      f"stride, offset): candidate build + float64 loss, dX, dW"
                      + (" of the e4m3 step" if e4m3 else "")}


if __name__ == "__main__":
    main()
