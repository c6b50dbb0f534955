"""Benchmark of the sampled-softmax cross-entropy step on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload stage01]

A step is one call of sampled_ce_forward_backward: candidate build, row gather,
logits GEMM, fused CE forward/backward, dX and dW GEMMs, dense scatter, over one
microbatch of synthetic inputs already resident in HBM. Prints ONE JSON line:
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
PEAK_TFLOPS = {"bf16": 2500.0, "f32": 157.3}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def stage_work(w, P_eff):
    """Algorithmic work of one launch of each stage: (kind, amount)."""
    es = 2 if w.dtype == "bf16" else 4
    ldz = (P_eff + 7) // 8 * 8
    flops = 2.0 * w.T * P_eff * w.d
    return {
        "logits": ("mfma", flops),
        "dx": ("mfma", flops),
        "dw": ("mfma", flops),
        # read Z once, write dZ once, plus labels and the row loss
        "ce": ("hbm", 2.0 * w.T * ldz * es + w.T * 12),

        # read the fp32 candidate-row gradient once, write the dense dW, read vocab_pos
        "scatter": ("hbm", P_eff * w.d * 4.0 + w.V * w.d * es + 4 * w.V),
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


def recorded_traffic(workload, stage):
    """HBM bytes per launch (calibrated FETCH_SIZE + WRITE_SIZE) recorded under profiles/
    for this workload and stage, or None when absent or taken from other kernel sources."""
    path = os.path.join(ROOT, "profiles", f"{workload}_traffic.json")
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
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-full-compare", action="store_true")
    ap.add_argument("--cpu-sample-tokens", type=int, default=16384)
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

    xd, Wd = to_dev(x), to_dev(W)
    yd = torch.from_numpy(y).to(dev)
    pd = torch.from_numpy(p).to(dev) if p is not None else None
    off = w.offset
    outs = {}

    def step(P):
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
    work = stage_work(w, P_eff)
    stages = {}
    for k, t in stage_ms.items():
        entry = {"ms": round(t, 5)}
        if k in work and t > 0.01:
            kind, amount = work[k]
            if kind == "mfma":
                ach = amount / (t * 1e-3) / 1e12
                entry.update(tflops=round(ach, 2), frac=round(ach / PEAK_TFLOPS[w.dtype], 4))
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
                "peak": PEAK_TFLOPS[w.dtype], "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_TFLOPS[w.dtype], 4),
                "traffic": recorded_traffic(w.name, dom)}
    else:
        achieved = amount / (stage_ms[dom] * 1e-3) / 1e9
        roof = {"kernel": dom, "bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
                "traffic": recorded_traffic(w.name, dom)}

    if args.calibrate_copy_mib:
        src = torch.empty(args.calibrate_copy_mib << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        src.fill_(1)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    full_cmp = None
    if not args.no_full_compare and w.P > 0:
        ms_v, _ = timed(w.V, max(5, args.steps // 5), 2)
        full_cmp = {"P": w.V, "ms_per_step": round(ms_v, 4), "speedup": round(ms_v / ms, 3)}
        log(f"[bench] same library at P=V: {ms_v:.4f} ms/step -> sampled speedup {ms_v / ms:.2f}x")
        del outs[w.V]
        torch.cuda.empty_cache()

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, x, W, y, p, args.cpu_sample_tokens)
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
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "T": w.T, "d": w.d, "V": w.V, "P": w.P,
                   "stride": w.stride, "offset": off, "targets": f"zipf({w.zipf_s})",
                   "prefix_targets": w.prefix},
        "roofline": roof,
        "stages": stages,
        "full_softmax_same_library": full_cmp,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def cpu_baseline(w, x, W, y, p, sample_tokens):
    """The float64 CPU oracle, as it stands, on the first `sample_tokens` tokens of the
    same microbatch: candidate build + dense loss and gradients."""
    from threadpoolctl import threadpool_info

    from oracle import build_candidates, ce
    from sampled_softmax_cross_amd import synth

    Ts = min(sample_tokens, w.T)
    xs = synth.to_f64(x[:Ts], w.dtype)
    Wf = synth.to_f64(W, w.dtype)
    ys = y[:Ts]
    ps = None if p is None else p[:Ts]
    t0 = time.perf_counter()
    cand = build_candidates(w.V, w.P, w.stride, w.offset, ys, ps)
    ce.forward_backward(xs, Wf, None if w.P == 0 else cand["C"], cand["target_pos"],
                        cand["prefix_pos"] if ps is not None else None)
    dt = time.perf_counter() - t0
    threads = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    return {"value": round(Ts / dt, 1), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "seconds": round(dt, 2),
            "sample": f"first {Ts} of {w.T} tokens of the {w.name} microbatch (same P, V, d, "
                      f"stride, offset): candidate build + float64 loss, dX, dW"}


if __name__ == "__main__":
    main()
