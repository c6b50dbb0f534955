"""Benchmark of the sampled-softmax cross-entropy step on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload stage01] [--dtype e4m3]

A step is one call of sampled_ce_forward_backward: candidate build, row gather,
logits GEMM, fused CE forward/backward, dX and dW GEMMs, dense scatter, over one
microbatch of synthetic inputs already resident in HBM. --dtype e4m3 times, on the same
microbatch, the e4m3 step from the bf16 weights (sampled_ce_forward_backward_fp8_bf16w:
the lm_head cache's scale and the codes of the candidate rows formed inside every step,
x quantised per call, e4m3 products); the full-cache refresh (sce_refresh_e4m3_cache) is
timed beside it. Prints ONE JSON line:
tokens/s of the whole step on the headline workload (stage-0/1, P = 10240), the
roofline fraction of its dominant kernel (timed live with HIP events the library
records on the call's stream), the same library at P = V for the speedup of the
sampled path, the other configurations the metric names (P = 14336 and 24576 at
T = 49152, and the full softmax) with theirs, and the CPU oracle on a bounded sample
of the headline workload. Every measurement follows ~100 ms of untimed steps
(`settle_steps`), so it sees the GPU's settled clock rather than the transient right
after an idle period.
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


def dw_split_rows(w, P_eff, cus):
    """Rows of dW_C that go through the k-split reduction (the scatter stage). The dW
    product (256 x 256 tiles, M = P_eff, N = d, K = T) stores whole rounds of tiles
    straight into dW when its tiles outnumber the CUs, its column tiles are at most 4
    and T >= 1024 (whole rounds trimmed to whole row blocks); the other rows are
    k-split. The fp32 step splits every row."""
    nbx, nby = -(-w.d // 256), -(-P_eff // 256)
    tiles = nbx * nby
    if w.dtype != "bf16" or nbx > 4 or tiles <= cus or w.T < 1024:
        return P_eff
    whole = (tiles // cus) * cus // nbx * nbx
    return P_eff - (whole // nbx) * 256


def stage_work(w, P_eff, e4m3=False, cus=256):
    """Algorithmic work of one launch of each stage: (kind, amount)."""
    es = 2 if w.dtype == "bf16" else 4
    ldz = (P_eff + 7) // 8 * 8
    flops = 2.0 * w.T * P_eff * w.d
    split_rows = dw_split_rows(w, P_eff, cus)
    # read Z once, write dZ once (e4m3 step: read bf16 Z, write the e4m3 gradient), plus
    # labels and the row loss
    ce_bytes = (w.T * ldz * 3.0 if e4m3 else 2.0 * w.T * ldz * es) + w.T * 12
    return {
        "logits": ("mfma", flops),
        "dx": ("mfma", flops),
        "dw": ("mfma", flops),
        "ce": ("hbm", ce_bytes),
        # read the fp32 gradient of the k-split candidate rows once, write those rows of
        # dense dW (the dW product stores the other candidate rows; the rows outside C are
        # cleared in the candidates stage)
        "scatter": ("hbm", split_rows * w.d * (4.0 + (2 if e4m3 else es))),
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


OTHER_CONFIGS = ("s2early", "s2late", "full")


def stage_table(stage_ms, work, ptype):
    """Per-stage times with the achieved rate and its fraction of the published peak."""
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
    return stages


def roofline_of(w, stage_ms, work, ptype, e4m3):
    """The dominant (slowest) kernel's algorithmic rate against its published peak."""
    dom = max((k for k in work if k in stage_ms), key=lambda k: stage_ms[k])
    kind, amount = work[dom]
    traffic = recorded_traffic(w.name, dom, e4m3)
    if kind == "mfma":
        achieved = amount / (stage_ms[dom] * 1e-3) / 1e12
        return {"kernel": dom, "bound": "mfma", "achieved": round(achieved, 2),
                "peak": PEAK_TFLOPS[ptype], "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_TFLOPS[ptype], 4), "traffic": traffic}
    achieved = amount / (stage_ms[dom] * 1e-3) / 1e9
    return {"kernel": dom, "bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
            "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": traffic}


class Bench:
    """One workload resident on the GPU, and the measurements of its step."""

    def __init__(self, w, dev, e4m3):
        import numpy as np
        import torch

        from sampled_softmax_cross_amd import synth

        self.w, self.dev, self.e4m3 = w, dev, e4m3
        self.torch = torch
        x, W = synth.make_weights(w)
        self.host = (x, W)

        def to_dev(a):
            if w.dtype == "bf16":
                return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
            return torch.from_numpy(a).to(dev)

        self.xd, self.Wd = to_dev(x), to_dev(W)
        # one label set per consecutive call of the workload (the 4-call workload advances
        # its candidate offset by P per call; a step takes the calls in turn)
        self.calls = []
        self.host_calls = []
        for c in range(w.calls):
            y, p = synth.make_labels(w, c)
            if c == 0:
                self.labels0 = (y, p)
            self.calls.append((torch.from_numpy(y).to(dev),
                               torch.from_numpy(p).to(dev) if p is not None else None,
                               w.call_offset(c)))
            self.host_calls.append((torch.from_numpy(y), torch.from_numpy(p) if p is not None else None,
                                    w.call_offset(c)))
        self.i = 0
        self.outs = {}
        if e4m3:
            from sampled_softmax_cross_amd import binding

            # the lm_head's e4m3 cache, rebuilt from the bf16 weights on the device at the
            # start of every step (the weights change at every optimizer step)
            self.rws = torch.empty(binding.REFRESH_WORKSPACE_BYTES, dtype=torch.uint8, device=dev)
            self.cache = binding.refresh_e4m3_cache(self.Wd, ws=self.rws)

    def step(self, P, outputs=None, ws=None):
        from sampled_softmax_cross_amd import binding

        w = self.w
        yd, pd, off = self.calls[self.i % len(self.calls)]
        self.i += 1
        o = self.outs.get(P) if outputs is None else outputs
        if self.e4m3:
            # the e4m3 step from the bf16 weights: the cache's scale and the candidate rows'
            # codes are formed inside the step (the weights change at every optimizer step)
            return binding.forward_backward_fp8_bf16w(self.xd, self.Wd, yd, pd, P, w.stride, off,
                                                      outputs=o, ws=ws)
        return binding.forward_backward(self.xd, self.Wd, yd, pd, P, w.stride, off, outputs=o,
                                        ws=ws)

    def refresh(self):
        from sampled_softmax_cross_amd import binding

        binding.refresh_e4m3_cache(self.Wd, outputs=self.cache, ws=self.rws)

    def refresh_us(self, reps):
        """The e4m3 cache refresh alone (microseconds per call), and its algorithmic HBM
        rate: W read once (bf16) and the codes written once, 3 V d bytes."""
        ms = _time_ms(self.refresh, reps=reps, warmup=3)
        nbytes = 3.0 * self.w.V * self.w.d
        if self.cache["status"].item() != 0:
            raise RuntimeError("device status in the e4m3 cache refresh")
        return {"us": round(ms * 1e3, 2), "gbs": round(nbytes / (ms * 1e-3) / 1e9, 1),
                "frac": round(nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                "algorithmic_bytes": int(nbytes)}

    def prepare(self, P):
        self.outs[P] = self.step(P)  # outputs and workspace allocated once
        self.torch.cuda.synchronize()

    def settle(self, P, ms=100.0):
        """Untimed steps for about `ms` milliseconds: after an idle period the GPU's clock
        overshoots and settles over the first ~25 steps (measured at stage-0/1: steps 5..25
        after 2 s idle 8% slower than the steady state), and every later measurement should
        see the steady state a training loop runs in. Returns the number of steps run."""
        torch = self.torch
        n, t0 = 0, time.perf_counter()
        while n < 4 or (time.perf_counter() - t0) * 1e3 < ms:
            for _ in range(4):
                self.step(P)
            torch.cuda.synchronize()
            n += 4
        return n

    def timed(self, P, steps, warmup):
        torch = self.torch
        for _ in range(warmup):
            self.step(P)
        torch.cuda.synchronize()
        s = torch.cuda.Event(enable_timing=True)
        e = torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        s.record()
        for _ in range(steps):
            self.step(P)
        e.record()
        torch.cuda.synchronize()
        return s.elapsed_time(e) / steps, time.perf_counter() - t0

    def pipelined_ms(self, steps, warmup):
        """The step with its candidate build off the critical path, the way the page runs
        it: while the GPU runs step i (sampled_ce_forward_backward_prebuilt), the host
        builds the set of microbatch i + 1 (sce_build_candidates_host) into pinned memory
        and a copy stream uploads it; step i + 1 waits only for that upload. Host and
        device buffers are double-buffered and ordered by events. Returns ms per step
        (sampled steps; the e4m3 step refreshes its cache and runs
        sampled_ce_forward_backward_fp8_prebuilt)."""
        from sampled_softmax_cross_amd import binding

        torch, w = self.torch, self.w
        main, copy = torch.cuda.current_stream(), torch.cuda.Stream()
        T, P = w.T, w.P
        pre = w.prefix

        def slot(pin):
            # one buffer per slot, so that one copy uploads the whole set: aux (int64 [4])
            # first, then C, the target and the prefix positions
            kw = dict(pin_memory=True) if pin else dict(device=self.dev)
            buf = torch.empty(8 + P + (2 if pre else 1) * T, dtype=torch.int32, **kw)
            return {"_buf": buf, "aux": buf[:8].view(torch.int64), "C": buf[8:8 + P],
                    "target_pos": buf[8 + P:8 + P + T],
                    "prefix_pos": buf[8 + P + T:8 + P + 2 * T] if pre else None}

        host, devb = [slot(True), slot(True)], [slot(False), slot(False)]
        copied = [torch.cuda.Event(), torch.cuda.Event()]
        used = [torch.cuda.Event(), torch.cuda.Event()]
        for e in used + copied:
            e.record(main)
        out = {"o": self.outs.get(P)}

        def build_upload(i):
            k = i % 2
            y, p, off = self.host_calls[i % len(self.host_calls)]
            copied[k].synchronize()  # the pinned slot's last upload has left it
            binding.build_candidates_host(y, p, w.V, P, w.stride, off, outputs=host[k])
            with torch.cuda.stream(copy):
                copy.wait_event(used[k])  # the step that read the device slot is done
                devb[k]["_buf"].copy_(host[k]["_buf"], non_blocking=True)
                copied[k].record(copy)

        def run(n, i0):
            for i in range(i0, i0 + n):
                main.wait_event(copied[i % 2])
                if self.e4m3:
                    self.refresh()
                    out["o"] = binding.forward_backward_fp8_prebuilt(
                        self.xd, self.cache["W8"], self.cache["w_scale"], devb[i % 2],
                        outputs=out["o"])
                else:
                    out["o"] = binding.forward_backward_prebuilt(self.xd, self.Wd, devb[i % 2],
                                                                 outputs=out["o"])
                used[i % 2].record(main)
                build_upload(i + 1)  # on the host while the GPU runs step i

        build_upload(0)
        run(warmup, 0)
        torch.cuda.synchronize()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        run(steps, warmup)
        e.record()
        torch.cuda.synchronize()
        if out["o"]["aux"][3].item() != 0:
            raise RuntimeError("device status in the overlapped-build steps")
        return s.elapsed_time(e) / steps

    def stage_ms(self, P, n):
        """Per-stage times from HIP events the library records on the call's stream."""
        from sampled_softmax_cross_amd import binding

        binding.profile_enable(True)
        for _ in range(n):
            self.step(P)
        binding.profile_enable(False)
        tot, ncalls = binding.profile_collect()
        return {k: v / ncalls for k, v in tot.items()}

    def graph_ms(self, P, reps):
        """The same call captured once in a HIP graph and replayed."""
        from sampled_softmax_cross_amd import binding

        torch, w = self.torch, self.w
        code = binding.SCE_E4M3_BF16W if self.e4m3 else binding.dtype_code(self.xd.dtype)
        ws = binding.workspace(binding.workspace_size(w.T, w.d, w.V, P, code), self.dev)
        o = self.outs[P]
        i0 = self.i
        call = lambda: self.step(P, outputs=o, ws=ws)
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            call()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        self.i = i0
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            call()
        # the first replays after a capture run slower; warm up past them
        gms = _time_ms(g.replay, reps=reps, warmup=20)
        del g
        return gms

    def check_status(self, P):
        aux = self.outs[P]["aux"].cpu().tolist()
        if aux[3] != 0:
            raise RuntimeError(f"device status {aux[3]} in the {self.w.name} step")

    def release(self):
        self.outs.clear()
        self.torch.cuda.empty_cache()


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
    ap.add_argument("--no-overlap", action="store_true",
                    help="skip the step with the candidate build overlapped on the host")
    ap.add_argument("--no-other-configs", action="store_true",
                    help="time only the headline workload (not the other configurations the "
                         "metric names)")
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

    import torch

    from sampled_softmax_cross_amd import synth

    if args.micro:
        micro(args.micro)
        return
    e4m3 = args.dtype == "e4m3"
    w = synth.workload(args.workload)
    if e4m3 and w.dtype != "bf16":
        raise SystemExit("--dtype e4m3 needs a bf16 workload")
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    ptype = "e4m3" if e4m3 else w.dtype
    log(f"[bench] workload {w.name}: T={w.T} d={w.d} V={w.V} P={w.P} {ptype}")
    b = Bench(w, dev, e4m3)
    b.prepare(w.P)
    P_eff = w.P if w.P else w.V
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    work = stage_work(w, P_eff, e4m3, cus)
    settled = b.settle(w.P)
    log(f"[bench] {settled} untimed steps while the clock settles")
    stage_ms = b.stage_ms(w.P, max(20, min(args.steps, 50)))
    stages = stage_table(stage_ms, work, ptype)
    log("[bench] stages: " + json.dumps(stages))
    roof = roofline_of(w, stage_ms, work, ptype, e4m3)
    gms = b.graph_ms(w.P, max(100, min(args.steps, 200)))
    log(f"[bench] as a replayed HIP graph: {gms:.4f} ms/step ({w.T / gms * 1e3 / 1e6:.2f} M tokens/s)")
    ms, wall = b.timed(w.P, args.steps, args.warmup)
    b.check_status(w.P)
    log(f"[bench] {ms:.4f} ms/step ({w.T / ms * 1e3 / 1e6:.2f} M tokens/s); wall {wall:.3f} s")
    refresh = None
    if e4m3:
        refresh = b.refresh_us(max(20, min(args.steps, 200)))
        refresh["in_step"] = False
        refresh["note"] = ("the timed step forms the scale and the candidate rows' codes itself; "
                           "the full-cache refresh runs in the overlapped-build leg")
        log(f"[bench] e4m3 full-cache refresh (beside the step): {refresh}")
    pipelined = None
    if w.P > 0 and not args.no_overlap:
        # its first steps run slower (host buffers and the copy stream warming up)
        pms = b.pipelined_ms(max(100, min(args.steps, 200)), max(20, args.warmup))
        pipelined = {"ms_per_step": round(pms, 5), "value": round(w.T / (pms * 1e-3), 1),
                     "how": "next microbatch's candidate set built on the host "
                            "(sce_build_candidates_host) and uploaded on a copy stream while the "
                            "GPU runs the step from the current one "
                            + ("(sce_refresh_e4m3_cache + sampled_ce_forward_backward_fp8_prebuilt)"
                               if e4m3 else "(sampled_ce_forward_backward_prebuilt)")}
        log(f"[bench] with the build overlapped: {pms:.4f} ms/step ({w.T / pms * 1e3 / 1e6:.2f} M tokens/s)")

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
        ref = achievable["gemm_tflops"] if roof["bound"] == "mfma" else achievable["copy_gbs"]
        achievable["dominant_frac"] = round(roof["achieved"] / ref, 4)
        if ptype == "bf16":
            lib = library_same_shapes(torch, dev, w)
            for k in lib:
                lib[k]["ours_us"] = round(stage_ms[k] * 1e3, 1)
            achievable["library_same_shapes"] = lib
        log(f"[bench] achievable on this GPU: {achievable}")

    full_cmp = None
    if not args.no_full_compare and w.P > 0:
        b.prepare(w.V)
        ms_v, _ = b.timed(w.V, max(5, args.steps // 5), 2)
        full_cmp = {"P": w.V, "ms_per_step": round(ms_v, 4), "speedup": round(ms_v / ms, 3)}
        log(f"[bench] same library at P=V: {ms_v:.4f} ms/step -> sampled speedup {ms_v / ms:.2f}x")
    x, W = b.host
    y, p = b.labels0
    b.release()
    del b

    others = None
    if not args.no_other_configs and args.workload == "stage01":
        others = {}
        for name in OTHER_CONFIGS:
            others[name] = other_config(synth.workload(name), dev, e4m3, args, torch)
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
                   "stride": w.stride, "offset": w.offset, "targets": f"zipf({w.zipf_s})",
                   "prefix_targets": w.prefix,
                   **({"operands": "e4m3 x and lm_head, bf16 logits; the lm_head's e4m3 "
                                   "scale and candidate-row codes formed from bf16 W in every "
                                   "step"}
                      if e4m3 else {})},
        "roofline": roof,
        "achievable": achievable,
        "settle_steps": settled,
        "graph_replay": {"ms_per_step": round(gms, 5), "value": round(w.T / (gms * 1e-3), 1)},
        "build_overlapped": pipelined,
        "e4m3_cache_refresh": refresh,
        "stages": stages,
        "full_softmax_same_library": full_cmp,
        "other_configs": others,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def other_config(w, dev, e4m3, args, torch):
    """The step on another configuration the metric names, in the same order of
    measurement (stage timing, then the timed steps), with its dominant kernel's roofline
    and, for a sampled configuration, the same library at P = V on the same microbatch."""
    ptype = "e4m3" if e4m3 else w.dtype
    log(f"[bench] workload {w.name}: T={w.T} d={w.d} V={w.V} P={w.P} {ptype}")
    b = Bench(w, dev, e4m3)
    b.prepare(w.P)
    P_eff = w.P if w.P else w.V
    work = stage_work(w, P_eff, e4m3, torch.cuda.get_device_properties(dev).multi_processor_count)
    settled = b.settle(w.P)
    stage_ms = b.stage_ms(w.P, 12)
    stages = stage_table(stage_ms, work, ptype)
    roof = roofline_of(w, stage_ms, work, ptype, e4m3)
    steps = max(8, args.steps // 2)
    ms, _ = b.timed(w.P, steps, max(4, args.warmup))
    b.check_status(w.P)
    res = {"T": w.T, "P": w.P, "calls": w.calls, "settle_steps": settled, "steps": steps,
           "ms_per_step": round(ms, 4),
           "tokens_per_s": round(w.T / (ms * 1e-3), 1), "roofline": roof, "stages": stages}
    log(f"[bench]   {ms:.4f} ms/step ({w.T / ms * 1e3 / 1e6:.2f} M tokens/s); dominant {roof['kernel']} "
        f"at {roof['frac']:.3f} of peak")
    if w.P > 0 and not args.no_full_compare:
        b.release()
        b.prepare(w.V)
        ms_v, _ = b.timed(w.V, max(4, steps // 2), 2)
        res["full_softmax_same_library"] = {"P": w.V, "ms_per_step": round(ms_v, 4),
                                            "speedup": round(ms_v / ms, 3)}
        log(f"[bench]   same library at P=V: {ms_v:.4f} ms/step -> {ms_v / ms:.2f}x")
    b.release()
    return res


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


def library_same_shapes(torch, dev, w):
    """The vendor library (hipBLASLt through torch.matmul, bf16, 2-D products) on the
    step's three products at this workload's shapes and operand layouts: logits
    x [T, d] @ W_C^T, dX dZ [T, P] @ W_C [P, d], dW dZ^T @ x; microseconds each and the
    fraction of the bf16 peak."""
    T, d, P = w.T, w.d, (w.P or w.V)
    x = torch.randn(T, d, device=dev, dtype=torch.bfloat16)
    Wc = (0.02 * torch.randn(P, d, device=dev)).to(torch.bfloat16)
    Z = (1e-4 * torch.randn(T, P, device=dev)).to(torch.bfloat16)
    fl = 2.0 * T * P * d
    out = {}
    for name, fn in (("logits", lambda: torch.matmul(x, Wc.t())), ("dx", lambda: torch.matmul(Z, Wc)),
                     ("dw", lambda: torch.matmul(Z.t(), x))):
        ms = _time_ms(fn, reps=20, warmup=3)
        out[name] = {"us": round(ms * 1e3, 1),
                     "frac": round(fl / (ms * 1e-3) / 1e12 / PEAK_TFLOPS["bf16"], 4)}
    del x, Wc, Z
    torch.cuda.empty_cache()
    return out


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
    # ~200 ms of device work before the first measurement, so that it sees the settled
    # clock rather than the transient right after an idle period
    a = torch.empty(1 << 28, dtype=torch.uint8, device=dev)
    b = torch.empty_like(a)
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < 0.2:
        for _ in range(10):
            b.copy_(a)
        torch.cuda.synchronize()
    del a, b
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
    """The CPU oracle, as it stands, on the first `sample_tokens` tokens of the same
    microbatch: candidate build (plain C) + dense loss and gradients (plain C, float64,
    OpenMP over token blocks; for the e4m3 step the float64 numpy e4m3 oracle)."""
    from oracle import build_candidates, ce_c, fp8
    from sampled_softmax_cross_amd import synth

    Ts = min(sample_tokens, w.T)
    xs = synth.to_f64(x[:Ts], w.dtype)
    Wf = synth.to_f64(W, w.dtype)
    ys = y[:Ts]
    ps = None if p is None else p[:Ts]
    if e4m3:
        W8, w_scale = fp8.e4m3_cache(Wf)
    t0 = time.perf_counter()
    cand = build_candidates(w.V, w.P, w.stride, w.offset, ys, ps)
    C = None if w.P == 0 else cand["C"]
    ppos = cand["prefix_pos"] if ps is not None else None
    if e4m3:
        fp8.forward_backward(xs, W8, w_scale, C, cand["target_pos"], ppos)
        from threadpoolctl import threadpool_info
        threads = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
        kind = "float64 numpy e4m3 oracle (BLAS threads)"
    else:
        ce_c.forward_backward(xs, Wf, C, cand["target_pos"], ppos)
        threads = ce_c.threads()
        kind = "plain C float64 oracle, OpenMP over token blocks"
    dt = time.perf_counter() - t0
    return {"value": round(Ts / dt, 1), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "nproc": os.cpu_count(), "seconds": round(dt, 2),
            "sample": f"first {Ts} of {w.T} tokens of the {w.name} microbatch (same P, V, d, "
                      f"stride, offset; C built from these tokens): candidate build + loss, dX, "
                      f"dW by the {kind}"}


if __name__ == "__main__":
    main()
