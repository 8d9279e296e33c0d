#!/usr/bin/env python3
"""Benchmark of the MoE layer hot path (route -> align -> SwiGLU grouped GEMM
-> combine) on one MI355X.

A step is one whole-layer call (moe_layer) over one batch of seeded synthetic
inputs already resident in HBM.  The default workload is the Mixtral-8x7B
shaped prefill layer (T=4096, H=4096, E=8, top-2, I=14336, bf16).  Right
after the K timed steps, K more layer calls each record six events of the
bench's around their five steps (moe_layer_aux.stage_events), which time
every step inside a layer call; the dominant kernel's roofline is computed
from its average there and its algorithmic flops/bytes.  Then K launches of each step
(through its own entry point) are captured in a HIP graph and replayed
between two HIP events, for each kernel's time launched back to back, and a
cold pass (after a 1 GiB write) gives each step's time with its inputs in
HBM.  The CPU oracle is timed on a bounded token
sample of the same workload on the host cores (a baseline, not the target).

Prints exactly one JSON line.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/s; grouped-GEMM % MFMA peak; route+combine % HBM BW"
PEAK_HBM_GBPS = 8000.0
# W4A16 ("i4") widens its int4 weights to bf16 and runs the bf16 MFMA
PEAK_TFLOPS = {"bf16": 2500.0, "i8": 5000.0, "f32": 157.3, "i4": 2500.0, "i4a8": 5000.0}
RIDGE = {k: v * 1e12 / (PEAK_HBM_GBPS * 1e9) for k, v in PEAK_TFLOPS.items()}   # flop per byte
CPU_SAMPLE = {1: 64, 2: 4096, 3: 64, 4: 16, 5: 512}
BYTES = {"f32": 4, "bf16": 2, "i8": 1, "i4": 0.5, "i4a8": 0.5}
A8 = ("i8", "i4a8")                  # schemes that quantise activations per token


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse() -> argparse.Namespace:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=2, help="workload 1..5 (default 2, Mixtral-shaped prefill)")
    ap.add_argument("--w-dtype", choices=("bf16", "i8", "i4", "i4a8"), default=None,
                    help="run the workload with these expert weights instead of its own (i4: W4A16 with "
                         "int4 codes and per-channel scales, packed on the device; i4a8: the same weights "
                         "with per-token int8 activations, W4A8)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--library-ref", action="store_true",
                    help="also time hipBLASLt (torch.bmm) on the same GEMM shapes, for context (off by default)")
    ap.add_argument("--cpu-sample", type=int, default=None, help="tokens in the oracle's timed sample")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (to calibrate HBM byte counters) and exit")
    return ap.parse_args()


def to_dev(a, torch):
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(a).cuda()


class Staged:
    """The layer as its separate launches with preallocated buffers, for
    per-kernel timing with events between launches."""

    def __init__(self, moe, torch, spec, d, C, from_route=False):
        import ctypes
        self.moe, self.torch, self.spec, self.d, self.C = moe, torch, spec, d, C
        # the layer's align step takes the route step's per-workgroup counts:
        # time route + align as moe_route_align runs them (the layer's
        # launches) and report align as that minus the route alone
        self.from_route = from_route
        L = moe.lib
        T, H, E, k, I = spec.T, spec.H, spec.E, spec.k, spec.I
        n = T * k
        dev = "cuda"
        i32, f32 = torch.int32, torch.float32
        wdt = "w4a8" if spec.w_dtype == "i4a8" else d["w13"].dtype
        self.wd = moe.binding._DT[wdt]
        self.quant = spec.w_dtype in A8
        self.ids = torch.empty((T, k), dtype=i32, device=dev)
        self.w = torch.empty((T, k), dtype=f32, device=dev)
        self.xq = torch.empty((T, H), dtype=torch.int8, device=dev) if self.quant else None
        self.xs = torch.empty(T, dtype=f32, device=dev) if self.quant else None
        self.bm = moe.ffn_block_m(T, H, I, E, k, wdt)
        mt = int(L.moe_align_max_tiles(T, k, E, self.bm))
        self.counts = torch.empty(E, dtype=i32, device=dev)
        self.offsets = torch.empty(E + 1, dtype=i32, device=dev)
        self.sorted_slot = torch.empty(n, dtype=i32, device=dev)
        self.pos = torch.empty(n, dtype=i32, device=dev)
        self.tiles = torch.empty((mt, 4), dtype=i32, device=dev)
        self.num_tiles = torch.empty(1, dtype=i32, device=dev)
        self.num_dropped = torch.empty(1, dtype=i32, device=dev)
        ydt = torch.float32 if spec.w_dtype == "f32" else torch.bfloat16
        self.y = torch.empty((n, H), dtype=ydt, device=dev)
        self.out = torch.empty((T, H), dtype=d["x"].dtype, device=dev)
        self.n_route = int(L.moe_route_workspace_size(T, H, E, k))
        self.n_align = int(L.moe_align_workspace_size(T, k, E))
        self.n_ffn = int(L.moe_ffn_workspace_size(T, H, I, E, k, self.wd))
        self.n_ra = int(L.moe_route_align_workspace_size(T, H, E, k))
        mx = max(self.n_route, self.n_align, self.n_ffn, self.n_ra, 1)
        self.ws = torch.empty(mx, dtype=torch.uint8, device=dev)
        self.P = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())
        self.DT = moe.binding._DT

    def stages(self):
        """(name, launch) for each step; each is idempotent once a full pass
        has filled its inputs."""
        L, P, DT, s, d = self.moe.lib, self.P, self.DT, self.spec, self.d
        T, H, E, k, I = s.T, s.H, s.E, s.k, s.I
        st = self.moe.binding._stream(d["x"].device)
        chk = self.moe.binding._check
        ws = P(self.ws)
        act = self.xq if self.quant else d["x"]

        def route():
            chk(L.moe_route(P(d["x"]), DT[d["x"].dtype], P(d["wg"]), DT[d["wg"].dtype], P(d["bias"]), T, H, E, k,
                            P(self.ids), P(self.w), None, P(self.xq), P(self.xs), ws, self.n_route, st))

        def align():
            chk(L.moe_align(P(self.ids), T, k, E, self.C, self.bm, P(self.counts), P(self.offsets),
                            P(self.sorted_slot), P(self.pos), P(self.tiles), P(self.num_tiles),
                            P(self.num_dropped), ws, self.n_align, st))

        def route_align():
            chk(L.moe_route_align(P(d["x"]), DT[d["x"].dtype], P(d["wg"]), DT[d["wg"].dtype], P(d["bias"]), T, H, E,
                                  k, self.C, self.bm, P(self.ids), P(self.w), None, P(self.xq), P(self.xs),
                                  P(self.counts), P(self.offsets), P(self.sorted_slot), P(self.pos), P(self.tiles),
                                  P(self.num_tiles), P(self.num_dropped), ws, self.n_ra, st))

        def up():
            chk(L.moe_ffn_up(P(act), DT[act.dtype], P(self.xs), P(d["w13"]), self.wd, P(d["s13"]),
                             P(self.sorted_slot), P(self.tiles), P(self.num_tiles), self.bm, T, H, I, E, k, ws,
                             self.n_ffn, st))

        def down():
            chk(L.moe_ffn_down(P(d["w2"]), self.wd, P(d["s2"]), P(self.sorted_slot), P(self.tiles),
                               P(self.num_tiles), self.bm, P(self.w), T, H, I, E, k, P(self.y), DT[self.y.dtype],
                               ws, self.n_ffn, st))

        def combine():
            chk(L.moe_combine(P(self.y), DT[self.y.dtype], P(self.pos), None, T, k, H, P(self.out),
                              DT[self.out.dtype], st))

        if self.from_route:
            return [("route", route), ("route_align", route_align), ("ffn_up", up), ("ffn_down", down),
                    ("combine", combine)]
        return [("route", route), ("align", align), ("ffn_up", up), ("ffn_down", down), ("combine", combine)]

    def run(self):
        for _, fn in self.stages():
            fn()

    def time_each(self, reps: int) -> dict:
        """Average GPU time of each step: `reps` launches of it captured in one
        HIP graph, replayed between two events on the replaying stream, so
        the host's per-call cost (ctypes, launch) does not enter the small
        kernels' times."""
        torch = self.torch
        out = {}
        for i, (name, fn) in enumerate(self.stages()):
            fn()
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                cap = self.stages()[i][1]      # bound to the capturing stream
                for _ in range(reps):
                    cap()
            g.replay()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            g.replay()
            e1.record()
            torch.cuda.synchronize()
            out[name] = e0.elapsed_time(e1) / reps
            del g
        return out


def traffic_for(workload: str, kernel_src: str):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they were
    taken on the current kernel source (else None)."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    sha = hashlib.sha256(open(kernel_src, "rb").read()).hexdigest()
    if rec.get("kernel_source_sha256") != sha:
        return None
    return rec.get("hbm_bytes_per_launch")


def library_gemm_reference(torch, spec, d, N: int, D: int):
    """hipBLASLt (torch.bmm) on the up and down GEMM shapes of this workload,
    for context: D experts x ceil(N/D) rows, no gather and no epilogue."""
    if spec.w_dtype != "bf16" or D == 0:
        return None
    m = -(-N // D)
    H, I = spec.H, spec.I
    e = torch.nonzero(torch.ones(spec.E)).flatten()[:D]
    res = {}
    for name, b, k_, n_ in (("up", d["w13"], H, 2 * I), ("down", d["w2"], I, H)):
        bt = b[e.to(b.device)].transpose(1, 2).contiguous()    # [D, K, N], contiguous right operand
        a = torch.randn(D, m, k_, device="cuda").to(torch.bfloat16)
        torch.bmm(a, bt)
        torch.cuda.synchronize()
        c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        c0.record()
        for _ in range(5):
            torch.bmm(a, bt)
        c1.record()
        torch.cuda.synchronize()
        ms = c0.elapsed_time(c1) / 5
        res[name] = {"shape": [D, m, k_, n_], "ms": ms,
                     "frac_of_peak": 2.0 * D * m * k_ * n_ / (ms * 1e-3) / 1e12 / PEAK_TFLOPS["bf16"]}
        del bt, a
    return res


def _cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _blas_threads() -> int | None:
    try:
        import threadpoolctl
        blas = [i["num_threads"] for i in threadpoolctl.threadpool_info() if i.get("user_api") == "blas"]
        return max(blas) if blas else None
    except Exception:
        return None


def routing_vs_oracle(ids_gpu: np.ndarray, r: dict) -> dict:
    """The near-tie accounting of the top-k contract: rows whose oracle
    k-th/(k+1)-th probability gap is below 1e-4 (the band), GPU ids that
    differ from the oracle's inside and outside the band, and rows outside it
    whose ids differ only in the order of selected experts with oracle
    probabilities within 1e-6 (the order of near-equal keys)."""
    ids_o = r["ids"]
    band = r["gap_p"] < 1e-4
    diff = ~(ids_gpu == ids_o).all(axis=1)
    swaps, other = 0, 0
    for t in np.nonzero(diff & ~band)[0]:
        pg = r["p"][t, ids_gpu[t]]
        if set(ids_gpu[t].tolist()) == set(ids_o[t].tolist()) and np.all(np.diff(pg) <= 1e-6):
            swaps += 1
        else:
            other += 1
    return {"tokens": int(len(ids_o)), "band_size": int(band.sum()), "band_logit_gap": int((r["gap_logit"] < 1e-4).sum()),
            "mismatched_in_band": int((diff & band).sum()), "order_swaps_outside_band": swaps,
            "mismatched_outside_band": other}


def cpu_baseline(cfg: int, sample_n: int, spec=None, ids_gpu=None) -> dict:
    """The CPU oracle on a bounded token sample of the workload, in whole
    passes until about 10 s have run; with the GPU's top-k ids, also the
    near-tie accounting against the oracle's routing of every token."""
    import moe_synth
    import oracle
    inp = moe_synth.config_inputs(cfg) if spec is None else moe_synth.make_inputs(spec, 1000 * cfg)
    T = inp.spec.T
    S = min(sample_n, T)
    sample = np.sort(np.random.default_rng(7).choice(T, size=S, replace=False))
    blas = _blas_threads()
    passes, t0 = 0, time.perf_counter()
    while True:
        res = oracle.layer_from_inputs(inp, sample_tokens=sample)
        passes += 1
        dt = time.perf_counter() - t0
        if dt >= 10.0:
            break
    out = {"value": passes * S / dt, "unit": "tokens/s", "cores": int(blas or os.cpu_count() or 1), "kind": "oracle",
           "sample": f"{passes} pass(es) over {S} of {T} tokens of {inp.spec.name} (routing and align over all "
                     f"{T} tokens, expert FFN and combine for the sample; fp64 NumPy/OpenBLAS), {dt:.1f} s",
           "cpu_model": _cpu_model(), "os_cpu_count": os.cpu_count(), "blas_threads": blas}
    if ids_gpu is not None:
        out["routing_vs_oracle"] = routing_vs_oracle(ids_gpu, res["route"])
    return out


def main() -> int:
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (the MoE path has no multi-GPU code); got --gpus {args.gpus}",
              file=sys.stderr)
        return 2
    import torch

    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "launches": 3}), flush=True)
        return 0

    import moe_synth
    import routing_dispatch_expert_gate_amd as moe

    cfg = args.config
    spec = moe_synth.CONFIGS[cfg]
    if args.w_dtype and args.w_dtype != spec.w_dtype:
        tag = {"bf16": "w16a16", "i8": "w8a8", "i4": "w4a16", "i4a8": "w4a8"}[args.w_dtype]
        spec = spec.replace(w_dtype=args.w_dtype, name=f"{spec.name}_{tag}")
    T, H, E, k, I = spec.T, spec.H, spec.E, spec.k, spec.I
    log(f"workload {cfg}: {spec.name}; generating inputs")
    inp = moe_synth.make_inputs(spec, 1000 * cfg)
    d = {n: to_dev(getattr(inp, n), torch) for n in ("x", "wg", "bias", "w13", "w2", "s13", "s2")}
    if spec.w_dtype in ("i4", "i4a8"):
        # offline weight preparation: int4 codes -> the packed layout
        d["w13"], d["w2"] = moe.pack_int4(d["w13"]), moe.pack_int4(d["w2"])
        inp.w13 = inp.w2 = None
        torch.cuda.synchronize()
    C = moe.capacity(T, k, E, spec.capacity_factor) if spec.capacity_factor > 0 else 0
    layer = moe.Layer(T, H, I, E, k, d["x"].dtype, "w4a8" if spec.w_dtype == "i4a8" else d["w13"].dtype)
    counts = torch.empty(E, dtype=torch.int32, device="cuda")
    offsets = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    out = torch.empty((T, H), dtype=d["x"].dtype, device="cuda")
    ids_buf = torch.empty((T, k), dtype=torch.int32, device="cuda")
    aux = {"counts": counts, "offsets": offsets, "topk_ids": ids_buf}

    def step(with_aux=False, events=None):
        layer(d["x"], d["wg"], d["w13"], d["w2"], C, d["bias"], d["s13"], d["s2"], out=out,
              aux=aux if with_aux else ({"stage_events": events} if events else None))

    step(True)
    torch.cuda.synchronize()
    dispatch = moe.last_dispatch()
    ids_gpu = ids_buf.cpu().numpy()
    off = offsets.cpu().numpy()
    kept = np.diff(off)
    N, D = int(off[-1]), int((kept > 0).sum())
    log(f"dispatch: {dispatch}; N={N} D={D}")

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    t0 = time.perf_counter()
    evs[0].record()
    for i in range(args.steps):
        step()
        evs[i + 1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps
    per_step = np.array([evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps)])
    gpu_ms = float(per_step.mean())
    log(f"layer: {ms_per_step:.3f} ms/step wall, {gpu_ms:.3f} ms/step on the stream "
        f"(p10 {np.percentile(per_step, 10):.3f}, median {np.median(per_step):.3f}, "
        f"p90 {np.percentile(per_step, 90):.3f})")
    # the same layer calls again, K of them right after the timed ones, each
    # recording six events of the bench's around its five steps
    # (moe_layer_aux.stage_events): every step timed inside a layer call, in
    # the layer's order and on the layer's stream.  The timed steps above
    # carry no events: each record costs ~3.5 us on the GPU's timeline (+4%
    # at the decode workload, +60% at the tiny one).
    ev_sets = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(args.steps)]
    for es in ev_sets:
        for e in es:
            e.record()                      # torch creates its events lazily, at the first record
    torch.cuda.synchronize()
    for es in ev_sets:
        step(events=[e.cuda_event for e in es])
    torch.cuda.synchronize()
    step_names = ("route", "align", "ffn_up", "ffn_down", "combine")
    in_layer = {n: float(np.mean([es[j].elapsed_time(es[j + 1]) for es in ev_sets]))
                for j, n in enumerate(step_names)}
    log("steps inside layer calls (ms): " + ", ".join(f"{n}={v:.4f}" for n, v in in_layer.items()))

    # per-kernel durations: each step (entry point) launched back to back
    # `steps` times between two events on the library's stream
    st = Staged(moe, torch, spec, d, C, from_route="align(from route counts" in dispatch)
    names = [n for n, _ in st.stages()]
    for _ in range(max(2, args.warmup)):
        st.run()
    torch.cuda.synchronize()
    stage_ms = st.time_each(args.steps)
    if st.from_route:
        stage_ms["align"] = stage_ms.pop("route_align") - stage_ms["route"]
    log("stages (ms): " + ", ".join(f"{n}={v:.4f}" for n, v in stage_ms.items()))

    # isolated cold: a 1 GiB write before each staged pass evicts L2 and the
    # last-level cache, so every stage reads its inputs from HBM (the host
    # queues the pass's launches while the write runs, so events between them
    # time the GPU)
    flush = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")

    def cold_pass(fns):
        acc = np.zeros(len(fns))
        for i in range(args.steps):
            flush.fill_(i & 0xFF)
            evs = [torch.cuda.Event(enable_timing=True) for _ in range(len(fns) + 1)]
            evs[0].record()
            for j, fn in enumerate(fns):
                fn()
                evs[j + 1].record()
            torch.cuda.synchronize()
            acc += [evs[j].elapsed_time(evs[j + 1]) for j in range(len(fns))]
        return (acc / args.steps).tolist()

    stage_fns = dict(st.stages())
    if st.from_route:
        # route alone, then (after another write) route + align as the layer
        # runs them and the rest: the align share is the difference
        route_cold = cold_pass([stage_fns["route"]])[0]
        rest = cold_pass([stage_fns[n] for n in ("route_align", "ffn_up", "ffn_down", "combine")])
        cold_ms = {"route": route_cold, "align": rest[0] - route_cold, "ffn_up": rest[1], "ffn_down": rest[2],
                   "combine": rest[3]}
    else:
        cold_ms = dict(zip(names, cold_pass([stage_fns[n] for n in names])))
    log("stages cold (ms): " + ", ".join(f"{n}={v:.4f}" for n, v in cold_ms.items()))
    # measured streaming rate: a 1 GiB device copy (read + write)
    dst = torch.empty_like(flush)
    dst.copy_(flush)
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0.record()
    for _ in range(5):
        dst.copy_(flush)
    c1.record()
    torch.cuda.synchronize()
    copy_GBps = 5 * 2 * flush.numel() / (c0.elapsed_time(c1) * 1e-3) / 1e9
    del flush, dst
    # measured MFMA rate: a dense loop of MFMA 32x32x16 bf16 from registers
    # (one workgroup of 4 waves per CU), best of three launches; the probe is
    # a bench-only library outside the MoE ABI
    probe_lib = ctypes.CDLL(os.path.join(ROOT, "routing_dispatch_expert_gate_amd", "libmoe_probe.so"))
    probe_lib.moe_probe_mfma_rate.restype = ctypes.c_int
    probe_lib.moe_probe_mfma_rate.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]
    probe = torch.empty(256 * 256, device="cuda")
    pst = moe.binding._stream(probe.device)
    mfma_iters, mfma_best = 20000, float("inf")
    for _ in range(4):
        m0, m1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        m0.record()
        rc = probe_lib.moe_probe_mfma_rate(256, mfma_iters, ctypes.c_void_p(probe.data_ptr()), pst)
        m1.record()
        torch.cuda.synchronize()
        if rc != 0:
            raise RuntimeError(f"moe_probe_mfma_rate returned {rc}")
        mfma_best = min(mfma_best, m0.elapsed_time(m1))
    mfma_TFLOPs = 256 * mfma_iters * 4 * 16 * 32768 / (mfma_best * 1e-3) / 1e12
    del probe
    log(f"measured: copy {copy_GBps:.0f} GB/s, dense MFMA bf16 loop {mfma_TFLOPs:.0f} TFLOP/s")
    lib_ref = library_gemm_reference(torch, spec, d, N, D) if args.library_ref else None

    # algorithmic work (bytes / flops the method must move or do)
    bx, bg, bw = BYTES[spec.x_dtype], BYTES[spec.wg_dtype], BYTES[spec.w_dtype]
    by = 4 if spec.w_dtype == "f32" else 2
    bo = BYTES[spec.out_dtype]
    ba = 1 if spec.w_dtype in A8 else bx                    # activation bytes the up GEMM reads
    bh = 1 if spec.w_dtype in A8 else by                    # h bytes the down GEMM reads
    up_flops = 4.0 * N * H * I
    down_flops = 2.0 * N * H * I
    up_bytes = D * 2 * I * H * bw + N * H * ba + N * I * by      # h is written in bf16 (fp32 for f32)
    down_bytes = D * H * I * bw + N * I * bh + N * H * by
    route_bytes = T * H * bx + E * H * bg + 8 * T * k + (T * H + 4 * T if spec.w_dtype in A8 else 0)
    align_bytes = 12 * T * k
    combine_bytes = N * H * by + T * H * bo + 4 * T * k
    dt = spec.w_dtype
    # the dominant kernel's time: its average inside the layer calls
    up_s = in_layer["ffn_up"] * 1e-3
    ai = up_flops / up_bytes
    if ai >= RIDGE[dt]:
        roof = {"bound": "mfma", "achieved": up_flops / up_s / 1e12, "peak": PEAK_TFLOPS[dt],
                "unit": "TFLOP/s" if dt not in A8 else "TOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": up_bytes / up_s / 1e9, "peak": PEAK_HBM_GBPS, "unit": "GB/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["kernel"] = "up GEMM: " + (dispatch.split("|")[2].strip().split("+")[0]
                                     if dispatch.count("|") >= 3 else "gg_kernel")
    roof["per_launch"] = {"flops": up_flops, "bytes": up_bytes, "ms": in_layer["ffn_up"],
                          "timed": "average inside K layer calls run right after the timed ones, between "
                                   "events the layer records around its steps",
                          "ms_back_to_back": stage_ms["ffn_up"]}
    roof["traffic"] = traffic_for(spec.name, os.path.join(ROOT, "routing_dispatch_expert_gate_amd", "csrc",
                                                          "ffn.hip"))
    gemm_s = (stage_ms["ffn_up"] + stage_ms["ffn_down"]) * 1e-3
    rac_s = (stage_ms["route"] + stage_ms["align"] + stage_ms["combine"]) * 1e-3
    rac_bytes = route_bytes + align_bytes + combine_bytes
    extra = {
        "grouped_gemm": {"flops": up_flops + down_flops, "ms": gemm_s * 1e3,
                         "tflops": (up_flops + down_flops) / gemm_s / 1e12,
                         "frac_of_peak": (up_flops + down_flops) / gemm_s / 1e12 / PEAK_TFLOPS[dt],
                         "peak_dtype": dt,
                         "hbm_GBps_alg": (up_bytes + down_bytes) / gemm_s / 1e9},
        "route_align_combine": {"bytes": rac_bytes, "ms": rac_s * 1e3,
                                "GBps": rac_bytes / rac_s / 1e9,
                                "frac_of_hbm": rac_bytes / rac_s / 1e9 / PEAK_HBM_GBPS},
        "stages_ms": stage_ms,
        "stages_ms_in_layer": in_layer,
        "stages_ms_cold": cold_ms,
        "route_align_combine_cold": {"ms": sum(cold_ms[n] for n in ("route", "align", "combine")),
                                     "frac_of_hbm": rac_bytes / (sum(cold_ms[n] for n in ("route", "align", "combine"))
                                                                 * 1e-3) / 1e9 / PEAK_HBM_GBPS},
        "layer_ms_p10_p50_p90": [float(np.percentile(per_step, 10)), float(np.median(per_step)),
                                 float(np.percentile(per_step, 90))],
        "measured_copy_GBps": copy_GBps,
        "measured_mfma_bf16_TFLOPs": mfma_TFLOPs,
        "library_bmm_same_shapes": lib_ref,
        "kept_rows_N": N, "active_experts_D": D, "capacity": C,
        "layer_gpu_ms": gpu_ms,
        "dispatch": dispatch,
    }

    cpu = None
    if not args.no_cpu_baseline:
        n = args.cpu_sample or CPU_SAMPLE[cfg]
        log(f"timing the CPU oracle on {n} tokens")
        cpu = cpu_baseline(cfg, n, spec, ids_gpu)

    rec = {
        "metric": METRIC, "value": T / (ms_per_step * 1e-3), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_per_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": {"bf16": "bf16", "i8": "int8 (W8A8)", "f32": "f32", "i4": "bf16 MFMA on int4 weights (W4A16)",
                  "i4a8": "int8 MFMA on int4 weights (W4A8)"}[spec.w_dtype],
        "data": "synthetic (seeded; random-init weights of the workload's shapes)",
        "config": {"workload": spec.name, "T": T, "H": H, "E": E, "top_k": k, "I": I,
                   "capacity": C, "x_dtype": spec.x_dtype, "w_dtype": spec.w_dtype,
                   "parallelism": "single GPU"},
        "roofline": roof,
        "cpu_baseline": cpu,
        "detail": extra,
    }
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
