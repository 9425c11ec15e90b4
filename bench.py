"""Benchmark: the exponent-compressed, Llama-3.1-8B-shaped MLP stack on one MI355X.

Workload: 32 SwiGLU MLP layers of Llama-3.1-8B's shape -- gate and up 14336 x 4096, down
4096 x 14336, bf16 weights ~ N(0, sigma_l) with sigma_l = 0.02 * U(0.8, 1.2) per layer,
synthetic and seeded -- every projection held exponent-compressed on the GPU and run
through the plan the autotuner measured for its shape and batch size (pipeline, GEMM
variant, K split). Every layer reads the same X (M x 4096 bf16 ~ N(0, 1)).

One step = one forward of the whole stack (per layer: gate, up, SwiGLU, down) for each
batch size M in {1, 16, 64}: the small-batch regime, bound by the weight bytes read from
HBM. value = the uncompressed-equivalent weight bytes of those three forwards (3 x 96
matrices x 2 N K bytes) per second of the step. Inputs are resident in HBM when the
timed region starts; the timed region is `steps` steps launched back to back between two
HIP events on the launch stream.

The JSON line also carries:
  roofline      the step's dominant kernel (the largest share of the step): algorithmic
                HBM bytes per launch / its mean launch duration (HIP events around back-
                to-back launches over the 32 layers, on the launch stream) vs 8 TB/s, and
                the read rate of a plain streaming kernel over the same planes
  large_m       the same stack forward at M = 1024 and 4096 (MFMA-bound): TFLOP/s and
                the fraction of the 2.5 PFLOP/s bf16 peak, and each projection's GEMM alone
  cpu_baseline  the CPU oracle (bit-serial decode + fp64 GEMM) on a bounded sample of the
                same workload, on one thread and on all host cores
  detail        the plans, and the single-matrix gate-shaped workload (14336 x 4096 with
                0.01% outliers) through every pipeline, and each decoder alone
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
SMALL_MS = (1, 16, 64)
LARGE_MS = (1024, 4096)
ROLES = ("gate", "up", "down")
# measured HBM traffic of the dominant kernel (rocprofv3 FETCH_SIZE / WRITE_SIZE runs,
# scaled by the counters of a copy of known size); used only while the GEMM sources
# still hash to what was profiled
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemm_gate_up_stack_traffic.json")
GEMM_SOURCES = ["decode_gemm_amd/csrc/uw_gemm.hip", "decode_gemm_amd/csrc/uw_recon.h",
                "decode_gemm_amd/csrc/uw_internal.h"]


def gemm_sources_sha256():
    import hashlib

    hsh = hashlib.sha256()
    for f in GEMM_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            hsh.update(fh.read())
    return hsh.hexdigest()


def measured_traffic(key):
    """HBM bytes per launch of `key` from the committed counter summary, or None when the
    summary is missing, does not cover `key`, or the kernel sources changed since."""
    try:
        with open(TRAFFIC_FILE) as fh:
            t = json.load(fh)
    except (OSError, ValueError):
        return None
    if t.get("sources_sha256") != gemm_sources_sha256():
        return None
    k = t.get("kernels", {}).get(key)
    return None if k is None else int(k["hbm_bytes_per_launch"])


def parse(argv=None):
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU-oracle baseline")
    p.add_argument("--no-detail", action="store_true", help="skip the single-matrix pipelines and decoders")
    p.add_argument("--no-large", action="store_true", help="skip the M = 1024 / 4096 stack forwards")
    p.add_argument("--plans", help="read the plans from this JSON file (written by --save-plans) instead of tuning")
    p.add_argument("--save-plans", help="write the measured plans to this JSON file")
    p.add_argument("--copy-probe", action="store_true", help="also launch a plain 256 MiB copy kernel (counter scale)")
    p.add_argument("--no-70b", action="store_true", help="skip the 70B-shaped layer")
    p.add_argument("--schedules", action="store_true",
                   help="also time the hard/easy stack: one stream, a decode stream, CU-split pairs, tuned end to end")
    return p.parse_args(argv)


# ---------------------------------------------------------------- byte accounting
def section_bytes(h):
    """Bytes of each section of the Huffman-format blob."""
    N, K = h.N, h.K
    return {"sm": N * K, "stream": h.bytes_stream, "offs": 4 * (h.n_chunks + 1), "bitmap": 4 * N * h.bitmap_words,
            "row_base": 4 * (N + 1), "raw": 64 * h.n_raw}


def direct_bytes(h):
    """Bytes of the load-time direct-palette plane (blocks, meta, raw side table)."""
    T, G = (h.N + 15) // 16, h.K // 64
    return 1536 * T * G + (8 * T * G + 63) // 64 * 64 + 64 * h.n_raw


def decode_bytes(h, mode):
    """HBM bytes a decoder must read and write: the blob sections it consumes and its output."""
    s = section_bytes(h)
    NK = h.N * h.K
    codes = s["stream"] + s["offs"] + s["bitmap"]
    return {"full": s["sm"] + codes + s["row_base"] + s["raw"] + 2 * NK,
            "exp": codes + s["row_base"] + s["raw"] + NK,
            "idx": codes + NK // 2,
            "direct": s["sm"] + codes + s["row_base"] + s["raw"] + direct_bytes(h),
            "expand": direct_bytes(h) + 2 * NK}[mode]


def gemm_bytes(h, M, src):
    """HBM bytes of the GEMM kernel alone: its weight planes, X and Y."""
    s = section_bytes(h)
    NK = h.N * h.K
    w = {0: 2 * NK, 1: 2 * NK, 2: NK // 2 + NK + s["bitmap"] + s["row_base"] + s["raw"], 3: direct_bytes(h)}[src]
    return w + 2 * M * h.K + 4 * M * h.N


def algorithmic_bytes(h, M, pipeline):
    """HBM bytes a pipeline must move per forward: the decoder's reads and writes (none for
    direct palette, whose plane is made at load) plus the GEMM's."""
    if pipeline == 3:
        return gemm_bytes(h, M, 3)
    mode, src = {0: ("full", 0), 1: ("exp", 1), 2: ("idx", 2), 4: ("expand", 0)}[pipeline]
    return decode_bytes(h, mode) + gemm_bytes(h, M, src)


def resident_bytes(h, pipeline, blob_bytes):
    """B_res: the resident bytes of the format a pipeline starts from (the Huffman blob for
    full / exponent / transcode, the direct plane for direct palette and expand)."""
    return direct_bytes(h) if pipeline in (3, 4) else blob_bytes


def gate_up_bytes(hg, hu, M):
    """The fused gate/up/SwiGLU launch: both direct planes, X, g and u (fp32), h (bf16)."""
    return direct_bytes(hg) + direct_bytes(hu) + 2 * M * hg.K + 4 * M * hg.N + 4 * M * hu.N + 2 * M * hg.N


# ---------------------------------------------------------------- the stack
class Stack:
    """MLP layers on the device (the 32-layer stack, or the one 70B-shaped layer): per (layer,
    role) the header, the blob and the direct plane made from it at load."""

    def __init__(self, uw, synth, torch, dev, log, cfg_name="stack"):
        import concurrent.futures as cf

        self.cfg = cfg = synth.CONFIGS[cfg_name]
        self.L = cfg.layers
        sig = synth.gen_stack_sigmas(cfg) if cfg.layers > 1 else None
        t0 = time.time()

        def make(i):
            layer, q = divmod(i, 3)
            return uw.encode(synth.gen_weight(cfg, ROLES[q], layer, sigma=None if sig is None else float(sig[layer])))

        self.h = [[None] * 3 for _ in range(self.L)]
        self.blob = [[None] * 3 for _ in range(self.L)]
        self.plane = [[None] * 3 for _ in range(self.L)]
        self.blob_bytes = [[0] * 3 for _ in range(self.L)]
        workers = max(1, min(16, os.cpu_count() or 8))
        with cf.ThreadPoolExecutor(workers) as ex:
            for i, b in enumerate(ex.map(make, range(3 * self.L))):
                layer, q = divmod(i, 3)
                h = uw.inspect(b)
                db = torch.from_numpy(b).to(dev)
                dp = torch.empty(uw.direct_plane_bytes(h), dtype=torch.uint8, device=dev)
                uw.prepare_direct(h, db, dp)
                self.h[layer][q], self.blob[layer][q], self.plane[layer][q] = h, db, dp
                self.blob_bytes[layer][q] = b.size
        torch.cuda.synchronize()
        self.Nff, self.K = self.h[0][0].N, self.h[0][0].K
        self.weight_bytes = sum(2 * h.N * h.K for row in self.h for h in row)
        self.macs = sum(h.N * h.K for row in self.h for h in row)
        blob_total = sum(sum(r) for r in self.blob_bytes)
        plane_total = sum(uw.direct_plane_bytes(h) for row in self.h for h in row)
        log(f"[bench] {cfg.name}: {3 * self.L} matrices encoded and prepared in {time.time() - t0:.1f}s; "
            f"Huffman {blob_total / 1e9:.2f} GB ({blob_total / self.weight_bytes * 2:.3f} B/w), direct planes "
            f"{plane_total / 1e9:.2f} GB ({plane_total / self.weight_bytes * 2:.3f} B/w), bf16 {self.weight_bytes / 1e9:.2f} GB")
        self.blob_total, self.plane_total = blob_total, plane_total

    def rot(self, uw, q):
        return [uw.proj(self.h[l][q], self.blob[l][q], d_direct=self.plane[l][q]) for l in range(self.L)]

    def layers(self, uw, plans_m):
        """uw_mlp_layer array with gate and up on plans_m['gate'], down on plans_m['down']."""
        rows = []
        for l in range(self.L):
            trip = []
            for q in range(3):
                p = plans_m["down" if q == 2 else "gate"]
                trip.append(uw.proj(self.h[l][q], self.blob[l][q], p["pipeline"], d_direct=self.plane[l][q],
                                    variant=p["variant"], split_k=p["split_k"]))
            rows.append(trip)
        return uw.mlp_layers(rows)


def fusable_mask(uw, torch, dev, stack, M):
    """Bit v set: the fused gate/up/SwiGLU launch takes variant v (with the variant's own K
    split) at M -- found by launching it once with each on layer 0."""
    K, N = stack.K, stack.Nff
    x = torch.zeros(M, K, dtype=torch.int16, device=dev)
    g = torch.empty(M, N, dtype=torch.float32, device=dev)
    u = torch.empty_like(g)
    h = torch.empty(M * N, dtype=torch.int16, device=dev)
    mask = 0
    for v in range(uw.variant_count()):
        try:
            uw.recon_gemm_gate_up(stack.h[0][0], stack.blob[0][0], stack.plane[0][0], stack.h[0][1], stack.blob[0][1],
                                  stack.plane[0][1], x, g, u, h, M, variant=v, split_k=0)
            mask |= 1 << v
        except uw.UwError as e:
            if e.status != uw.EUNSUPPORTED:
                raise
    torch.cuda.synchronize()
    return mask


def tune_fused(uw, torch, dev, stack, M, vmask, stream):
    """The fused gate/up/SwiGLU launch's variant at M: each variant in vmask timed as the
    stack runs it (the 32 layers back to back, HIP-graph replay), the fastest kept.
    Returns (variant, ms per launch)."""
    K, N = stack.K, stack.Nff
    x = torch.from_numpy(np.zeros((M, K), np.int16)).to(dev)
    g = torch.empty(M, N, dtype=torch.float32, device=dev)
    u = torch.empty_like(g)
    h = torch.empty(M * N, dtype=torch.int16, device=dev)
    best = (None, float("inf"))
    for v in range(uw.variant_count()):
        if not (vmask >> v) & 1:
            continue
        fn = (lambda v: lambda l: uw.recon_gemm_gate_up(
            stack.h[l][0], stack.blob[l][0], stack.plane[l][0], stack.h[l][1], stack.blob[l][1], stack.plane[l][1], x,
            g, u, h, M, variant=v, split_k=0))(v)
        ms = min(time_op(torch, stream, stack, fn, 3, graph=True) for _ in range(2))
        if ms < best[1]:
            best = (v, ms)
    return best


def tune_plans(uw, synth, torch, dev, stack, Ms, log):
    """uw_autotune per (M, role) with the 32 layers of that role as its rotation set, every
    pipeline, variant and K split; up runs on gate's plan (same shape and statistics). For
    M <= 64 the stack forward runs gate, up and the SwiGLU as one launch, so gate's plan is
    that launch's: direct planes, the variant under which the fused launch itself runs
    fastest (one K slice). Past M = 64, where a pick runs with preprocessing (expand,
    decode), the best plan without it is tuned too and the stack forward chooses."""
    plans, alts = {}, {}
    stream = torch.cuda.current_stream()
    for M in Ms:
        plans[M] = {}
        for role, q in (("gate", 0), ("down", 2)):
            h0 = stack.h[0][q]
            t0 = time.time()
            if role == "gate" and M <= 64:
                v, ms = tune_fused(uw, torch, dev, stack, M, fusable_mask(uw, torch, dev, stack, M), stream)
                if v is not None:
                    plans[M][role] = {"pipeline": uw.PIPE_DIRECT, "variant": v, "split_k": 0, "t_ms": ms}
                    log(f"[bench] plan M={M} gate+up fused: direct / {uw.variant_name(v)}: {ms * 1e3:.1f} us "
                        f"({time.time() - t0:.1f}s)")
                    continue
            x = torch.from_numpy(synth.gen_x(stack.cfg, M, h0.K).view(np.int16)).to(dev)
            y = torch.empty(M, h0.N, dtype=torch.float32, device=dev)
            ws = torch.empty(uw.workspace_bytes(h0, uw.PIPE_FULL), dtype=torch.uint8, device=dev)
            reps, trials = (10, 3) if M <= 64 else (3, 2) if M <= 1024 else (2, 2)
            pl = uw.autotune(h0, stack.blob[0][q], x, y, [M], d_ws=ws, ws_bytes=ws.numel(), reps=reps, warmup=1,
                             trials=trials, rot=stack.rot(uw, q))[0]
            plans[M][role] = {"pipeline": pl.pipeline, "variant": pl.variant, "split_k": pl.split_k, "t_ms": pl.t_ms}
            log(f"[bench] plan M={M} {role}: {uw.PIPELINE_NAMES[pl.pipeline]} / {uw.variant_name(pl.variant)} / "
                f"split {pl.split_k}: {pl.t_ms * 1e3:.1f} us ({time.time() - t0:.1f}s)")
            if M > 64 and pl.pipeline != uw.PIPE_DIRECT:
                # the best plan without preprocessing too: launch by launch the two can be within
                # noise of each other while the forward, where each expand precedes its GEMM,
                # is not; the forward decides between them below
                pd = uw.autotune(h0, stack.blob[0][q], x, y, [M], d_ws=ws, ws_bytes=ws.numel(), reps=reps, warmup=1,
                                 trials=trials, rot=stack.rot(uw, q), pipeline_mask=1 << uw.PIPE_DIRECT)[0]
                alts.setdefault(M, {})[role] = {"pipeline": pd.pipeline, "variant": pd.variant, "split_k": pd.split_k,
                                                "t_ms": pd.t_ms}
            del x, y, ws
        if M in alts:
            plans[M] = fastest_forward(uw, synth, torch, dev, stack, M, plans[M], alts[M], log)
    return plans


def fastest_forward(uw, synth, torch, dev, stack, M, best, alts, log):
    """Among the per-launch picks and the same with any role on its best plan without
    preprocessing, the plans whose whole stack forward at M (one stream) is fastest."""
    cands = [best]
    for roles in (("gate",), ("down",), ("gate", "down")):
        if all(r in alts for r in roles):
            c = dict(best)
            for r in roles:
                c[r] = alts[r]
            cands.append(c)
    x = torch.from_numpy(synth.gen_x(stack.cfg, M, stack.K).view(np.int16)).to(dev)
    y = torch.empty(M, stack.K, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    times = []
    for c in cands:
        arr = stack.layers(uw, c)
        nb = uw.mlp_stack_workspace(arr, M)
        ws = torch.empty(nb, dtype=torch.uint8, device=dev)
        uw.mlp_stack_forward(arr, M, x, y, ws, nb, stream=stream)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(2):
            uw.mlp_stack_forward(arr, M, x, y, ws, nb, stream=stream)
        b.record(stream)
        torch.cuda.synchronize()
        times.append(a.elapsed_time(b) / 2)
        del ws
    i = min(range(len(cands)), key=lambda k: times[k])
    desc = lambda c: ", ".join(f"{r} {uw.PIPELINE_NAMES[c[r]['pipeline']]} / {uw.variant_name(c[r]['variant'])}"
                               for r in ("gate", "down"))
    log(f"[bench] plans M={M} by forward: " + "; ".join(f"{desc(c)}: {t:.3f} ms" for c, t in zip(cands, times))
        + f" -> {desc(cands[i])}")
    del x, y
    return cands[i]


def plans_to_json(uw, plans):
    return {str(M): {r: {"pipeline": uw.PIPELINE_NAMES[p["pipeline"]], "variant": uw.variant_name(p["variant"]),
                         "split_k": p["split_k"], "t_ms": round(float(p["t_ms"]), 5)} for r, p in pm.items()}
            for M, pm in plans.items()}


def plans_from_json(uw, d):
    names = {uw.variant_name(v): v for v in range(uw.variant_count())}
    pipes = {v: k for k, v in uw.PIPELINE_NAMES.items()}
    return {int(M): {r: {"pipeline": pipes[p["pipeline"]], "variant": names[p["variant"]], "split_k": p["split_k"],
                         "t_ms": p.get("t_ms", 0.0)} for r, p in pm.items()} for M, pm in d.items()}


def step_ops(uw, torch, dev, stack, plans_m, M, x, bufs):
    """The launches one stack forward at M is made of, as callables over a layer index, with
    their algorithmic bytes: the fused gate/up/SwiGLU launch where the stack uses it (both
    direct planes, M <= 64, a variant with a fused form, no K split), otherwise gate and up
    through their pipeline and the SwiGLU; then down."""
    pg, pd = plans_m["gate"], plans_m["down"]
    g, u, hbuf, yd, ws = bufs
    ops = []
    fused = pg["pipeline"] == uw.PIPE_DIRECT and M <= 64
    if fused:
        try:
            l = 0
            uw.recon_gemm_gate_up(stack.h[l][0], stack.blob[l][0], stack.plane[l][0], stack.h[l][1], stack.blob[l][1],
                                  stack.plane[l][1], x, g, u, hbuf, M, variant=pg["variant"], split_k=pg["split_k"])
        except uw.UwError as e:
            if e.status != uw.EUNSUPPORTED:
                raise
            fused = False
    if fused:
        ops.append(("gate_up fused", pg, lambda l: uw.recon_gemm_gate_up(
            stack.h[l][0], stack.blob[l][0], stack.plane[l][0], stack.h[l][1], stack.blob[l][1], stack.plane[l][1], x,
            g, u, hbuf, M, variant=pg["variant"], split_k=pg["split_k"]),
            gate_up_bytes(stack.h[0][0], stack.h[0][1], M)))
    else:
        for q, out in ((0, g), (1, u)):
            ops.append((ROLES[q], pg, (lambda q, out: lambda l: uw.run_pipeline(
                pg["pipeline"], stack.h[l][q], stack.blob[l][q], x, out, M, d_direct=stack.plane[l][q], d_ws=ws,
                ws_bytes=ws.numel(), variant=pg["variant"], split_k=pg["split_k"]))(q, out),
                algorithmic_bytes(stack.h[0][q], M, pg["pipeline"])))
        ops.append(("swiglu", None, lambda l: uw.swiglu(g, u, hbuf, M * stack.Nff), 10 * M * stack.Nff))
    ops.append(("down", pd, lambda l: uw.run_pipeline(
        pd["pipeline"], stack.h[l][2], stack.blob[l][2], hbuf, yd, M, d_direct=stack.plane[l][2], d_ws=ws,
        ws_bytes=ws.numel(), variant=pd["variant"], split_k=pd["split_k"]),
        algorithmic_bytes(stack.h[0][2], M, pd["pipeline"])))
    return ops


def time_op(torch, stream, stack, fn, reps, graph=False):
    """Mean duration (ms) of fn(layer) launched back to back over the layers, `reps` times
    round, between two HIP events on the launch stream. graph: also replay the 32 launches
    from a HIP graph (fn must launch on the current stream), so that a launch shorter than
    the Python call that issues it is not timed at the call's pace; the lower of the two is
    returned."""
    for l in range(stack.L):
        fn(l)
    torch.cuda.synchronize()

    def timed(run):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for r in range(reps):
            run()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / (reps * stack.L)

    def eager():
        for l in range(stack.L):
            fn(l)

    ms = timed(eager)
    if graph:
        try:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for l in range(stack.L):
                    fn(l)
            g.replay()
            torch.cuda.synchronize()
            ms = min(ms, timed(g.replay))
        except Exception as e:  # (eager timing stands)
            print(f"[bench] graph timing unavailable: {e}", file=sys.stderr, flush=True)
    return ms


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU; multi-GPU sharding is described in DESIGN.md but not run",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    import torch

    if not torch.cuda.is_available():
        print("bench.py needs a ROCm GPU", file=sys.stderr)
        sys.exit(1)
    import decode_gemm_amd as uw
    import synth

    log = lambda *a: print(*a, file=sys.stderr, flush=True)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    stack = Stack(uw, synth, torch, dev, log)
    Ms_all = SMALL_MS + (() if args.no_large else LARGE_MS)
    if args.plans:
        with open(args.plans) as fh:
            plans = plans_from_json(uw, json.load(fh)["plans"])
        log(f"[bench] plans read from {args.plans}")
    else:
        plans = tune_plans(uw, synth, torch, dev, stack, Ms_all, log)
    if args.save_plans:
        with open(args.save_plans, "w") as fh:
            json.dump({"format": "uw-stack-plans-1", "workload": "8B-shaped 32-layer SwiGLU MLP stack",
                       "plans": plans_to_json(uw, plans)}, fh, indent=1)

    # ---- the timed step: one stack forward at each small M
    Nff, K, L = stack.Nff, stack.K, stack.L
    arrs = {M: stack.layers(uw, plans[M]) for M in SMALL_MS}
    xs = {M: torch.from_numpy(synth.gen_x(stack.cfg, M, K).view(np.int16)).to(dev) for M in SMALL_MS}
    ys = {M: torch.empty(M, K, dtype=torch.float32, device=dev) for M in SMALL_MS}
    nbs = {M: uw.mlp_stack_workspace(arrs[M], M) for M in SMALL_MS}
    ws = torch.empty(max(nbs.values()), dtype=torch.uint8, device=dev)

    def step():
        for M in SMALL_MS:
            uw.mlp_stack_forward(arrs[M], M, xs[M], ys[M], ws, nbs[M], stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    ms_per_step = ev0.elapsed_time(ev1) / args.steps
    value = len(SMALL_MS) * stack.weight_bytes / (ms_per_step * 1e-3) / 1e9
    # each M's forward alone, back to back
    fwd_ms = {}
    for M in SMALL_MS:
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(max(3, args.steps // 2)):
            uw.mlp_stack_forward(arrs[M], M, xs[M], ys[M], ws, nbs[M], stream=stream)
        b.record(stream)
        torch.cuda.synchronize()
        fwd_ms[M] = a.elapsed_time(b) / max(3, args.steps // 2)
    log(f"[bench] step {ms_per_step:.3f} ms = {value:.0f} GB/s uncompressed-equivalent; forwards (ms): "
        + ", ".join(f"M={M} {fwd_ms[M]:.3f}" for M in SMALL_MS))

    # ---- the launches of the step, each timed back to back over the layers; the dominant
    # kernel is the group of launches of one kernel build (same op, plan and 16-column tile
    # count) with the largest share of the step
    groups = {}
    op_rows = {}
    for M in SMALL_MS:
        g = torch.empty(M, Nff, dtype=torch.float32, device=dev)
        u = torch.empty_like(g)
        hbuf = torch.empty(M * Nff, dtype=torch.int16, device=dev)
        yd = torch.empty(M, K, dtype=torch.float32, device=dev)
        wsp = torch.empty(uw.workspace_bytes(stack.h[0][0], uw.PIPE_FULL), dtype=torch.uint8, device=dev)
        for name, plan, fn, nbytes in step_ops(uw, torch, dev, stack, plans[M], M, xs[M], (g, u, hbuf, yd, wsp)):
            ms = time_op(torch, stream, stack, fn, max(3, args.steps // 2), graph=True)
            pipe = uw.PIPELINE_NAMES[plan["pipeline"]] if plan else "-"
            var = uw.variant_name(plan["variant"]) if plan else "-"
            split = plan["split_k"] if plan else 1
            key = (name, pipe, var, split > 1, (M + 15) // 16)
            grp = groups.setdefault(key, {"ms": 0.0, "bytes": 0, "launches": 0, "Ms": []})
            grp["ms"] += ms * L
            grp["bytes"] += nbytes * L
            grp["launches"] += L
            grp["Ms"].append(M)
            op_rows[f"M={M} {name}"] = {"pipeline": pipe, "variant": var, "split_k": split, "us": round(ms * 1e3, 2),
                                        "bytes": int(nbytes),
                                        "hbm_frac": round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
        del g, u, hbuf, yd, wsp
    dom = max(groups, key=lambda k: groups[k]["ms"])
    dg = groups[dom]
    mean_us = dg["ms"] / dg["launches"] * 1e3
    achieved = dg["bytes"] / (dg["ms"] * 1e-3) / 1e9
    dom_key = f"{dom[0]}, {dom[1]}, {dom[2]}{' (K split)' if dom[3] else ''}, M={'/'.join(map(str, dg['Ms']))}"
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": measured_traffic(dom_key), "kernel": dom_key,
                "bytes_per_launch": int(dg["bytes"] / dg["launches"]), "mean_launch_us": round(mean_us, 2),
                "launches_per_step": dg["launches"], "share_of_step": round(dg["ms"] / ms_per_step, 4)}
    # the read rate of a plain streaming kernel over the same planes (no other work)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    pb = uw.direct_plane_bytes(stack.h[0][0]) // 16 * 16
    read_ms = time_op(torch, stream, stack, lambda l: uw.stream_read(stack.plane[l][0], sink, pb, stream=stream), 3)
    read_gbs = pb / (read_ms * 1e-3) / 1e9
    roofline["read_ceiling_GBs"] = round(read_gbs, 1)
    roofline["frac_of_read_ceiling"] = round(achieved / read_gbs, 4)
    log(f"[bench] dominant: {dom_key}: {mean_us:.2f} us/launch, {achieved:.0f} GB/s = {achieved / HBM_PEAK_GBS:.3f} "
        f"of 8 TB/s ({achieved / read_gbs:.3f} of the {read_gbs:.0f} GB/s read ceiling); launches: {op_rows}")

    large = None if args.no_large else large_m(uw, synth, torch, dev, stream, stack, plans, log)
    sched = schedules(uw, synth, torch, dev, stream, stack, plans, log) if args.schedules else None
    l70 = None if args.no_70b else layer_70b(uw, synth, torch, dev, stream, log)
    detail = {"plans": plans_to_json(uw, plans), "launches": op_rows,
              "forward_ms": {str(M): round(fwd_ms[M], 4) for M in SMALL_MS},
              "blob_bytes_per_weight": round(2 * stack.blob_total / stack.weight_bytes, 4),
              "direct_plane_bytes_per_weight": round(2 * stack.plane_total / stack.weight_bytes, 4)}
    for M in SMALL_MS:
        # the forward's HBM fraction on the resident bytes it starts from (every plane it
        # reads once, X, the final Y) and on everything it moves
        res = stack.plane_total + 2 * M * K + 4 * M * K
        detail.setdefault("forward_hbm_frac", {})[str(M)] = round(res / (fwd_ms[M] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)
    if not args.no_detail:
        del arrs, ws
        torch.cuda.empty_cache()
        detail["single_matrix"] = single_matrix_detail(uw, synth, torch, dev, stream, log)

    cpu = None if args.no_cpu else cpu_baseline(synth, log)

    if args.copy_probe:
        a = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        a.fill_(1)
        torch.cuda.synchronize()
        b.copy_(a)
        torch.add(a, 1, out=b)
        torch.cuda.synchronize()

    out = {
        "metric": "uncompressed-equiv weight GB/s of decode+GEMM vs HBM roof; TFLOP/s at M>=1024",
        "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "Llama-3.1-8B-shaped MLP stack: 32 SwiGLU layers (gate, up 14336x4096; down 4096x14336) "
                               "bf16 N(0, 0.02*U(0.8,1.2)) exponent-compressed; one step = a stack forward at each "
                               "M in {1,16,64}; autotuned plan per (M, projection)",
                   "global_batch": int(sum(SMALL_MS)), "seq_len": 1, "parallelism": "single GPU",
                   "layers": L, "Ms": list(SMALL_MS)},
        "roofline": roofline,
        "large_m": large,
        "schedules": sched,
        "layer_70b": l70,
        "cpu_baseline": cpu,
        "detail": detail,
    }
    print(json.dumps(out))


def layer_70b(uw, synth, torch, dev, stream, log, reps=10):
    """The 70B-shaped MLP layer (gate and up 28672x8192, down 8192x28672; Student-t(4) weights
    with 1% of 64-weight rows holding an outlier exponent) at M in {1, 64, 512, 2048}: plans
    chosen as for the stack (uw_autotune per projection, the fused gate/up launch timed itself
    at M <= 64), then the layer's forward launched back to back between HIP events:
    uncompressed-equivalent GB/s at M <= 64, TFLOP/s and the bf16-peak fraction above."""
    st = Stack(uw, synth, torch, dev, log, "70b")
    Ms = st.cfg.Ms
    plans = tune_plans(uw, synth, torch, dev, st, Ms, log)
    pj = plans_to_json(uw, plans)
    out = {"workload": "70B-shaped SwiGLU MLP layer: gate/up 28672x8192, down 8192x28672 bf16 Student-t(4)*0.01, "
                       "1% of 64-weight rows with an outlier exponent",
           "n_raw": [int(h.n_raw) for h in st.h[0]]}
    for M in Ms:
        arr = st.layers(uw, plans[M])
        nb = uw.mlp_stack_workspace(arr, M)
        ws = torch.empty(max(nb, 256), dtype=torch.uint8, device=dev)
        x = torch.from_numpy(synth.gen_x(st.cfg, M, st.K).view(np.int16)).to(dev)
        y = torch.empty(M, st.K, dtype=torch.float32, device=dev)
        uw.mlp_stack_forward(arr, M, x, y, ws, nb, stream=stream)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(reps):
            uw.mlp_stack_forward(arr, M, x, y, ws, nb, stream=stream)
        b.record(stream)
        torch.cuda.synchronize()
        ms = a.elapsed_time(b) / reps
        row = {"forward_ms": round(ms, 4), "plans": pj[str(M)]}
        if M <= 64:
            row["uncompressed_GBs"] = round(st.weight_bytes / (ms * 1e-3) / 1e9, 1)
            res = st.plane_total + 2 * M * st.K + 4 * M * st.K
            row["hbm_frac"] = round(res / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)
        else:
            tf = 2.0 * M * st.macs / (ms * 1e-3) / 1e12
            row["tflops"] = round(tf, 1)
            row["mfma_frac"] = round(tf / BF16_PEAK_TFLOPS, 4)
        out[str(M)] = row
        log(f"[bench] 70B layer M={M}: {row}")
        del ws, x, y
    del st
    torch.cuda.empty_cache()
    return out


def schedules(uw, synth, torch, dev, stream, stack, plans, log, Ms=SMALL_MS, reps=5):
    """The stack with hard layers ("Sharing the GPU between decode and compute"): every 4th layer
    keeps only its Huffman blobs, so each of its projections needs preprocessing (full decode to
    start with), while the others run their direct planes on the tuned plans. ms per forward at
    each M, back to back between HIP events on the forward's stream: one stream; the decodes on a
    second stream with 3 workspace slots (in order, then each layer's down first); the same on
    CU-split stream pairs (decode on 32 or 64 of the CUs); then uw_mlp_stack_autotune's plan
    (decode stream, 3 slots), against the stack with no hard layer."""
    L = stack.L
    hard = [l for l in range(L) if l % 4 == 3]
    side = torch.cuda.Stream()
    out = {"hard_layers": hard, "slots": 3}
    for M in Ms:
        pm = plans[M]
        rows = []
        for l in range(L):
            trip = []
            for q in range(3):
                p = pm["down" if q == 2 else "gate"]
                if l in hard:
                    trip.append(uw.proj(stack.h[l][q], stack.blob[l][q], uw.PIPE_FULL))
                else:
                    trip.append(uw.proj(stack.h[l][q], stack.blob[l][q], p["pipeline"], d_direct=stack.plane[l][q],
                                        variant=p["variant"], split_k=p["split_k"]))
            rows.append(trip)
        arr = uw.mlp_layers(rows)
        easy = stack.layers(uw, pm)
        full = uw.mlp_layers([[uw.proj(stack.h[l][q], stack.blob[l][q], uw.PIPE_FULL) for q in range(3)]
                              for l in range(L)])
        nb = max(uw.mlp_stack_workspace_ex(full, M, slots=3, down_first=df) for df in (False, True))
        ws = torch.empty(nb, dtype=torch.uint8, device=dev)
        x = torch.from_numpy(synth.gen_x(stack.cfg, M, stack.K).view(np.int16)).to(dev)
        y = torch.empty(M, stack.K, dtype=torch.float32, device=dev)
        torch.cuda.synchronize()

        def timed(fwd, st):
            fwd()
            torch.cuda.synchronize()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(st)
            for _ in range(reps):
                fwd()
            b.record(st)
            torch.cuda.synchronize()
            return round(a.elapsed_time(b) / reps, 4)

        row = {"no_hard_layer": timed(lambda: uw.mlp_stack_forward(easy, M, x, y, ws, nb, stream=stream), stream),
               "one_stream": timed(lambda: uw.mlp_stack_forward_ex(arr, M, x, y, ws, nb, stream=stream, slots=3),
                                   stream)}
        for df in (False, True):
            row["decode_stream" + ("_down_first" if df else "")] = timed(
                lambda: uw.mlp_stack_forward_ex(arr, M, x, y, ws, nb, stream=stream, decode_stream=side, slots=3,
                                                down_first=df), stream)
        for cus in (32, 64):
            g, d = uw.stream_pair_create(cus)
            try:
                gs = torch.cuda.ExternalStream(g)
                row[f"cu_split_{cus}"] = timed(lambda: uw.mlp_stack_forward_ex(
                    arr, M, x, y, ws, nb, stream=g, decode_stream=d, slots=3, down_first=True), gs)
            finally:
                torch.cuda.synchronize()
                uw.stream_destroy(g)
                uw.stream_destroy(d)
        t0 = time.time()
        a = uw.mlp_stack_autotune(arr, M, x, y, ws, nb, stream=stream, decode_stream=side, slots=3, reps=3, warmup=1)
        torch.cuda.synchronize()
        tune_s = time.time() - t0
        df = bool(a.opts.down_first)
        row["tuned"] = timed(lambda: uw.mlp_stack_forward_ex(arr, M, x, y, ws, nb, stream=stream, decode_stream=side,
                                                             slots=3, down_first=df), stream)
        row["tuned_plan"] = {cls: {r: uw.PIPELINE_NAMES[getattr(arr[l], r).pipeline] for r in ("gate", "up", "down")}
                             for cls, l in (("easy", 0), ("hard", hard[0]))}
        row["tuned_down_first"] = df
        row["tune"] = {"passes": a.passes, "trials": a.trials, "seconds": round(tune_s, 1)}
        out[str(M)] = row
        log(f"[bench] hard/easy stack M={M} (ms per forward): {row}")
        del ws, x, y
    return out


def large_m(uw, synth, torch, dev, stream, stack, plans, log):
    """The stack forward at M = 1024 and 4096 on its plans: TFLOP/s (2 M x every matrix's
    N K per forward) vs the bf16 peak, and each projection's GEMM alone (back to back over
    the layers)."""
    res = {"unit": "TFLOP/s", "peak": BF16_PEAK_TFLOPS}
    for M in LARGE_MS:
        arr = stack.layers(uw, plans[M])
        x = torch.from_numpy(synth.gen_x(stack.cfg, M, stack.K).view(np.int16)).to(dev)
        y = torch.empty(M, stack.K, dtype=torch.float32, device=dev)
        nb = uw.mlp_stack_workspace(arr, M)
        ws = torch.empty(nb, dtype=torch.uint8, device=dev)
        uw.mlp_stack_forward(arr, M, x, y, ws, nb, stream=stream)
        torch.cuda.synchronize()
        reps = 3 if M <= 1024 else 2
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(reps):
            uw.mlp_stack_forward(arr, M, x, y, ws, nb, stream=stream)
        b.record(stream)
        torch.cuda.synchronize()
        ms = a.elapsed_time(b) / reps
        schedule = "one stream"
        del ws
        # plans with preprocessing (expand, decode): also the stack scheduler's form that runs
        # it on a second stream into three workspace slots, ahead of the GEMMs that use it
        if any(plans[M][r]["pipeline"] != uw.PIPE_DIRECT for r in ("gate", "down")):
            side = torch.cuda.Stream()
            nb = uw.mlp_stack_workspace_ex(arr, M, slots=3)
            ws = torch.empty(nb, dtype=torch.uint8, device=dev)
            fwd = lambda: uw.mlp_stack_forward_ex(arr, M, x, y, ws, nb, stream=stream, decode_stream=side, slots=3)
            fwd()
            torch.cuda.synchronize()
            a.record(stream)
            for _ in range(reps):
                fwd()
            b.record(stream)
            torch.cuda.synchronize()
            ms2 = a.elapsed_time(b) / reps
            log(f"[bench] stack M={M}: one stream {ms:.3f} ms, preprocessing on a second stream {ms2:.3f} ms")
            if ms2 < ms:
                ms, schedule = ms2, "preprocessing on a second stream, 3 slots"
            del ws
        tf = 2.0 * M * stack.macs / (ms * 1e-3) / 1e12
        row = {"forward_ms": round(ms, 3), "tflops": round(tf, 1), "mfma_frac": round(tf / BF16_PEAK_TFLOPS, 4),
               "tokens_per_s": round(M / (ms * 1e-3), 1), "schedule": schedule,
               "plans": plans_to_json(uw, {M: plans[M]})[str(M)]}
        g = torch.empty(M, stack.Nff, dtype=torch.float32, device=dev)
        hb = torch.empty(M * stack.Nff, dtype=torch.int16, device=dev)
        hb.zero_()
        wsp = torch.empty(uw.workspace_bytes(stack.h[0][0], uw.PIPE_FULL), dtype=torch.uint8, device=dev)
        for role, q, xin, out, N, Kin in (("gate", 0, x, g, stack.Nff, stack.K), ("down", 2, hb, y, stack.K, stack.Nff)):
            p = plans[M][role]
            fn = lambda l: uw.run_pipeline(p["pipeline"], stack.h[l][q], stack.blob[l][q], xin, out, M,
                                           d_direct=stack.plane[l][q], d_ws=wsp, ws_bytes=wsp.numel(),
                                           variant=p["variant"], split_k=p["split_k"])
            oms = time_op(torch, stream, stack, fn, 1, graph=True)
            otf = 2.0 * M * N * Kin / (oms * 1e-3) / 1e12
            row[role] = {"us": round(oms * 1e3, 1), "tflops": round(otf, 1), "mfma_frac": round(otf / BF16_PEAK_TFLOPS, 4)}
        del g, hb, wsp, x, y
        torch.cuda.empty_cache()
        res[str(M)] = row
        log(f"[bench] stack M={M}: {row}")
    return res


def single_matrix_detail(uw, synth, torch, dev, stream, log, copies=6):
    """The single-matrix gate-shaped workload (14336 x 4096, 0.01% outliers x 2^+-10) at M in
    {1, 16, 64}: each pipeline's best plan (rotated copies, back to back), its HBM fraction on
    the resident bytes it starts from plus X and Y (and on all the bytes it moves), and each
    decoder alone."""
    cfg = synth.CONFIGS["gate"]
    w = synth.gen_weight(cfg, "gate")
    blob = uw.encode(w)
    del w
    h = uw.inspect(blob)
    N, K = h.N, h.K
    blobs, planes = [], []
    for _ in range(copies):
        b = torch.from_numpy(blob).to(dev)
        d = torch.empty(uw.direct_plane_bytes(h), dtype=torch.uint8, device=dev)
        uw.prepare_direct(h, b, d)
        blobs.append(b)
        planes.append(d)
    rot = [uw.proj(h, blobs[r], d_direct=planes[r]) for r in range(copies)]
    ws = torch.empty(uw.workspace_bytes(h, uw.PIPE_FULL), dtype=torch.uint8, device=dev)
    pip = {}
    for M in SMALL_MS:
        x = torch.from_numpy(synth.gen_x(cfg, M, K).view(np.int16)).to(dev)
        y = torch.empty(M, N, dtype=torch.float32, device=dev)
        for p in range(5):
            pl = uw.autotune(h, blobs[0], x, y, [M], d_ws=ws, ws_bytes=ws.numel(), reps=12, warmup=2, trials=3, rot=rot,
                             pipeline_mask=1 << p, tune_split=True)[0]
            us = pl.t_ms * 1e3
            res = resident_bytes(h, p, blob.size) + 2 * M * K + 4 * M * N
            pip[f"M={M} {uw.PIPELINE_NAMES[p]}"] = {
                "variant": uw.variant_name(pl.variant), "split_k": pl.split_k, "us": round(us, 2),
                "uncompressed_GBs": round(2 * N * K / (us * 1e-6) / 1e9, 1),
                "hbm_frac": round(res / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                "moved_frac": round(algorithmic_bytes(h, M, p) / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
    log(f"[bench] single matrix: {pip}")
    return {"workload": "gate_proj shape W 14336x4096 bf16 N(0,0.02) + 0.01% 2^+-10 outliers, M in {1,16,64}",
            "blob_bytes_per_weight": round(blob.size / (N * K), 4),
            "pipelines": pip, "decoders": decoder_detail(uw, torch, h, blobs, stream, log, planes=planes)}


def decoder_detail(uw, torch, h, blobs, stream, log, planes=None):
    """Each decoder alone, launched back to back over rotated copies of the blob (the expand
    kernel over rotated copies of its direct plane): mean time, the bytes it must move, and
    the fraction of the HBM roof that rate is."""
    N, K = h.N, h.K
    outs = {"full": torch.empty(2 * N * K, dtype=torch.uint8, device=blobs[0].device),
            "exp": torch.empty(N * K, dtype=torch.uint8, device=blobs[0].device),
            "idx": torch.empty(N * K // 2, dtype=torch.uint8, device=blobs[0].device),
            "direct": torch.empty(uw.direct_plane_bytes(h), dtype=torch.uint8, device=blobs[0].device)}
    fns = {"full": lambda b, o: uw.decode_full(h, b, o, stream=stream),
           "exp": lambda b, o: uw.decode_exponent(h, b, o, stream=stream),
           "idx": lambda b, o: uw.transcode_palette(h, b, o, stream=stream),
           "direct": lambda b, o: uw.prepare_direct(h, b, o, stream=stream)}
    srcs = {mode: blobs for mode in fns}
    if planes:
        outs["expand"] = outs["full"]
        fns["expand"] = lambda p, o: uw.expand_direct(h, p, o, stream=stream)
        srcs["expand"] = planes
    res = {}
    for mode, fn in fns.items():
        src = srcs[mode]
        R = len(src)
        for r in range(R):
            fn(src[r], outs[mode])
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for r in range(4 * R):
            fn(src[r % R], outs[mode])
        b.record(stream)
        torch.cuda.synchronize()
        us = a.elapsed_time(b) / (4 * R) * 1e3
        nbytes = decode_bytes(h, mode)
        gbs = nbytes / (us * 1e-6) / 1e9
        res[mode] = {"us": round(us, 2), "bytes": int(nbytes), "GBs": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4)}
    log(f"[bench] decoders: {res}")
    return res


def cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(synth, log):
    """The CPU oracle as it stands (plain scalar C, one call per matrix) on a bounded sample
    of the step: projections of the stack at M = 1, 16 and 64, each forward a bit-serial
    decode of its Huffman blob to bf16 W and an fp64 GEMM. One thread on layer 0's gate and
    down; then two projections per thread on all host cores (up to 16), started together.
    The encode is not timed. Also the M = 1024 forward, extrapolated from a 16-row (1/64)
    sample of X."""
    import concurrent.futures as cf
    import threading

    import oracle

    cfg = synth.CONFIGS["stack"]
    sig = synth.gen_stack_sigmas(cfg)

    def prep(i):
        layer, q = divmod(i, 3)
        w = synth.gen_weight(cfg, ROLES[q], layer, sigma=float(sig[layer]))
        blob = oracle.encode(w, chunk=256)
        xs = {M: synth.gen_x(cfg, M, w.shape[1]) for M in SMALL_MS}
        return blob, xs, w.shape

    def work(item):
        blob, xs, _ = item
        for M in SMALL_MS:
            d = oracle.decode(blob, want=("w",))
            oracle.gemm(xs[M], d["w"])

    one = prep(0)
    N, K = one[2]
    two = prep(2)
    t = time.perf_counter()
    work(one)
    work(two)
    t1 = time.perf_counter() - t
    v1 = 2 * len(SMALL_MS) * 2.0 * N * K / t1 / 1e9
    # M = 1024: decode once, GEMM on 16 of its 1024 rows, scaled by 64
    x16 = synth.gen_x(cfg, 1024, K)[:16]
    t = time.perf_counter()
    d = oracle.decode(one[0], want=("w",))
    td = time.perf_counter() - t
    t = time.perf_counter()
    oracle.gemm(x16, d["w"])
    tg = time.perf_counter() - t
    del d
    t1024 = td + 64 * tg
    log(f"[bench] cpu oracle, 1 thread: {t1:.1f}s -> {v1:.4f} GB/s; M=1024 extrapolated {t1024:.1f}s")
    del one, two
    threads = max(1, min(16, os.cpu_count() or 1))
    per = 2  # projections per thread
    with cf.ThreadPoolExecutor(threads) as ex:
        items = list(ex.map(prep, range(per * threads)))
    barrier = threading.Barrier(threads)
    ends = [0.0] * threads

    def run(i):
        barrier.wait()
        for k in range(per):
            work(items[per * i + k])
        ends[i] = time.perf_counter()

    start = [0.0]

    def run0():
        barrier.wait()
        start[0] = time.perf_counter()
        for k in range(per):
            work(items[k])
        ends[0] = time.perf_counter()

    with cf.ThreadPoolExecutor(threads) as ex:
        futs = [ex.submit(run0)] + [ex.submit(run, i) for i in range(1, threads)]
        for f in futs:
            f.result()
    tall = max(ends) - start[0]
    vall = per * threads * len(SMALL_MS) * 2.0 * N * K / tall / 1e9
    log(f"[bench] cpu oracle, {threads} threads: {tall:.1f}s -> {vall:.4f} GB/s")
    return {"value": round(vall, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "cpu_model": cpu_model(), "host_cpus": os.cpu_count(),
            "sample": f"{per * threads} projections of the stack (layers 0..{(per * threads - 1) // 3}), {per} per "
                      f"thread, each a forward at M = 1, 16, 64 (bit-serial decode + fp64 GEMM per forward), {tall:.1f} s",
            "single_thread": {"value": round(v1, 4), "unit": "GB/s", "cores": 1,
                              "sample": f"layer 0 gate 14336x4096 and down 4096x14336 at M = 1, 16, 64, {t1:.1f} s"},
            "large_m_extrapolated": {
                "tflops": round(2.0 * 1024 * N * K / t1024 / 1e12, 6), "unit": "TFLOP/s", "cores": 1,
                "sample": f"layer 0 gate at M = 1024: decode {td:.1f} s + fp64 GEMM on 16 of the 1024 rows "
                          f"{tg:.1f} s x 64 (extrapolated)"}}


if __name__ == "__main__":
    main()
