"""Benchmark: decode + GEMM throughput of the exponent-compressed gate projection on one
MI355X, as uncompressed-equivalent weight GB/s (2 * N * K bytes per forward / time).

Workload (the small-batch, decode-bound case): a Llama-3.1-8B gate_proj-shaped matrix,
W 14336 x 4096 bf16 ~ N(0, 0.02) with 0.01% of entries pushed by 2^+-10, synthetic and
seeded; X M x 4096 bf16 ~ N(0, 1). One step = one forward of the matrix for each batch
size M in {1, 16, 64}, each through the pipeline the autotuner picked for that M
(full decode + GEMM, exponent-only, palette transcode or direct palette), with the
weights' compressed planes rotated over enough copies that the 256 MB Infinity Cache
cannot serve them. Inputs are resident in HBM when the timed region starts.

The JSON line also carries:
  roofline      the dominant kernel's algorithmic HBM bytes per launch / its mean
                duration (HIP events on its stream, inside the timed region) vs 8 TB/s
  cpu_baseline  the CPU oracle (bit-serial decode + fp64 GEMM) timed on one host core
                on one full step of the same workload
  detail        per-M plans and the time of each of the four pipelines
  large_m       TFLOP/s of the down_proj-shaped (4096 x 14336) GEMM at M = 4096
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
# measured HBM traffic of the dominant kernel (rocprofv3 FETCH_SIZE / WRITE_SIZE runs,
# scaled by the counters of a copy of known size); used only while the GEMM sources
# still hash to what was profiled
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemm_direct_gate_traffic.json")
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


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--copies", type=int, default=6, help="rotated copies of the compressed weights")
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU-oracle baseline")
    p.add_argument("--no-detail", action="store_true", help="skip per-pipeline detail and the large-M line")
    p.add_argument("--copy-probe", action="store_true", help="also launch a plain 256 MiB copy kernel (counter scale)")
    p.add_argument("--configs", action="store_true",
                   help="also sweep the down_proj, 70B-layer and 32-layer-stack workloads (a few minutes more)")
    return p.parse_args()


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

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    cfg = synth.CONFIGS["gate"]
    Ms = list(cfg.Ms)
    t0 = time.time()
    w = synth.gen_weight(cfg, "gate")
    blob = uw.encode(w)
    h = uw.inspect(blob)
    N, K = h.N, h.K
    log = lambda *a: print(*a, file=sys.stderr, flush=True)
    log(f"[bench] gate {N}x{K}: blob {blob.size / 1e6:.1f} MB ({blob.size / (N * K):.3f} B/w), raw groups {h.n_raw}, "
        f"prep {time.time() - t0:.1f}s")

    # R copies of the blob and of its load-time direct-palette plane
    R = args.copies
    d_blob = torch.from_numpy(blob).to(dev)
    blobs, idxs = [], []
    for r in range(R):
        b = d_blob.clone()
        i = torch.empty(uw.direct_plane_bytes(h), dtype=torch.uint8, device=dev)
        uw.prepare_direct(h, b, i)
        blobs.append(b)
        idxs.append(i)
    del d_blob
    xs = {M: torch.from_numpy(synth.gen_x(cfg, M, K).view(np.int16)).to(dev) for M in Ms}
    ys = {M: torch.empty(M, N, dtype=torch.float32, device=dev) for M in Ms}
    ws_bytes = uw.workspace_bytes(h, uw.PIPE_FULL)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    scrub = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    # plans: uw_autotune per M (single launches, cold caches: the scrub buffer is
    # overwritten before each rep), then the timed step's own conditions decide between
    # its pick and every direct-palette variant: launches back to back over the rotated
    # copies, X resident, as in the timed region
    tuned = {}
    for M in Ms:
        tuned[M] = uw.autotune(h, blobs[0], xs[M], ys[M], [M], d_direct=idxs[0], d_ws=ws, ws_bytes=ws_bytes, reps=10,
                               warmup=2, d_scrub=scrub, scrub_bytes=scrub.numel())[0]
    log("[bench] autotune: " + ", ".join(f"M={M}: {tuned[M]!r} ({uw.variant_name(tuned[M].variant)})" for M in Ms))

    def back_to_back_us(pipeline, variant, M, n):
        for r in range(R):
            uw.run_pipeline(pipeline, h, blobs[r], xs[M], ys[M], M, d_direct=idxs[r], d_ws=ws, ws_bytes=ws_bytes,
                            variant=variant, stream=stream)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for r in range(n):
            uw.run_pipeline(pipeline, h, blobs[r % R], xs[M], ys[M], M, d_direct=idxs[r % R], d_ws=ws,
                            ws_bytes=ws_bytes, variant=variant, stream=stream)
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / n * 1e3

    plans, choice = {}, {}
    for M in Ms:
        cands = [(tuned[M].pipeline, tuned[M].variant)]
        cands += [(uw.PIPE_DIRECT, v) for v in range(uw.variant_count())
                  if uw.variant_supports(v, N, K, M, uw.W_DIRECT) and (uw.PIPE_DIRECT, v) != cands[0]]
        times = {c: back_to_back_us(c[0], c[1], M, 4 * R) for c in cands}
        best = min(times, key=times.get)
        plans[M] = uw.Plan(best[0], best[1], times[best] / 1e3, 0)
        choice[M] = {"autotune": f"{uw.PIPELINE_NAMES[cands[0][0]]} / {uw.variant_name(cands[0][1])}",
                     "autotune_back_to_back_us": round(times[cands[0]], 2), "candidates": len(cands)}
    log("[bench] plans: " + ", ".join(f"M={M}: {plans[M]!r} ({uw.variant_name(plans[M].variant)})" for M in Ms))

    seq = [0]

    def launch(M):
        c = seq[0] % R
        seq[0] += 1
        p = plans[M]
        uw.run_pipeline(p.pipeline, h, blobs[c], xs[M], ys[M], M, d_direct=idxs[c], d_ws=ws, ws_bytes=ws_bytes,
                        variant=p.variant, stream=stream)

    def step():
        for M in Ms:
            launch(M)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # timed region: K steps back to back, HIP events on the launch stream at both ends only
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    ms_per_step = ev0.elapsed_time(ev1) / args.steps
    uncompressed = 2.0 * N * K * len(Ms)
    value = uncompressed / (ms_per_step * 1e-3) / 1e9

    # per-M launch durations: each M's pipeline launched K times back to back (rotated
    # copies), events at both ends, so no event sits between two launches
    mean_ms = {}
    for M in Ms:
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(args.steps):
            launch(M)
        b.record(stream)
        torch.cuda.synchronize()
        mean_ms[M] = a.elapsed_time(b) / args.steps

    # dominant kernel: the pipeline launch with the largest share of the step; when the
    # pipeline is direct palette this is exactly one GEMM kernel launch
    Mdom = max(Ms, key=lambda M: mean_ms[M])
    pdom = plans[Mdom]
    alg = algorithmic_bytes(h, Mdom, pdom.pipeline)
    achieved = alg / (mean_ms[Mdom] * 1e-3) / 1e9
    dom_key = f"{uw.PIPELINE_NAMES[pdom.pipeline]} pipeline, {uw.variant_name(pdom.variant)}, M={Mdom}"
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": measured_traffic(dom_key),
                "kernel": dom_key,
                "bytes_per_launch": int(alg), "mean_launch_us": round(mean_ms[Mdom] * 1e3, 2)}
    # the practical read ceiling beside the published peak: a plain streaming read of the
    # same rotated planes (uw_stream_read, no other work), back to back like the GEMMs
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    pbytes = uw.direct_plane_bytes(h) // 16 * 16
    for r in range(R):
        uw.stream_read(idxs[r], sink, pbytes, stream=stream)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for r in range(4 * R):
        uw.stream_read(idxs[r % R], sink, pbytes, stream=stream)
    b.record(stream)
    torch.cuda.synchronize()
    read_us = a.elapsed_time(b) / (4 * R) * 1e3
    read_gbs = pbytes / (read_us * 1e-6) / 1e9
    roofline["read_ceiling_GBs"] = round(read_gbs, 1)
    roofline["frac_of_read_ceiling"] = round(achieved / read_gbs, 4)
    log(f"[bench] plain streaming read of one plane: {read_us:.1f} us = {read_gbs:.0f} GB/s "
        f"({read_gbs / HBM_PEAK_GBS:.3f} of the peak); dominant kernel at {achieved / read_gbs:.3f} of it")
    log(f"[bench] step {ms_per_step * 1e3:.1f} us, {value:.0f} GB/s uncompressed-equivalent; per-M us: "
        + ", ".join(f"{M}: {mean_ms[M] * 1e3:.1f}" for M in Ms))

    detail = {"plans": {str(M): {"pipeline": uw.PIPELINE_NAMES[plans[M].pipeline], "variant": uw.variant_name(plans[M].variant),
                                 "us": round(mean_ms[M] * 1e3, 2), "selection": choice[M],
                                 "hbm_frac_compressed": round(algorithmic_bytes(h, M, plans[M].pipeline) / (mean_ms[M] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
                        for M in Ms},
              "blob_bytes_per_weight": round(blob.size / (N * K), 4),
              "direct_plane_bytes_per_weight": round(uw.direct_plane_bytes(h) / (N * K), 4)}
    large_m = None
    if not args.no_detail:
        # every pipeline at every M (best variant each), cold weights via rotation
        pip = {}
        for M in Ms:
            for p in range(5):
                pl = uw.autotune(h, blobs[0], xs[M], ys[M], [M], d_direct=idxs[0], d_ws=ws, ws_bytes=ws_bytes, reps=5,
                                 warmup=1, pipeline_mask=1 << p, d_scrub=scrub, scrub_bytes=scrub.numel())[0]
                ts = []
                for r in range(3 * R):
                    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    c = r % R
                    a.record(stream)
                    uw.run_pipeline(p, h, blobs[c], xs[M], ys[M], M, d_direct=idxs[c], d_ws=ws, ws_bytes=ws_bytes,
                                    variant=pl.variant, stream=stream)
                    b.record(stream)
                    ts.append((a, b))
                torch.cuda.synchronize()
                us = float(np.median([a.elapsed_time(b) for a, b in ts])) * 1e3
                pip[f"M={M} {uw.PIPELINE_NAMES[p]}"] = {
                    "variant": uw.variant_name(pl.variant), "us": round(us, 2),
                    "uncompressed_GBs": round(2 * N * K / (us * 1e-6) / 1e9, 1),
                    "hbm_frac_compressed": round(algorithmic_bytes(h, M, p) / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
        detail["pipelines"] = pip
        detail["decoders"] = decoder_detail(uw, torch, h, blobs, stream, log, planes=idxs)
        large_m = large_m_line(uw, synth, torch, dev, stream, log)

    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(synth, cfg, w, Ms, log)

    sweep = configs_sweep(uw, synth, torch, dev, stream, log) if args.configs else None

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
        "config": {"workload": "Llama-3.1-8B gate_proj shape, W 14336x4096 bf16 N(0,0.02) + 0.01% 2^+-10 outliers, "
                               "exponent-compressed; X Mx4096 bf16, M in {1,16,64}; autotuned pipeline per M",
                   "global_batch": int(sum(Ms)), "seq_len": 1, "parallelism": "single GPU"},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "detail": detail,
        "large_m": large_m,
    }
    if sweep is not None:
        out["configs"] = sweep
    print(json.dumps(out))


def decoder_detail(uw, torch, h, blobs, stream, log, planes=None):
    """Each decoder alone on rotated copies of the gate blob (and the expand kernel on rotated
    copies of its direct plane): median time, the bytes it must move, and the fraction of the
    HBM roof that rate is."""
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
        fn(src[0], outs[mode])
        ts = []
        for r in range(3 * R):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            fn(src[r % R], outs[mode])
            b.record(stream)
            ts.append((a, b))
        torch.cuda.synchronize()
        us = float(np.median([a.elapsed_time(b) for a, b in ts])) * 1e3
        nbytes = decode_bytes(h, mode)
        gbs = nbytes / (us * 1e-6) / 1e9
        res[mode] = {"us": round(us, 2), "bytes": int(nbytes), "GBs": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4)}
    log(f"[bench] decoders: {res}")
    return res


def timed(torch, stream, fn, reps=10):
    """Median of per-launch HIP-event times (ms) of fn(rep)."""
    ev = []
    for r in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        fn(r)
        b.record(stream)
        ev.append((a, b))
    torch.cuda.synchronize()
    return float(np.median([a.elapsed_time(b) for a, b in ev]))


def shape_sweep(uw, synth, torch, dev, stream, log, cfg, proj, Ms, copies=2):
    """One projection shape: the autotuned plan and each pipeline's best per M, timed over
    rotated copies of the compressed weights."""
    w = synth.gen_weight(cfg, proj)
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
    ws_bytes = uw.workspace_bytes(h, uw.PIPE_FULL)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    rows = {}
    for M in Ms:
        x = torch.from_numpy(synth.gen_x(cfg, M, K).view(np.int16)).to(dev)
        y = torch.empty(M, N, dtype=torch.float32, device=dev)
        per = {}
        for p in range(5):
            pl = uw.autotune(h, blobs[0], x, y, [M], d_direct=planes[0], d_ws=ws, ws_bytes=ws_bytes, reps=5, warmup=2,
                             pipeline_mask=1 << p)[0]
            ms = timed(torch, stream, lambda r: uw.run_pipeline(p, h, blobs[r % copies], x, y, M, d_direct=planes[r % copies],
                                                                d_ws=ws, ws_bytes=ws_bytes, variant=pl.variant,
                                                                stream=stream))
            alg = algorithmic_bytes(h, M, p)
            per[uw.PIPELINE_NAMES[p]] = {
                "variant": uw.variant_name(pl.variant), "us": round(ms * 1e3, 2),
                "uncompressed_GBs": round(2 * N * K / (ms * 1e-3) / 1e9, 1),
                "hbm_frac_compressed": round(alg / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                "tflops": round(2.0 * M * N * K / (ms * 1e-3) / 1e12, 1),
                "mfma_frac": round(2.0 * M * N * K / (ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4)}
        best = min(per, key=lambda k: per[k]["us"])
        rows[str(M)] = {"best": best, **per}
        log(f"[bench] {cfg.name}/{proj} {N}x{K} M={M}: best {best} {per[best]}")
    return {"shape": [N, K], "blob_bytes_per_weight": round(blob.size / (N * K), 4), "by_M": rows}


def stack_sweep(uw, synth, torch, dev, stream, log, Ms):
    """The 32-layer SwiGLU stack through uw_mlp_stack_forward: per M, plans autotuned on
    layer 0's gate and down shapes, one forward timed with one stream and with a separate
    decode stream."""
    import concurrent.futures as cf

    cfg = synth.CONFIGS["stack"]
    sig = synth.gen_stack_sigmas(cfg)
    L = cfg.layers
    t0 = time.time()

    def make(i):
        layer, q = divmod(i, 3)
        proj = ("gate", "up", "down")[q]
        return uw.encode(synth.gen_weight(cfg, proj, layer, sigma=float(sig[layer])))

    with cf.ThreadPoolExecutor(max(1, min(16, (os.cpu_count() or 8)))) as ex:
        blobs_h = list(ex.map(make, range(3 * L)))
    hs = [uw.inspect(b) for b in blobs_h]
    d_blobs, d_planes = [], []
    for b, h in zip(blobs_h, hs):
        db = torch.from_numpy(b).to(dev)
        dp = torch.empty(uw.direct_plane_bytes(h), dtype=torch.uint8, device=dev)
        uw.prepare_direct(h, db, dp)
        d_blobs.append(db)
        d_planes.append(dp)
    del blobs_h
    torch.cuda.synchronize()
    log(f"[bench] stack: {3 * L} matrices encoded and prepared in {time.time() - t0:.1f}s")
    Nff, K = hs[0].N, hs[0].K
    weight_bytes = sum(2 * h.N * h.K for h in hs)
    ws_t = torch.empty(uw.workspace_bytes(hs[0], uw.PIPE_FULL), dtype=torch.uint8, device=dev)
    side = torch.cuda.Stream()
    rows = {}
    for M in Ms:
        plans = {}
        for q, Kin, Nout in ((0, K, Nff), (2, Nff, K)):
            x = torch.from_numpy(synth.gen_x(cfg, M, Kin).view(np.int16)).to(dev)
            y = torch.empty(M, Nout, dtype=torch.float32, device=dev)
            plans[q] = uw.autotune(hs[q], d_blobs[q], x, y, [M], d_direct=d_planes[q], d_ws=ws_t, ws_bytes=ws_t.numel(),
                                   reps=5, warmup=2)[0]
        layers = []
        for layer in range(L):
            trip = []
            for q in range(3):
                i = 3 * layer + q
                pl = plans[0 if q < 2 else 2]
                trip.append(uw.proj(hs[i], d_blobs[i], pl.pipeline, d_direct=d_planes[i], variant=pl.variant))
            layers.append(trip)
        arr = uw.mlp_layers(layers)
        x = torch.from_numpy(synth.gen_x(cfg, M, K).view(np.int16)).to(dev)
        y = torch.empty(M, K, dtype=torch.float32, device=dev)
        row = {"gate_up_plan": f"{uw.PIPELINE_NAMES[plans[0].pipeline]} / {uw.variant_name(plans[0].variant)}",
               "down_plan": f"{uw.PIPELINE_NAMES[plans[2].pipeline]} / {uw.variant_name(plans[2].variant)}"}
        for two in (False, True):
            nb = uw.mlp_stack_workspace(arr, M, two_slots=two)
            ws = torch.empty(nb, dtype=torch.uint8, device=dev)
            fwd = lambda r: uw.mlp_stack_forward(arr, M, x, y, ws, nb, stream=stream, decode_stream=side if two else None)
            fwd(0)
            ms = timed(torch, stream, fwd, reps=3)
            key = "two_streams" if two else "one_stream"
            row[key] = {"ms": round(ms, 3), "tokens_per_s": round(M / (ms * 1e-3), 1),
                        "uncompressed_GBs": round(weight_bytes / (ms * 1e-3) / 1e9, 1),
                        "tflops": round(2.0 * M * weight_bytes / 2 / (ms * 1e-3) / 1e12, 1)}
            del ws
        rows[str(M)] = row
        log(f"[bench] stack M={M}: {row}")

    # decode-first plans (the best of full / exponent / transcode per shape) with the
    # preprocessing on one stream, on a second stream, and on CU-split stream pairs
    split = {}
    for M in (1, 16, 64):
        plans = {}
        for q, Kin, Nout in ((0, K, Nff), (2, Nff, K)):
            xq = torch.from_numpy(synth.gen_x(cfg, M, Kin).view(np.int16)).to(dev)
            yq = torch.empty(M, Nout, dtype=torch.float32, device=dev)
            plans[q] = uw.autotune(hs[q], d_blobs[q], xq, yq, [M], d_ws=ws_t, ws_bytes=ws_t.numel(), reps=5,
                                   warmup=2, pipeline_mask=0b0111)[0]
        arr = uw.mlp_layers([[uw.proj(hs[3 * l + q], d_blobs[3 * l + q], plans[0 if q < 2 else 2].pipeline,
                                      variant=plans[0 if q < 2 else 2].variant) for q in range(3)] for l in range(L)])
        x = torch.from_numpy(synth.gen_x(cfg, M, K).view(np.int16)).to(dev)
        y = torch.empty(M, K, dtype=torch.float32, device=dev)
        row = {"gate_up_plan": f"{uw.PIPELINE_NAMES[plans[0].pipeline]} / {uw.variant_name(plans[0].variant)}",
               "down_plan": f"{uw.PIPELINE_NAMES[plans[2].pipeline]} / {uw.variant_name(plans[2].variant)}"}
        for mode in ("one_stream", "two_streams", "cu_split_32", "cu_split_64", "cu_split_128"):
            two = mode != "one_stream"
            nb = uw.mlp_stack_workspace(arr, M, two_slots=two)
            ws = torch.empty(nb, dtype=torch.uint8, device=dev)
            pair = uw.stream_pair_create(int(mode.rsplit("_", 1)[1])) if mode.startswith("cu_split") else None
            main = torch.cuda.ExternalStream(pair[0]) if pair else stream
            dec = pair[1] if pair else (side if two else None)
            torch.cuda.synchronize()
            fwd = lambda r: uw.mlp_stack_forward(arr, M, x, y, ws, nb, stream=main, decode_stream=dec)
            fwd(0)
            ms = timed(torch, main, fwd, reps=3)
            torch.cuda.synchronize()
            if pair:
                uw.stream_destroy(pair[0])
                uw.stream_destroy(pair[1])
            row[mode] = {"ms": round(ms, 3), "uncompressed_GBs": round(weight_bytes / (ms * 1e-3) / 1e9, 1)}
            del ws
        split[str(M)] = row
        log(f"[bench] stack decode-first M={M}: {row}")

    # hard / easy layers: every 4th layer keeps only its Huffman blobs (no direct planes, so
    # it always needs preprocessing); the others hold direct planes. Start: direct palette on
    # the easy layers, full decode on the hard ones; uw_mlp_stack_autotune then tunes the
    # per-class, per-role pipelines and the decode order end to end (decode stream, 3 slots).
    hard = {}
    for M in (1, 16, 64, 256):
        layers = []
        for l in range(L):
            is_hard = l % 4 == 3
            layers.append([uw.proj(hs[3 * l + q], d_blobs[3 * l + q], uw.PIPE_FULL if is_hard else uw.PIPE_DIRECT,
                                   d_direct=None if is_hard else d_planes[3 * l + q]) for q in range(3)])
        arr = uw.mlp_layers(layers)
        full = uw.mlp_layers([[uw.proj(hs[3 * l + q], d_blobs[3 * l + q], uw.PIPE_FULL) for q in range(3)]
                              for l in range(L)])
        nb = uw.mlp_stack_workspace_ex(full, M, slots=3)
        ws = torch.empty(nb, dtype=torch.uint8, device=dev)
        x = torch.from_numpy(synth.gen_x(cfg, M, K).view(np.int16)).to(dev)
        y = torch.empty(M, K, dtype=torch.float32, device=dev)
        torch.cuda.synchronize()
        t0 = time.time()
        a = uw.mlp_stack_autotune(arr, M, x, y, ws, nb, stream=stream, decode_stream=side, slots=3, reps=3, warmup=1)
        torch.cuda.synchronize()
        tune_s = time.time() - t0
        plan = {}
        for cls, l in (("easy", 0), ("hard", 3)):
            plan[cls] = {r: uw.PIPELINE_NAMES[getattr(arr[l], r).pipeline] for r in ("gate", "up", "down")}
        fwd = lambda r: uw.mlp_stack_forward_ex(arr, M, x, y, ws, nb, stream=stream, decode_stream=side, slots=3,
                                                down_first=bool(a.opts.down_first))
        fwd(0)
        ms = timed(torch, stream, fwd, reps=3)
        hard[str(M)] = {"hard_layers": L // 4, "plan": plan, "down_first": bool(a.opts.down_first),
                        "start_ms": round(a.t_start_ms, 3), "tuned_ms": round(ms, 3), "passes": a.passes,
                        "trials": a.trials, "tune_seconds": round(tune_s, 1),
                        "uncompressed_GBs": round(weight_bytes / (ms * 1e-3) / 1e9, 1)}
        del ws
        log(f"[bench] stack hard/easy M={M}: {hard[str(M)]}")
    return {"layers": L, "shapes": {"gate_up": [Nff, K], "down": [K, Nff]}, "by_M": rows, "decode_first": split,
            "hard_easy_tuned": hard}


def configs_sweep(uw, synth, torch, dev, stream, log):
    """The other workloads: down_proj (M 256..4096), the 70B-shaped layer (gate and down,
    M 1..2048), the 32-layer stack (M sweep), and PyTorch's bf16 matmul on plain bf16
    weights of the large-M shapes as a reference point."""
    out = {}
    out["down"] = shape_sweep(uw, synth, torch, dev, stream, log, synth.CONFIGS["down"], "down", (256, 1024, 4096))
    c70 = synth.CONFIGS["70b"]
    out["70b_gate"] = shape_sweep(uw, synth, torch, dev, stream, log, c70, "gate", c70.Ms)
    out["70b_down"] = shape_sweep(uw, synth, torch, dev, stream, log, c70, "down", c70.Ms)
    torch.cuda.empty_cache()
    out["stack"] = stack_sweep(uw, synth, torch, dev, stream, log, (1, 4, 16, 64, 256, 1024, 4096))
    ref = {}
    for (N, K, M) in ((4096, 14336, 4096), (14336, 4096, 4096), (8192, 28672, 2048)):
        a = torch.randn(M, K, device=dev, dtype=torch.bfloat16)
        b = torch.randn(N, K, device=dev, dtype=torch.bfloat16)
        ms = timed(torch, stream, lambda r: torch.matmul(a, b.t()), reps=10)
        ref[f"M={M} N={N} K={K}"] = {"us": round(ms * 1e3, 1), "tflops": round(2.0 * M * N * K / (ms * 1e-3) / 1e12, 1)}
        del a, b
    # small M on the gate shape: plain bf16 weights (2 B/w) over 6 rotated copies, launches
    # back to back between two events, as the headline step is timed
    ws = [torch.randn(14336, 4096, device=dev, dtype=torch.bfloat16) for _ in range(6)]
    for M in (1, 16, 64):
        a = torch.randn(M, 4096, device=dev, dtype=torch.bfloat16)
        for r in range(6):
            torch.matmul(a, ws[r].t())
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for r in range(48):
            torch.matmul(a, ws[r % 6].t())
        e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) / 48 * 1e3
        ref[f"M={M} N=14336 K=4096 (bf16 weights, rotated)"] = {
            "us": round(us, 2), "weight_GBs": round(2 * 14336 * 4096 / (us * 1e-6) / 1e9, 1)}
    del ws
    out["vendor_bf16_matmul_reference"] = ref
    log(f"[bench] vendor reference: {ref}")
    return out


def large_m_line(uw, synth, torch, dev, stream, log):
    """TFLOP/s on the down_proj shape at M = 4096 (MFMA-bound) of the direct-palette pipeline,
    the full-decode pipeline and the expand pipeline (bf16 weights rebuilt in HBM from the
    Huffman stream or from the direct plane, then the best plain bf16 GEMM: ours or the vendor
    library's), each with its autotuned variant, vs the 2.5 PFLOP/s bf16 peak."""
    cfg = synth.CONFIGS["down"]
    w = synth.gen_weight(cfg, "down")
    blob = uw.encode(w)
    h = uw.inspect(blob)
    N, K, M = h.N, h.K, 4096
    b = torch.from_numpy(blob).to(dev)
    idx = torch.empty(uw.direct_plane_bytes(h), dtype=torch.uint8, device=dev)
    uw.prepare_direct(h, b, idx)
    x = torch.from_numpy(synth.gen_x(cfg, M, K).view(np.int16)).to(dev)
    y = torch.empty(M, N, dtype=torch.float32, device=dev)
    ws = torch.empty(uw.workspace_bytes(h, uw.PIPE_FULL), dtype=torch.uint8, device=dev)
    res = {}
    for p in (uw.PIPE_DIRECT, uw.PIPE_FULL, uw.PIPE_EXPAND):
        pl = uw.autotune(h, b, x, y, [M], d_direct=idx, d_ws=ws, ws_bytes=ws.numel(), reps=5, warmup=2,
                         pipeline_mask=1 << p)[0]
        ts = []
        for _ in range(10):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            uw.run_pipeline(p, h, b, x, y, M, d_direct=idx, d_ws=ws, ws_bytes=ws.numel(), variant=pl.variant, stream=stream)
            e1.record(stream)
            ts.append((e0, e1))
        torch.cuda.synchronize()
        ms = float(np.median([a.elapsed_time(c) for a, c in ts]))
        tf = 2.0 * M * N * K / (ms * 1e-3) / 1e12
        res[uw.PIPELINE_NAMES[p]] = {"variant": uw.variant_name(pl.variant), "ms": round(ms, 4), "tflops": round(tf, 1),
                                     "mfma_frac": round(tf / BF16_PEAK_TFLOPS, 4)}
    log(f"[bench] large M: {res}")
    return {"workload": "down_proj shape W 4096x14336, M=4096", "unit": "TFLOP/s", **res}


def cpu_baseline(synth, cfg, w, Ms, log, steps=3):
    """The CPU oracle on `steps` full steps of the same workload: for each M, bit-serial
    decode of the Huffman blob to bf16 W, then the fp64 GEMM; single-threaded C (about
    15 s on the host cores)."""
    import oracle

    blob = oracle.encode(w, chunk=256)
    xs = {M: synth.gen_x(cfg, M, w.shape[1]) for M in Ms}
    t = time.time()
    for _ in range(steps):
        for M in Ms:
            d = oracle.decode(blob, want=("w",))
            oracle.gemm(xs[M], d["w"])
    dt = time.time() - t
    N, K = w.shape
    v = 2.0 * N * K * len(Ms) * steps / dt / 1e9
    log(f"[bench] cpu oracle {steps} steps {dt:.1f}s -> {v:.3f} GB/s")
    return {"value": round(v, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{steps} full steps (M in {{{', '.join(map(str, Ms))}}}: decode + fp64 GEMM each), {dt:.1f} s"}


if __name__ == "__main__":
    main()
