"""Full-shape parity of the 8B-shaped MLP stack workload (32 SwiGLU layers of gate and up
14336 x 4096 and down 4096 x 14336, sigma_l = 0.02 * U(0.8, 1.2)), through the C ABI.

- Every loader (bf16, exponent, index, direct plane), every large-batch GEMM variant and
  several K splits on the gate and down shapes at M = 256, 1024 and 4096: a seeded sample
  of Y against the fp64 oracle (1e-3 * sum|x w|), and no unwritten output.
- The whole 32-layer uw_mlp_stack_forward at M = 64 (the plans the bench measures there:
  fused gate/up, down with a K split) and at M = 1024 (every pipeline, layers cycling
  through them; the SwiGLU in the up GEMM's epilogue): the layer run last is checked
  teacher-forced (its g against the oracle on X, h against the SwiGLU of the GPU's g and
  the oracle's u within the GEMM tolerance and one bf16 rounding, Y against the oracle on
  the GPU's h), with the layer order rotated so that several layers, one of each
  pipeline, are the last one; and one layer at M = 4096 on expand + the 256x256 DMA GEMM
  (three whole rounds of the CUs and a 256x128 tail per launch).
"""
import concurrent.futures as cf
import os

import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import check_gemm, dev, empty_f32, empty_u8, empty_u16, host, log, torch_cuda, zeros_u32

pytestmark = pytest.mark.gpu

uw = None
CFG = synth.CONFIGS["stack"]
ROLES = ("gate", "up", "down")


def setup_module():
    global uw
    torch_cuda()
    import decode_gemm_amd

    uw = decode_gemm_amd
    oracle.build(force=False)


def _variant(name):
    names = [uw.variant_name(v) for v in range(uw.variant_count())]
    return names.index(name)


def _weight(layer, role):
    sig = synth.gen_stack_sigmas(CFG)
    return synth.gen_weight(CFG, role, layer, sigma=float(sig[layer]))


def _sample(t, mi, ni):
    """Y[mi, ni] gathered on the device, to host float32."""
    torch = torch_cuda()
    return t[torch.from_numpy(mi).cuda(), torch.from_numpy(ni).cuda()].cpu().numpy()


def _all_finite(t):
    torch = torch_cuda()
    return bool(torch.isfinite(t).all().item())


@pytest.mark.parametrize("role", ["gate", "down"])
def test_stack_shapes_large_m_every_loader_variant_and_split(role):
    w = _weight(0, role)
    N, K = w.shape
    blob = uw.encode(w)
    h = uw.inspect(blob)
    d_blob = dev(blob)
    err = zeros_u32()
    planes = {uw.W_BF16: empty_u16(N * K), uw.W_EXP: empty_u8(N * K), uw.W_IDX: empty_u8(N * K // 2),
              uw.W_DIRECT: empty_u8(uw.direct_plane_bytes(h))}
    uw.decode_full(h, d_blob, planes[uw.W_BF16], err)
    uw.decode_exponent(h, d_blob, planes[uw.W_EXP], err)
    uw.transcode_palette(h, d_blob, planes[uw.W_IDX], err)
    uw.prepare_direct(h, d_blob, planes[uw.W_DIRECT], err)
    torch_cuda().cuda.synchronize()
    assert int(host(err)[0]) == 0
    rng = np.random.default_rng(4242)
    for M in (256, 1024, 4096):
        x = synth.gen_x(CFG, M, K)
        d_x = dev(x)
        mi, ni = rng.integers(0, M, 4096), rng.integers(0, N, 4096)
        y_ref, a_ref = oracle.gemm_pairs(x, w, mi, ni)
        y = empty_f32(M, N)
        for src, plane in planes.items():
            for v in range(uw.variant_count()):
                if not uw.variant_supports(v, N, K, M, src):
                    continue
                for ks in (0, 1, 2, 4):
                    what = f"{role} M={M} src={src} {uw.variant_name(v)} split={ks} ({uw.split_count(v, N, K, M, ks)})"
                    log(f"  {what}")
                    y.fill_(float("nan"))
                    uw.recon_gemm(h, d_blob, src, plane, d_x, y, M, variant=v, split_k=ks)
                    check_gemm(_sample(y, mi, ni), y_ref, a_ref, what)
                    assert _all_finite(y), f"{what}: unwritten outputs"
        if role == "gate" and M == 4096:
            # 896 tiles of 256 x 256 are 3.5 rounds of 256 CUs: the DMA launch runs three whole
            # rounds and its last column blocks as 256 x 128 tiles. Every output is summed over K
            # in the same order as by the 256 x 128 variant alone, so the two agree bit for bit.
            names = [uw.variant_name(v) for v in range(uw.variant_count())]
            y2 = empty_f32(M, N)
            y2.fill_(float("nan"))
            y.fill_(float("nan"))
            uw.recon_gemm(h, d_blob, uw.W_BF16, planes[uw.W_BF16], d_x, y, M, variant=names.index("dma 256x256"),
                          split_k=1)
            uw.recon_gemm(h, d_blob, uw.W_BF16, planes[uw.W_BF16], d_x, y2, M,
                          variant=names.index("dma 256x128 s3"), split_k=1)
            assert torch_cuda().equal(y, y2), "dma 256x256 in whole rounds differs from dma 256x128 s3"
            del y2
        del d_x, y


class _Stack:
    """The 32 layers on the device: headers, blobs, direct planes (host weights are
    regenerated from the seeds when a layer is checked)."""

    def __init__(self):
        def make(i):
            layer, q = divmod(i, 3)
            return uw.encode(_weight(layer, ROLES[q]))

        self.h, self.blob, self.plane = {}, {}, {}
        with cf.ThreadPoolExecutor(max(1, min(16, os.cpu_count() or 8))) as ex:
            for i, b in enumerate(ex.map(make, range(3 * CFG.layers))):
                key = divmod(i, 3)
                h = uw.inspect(b)
                self.h[key] = h
                self.blob[key] = dev(b)
                p = empty_u8(uw.direct_plane_bytes(h))
                uw.prepare_direct(h, self.blob[key], p)
                self.plane[key] = p
        torch_cuda().cuda.synchronize()

    def arr(self, order, plan_of):
        rows = []
        for l in order:
            trip = []
            for q in range(3):
                pipe, var, ks = plan_of(l, q)
                trip.append(uw.proj(self.h[(l, q)], self.blob[(l, q)], pipe, d_direct=self.plane[(l, q)],
                                    variant=var, split_k=ks))
            rows.append(trip)
        return uw.mlp_layers(rows)


def _check_last(st, last, x, y, ws, M, rng, what):
    """Teacher-forced check of the layer run last: g and h are left in the workspace (u
    only where the up GEMM ran without the SwiGLU epilogue, so it is not read here)."""
    torch = torch_cuda()
    F, K = st.h[(0, 0)].N, st.h[(0, 0)].K
    a256 = lambda v: (v + 255) // 256 * 256
    g = ws[: 4 * M * F].view(torch.float32).reshape(M, F)
    ho = 2 * a256(4 * M * F)
    hg = ws[ho: ho + 2 * M * F].view(torch.int16).reshape(M, F)
    mi, fi = rng.integers(0, M, 4096), rng.integers(0, F, 4096)
    yr, ar = oracle.gemm_pairs(x, _weight(last, "gate"), mi, fi)
    gs = _sample(g, mi, fi)
    check_gemm(gs, yr, ar, f"{what}: layer {last} gate")
    # h = bf16(silu(g) u) with the GPU's g and u within 1e-3 sum|x w| of the oracle's u:
    # |h - silu(g) u_oracle| <= |silu(g)| 1e-3 sum|x w| + the bf16 rounding of h (2^-8 |h|,
    # which also covers the fp32 arithmetic of silu)
    ur, ua = oracle.gemm_pairs(x, _weight(last, "up"), mi, fi)
    hs = _sample(hg, mi, fi).view(np.uint16)
    hv = (hs.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    g64 = gs.astype(np.float64)
    sg = g64 / (1.0 + np.exp(-g64))
    err = np.abs(hv - sg * ur)
    bound = np.abs(sg) * 1e-3 * ua + 2.0 ** -8 * np.abs(hv) + 1e-30
    assert (err <= bound).all(), f"{what}: layer {last} up + SwiGLU, worst {float(np.max(err - bound))}"
    hh = host(hg).view(np.uint16)
    ni = rng.integers(0, K, 4096)
    yr, ar = oracle.gemm_pairs(hh, _weight(last, "down"), mi, ni)
    check_gemm(_sample(y, mi, ni), yr, ar, f"{what}: layer {last} down")
    assert _all_finite(y)


def test_stack_32_layers_forward_teacher_forced():
    st = _Stack()
    L = CFG.layers
    rng = np.random.default_rng(7)
    torch = torch_cuda()
    xs = synth.gen_x(CFG, 4096, st.h[(0, 0)].K)
    # M = 64: the plans the bench measures there (fused gate/up; down with four K slices)
    xt, ks4 = _variant("skinny rt4 u2 w4 xt"), _variant("skinny rt4 u2 w4 xt ks")
    plan64 = lambda l, q: (uw.PIPE_DIRECT, ks4, 4) if q == 2 else (uw.PIPE_DIRECT, xt, 0)
    # M = 1024: every pipeline, layers cycling through them; direct layers on the 256x256
    # tile with explicit splits, the others on their default variant
    wide = _variant("wide 256x256")
    pipes = (uw.PIPE_FULL, uw.PIPE_EXP, uw.PIPE_TRANSCODE, uw.PIPE_DIRECT, uw.PIPE_EXPAND)

    def plan1024(l, q):
        p = pipes[l % 5]
        if p == uw.PIPE_DIRECT:
            return p, wide, 4 if q == 2 else 1
        return p, -1, 0

    # M = 4096, one layer: expand + the 256 x 256 DMA GEMM (gate and up: three whole rounds of
    # 256 CUs and a 256 x 128 tail, the SwiGLU in up's epilogue through both launches)
    dma = _variant("dma 256x256")
    plan4096 = lambda l, q: (uw.PIPE_EXPAND, dma, 1)
    for M, plan_of, lasts in ((64, plan64, (L - 1, 0, 13)), (1024, plan1024, (L - 1, 0, 1, 2, 3, 4)),
                              (4096, plan4096, (5,))):
        x = xs[:M]
        d_x = dev(x)
        y = empty_f32(M, st.h[(0, 2)].N)
        for last in lasts:
            order = [l for l in range(L) if l != last] + [last] if M < 4096 else [last]
            arr = st.arr(order, plan_of)
            nb = uw.mlp_stack_workspace(arr, M)
            ws = empty_u8(nb)
            y.fill_(float("nan"))
            log(f"  stack forward M={M}, layer {last} last ({uw.PIPELINE_NAMES[plan_of(last, 0)[0]]})")
            uw.mlp_stack_forward(arr, M, d_x, y, ws, nb)
            torch.cuda.synchronize()
            _check_last(st, last, x, y, ws, M, rng, f"M={M}")
            del ws


class _Loaded:
    """Stack layers taken from a loaded bundle ({name: (Header, d_blob, d_direct)})."""

    def __init__(self, loaded):
        self.h, self.blob, self.plane = {}, {}, {}
        for l in range(CFG.layers):
            for q in range(3):
                h, b, p = loaded[f"layers.{l}.mlp.{ROLES[q]}_proj"]
                self.h[(l, q)], self.blob[(l, q)], self.plane[(l, q)] = h, b, p

    arr = _Stack.arr


def test_stack_bundle_round_trip_load_and_forward():
    """The 32-layer stack written as one bundle (96 Huffman blobs and the plans at M = 64
    and 1024), opened with full verification and loaded with transcode at load
    (uw_prepare_direct per projection): the planes equal those made from the original
    blobs, and the forward on the bundle's own plans matches the oracle (last layer
    teacher-forced)."""
    torch = torch_cuda()

    def make(i):
        layer, q = divmod(i, 3)
        return uw.encode(_weight(layer, ROLES[q]))

    with cf.ThreadPoolExecutor(max(1, min(16, os.cpu_count() or 8))) as ex:
        blobs = list(ex.map(make, range(3 * CFG.layers)))
    names = [f"layers.{l}.mlp.{r}_proj" for l in range(CFG.layers) for r in ROLES]
    F, K = 14336, 4096
    plans = [dict(N=F, K=K, M=64, pipeline=uw.PIPE_DIRECT, split_k=0, variant="skinny rt4 u2 w4 xt"),
             dict(N=K, K=F, M=64, pipeline=uw.PIPE_DIRECT, split_k=4, variant="skinny rt4 u2 w4 xt ks"),
             dict(N=F, K=K, M=1024, pipeline=uw.PIPE_EXPAND, split_k=0, variant="wide 256x256"),
             dict(N=K, K=F, M=1024, pipeline=uw.PIPE_DIRECT, split_k=4, variant="wide 256x256")]
    buf = uw.bundle_write(list(zip(names, blobs)), plans)
    total = sum(b.size for b in blobs)
    log(f"  bundle {buf.size / 1e9:.2f} GB for {total / 1e9:.2f} GB of blobs")
    assert total <= buf.size < total + 256 * (len(blobs) + 64)
    info = uw.bundle_open(buf, verify=True)
    assert info.n_items == 96 and info.n_plans == 4
    loaded = uw.load_bundle(buf)
    st = _Loaded(loaded)
    for l, q in ((0, 0), (17, 2), (31, 1)):
        ref = empty_u8(uw.direct_plane_bytes(st.h[(l, q)]))
        uw.prepare_direct(st.h[(l, q)], dev(blobs[3 * l + q]), ref)
        assert torch.equal(ref, st.plane[(l, q)]), f"layer {l} {ROLES[q]}: plane from the bundle differs"
    del blobs
    bplans = uw.bundle_plans(buf)
    rng = np.random.default_rng(11)
    xs = synth.gen_x(CFG, 1024, K)
    for M in (64, 1024):
        by = {(p["N"], p["K"]): p for p in bplans if p["M"] == M}
        plan_of = lambda l, q: (lambda p: (p["pipeline"], p["variant"], p["split_k"]))(by[(K, F)] if q == 2 else by[(F, K)])
        order = list(range(CFG.layers))
        arr = st.arr(order, plan_of)
        nb = uw.mlp_stack_workspace(arr, M)
        ws = empty_u8(nb)
        y = empty_f32(M, K)
        y.fill_(float("nan"))
        x = xs[:M]
        log(f"  bundle stack forward M={M}")
        uw.mlp_stack_forward(arr, M, dev(x), y, ws, nb)
        torch.cuda.synchronize()
        _check_last(st, CFG.layers - 1, x, y, ws, M, rng, f"bundle M={M}")
        del ws
