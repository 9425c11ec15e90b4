"""GPU parity: every kernel of libuw against the CPU oracle, through the C ABI.

Decoded planes must be bit-exact (the method is lossless); GEMM outputs must lie
within 1e-3 * sum_k |x_k w_k| of the fp64 oracle elementwise. Small cases span several
tiles and ragged tails; the full-size workloads (gate 14336x4096, down 4096x14336,
70B-shaped 28672x8192 / 8192x28672) compare decoded planes in full and a seeded sample
of GEMM outputs, in the launch configurations the bench uses.
"""
import numpy as np
import pytest

import oracle
import synth
from tests import direct_layout
from tests.gpu_util import check_gemm, dev, empty_f32, empty_u8, empty_u16, host, log, torch_cuda, zeros_u32

pytestmark = pytest.mark.gpu

uw = None


def setup_module():
    global uw
    torch_cuda()
    import decode_gemm_amd

    uw = decode_gemm_amd
    oracle.build(force=False)


def _sync():
    torch_cuda().cuda.synchronize()


class Mat:
    """A weight matrix uploaded with its library blob, plus oracle reference planes."""

    def __init__(self, w, chunk=0, lmax=0, blob=None):
        self.w = np.ascontiguousarray(w, dtype=np.uint16)
        self.N, self.K = self.w.shape
        self.blob = uw.encode(self.w, chunk=chunk, lmax=lmax) if blob is None else blob
        self.h = uw.inspect(self.blob)
        self.d_blob = dev(self.blob)
        self._ref = None

    def ref(self):
        if self._ref is None:
            self._ref = oracle.decode(self.blob, want=("exp", "idx"))
        return self._ref

    def decode(self, mode):
        n = self.N * self.K
        err = zeros_u32()
        if mode == "full":
            out = empty_u16(n)
            uw.decode_full(self.h, self.d_blob, out, err)
        elif mode == "exp":
            out = empty_u8(n)
            uw.decode_exponent(self.h, self.d_blob, out, err)
        elif mode == "direct":
            out = empty_u8(uw.direct_plane_bytes(self.h))
            out.fill_(0xA5)  # every byte must be written by uw_prepare_direct
            uw.prepare_direct(self.h, self.d_blob, out, err)
        else:
            out = empty_u8(n // 2)
            uw.transcode_palette(self.h, self.d_blob, out, err)
        _sync()
        return out, int(host(err)[0])


def _check_decoders(m: Mat, what: str):
    log(f"  decode {what} N={m.N} K={m.K} chunk={m.h.chunk} lmax={m.h.lmax} raw={m.h.n_raw}")
    out, err = m.decode("full")
    assert err == 0, f"{what}: error flags {err}"
    assert (host(out, np.uint16).reshape(m.N, m.K) == m.w).all(), f"{what}: full decode differs"
    ref = m.ref()
    out, err = m.decode("exp")
    assert err == 0 and (host(out).reshape(m.N, m.K) == ref["exp"]).all(), f"{what}: exponent plane differs"
    out, err = m.decode("idx")
    assert err == 0 and (host(out) == ref["idx"]).all(), f"{what}: index plane differs"
    # the direct plane is a GPU operand layout, not a step of the method: it is checked by
    # what it must hold (W itself through the format's reader, the raw-group rule of the
    # oracle, the bytes the format fixes to zero), not against an oracle copy of the layout
    out, err = m.decode("direct")
    plane = host(out)
    assert err == 0, f"{what}: direct plane error flags {err}"
    assert plane.size == direct_layout.plane_bytes(m.N, m.K, m.h.n_raw), f"{what}: direct plane size"
    pal_sorted = sorted(int(v) for v in m.h.palette[: m.h.n_pal])
    assert (direct_layout.rebuild(plane, pal_sorted, m.N, m.K) == m.w).all(), f"{what}: direct plane does not hold W"
    assert direct_layout.zero_bytes_ok(plane, m.N, m.K) == [], f"{what}: direct plane format"
    _, e_ref = oracle.split(m.w)
    pal_ref, _ = oracle.palette(e_ref)
    bitmap, _, _ = oracle.raw_groups(e_ref.reshape(m.N, m.K), pal_ref)
    G = m.K // 64
    raw_ref = ((bitmap[:, np.arange(G) // 32] >> (np.arange(G) % 32).astype(np.uint32)) & 1).astype(bool)
    assert (direct_layout.raw_masks(plane, m.N, m.K) == raw_ref).all(), f"{what}: raw rows of the direct plane"
    # the direct plane expanded back to bf16 is the original matrix, bit for bit
    wx = empty_u16(m.N * m.K)
    wx.fill_(0x5A5A)  # every weight must be written
    uw.expand_direct(m.h, out, wx)
    _sync()
    assert (host(wx, np.uint16).reshape(m.N, m.K) == m.w).all(), f"{what}: expanded direct plane differs"


def test_decoders_tiny_library_and_oracle_blobs():
    w = synth.gen_weight(synth.CONFIGS["tiny"], "w")
    for chunk, lmax in ((64, 12), (256, 12), (1024, 12), (192, 7), (512, 14), (128, 4)):
        _check_decoders(Mat(w, chunk, lmax), f"lib chunk={chunk} lmax={lmax}")
        _check_decoders(Mat(w, blob=oracle.encode(w, chunk=chunk, lmax=lmax)), f"oracle chunk={chunk} lmax={lmax}")


def test_decoders_edge_matrices():
    rng = np.random.default_rng(31)
    _check_decoders(Mat(np.full((3, 192), 0x3C01, np.uint16), 128), "single symbol")
    e = rng.integers(100, 116, size=(5, 128)).astype(np.uint16)
    e[:, 5] = 200 + np.arange(5)
    e[:, 70] = 210 + np.arange(5)
    w = ((e << 7) | rng.integers(0, 256, size=e.shape).astype(np.uint16) & 0x807F).astype(np.uint16)
    m = Mat(w, 64)
    assert m.h.total_bits == 0
    _check_decoders(m, "all raw")
    w = synth.f32_to_bf16_bits(rng.standard_normal((37, 320), dtype=np.float32) * 0.02)
    w.reshape(-1)[rng.choice(w.size, 80, replace=False)] = np.array(
        [0, 0x8000, 1, 0x807F, 0x7F80, 0xFF80, 0x7FC1, 0xFFFF], np.uint16)[np.arange(80) % 8]
    _check_decoders(Mat(w, 1024), "specials, ragged last chunk")
    _check_decoders(Mat(w, 64 * 7), "chunk 448")
    e = rng.integers(110, 126, size=(6, 4096)).astype(np.uint16)
    e[1, 64 * 33 + 3] = 230
    e[3, 64 * 63] = 231
    e[5, 64 * 31 + 63] = 232
    w = ((e << 7) | rng.integers(0, 128, size=e.shape).astype(np.uint16)).astype(np.uint16)
    _check_decoders(Mat(w, 256), "raw groups in the second bitmap word")
    # one wave's worth of chunks and more: several workgroups, partial last wave
    w = synth.gen_weight(synth.CONFIGS["tiny"], "w")
    w2 = np.concatenate([w, w[:100]], axis=0)
    _check_decoders(Mat(w2, 64), "612 rows, 2448 chunks")


def test_decoder_reports_corruption():
    w = synth.gen_weight(synth.CONFIGS["tiny"], "w")
    m = Mat(w, 256)
    bad = m.blob.copy()
    oc = m.h.off_chunk + 4 * 5
    v = int(np.frombuffer(bad[oc : oc + 4].tobytes(), "<u4")[0])
    bad[oc : oc + 4] = np.frombuffer(np.uint32(v + 3).tobytes(), np.uint8)  # chunk 5 starts 3 bits late
    mb = Mat(w, blob=bad)
    _, err = mb.decode("idx")
    assert err & uw.DERR_CHUNKLEN
    # one used symbol has the code '0': a '1' bit in its stream is no code
    ws = np.full((2, 128), 0x3C01, np.uint16)
    ms = Mat(ws, 128)
    bad = ms.blob.copy()
    bad[ms.h.off_stream + 3] |= 0x80  # bit 0 of the first word (MSB) set
    _, err = Mat(ws, blob=bad).decode("exp")
    assert err & uw.DERR_BADCODE


def test_corrupt_raw_bookkeeping_stays_inside_the_buffers():
    """A device blob whose row_base and bitmap claim raw groups past the raw table (only the
    header is validated for device blobs): uw_prepare_direct drops those rows, reports
    UW_DERR_RAWINDEX and writes nothing past the plane (a sentinel guard region after it
    is untouched); the GEMMs that read raw groups through the corrupt blob or plane clamp
    their reads and finish (their values are meaningless)."""
    w = synth.gen_weight(synth.CONFIGS["tiny"], "w")
    m = Mat(w, 256)
    assert m.h.n_raw > 0
    bad = m.blob.copy()
    N, K = m.N, m.K
    rb = np.frombuffer(bad[m.h.off_rowbase: m.h.off_rowbase + 4 * (N + 1)].tobytes(), "<u4").copy()
    rb[300:] += 10000  # rows 300.. claim raw groups far past the table
    bad[m.h.off_rowbase: m.h.off_rowbase + 4 * (N + 1)] = np.frombuffer(rb.tobytes(), np.uint8)
    bw = m.h.bitmap_words
    bm = np.frombuffer(bad[m.h.off_bitmap: m.h.off_bitmap + 4 * N * bw].tobytes(), "<u4").copy().reshape(N, bw)
    bm[N - 3:] = 0xFFFFFFFF  # the last rows: every group raw (more than the table holds)
    bad[m.h.off_bitmap: m.h.off_bitmap + 4 * N * bw] = np.frombuffer(bm.tobytes(), np.uint8)
    # uw_inspect rejects this blob on the host; a blob already on the device is only
    # header-checked, so it is uploaded as is with the (unchanged) header
    with pytest.raises(uw.UwError):
        uw.inspect(bad)
    d_bad = dev(bad)
    pb = uw.direct_plane_bytes(m.h)
    guard = 4096
    buf = empty_u8(pb + guard)
    buf.fill_(0xA5)
    err = zeros_u32()
    uw.prepare_direct(m.h, d_bad, buf, err)
    _sync()
    assert int(host(err)[0]) & uw.DERR_RAWINDEX
    assert (host(buf)[pb:] == 0xA5).all(), "uw_prepare_direct wrote past the plane"
    # GEMMs over the corrupt blob (index plane, raw groups from row_base / bitmap) and over
    # the plane with corrupt side-table bases: every variant finishes, Y's guard is intact
    idx = empty_u8(N * K // 2)
    uw.transcode_palette(m.h, d_bad, idx, err)
    meta_off = 1536 * ((N + 15) // 16) * (K // 64)
    plane = host(buf)[:pb].copy()
    meta = np.frombuffer(plane[meta_off: meta_off + 8 * ((N + 15) // 16) * (K // 64)].tobytes(), "<u4").copy()
    meta[1::2] += 5000  # side-table bases past the table
    plane[meta_off: meta_off + meta.size * 4] = np.frombuffer(meta.tobytes(), np.uint8)
    d_plane = dev(plane)
    for src, wp in ((uw.W_IDX, idx), (uw.W_DIRECT, d_plane)):
        for M in (1, 16, 200):
            x = dev(synth.gen_x(synth.CONFIGS["tiny"], M, K))
            for v in _variants_for(m, M, src):
                yg = empty_f32(M * N + guard // 4)
                yg.fill_(1.5)
                uw.recon_gemm(m.h, d_bad, src, wp, x, yg, M, variant=v)
                _sync()
                assert (host(yg)[M * N:] == 1.5).all(), f"src {src} variant {v} M={M} wrote past Y"


# ---------------------------------------------------------------- GEMM
def _planes(m: Mat):
    """Device planes for each GEMM source, produced by the GPU decoders."""
    full, _ = m.decode("full")
    exp, _ = m.decode("exp")
    idx, _ = m.decode("idx")
    direct, _ = m.decode("direct")
    return {uw.W_BF16: full, uw.W_EXP: exp, uw.W_IDX: idx, uw.W_DIRECT: direct}


def _run_gemm(m, planes, src, x, variant):
    M = x.shape[0]
    d_x = dev(x)
    y = empty_f32(M, m.N)
    y.fill_(float("nan"))
    uw.recon_gemm(m.h, m.d_blob, src, planes[src], d_x, y, M, variant=variant)
    _sync()
    return host(y)


def _variants_for(m, M, src):
    return [v for v in range(uw.variant_count()) if uw.variant_supports(v, m.N, m.K, M, src)]


def test_gemm_one_hot_rows_give_weights_exactly():
    """X rows one-hot at k: Y[m][n] = W[n][k] exactly, through every loader and variant
    (pins the rebuild of sign, exponent, mantissa and the raw overlay)."""
    w = synth.gen_weight(synth.CONFIGS["tiny"], "w")
    m = Mat(w, 256)
    planes = _planes(m)
    wf = synth.bf16_bits_to_f32(w)
    ks = np.array([0, 1, 15, 16, 63, 64, 100, 127, 128, 200, 255] * 6)[:66]
    for M in (1, 16, 66):
        x = np.zeros((M, m.K), np.uint16)
        for r in range(M):
            x[r, ks[r % len(ks)]] = 0x3F80
        for src in (uw.W_BF16, uw.W_EXP, uw.W_IDX, uw.W_DIRECT):
            for v in _variants_for(m, M, src):
                log(f"  one-hot M={M} src={src} variant={v}")
                y = _run_gemm(m, planes, src, x, v)
                ref = np.stack([wf[:, ks[r % len(ks)]] for r in range(M)])
                assert np.array_equal(y, ref), f"one-hot M={M} src={src} variant={v}"


def test_gemm_direct_raw_heavy_blocks():
    """Direct plane with blocks of very different raw density: a few raw groups in some
    16-row tiles, rows 64..95 raw in every group (hundreds of side-table rows per
    workgroup). One-hot X rows give the weights exactly through every direct variant and
    the fused gate/up launch."""
    torch = torch_cuda()
    rng = np.random.default_rng(97)
    N, K = 160, 1152
    e = rng.integers(110, 126, size=(N, K)).astype(np.uint16)
    e[64:96, ::64] = 200 + (np.arange(32) % 20)[:, None]  # rows 64..95: raw in all 18 groups
    e[5, 64 * 3 + 7] = 221
    e[40, 64 * 10] = 222
    e[130, 64 * 17 + 63] = 223
    w = (((e << 7) | (rng.integers(0, 256, size=e.shape).astype(np.uint16) & 0x807F)) & 0xFFFF).astype(np.uint16)
    m = Mat(w, 256)
    assert m.h.n_raw == 32 * 18 + 3
    direct = m.decode("direct")[0]
    planes = {uw.W_DIRECT: direct}
    wf = synth.bf16_bits_to_f32(w)
    ks = np.array([0, 7, 63, 64 * 3 + 7, 64 * 10, 64 * 17 + 63, 640, 1151])
    for M in (1, 16, 64):
        x = np.zeros((M, K), np.uint16)
        for r in range(M):
            x[r, ks[r % len(ks)]] = 0x3F80
        ref = np.stack([wf[:, ks[r % len(ks)]] for r in range(M)])
        for v in _variants_for(m, M, uw.W_DIRECT):
            log(f"  raw rows M={M} variant={v}")
            assert np.array_equal(_run_gemm(m, planes, uw.W_DIRECT, x, v), ref), f"M={M} variant={v}"
        d_x = dev(x)
        yg, yu = empty_f32(M, N), empty_f32(M, N)
        h = torch.empty(M, N, dtype=torch.int16, device="cuda")
        # (8 waves with X rings have no fused form past M = 32: their LDS would not fit)
        xd = [v for v in range(uw.variant_count())
              if uw.variant_name(v) == "skinny rt4 u2 w4 xd" or (uw.variant_name(v) == "skinny rt4 u2 w8 xd" and M <= 32)]
        for v in [-1, 5, 14, 3, 2] + xd:
            log(f"  raw rows fused M={M} variant={v}")
            yg.fill_(float("nan"))
            yu.fill_(float("nan"))
            uw.recon_gemm_gate_up(m.h, m.d_blob, direct, m.h, m.d_blob, direct, d_x, yg, yu, h, M, variant=v)
            _sync()
            assert np.array_equal(host(yg), ref) and np.array_equal(host(yu), ref), f"fused M={M} variant={v}"


def test_gemm_small_integers_exact():
    rng = np.random.default_rng(41)
    N, K = 200, 320
    wi = rng.integers(-8, 9, size=(N, K))
    w = synth.f32_to_bf16_bits(wi.astype(np.float32))
    m = Mat(w, 128)
    planes = _planes(m)
    for M in (3, 40, 130):
        xi = rng.integers(-8, 9, size=(M, K))
        x = synth.f32_to_bf16_bits(xi.astype(np.float32))
        ref = (xi @ wi.T).astype(np.float32)
        for src in (uw.W_BF16, uw.W_EXP, uw.W_IDX, uw.W_DIRECT):
            for v in _variants_for(m, M, src):
                log(f"  integers M={M} src={src} variant={v}")
                assert np.array_equal(_run_gemm(m, planes, src, x, v), ref), f"M={M} src={src} v={v}"


def test_gemm_k_slices_one_hot_exact():
    """K = 4160 (65 groups of 64) with raw groups: the tiled and wide launches cut K into
    slices that start inside a bitmap word and end ragged, and add their partial sums
    into Y. One-hot X rows must still give the weights exactly."""
    cfg = synth.Config("kslice", 8, (("w", 333, 4160),), 0.02, "normal", 0.002, 0.0, 12, (1,))
    w = synth.gen_weight(cfg, "w")
    m = Mat(w, 256)
    assert m.h.n_raw > 0
    planes = _planes(m)
    wf = synth.bf16_bits_to_f32(w)
    rng = np.random.default_rng(7)
    for M in (17, 130, 300):
        ks = rng.integers(0, m.K, M)
        x = np.zeros((M, m.K), np.uint16)
        x[np.arange(M), ks] = 0x3F80
        ref = wf[:, ks].T
        for src in (uw.W_BF16, uw.W_EXP, uw.W_IDX, uw.W_DIRECT):
            for v in _variants_for(m, M, src):
                log(f"  k-slices one-hot M={M} src={src} variant={v}")
                assert np.array_equal(_run_gemm(m, planes, src, x, v), ref), f"M={M} src={src} v={v}"


@pytest.mark.parametrize("N,K", [(512, 256), (200, 192), (333, 4160)])
def test_gemm_parity_ragged(N, K):
    cfg = synth.Config("rag", 7, (("w", N, K),), 0.02, "normal", 0.001, 0.0, 12, (1,))
    w = synth.gen_weight(cfg, "w")
    m = Mat(w, 256)
    assert m.h.n_raw > 0
    planes = _planes(m)
    for M in (1, 4, 16, 17, 33, 64, 65, 129, 300):
        x = synth.gen_x(cfg, M, K)
        y_ref, a_ref = oracle.gemm(x, w)
        for src in (uw.W_BF16, uw.W_EXP, uw.W_IDX, uw.W_DIRECT):
            for v in _variants_for(m, M, src):
                log(f"  ragged N={N} K={K} M={M} src={src} variant={v}")
                check_gemm(_run_gemm(m, planes, src, x, v), y_ref, a_ref, f"N={N} K={K} M={M} src={src} v={v}")


def test_dma_whole_rounds_ragged_tail():
    """The 256x256 DMA launch in whole rounds of the CUs with a 256x128 tail launch, on ragged
    N and M: N = 4296 (17 column blocks, the last 200 rows wide), M = 4046 (16 row blocks, the
    last 206 rows) make 272 tiles; with 256 CUs the first 16 column blocks fill one round and
    the last one goes out as 32 tiles of 256x128. Y matches the oracle on a sample, every
    output is written, and the 256x128 variant alone gives the same bits."""
    torch = torch_cuda()
    N, K, M = 4296, 256, 4046
    cfg = synth.Config("rounds", 11, (("w", N, K),), 0.02, "normal", 0.001, 0.0, 12, (1,))
    w = synth.gen_weight(cfg, "w")
    m = Mat(w, 256)
    plane = dev(w)
    x = synth.gen_x(cfg, M, K)
    d_x = dev(x)
    names = [uw.variant_name(v) for v in range(uw.variant_count())]
    ys = []
    for vname in ("dma 256x256", "dma 256x128 s3"):
        y = empty_f32(M, N)
        y.fill_(float("nan"))
        log(f"  {vname} N={N} K={K} M={M}")
        uw.recon_gemm(m.h, m.d_blob, uw.W_BF16, plane, d_x, y, M, variant=names.index(vname), split_k=1)
        _sync()
        assert bool(torch.isfinite(y).all().item()), f"{vname}: unwritten outputs"
        ys.append(y)
    assert torch.equal(ys[0], ys[1]), "whole rounds + tail differ from the 256x128 variant"
    rng = np.random.default_rng(5)
    mi, ni = rng.integers(0, M, 4096), rng.integers(0, N, 4096)
    mi[:8], ni[:8] = M - 1, N - 1 - np.arange(8)  # the ragged corner of the tail launch
    yr, ar = oracle.gemm_pairs(x, w, mi, ni)
    yg = ys[0][torch.from_numpy(mi).cuda(), torch.from_numpy(ni).cuda()].cpu().numpy()
    check_gemm(yg, yr, ar, "dma whole rounds, ragged")


def test_gemm_padded_leading_dimensions():
    """X and Y as rows of wider buffers (ldx > K, ldy > N): every loader and variant reads
    only the first K of each X row (the rest holds NaN, which would poison any output it
    reached), writes only the first N of each Y row (the rest keeps its sentinel) and
    matches the oracle there."""
    cfg = synth.Config("pad", 9, (("w", 200, 320),), 0.02, "normal", 0.001, 0.0, 12, (1,))
    w = synth.gen_weight(cfg, "w")
    m = Mat(w, 256)
    planes = _planes(m)
    ldx, ldy = m.K + 72, m.N + 12
    for M in (1, 17, 64, 130):
        x = synth.gen_x(cfg, M, m.K)
        xp = np.full((M, ldx), 0x7FC0, np.uint16)
        xp[:, : m.K] = x
        d_x = dev(xp)
        y_ref, a_ref = oracle.gemm(x, w)
        for src in (uw.W_BF16, uw.W_EXP, uw.W_IDX, uw.W_DIRECT):
            for v in _variants_for(m, M, src):
                log(f"  padded M={M} src={src} variant={v}")
                y = empty_f32(M, ldy)
                y.fill_(12345.0)
                uw.recon_gemm(m.h, m.d_blob, src, planes[src], d_x, y, M, ldx=ldx, ldy=ldy, variant=v)
                _sync()
                yh = host(y).reshape(M, ldy)
                check_gemm(yh[:, : m.N], y_ref, a_ref, f"padded M={M} src={src} v={v}")
                assert (yh[:, m.N:] == 12345.0).all(), f"padded M={M} src={src} v={v}: wrote past N"


def test_pipelines_tiny():
    cfg = synth.CONFIGS["tiny"]
    w = synth.gen_weight(cfg, "w")
    m = Mat(w)
    direct, _ = m.decode("direct")
    ws = empty_u8(uw.workspace_bytes(m.h, uw.PIPE_FULL))
    for M in (4, 1, 64, 200):
        x = synth.gen_x(cfg, M, m.K)
        y_ref, a_ref = oracle.gemm(x, w)
        for p in range(5):
            log(f"  pipeline {p} M={M}")
            y = empty_f32(M, m.N)
            err = zeros_u32()
            uw.run_pipeline(p, m.h, m.d_blob, dev(x), y, M, d_direct=direct, d_ws=ws, ws_bytes=ws.numel(), d_err=err)
            _sync()
            assert int(host(err)[0]) == 0
            check_gemm(host(y), y_ref, a_ref, f"pipeline {p} M={M}")


def test_run_pipeline_error_paths():
    w = synth.gen_weight(synth.CONFIGS["tiny"], "w")
    m = Mat(w)
    x = dev(synth.gen_x(synth.CONFIGS["tiny"], 4, m.K))
    y = empty_f32(4, m.N)
    with pytest.raises(uw.UwError) as e:
        uw.run_pipeline(uw.PIPE_FULL, m.h, m.d_blob, x, y, 4, d_ws=empty_u8(16), ws_bytes=16)
    assert e.value.status == uw.ENOSPACE
    with pytest.raises(uw.UwError) as e:
        uw.run_pipeline(uw.PIPE_DIRECT, m.h, m.d_blob, x, y, 4)
    assert e.value.status == uw.EINVAL
    ws = empty_u8(uw.workspace_bytes(m.h, uw.PIPE_EXPAND))
    with pytest.raises(uw.UwError) as e:  # expand without the direct plane
        uw.run_pipeline(uw.PIPE_EXPAND, m.h, m.d_blob, x, y, 4, d_ws=ws, ws_bytes=ws.numel())
    assert e.value.status == uw.EINVAL
    with pytest.raises(uw.UwError) as e:  # expand into a workspace too small
        uw.run_pipeline(uw.PIPE_EXPAND, m.h, m.d_blob, x, y, 4, d_direct=m.decode("direct")[0], d_ws=ws,
                        ws_bytes=ws.numel() - 16)
    assert e.value.status == uw.ENOSPACE
    with pytest.raises(uw.UwError) as e:
        uw.recon_gemm(m.h, m.d_blob, uw.W_IDX, empty_u8(m.N * m.K // 2), x, y, 4, ldx=m.K - 8)
    assert e.value.status == uw.EINVAL
    with pytest.raises(uw.UwError) as e:
        uw.recon_gemm(m.h, m.d_blob, uw.W_IDX, empty_u8(m.N * m.K // 2), x, y, 4, variant=99)
    assert e.value.status == uw.EINVAL
    with pytest.raises(uw.UwError) as e:
        uw.recon_gemm(m.h, m.d_blob, uw.W_IDX, empty_u8(m.N * m.K // 2), x, y, 100, variant=0)
    assert e.value.status == uw.EUNSUPPORTED
    uw.recon_gemm(m.h, m.d_blob, uw.W_IDX, empty_u8(m.N * m.K // 2), x, y, 0)  # M = 0: no-op


def test_stream_read_sizes_and_argument_errors():
    """The bench's read-ceiling helper: ragged and empty sizes run to completion, and
    misaligned or NULL arguments are rejected on the host before any launch."""
    buf = empty_u8(3 << 20)
    sink = zeros_u32(1)
    for n in (0, 16, 4096 + 16, (1 << 20) + 48, 3 << 20):
        uw.stream_read(buf, sink, n)
    _sync()
    with pytest.raises(uw.UwError) as e:
        uw.stream_read(buf.data_ptr() + 4, sink, 64)
    assert e.value.status == uw.EINVAL
    with pytest.raises(uw.UwError) as e:
        uw.stream_read(buf, sink, 40)
    assert e.value.status == uw.EINVAL
    with pytest.raises(uw.UwError) as e:
        uw.stream_read(buf, None, 64)
    assert e.value.status == uw.EINVAL


# ---------------------------------------------------------------- full sizes
def _full_size_case(cfg, proj, Ms, n_samples=4096, splits=(0, 2)):
    """Decoded planes in full, then every GEMM variant the shape and M allow (the ones the
    plans pick among), through every loader, at the variant's own K split and at the
    splits listed: a seeded sample of Y against the oracle, gathered on the device."""
    torch = torch_cuda()
    w = synth.gen_weight(cfg, proj)
    log(f"  {cfg.name}/{proj}: encoding {w.shape}")
    m = Mat(w)
    _check_decoders(m, f"{cfg.name}/{proj}")
    planes = _planes(m)
    m._ref = None
    rng = np.random.default_rng(12345)
    for M in Ms:
        x = synth.gen_x(cfg, M, m.K)
        d_x = dev(x)
        mi = rng.integers(0, M, n_samples)
        ni = rng.integers(0, m.N, n_samples)
        y_ref, a_ref = oracle.gemm_pairs(x, w, mi, ni)
        d_mi, d_ni = torch.from_numpy(mi).cuda(), torch.from_numpy(ni).cuda()
        y = empty_f32(M, m.N)
        for src in (uw.W_BF16, uw.W_EXP, uw.W_IDX, uw.W_DIRECT):
            for v in _variants_for(m, M, src):
                for ks in splits:
                    what = f"{cfg.name}/{proj} M={M} src={src} {uw.variant_name(v)} split={ks}"
                    log(f"  {what}")
                    y.fill_(float("nan"))
                    uw.recon_gemm(m.h, m.d_blob, src, planes[src], d_x, y, M, variant=v, split_k=ks)
                    check_gemm(y[d_mi, d_ni].cpu().numpy(), y_ref, a_ref, what)
                    assert bool(torch.isfinite(y).all().item()), f"{what}: unwritten outputs"


def test_full_size_gate():
    _full_size_case(synth.CONFIGS["gate"], "gate", (1, 16, 64))


def test_full_size_down():
    _full_size_case(synth.CONFIGS["down"], "down", (1, 16, 64, 256, 1024, 4096))


def test_full_size_70b():
    cfg = synth.CONFIGS["70b"]
    _full_size_case(cfg, "gate", (1, 64, 512, 2048), splits=(0,))
    _full_size_case(cfg, "down", (1, 64, 512, 2048), n_samples=2048, splits=(0,))


# ---------------------------------------------------------------- glue, autotune
def test_swiglu_against_oracle():
    torch = torch_cuda()
    rng = np.random.default_rng(51)
    for n in (8, 13, 4096 * 3 + 5):
        g = (rng.standard_normal(n) * 4).astype(np.float32)
        u = (rng.standard_normal(n) * 4).astype(np.float32)
        g[:3] = [0.0, -0.0, 30.0]
        h = torch.empty(n + 8, dtype=torch.int16, device="cuda")
        uw.swiglu(dev(g), dev(u), h, n)
        _sync()
        got = host(h, np.uint16)[:n].astype(np.int32)
        ref = oracle.swiglu(g, u).astype(np.int32)
        # within one bf16 ulp of the correctly rounded fp64 value (same sign)
        assert (np.abs(got - ref) <= 1).all()


def test_autotune_picks_the_fastest_and_the_choice_is_correct():
    """uw_autotune times candidates back to back over a rotation set (here four matrices of
    one shape, as a model's layers): its pick is within 1.25x + 2 us of the best time each
    pipeline reaches when tuned on its own, its K split is one the launch can use, and the
    chosen plan computes the right Y on every matrix of the set."""
    cfg = synth.CONFIGS["tiny"]
    mats = []
    for i in range(4):
        w = synth.gen_weight(cfg, "w") if i == 0 else np.roll(synth.gen_weight(cfg, "w"), 37 * i, axis=1)
        m = Mat(w)
        m.direct, _ = m.decode("direct")
        mats.append(m)
    m0 = mats[0]
    rot = [uw.proj(m.h, m.d_blob, d_direct=m.direct) for m in mats]
    Ms = [1, 64, 256]
    x = synth.gen_x(cfg, max(Ms), m0.K)
    d_x = dev(x)
    y = empty_f32(max(Ms), m0.N)
    ws = empty_u8(uw.workspace_bytes(m0.h, uw.PIPE_FULL))
    kw = dict(d_ws=ws, ws_bytes=ws.numel(), reps=20, warmup=3, trials=5, rot=rot, tune_split=True)
    plans = uw.autotune(m0.h, m0.d_blob, d_x, y, Ms, **kw)
    log(f"  plans {plans}")
    for M, plan in zip(Ms, plans):
        assert 0 <= plan.pipeline <= 4 and plan.t_ms > 0
        assert plan.split_k == uw.split_count(plan.variant, m0.N, m0.K, M, plan.split_k) >= 1
        per = [uw.autotune(m0.h, m0.d_blob, d_x, y, [M], pipeline_mask=1 << p, **kw)[0].t_ms for p in range(5)]
        assert plan.t_ms <= min(per) * 1.25 + 0.002, (M, plan, per)
        # the chosen plan computes the right result on every matrix it was timed on
        for m in mats:
            yy = empty_f32(M, m.N)
            uw.run_pipeline(plan.pipeline, m.h, m.d_blob, dev(x[:M]), yy, M, d_direct=m.direct, d_ws=ws,
                            ws_bytes=ws.numel(), variant=plan.variant, split_k=plan.split_k)
            _sync()
            y_ref, a_ref = oracle.gemm(x[:M], m.w)
            check_gemm(host(yy), y_ref, a_ref, f"autotuned M={M}")


def test_autotune_rejects_rotation_of_another_shape():
    cfg = synth.CONFIGS["tiny"]
    w = synth.gen_weight(cfg, "w")
    m, m2 = Mat(w), Mat(w[:256])
    x = dev(synth.gen_x(cfg, 4, m.K))
    y = empty_f32(4, m.N)
    with pytest.raises(uw.UwError) as e:
        uw.autotune(m.h, m.d_blob, x, y, [4], rot=[uw.proj(m.h, m.d_blob), uw.proj(m2.h, m2.d_blob)],
                    pipeline_mask=1 << uw.PIPE_TRANSCODE, d_ws=empty_u8(m.N * m.K), ws_bytes=m.N * m.K)
    assert e.value.status == uw.EINVAL


def test_explicit_k_splits_match_the_oracle():
    """Every variant at several explicit K splits (1, 2, 3, 5 slices and the most the shape
    allows) on a long-K shape, through each loader: Y within the bound of the oracle."""
    rng = np.random.default_rng(83)
    w = synth.f32_to_bf16_bits(rng.standard_normal((200, 64 * 23), dtype=np.float32) * 0.02)
    w.reshape(-1)[rng.choice(w.size, 30, replace=False)] ^= 0x0A00  # out-of-palette exponents
    m = Mat(w)
    planes = _planes(m)
    for M in (1, 33, 130):
        x = synth.f32_to_bf16_bits(rng.standard_normal((M, m.K), dtype=np.float32))
        y_ref, a_ref = oracle.gemm(x, w)
        d_x = dev(x)
        for src in (uw.W_BF16, uw.W_EXP, uw.W_IDX, uw.W_DIRECT):
            for v in _variants_for(m, M, src):
                for ks in (1, 2, 3, 5, 23):
                    assert uw.split_count(v, m.N, m.K, M, ks) == ks
                    y = empty_f32(M, m.N)
                    y.fill_(float("nan"))
                    uw.recon_gemm(m.h, m.d_blob, src, planes[src], d_x, y, M, variant=v, split_k=ks)
                    _sync()
                    check_gemm(host(y), y_ref, a_ref, f"M={M} src={src} variant={v} split={ks}")


def test_stack_layers_teacher_forced():
    """Two layers of the 8B-shaped SwiGLU MLP stack: gate and up from the same X, the
    SwiGLU glue, then down on the glue output, each step checked against the oracle on
    the GPU's own inputs (teacher forcing)."""
    cfg = synth.CONFIGS["stack"]
    sig = synth.gen_stack_sigmas(cfg)
    M = 4
    x = synth.gen_x(cfg, M, 4096)
    rng = np.random.default_rng(61)
    torch = torch_cuda()
    for layer in range(2):
        mats = {p: Mat(synth.gen_weight(cfg, p, layer, sigma=float(sig[layer]))) for p in ("gate", "up", "down")}
        dpl = {p: mats[p].decode("direct")[0] for p in mats}
        ys = {}
        for p in ("gate", "up"):
            y = empty_f32(M, 14336)
            uw.run_pipeline(uw.PIPE_DIRECT, mats[p].h, mats[p].d_blob, dev(x), y, M, d_direct=dpl[p])
            ys[p] = y
        hbuf = torch.empty(M * 14336, dtype=torch.int16, device="cuda")
        uw.swiglu(ys["gate"], ys["up"], hbuf, M * 14336)
        yd = empty_f32(M, 4096)
        uw.run_pipeline(uw.PIPE_DIRECT, mats["down"].h, mats["down"].d_blob, hbuf, yd, M, d_direct=dpl["down"])
        _sync()
        mi = rng.integers(0, M, 1024)
        for p in ("gate", "up"):
            ni = rng.integers(0, 14336, 1024)
            yr, ar = oracle.gemm_pairs(x, mats[p].w, mi, ni)
            check_gemm(host(ys[p])[mi, ni], yr, ar, f"layer {layer} {p}")
        g, u = host(ys["gate"]), host(ys["up"])
        href = oracle.swiglu(g, u).reshape(M, 14336)
        hg = host(hbuf, np.uint16).reshape(M, 14336)
        assert (np.abs(hg.astype(np.int32) - href.astype(np.int32)) <= 1).all()
        ni = rng.integers(0, 4096, 1024)
        yr, ar = oracle.gemm_pairs(hg, mats["down"].w, mi, ni)
        check_gemm(host(yd)[mi, ni], yr, ar, f"layer {layer} down")


def test_mlp_stack_forward_one_and_two_streams():
    """uw_mlp_stack_forward over 3 layers with mixed pipelines: one stream and a separate
    decode stream give bit-identical Y; the last layer's g, u, h (left in the workspace)
    and Y are checked against the oracle on the GPU's own inputs."""
    torch = torch_cuda()
    rng = np.random.default_rng(71)
    K, F, M = 256, 512, 5
    x = synth.f32_to_bf16_bits(rng.standard_normal((M, K), dtype=np.float32))
    pipes = [(uw.PIPE_FULL, uw.PIPE_FULL, uw.PIPE_EXP), (uw.PIPE_DIRECT, uw.PIPE_TRANSCODE, uw.PIPE_DIRECT),
             (uw.PIPE_EXP, uw.PIPE_DIRECT, uw.PIPE_FULL), (uw.PIPE_EXPAND, uw.PIPE_DIRECT, uw.PIPE_EXPAND)]
    mats, keep, layers = [], [], []
    for l, pp in enumerate(pipes):
        trip = []
        for q, (n, k) in enumerate(((F, K), (F, K), (K, F))):
            w = synth.f32_to_bf16_bits(rng.standard_normal((n, k), dtype=np.float32) * 0.05)
            m = Mat(w, 256)
            d = m.decode("direct")[0] if pp[q] in (uw.PIPE_DIRECT, uw.PIPE_EXPAND) else None
            keep.append((m, d))
            trip.append(uw.proj(m.h, m.d_blob, pp[q], d_direct=d))
        mats.append([t[0] for t in keep[-3:]])
        layers.append(trip)
    arr = uw.mlp_layers(layers)
    d_x = dev(x)
    outs = []
    for two in (False, True):
        nbytes = uw.mlp_stack_workspace(arr, M, two_slots=two)
        ws = empty_u8(nbytes + 256)
        y = empty_f32(M, K)
        y.fill_(float("nan"))
        side = torch.cuda.Stream() if two else None
        log(f"  stack forward, decode stream: {two}, workspace {nbytes} B")
        uw.mlp_stack_forward(arr, M, d_x, y, ws, nbytes, decode_stream=side)
        _sync()
        outs.append((host(y), host(ws)))
    assert np.array_equal(outs[0][0], outs[1][0]), "one stream and two streams differ"
    y, wsb = outs[1]
    gate, up, down = mats[-1]
    a256 = lambda v: (v + 255) // 256 * 256
    g = wsb[: 4 * M * F].view(np.float32).reshape(M, F)
    u = wsb[a256(4 * M * F): a256(4 * M * F) + 4 * M * F].view(np.float32).reshape(M, F)
    ho = 2 * a256(4 * M * F)
    hg = wsb[ho: ho + 2 * M * F].view(np.uint16).reshape(M, F)
    for name, got, wm in (("gate", g, gate), ("up", u, up)):
        yr, ar = oracle.gemm(x, wm.w)
        check_gemm(got, yr, ar, f"stack last layer {name}")
    href = oracle.swiglu(g, u).reshape(M, F)
    assert (np.abs(hg.astype(np.int32) - href.astype(np.int32)) <= 1).all()
    yr, ar = oracle.gemm(hg, down.w)
    check_gemm(y, yr, ar, "stack last layer down")


def test_stack_up_gemm_swiglu_epilogue_matches_two_steps():
    """Past M = 64 the stack forward runs the SwiGLU in the up projection's GEMM epilogue
    (tiled, wide and dma variants, one K slice; u is never stored): g, h and Y equal, bit for
    bit, the up GEMM into u followed by uw_swiglu and then down, on one stream and with a
    decode stream. An up projection cut into two K slices takes the two steps. Ragged M
    and N_ff (130 rows, 576 = 2 x 256 + 64 columns), and h checked against the oracle's
    SwiGLU of the two-step g and u."""
    torch = torch_cuda()
    rng = np.random.default_rng(97)
    K, F, M = 256, 576, 130
    x = synth.f32_to_bf16_bits(rng.standard_normal((M, K), dtype=np.float32))
    d_x = dev(x)
    mats = [Mat(synth.f32_to_bf16_bits(rng.standard_normal(shape, dtype=np.float32) * 0.05), 256)
            for shape in ((F, K), (F, K), (K, F))]
    planes = [m.decode("direct")[0] for m in mats]
    names = [uw.variant_name(v) for v in range(uw.variant_count())]
    vdown = names.index("tiled 128x128")
    side = torch.cuda.Stream()
    for pipe, vname, up_split in ((uw.PIPE_DIRECT, "tiled 128x128", 1), (uw.PIPE_DIRECT, "tiled 256x128", 1),
                                  (uw.PIPE_DIRECT, "wide 256x256", 1), (uw.PIPE_EXP, "tiled 128x64", 1),
                                  (uw.PIPE_TRANSCODE, "wide 256x256", 1), (uw.PIPE_FULL, "dma 256x256", 1),
                                  (uw.PIPE_EXPAND, "dma 256x128 s3", 1), (uw.PIPE_DIRECT, "wide 256x256", 2)):
        v = names.index(vname)
        what = f"{uw.PIPELINE_NAMES[pipe]} / {vname} / up split {up_split}"
        log(f"  up GEMM + SwiGLU: {what}")
        d = lambda q: planes[q] if pipe in (uw.PIPE_DIRECT, uw.PIPE_EXPAND) else None
        # two steps: gate, up into u, uw_swiglu, down
        nws = max(uw.workspace_bytes(m.h, pipe) for m in mats[:2])
        wsr = empty_u8(max(nws, 256))
        g_ref, u_ref, y_ref = empty_f32(M, F), empty_f32(M, F), empty_f32(M, K)
        h_ref = empty_u16(M * F)
        for q, out, ks in ((0, g_ref, 1), (1, u_ref, up_split)):
            uw.run_pipeline(pipe, mats[q].h, mats[q].d_blob, d_x, out, M, d_direct=d(q), d_ws=wsr, ws_bytes=nws,
                            variant=v, split_k=ks)
        uw.swiglu(g_ref, u_ref, h_ref, M * F)
        uw.run_pipeline(uw.PIPE_DIRECT, mats[2].h, mats[2].d_blob, h_ref, y_ref, M, d_direct=planes[2],
                        variant=vdown, split_k=1)
        _sync()
        gr, ur, hr, yr = host(g_ref), host(u_ref), host(h_ref, np.uint16).reshape(M, F), host(y_ref)
        assert (np.abs(hr.astype(np.int32) - oracle.swiglu(gr, ur).reshape(M, F).astype(np.int32)) <= 1).all(), what
        arr = uw.mlp_layers([(uw.proj(mats[0].h, mats[0].d_blob, pipe, d_direct=d(0), variant=v, split_k=1),
                              uw.proj(mats[1].h, mats[1].d_blob, pipe, d_direct=d(1), variant=v, split_k=up_split),
                              uw.proj(mats[2].h, mats[2].d_blob, uw.PIPE_DIRECT, d_direct=planes[2], variant=vdown,
                                      split_k=1))])
        for two in (False, True):
            nb = uw.mlp_stack_workspace(arr, M, two_slots=two)
            ws = empty_u8(nb)
            ws.fill_(0xFF)
            y = empty_f32(M, K)
            y.fill_(float("nan"))
            uw.mlp_stack_forward(arr, M, d_x, y, ws, nb, decode_stream=side if two else None)
            _sync()
            wsb = host(ws)
            a256 = lambda n: (n + 255) // 256 * 256
            g = wsb[: 4 * M * F].view(np.float32).reshape(M, F)
            u = wsb[a256(4 * M * F): a256(4 * M * F) + 4 * M * F].view(np.float32).reshape(M, F)
            ho = 2 * a256(4 * M * F)
            hg = wsb[ho: ho + 2 * M * F].view(np.uint16).reshape(M, F)
            assert np.array_equal(g, gr), f"{what}, decode stream {two}: g"
            assert np.array_equal(hg, hr), f"{what}, decode stream {two}: h"
            assert np.array_equal(host(y), yr), f"{what}, decode stream {two}: Y"
            if up_split == 1:
                assert np.isnan(u).all(), f"{what}: u was stored although the epilogue took the SwiGLU"
            else:
                assert np.array_equal(u, ur), f"{what}: u of the two-step path"


def _hard_easy_stack(rng, K, F, hard_pipes):
    """A stack whose layers alternate easy (three projections with direct planes, run on
    them) and hard (Huffman blobs only; decode-first pipelines from hard_pipes in turn).
    Returns (layer array, per-layer Mat triples, objects to keep alive)."""
    keep, mats, layers = [], [], []
    for l in range(2 * len(hard_pipes)):
        easy = l % 2 == 0
        trip, tm = [], []
        for q, (n, k) in enumerate(((F, K), (F, K), (K, F))):
            w = synth.f32_to_bf16_bits(rng.standard_normal((n, k), dtype=np.float32) * 0.05)
            m = Mat(w, 256)
            d = m.decode("direct")[0] if easy else None
            keep.append((m, d))
            tm.append(m)
            trip.append(uw.proj(m.h, m.d_blob, uw.PIPE_DIRECT if easy else hard_pipes[l // 2][q], d_direct=d))
        mats.append(tm)
        layers.append(trip)
    return uw.mlp_layers(layers), mats, keep


def _check_last_layer(x, y, wsb, mats, M, F, what):
    """Teacher-forced check of the last layer: g, u, h (left in the workspace) and Y."""
    gate, up, down = mats[-1]
    a256 = lambda v: (v + 255) // 256 * 256
    g = wsb[: 4 * M * F].view(np.float32).reshape(M, F)
    u = wsb[a256(4 * M * F): a256(4 * M * F) + 4 * M * F].view(np.float32).reshape(M, F)
    ho = 2 * a256(4 * M * F)
    hg = wsb[ho: ho + 2 * M * F].view(np.uint16).reshape(M, F)
    for name, got, wm in (("gate", g, gate), ("up", u, up)):
        yr, ar = oracle.gemm(x, wm.w)
        check_gemm(got, yr, ar, f"{what}: last layer {name}")
    href = oracle.swiglu(g, u).reshape(M, F)
    assert (np.abs(hg.astype(np.int32) - href.astype(np.int32)) <= 1).all()
    yr, ar = oracle.gemm(hg, down.w)
    check_gemm(y, yr, ar, f"{what}: last layer down")


def test_stack_schedules_hard_easy_bit_identical():
    """Hard layers (decode-first only) between easy ones (direct planes): every decode
    schedule (one stream; a decode stream with 1..4 slots, in order or down first) gives
    bit-identical Y, equal to uw_mlp_stack_forward's, and the last layer matches the
    oracle."""
    torch = torch_cuda()
    rng = np.random.default_rng(83)
    K, F, M = 256, 512, 5
    arr, mats, keep = _hard_easy_stack(rng, K, F, [(uw.PIPE_FULL, uw.PIPE_EXP, uw.PIPE_TRANSCODE),
                                                  (uw.PIPE_TRANSCODE, uw.PIPE_FULL, uw.PIPE_EXP)])
    x = synth.f32_to_bf16_bits(rng.standard_normal((M, K), dtype=np.float32))
    d_x = dev(x)
    side = torch.cuda.Stream()
    ys = {}
    last_ws = None
    for slots, down_first, two in ((1, False, False), (1, False, True), (2, False, True), (3, False, True),
                                   (3, True, True), (4, True, True), (4, False, True)):
        nbytes = uw.mlp_stack_workspace_ex(arr, M, slots=slots)
        ws = empty_u8(nbytes + 256)
        y = empty_f32(M, K)
        y.fill_(float("nan"))
        log(f"  stack forward_ex: slots {slots}, down first {down_first}, decode stream {two}")
        uw.mlp_stack_forward_ex(arr, M, d_x, y, ws, nbytes, decode_stream=side if two else None, slots=slots,
                                down_first=down_first)
        _sync()
        ys[(slots, down_first, two)] = host(y)
        last_ws = host(ws)
    nbytes = uw.mlp_stack_workspace(arr, M, two_slots=True)
    ws = empty_u8(nbytes + 256)
    y = empty_f32(M, K)
    uw.mlp_stack_forward(arr, M, d_x, y, ws, nbytes, decode_stream=side)
    _sync()
    ref = host(y)
    for k, v in ys.items():
        assert np.array_equal(v, ref), f"schedule {k} differs from uw_mlp_stack_forward"
    _check_last_layer(x, ref, last_ws, mats, M, F, "hard/easy stack")


def test_stack_autotune_coordinate_descent():
    """uw_mlp_stack_autotune on a hard/easy stack from an all-full-decode start: the
    tuned plan is never slower than the start, keeps direct palette off the hard layers
    (they have no direct planes), and its forward matches the oracle."""
    torch = torch_cuda()
    rng = np.random.default_rng(89)
    K, F, M = 256, 512, 4
    arr, mats, keep = _hard_easy_stack(rng, K, F, [(uw.PIPE_FULL,) * 3, (uw.PIPE_FULL,) * 3])
    for l in range(len(arr)):
        for r in ("gate", "up", "down"):
            getattr(arr[l], r).pipeline = uw.PIPE_FULL  # start: full decode everywhere
    x = synth.f32_to_bf16_bits(rng.standard_normal((M, K), dtype=np.float32))
    d_x = dev(x)
    side = torch.cuda.Stream()
    nbytes = uw.mlp_stack_workspace_ex(arr, M, slots=3)  # all-full plan: every candidate fits
    ws = empty_u8(nbytes + 256)
    y = empty_f32(M, K)
    log("  stack autotune: 4 layers, decode stream, 3 slots")
    a = uw.mlp_stack_autotune(arr, M, d_x, y, ws, nbytes, decode_stream=side, slots=3, reps=3, warmup=1,
                              max_passes=3)
    _sync()
    plan = [[getattr(arr[l], r).pipeline for r in ("gate", "up", "down")] for l in range(len(arr))]
    log(f"  tuned: {plan}, down first {a.opts.down_first}, {a.t_start_ms:.3f} -> {a.t_ms:.3f} ms, "
        f"{a.passes} passes, {a.trials} trials")
    assert a.t_ms <= a.t_start_ms
    assert 1 <= a.passes <= 3 and a.trials >= 2
    for l, pp in enumerate(plan):
        assert all(0 <= p <= 3 for p in pp)
        if l % 2 == 1:
            assert uw.PIPE_DIRECT not in pp, f"hard layer {l} given direct palette"
    y.fill_(float("nan"))
    uw.mlp_stack_forward_ex(arr, M, d_x, y, ws, nbytes, decode_stream=side, slots=3, down_first=bool(a.opts.down_first))
    _sync()
    _check_last_layer(x, host(y), host(ws), mats, M, F, "tuned stack")


def test_gate_up_fused_matches_separate_launches():
    """uw_recon_gemm_gate_up gives the same bits as the two GEMMs (same variant) and
    uw_swiglu, for every variant with a fused form, ragged N, raw rows, M = 1..64; the
    stack forward takes the fused path for direct gate/up and still equals the projection-
    by-projection result; unsupported cases are refused."""
    torch = torch_cuda()
    cfg = synth.Config("gu", 9, (("gate", 700, 4160), ("up", 700, 4160)), 0.02, "normal", 0.0005, 0.0, 12, (1,))
    mg, mu = Mat(synth.gen_weight(cfg, "gate")), Mat(synth.gen_weight(cfg, "up"))
    assert mg.h.n_raw > 0 and mu.h.n_raw > 0
    for m in (mg, mu):  # the fused form needs palettes of consecutive exponents
        pal = sorted(np.frombuffer(bytes(m.h.palette), np.uint8)[: m.h.n_pal])
        assert pal == list(range(pal[0], pal[0] + len(pal)))
    dg, du = mg.decode("direct")[0], mu.decode("direct")[0]
    N, K = mg.N, mg.K
    fused = ["skinny rt4 u2 w4", "skinny rt4 u2 w4 xt", "skinny rt2 u4 w4", "skinny rt1 u4 w4", "skinny rt1 u4 w8",
             "skinny rt4 u2 w4 xd", "skinny rt4 u2 w8 xd"]
    names = {uw.variant_name(v): v for v in range(uw.variant_count())}
    for M in (1, 5, 16, 17, 33, 64):
        x = dev(synth.gen_x(cfg, M, K))
        for v in [-1] + [names[n] for n in fused if not (n.endswith("w8 xd") and M > 32)]:
            log(f"  gate/up fused M={M} variant={v}")
            yg, yu, yg2, yu2 = (empty_f32(M, N) for _ in range(4))
            h = torch.empty(M, N, dtype=torch.int16, device="cuda")
            h2 = torch.empty(M, N, dtype=torch.int16, device="cuda")
            for t in (yg, yu, yg2, yu2):
                t.fill_(float("nan"))
            uw.recon_gemm_gate_up(mg.h, mg.d_blob, dg, mu.h, mu.d_blob, du, x, yg, yu, h, M, variant=v)
            uw.recon_gemm(mg.h, mg.d_blob, uw.W_DIRECT, dg, x, yg2, M, variant=v)
            uw.recon_gemm(mu.h, mu.d_blob, uw.W_DIRECT, du, x, yu2, M, variant=v)
            uw.swiglu(yg2, yu2, h2, M * N)
            _sync()
            assert np.array_equal(host(yg), host(yg2)) and np.array_equal(host(yu), host(yu2)), f"M={M} v={v}"
            assert np.array_equal(host(h, np.uint16), host(h2, np.uint16)), f"M={M} v={v}: h"
        yr, ar = oracle.gemm(synth.gen_x(cfg, M, K), mg.w)
        check_gemm(host(yg), yr, ar, f"fused gate M={M}")
    x = dev(synth.gen_x(cfg, 65, K))
    y = empty_f32(65, N)
    hh = torch.empty(65, N, dtype=torch.int16, device="cuda")
    with pytest.raises(uw.UwError) as e:
        uw.recon_gemm_gate_up(mg.h, mg.d_blob, dg, mu.h, mu.d_blob, du, x, y, y, hh, 65)
    assert e.value.status == uw.EUNSUPPORTED
    with pytest.raises(uw.UwError) as e:
        uw.recon_gemm_gate_up(mg.h, mg.d_blob, dg, mu.h, mu.d_blob, du, x, y, y, hh, 8, variant=names["tiled 128x128"])
    assert e.value.status == uw.EUNSUPPORTED

    # stack forward: direct gate/up (fused) with a down projection, vs the same kernels one by one
    cs = synth.Config("gus", 10, (("gate", 704, 512), ("up", 704, 512)), 0.02, "normal", 0.0, 0.0, 0, (1,))
    mg, mu = Mat(synth.gen_weight(cs, "gate")), Mat(synth.gen_weight(cs, "up"))
    dg, du = mg.decode("direct")[0], mu.decode("direct")[0]
    N, K = mg.N, mg.K
    wd = synth.f32_to_bf16_bits(np.random.default_rng(5).standard_normal((K, N), dtype=np.float32) * 0.02)
    md = Mat(wd)
    ddn = md.decode("direct")[0]
    cfg = cs
    for M, v in ((3, -1), (40, names["skinny rt4 u2 w4 xt"])):
        layer = [uw.proj(mg.h, mg.d_blob, uw.PIPE_DIRECT, d_direct=dg, variant=v),
                 uw.proj(mu.h, mu.d_blob, uw.PIPE_DIRECT, d_direct=du, variant=v),
                 uw.proj(md.h, md.d_blob, uw.PIPE_DIRECT, d_direct=ddn)]
        arr = uw.mlp_layers([layer, layer])
        x = dev(synth.gen_x(cfg, M, K))
        nbytes = uw.mlp_stack_workspace(arr, M)
        ws = empty_u8(nbytes + 256)
        y = empty_f32(M, K)
        uw.mlp_stack_forward(arr, M, x, y, ws, nbytes)
        yg2, yu2 = empty_f32(M, N), empty_f32(M, N)
        h2 = torch.empty(M, N, dtype=torch.int16, device="cuda")
        y2 = empty_f32(M, K)
        uw.recon_gemm(mg.h, mg.d_blob, uw.W_DIRECT, dg, x, yg2, M, variant=v)
        uw.recon_gemm(mu.h, mu.d_blob, uw.W_DIRECT, du, x, yu2, M, variant=v)
        uw.swiglu(yg2, yu2, h2, M * N)
        uw.recon_gemm(md.h, md.d_blob, uw.W_DIRECT, ddn, h2, y2, M)
        _sync()
        assert np.array_equal(host(y), host(y2)), f"stack M={M}"


def test_cu_split_streams_decode_and_stack_forward():
    """Streams on disjoint compute units: their CU counts add up to the device's, the
    persistent decoder on the decode slice is still bit-exact, and the stack forward with
    its preprocessing on the decode slice gives the same Y as on one stream."""
    torch = torch_cuda()
    total = uw.stream_cu_count(0)
    gs, ds = uw.stream_pair_create(48)
    try:
        assert uw.stream_cu_count(ds) == 48
        assert uw.stream_cu_count(gs) == total - 48
        w = synth.gen_weight(synth.CONFIGS["tiny"], "w")
        m = Mat(w, 256)
        ref = m.ref()
        out = empty_u8(m.N * m.K // 2)
        err = zeros_u32()
        uw.transcode_palette(m.h, m.d_blob, out, err, stream=ds)
        _sync()
        assert int(host(err)[0]) == 0 and (host(out) == ref["idx"]).all()
        rng = np.random.default_rng(73)
        K, F, M = 256, 512, 9
        x = synth.f32_to_bf16_bits(rng.standard_normal((M, K), dtype=np.float32))
        keep, layers = [], []
        for l in range(3):
            trip = []
            for q, (n, k) in enumerate(((F, K), (F, K), (K, F))):
                wl = synth.f32_to_bf16_bits(rng.standard_normal((n, k), dtype=np.float32) * 0.05)
                ml = Mat(wl, 256)
                keep.append(ml)
                trip.append(uw.proj(ml.h, ml.d_blob, (uw.PIPE_TRANSCODE, uw.PIPE_EXP, uw.PIPE_FULL)[(l + q) % 3]))
            layers.append(trip)
        arr = uw.mlp_layers(layers)
        d_x = dev(x)
        ys = []
        for split in (False, True):
            nbytes = uw.mlp_stack_workspace(arr, M, two_slots=split)
            ws = empty_u8(nbytes + 256)
            y = empty_f32(M, K)
            y.fill_(float("nan"))
            _sync()
            log(f"  stack forward on CU-split streams: {split}")
            if split:
                uw.mlp_stack_forward(arr, M, d_x, y, ws, nbytes, stream=gs, decode_stream=ds)
            else:
                uw.mlp_stack_forward(arr, M, d_x, y, ws, nbytes)
            _sync()
            ys.append(host(y))
        assert np.isfinite(ys[0]).all()
        assert np.array_equal(ys[0], ys[1])
        del torch
    finally:
        _sync()
        uw.stream_destroy(gs)
        uw.stream_destroy(ds)


def test_graft_smoke_entry():
    """The packaged smoke check (one tiny decode + direct-palette GEMM against the oracle)."""
    import __graft_entry__

    __graft_entry__.smoke()
