"""uw_run_pipeline_noalloc (the entry point for callers that cannot allocate device memory)
against uw_run_pipeline with a caller workspace, through the C ABI: two calls in a row per
pipeline, the second on a smaller input, each bit-identical to the workspace entry point
(the same kernels) and within 1e-3 * sum|x w| of the fp64 oracle on sampled outputs."""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import check_gemm, dev, empty_f32, empty_u8, host, log, torch_cuda, zeros_u32

pytestmark = pytest.mark.gpu


def _case(uw, cfg, proj, M, rng):
    w = synth.gen_weight(cfg, proj)
    blob = uw.encode(w)
    h = uw.inspect(blob)
    d_blob = dev(blob)
    direct = empty_u8(uw.direct_plane_bytes(h))
    uw.prepare_direct(h, d_blob, direct)
    x = synth.gen_x(cfg, M, h.K)
    n = min(2048, M * h.N)
    mi, ni = rng.integers(0, M, n), rng.integers(0, h.N, n)
    y_ref, a_ref = oracle.gemm_pairs(x, w, mi, ni)
    return h, d_blob, direct, dev(x), (mi, ni, y_ref, a_ref)


def test_noalloc_matches_the_workspace_entry_point():
    torch_cuda()
    import decode_gemm_amd as uw

    oracle.build(force=False)
    rng = np.random.default_rng(97)
    assert uw.noalloc_scratch_bytes() == 128 << 20
    big = _case(uw, synth.CONFIGS["gate"], "gate", 16, rng)   # first call: 14336 x 4096, M = 16
    small = _case(uw, synth.CONFIGS["tiny"], "w", 4, rng)     # second call: 512 x 256, M = 4
    for p in range(5):
        for what, (h, d_blob, direct, d_x, (mi, ni, y_ref, a_ref)) in (("gate M=16", big), ("tiny M=4", small)):
            M = d_x.shape[0]
            log(f"  noalloc pipeline {uw.PIPELINE_NAMES[p]} {what}")
            ws = empty_u8(max(1, uw.workspace_bytes(h, p)))
            err_a, err_b = zeros_u32(), zeros_u32()
            ya, yb = empty_f32(M, h.N), empty_f32(M, h.N)
            ya.fill_(float("nan"))
            yb.fill_(float("nan"))
            uw.run_pipeline(p, h, d_blob, d_x, ya, M, d_direct=direct, d_ws=ws, ws_bytes=ws.numel(), d_err=err_a)
            uw.run_pipeline_noalloc(p, h, d_blob, d_x, yb, M, d_direct=direct, d_err=err_b)
            torch_cuda().cuda.synchronize()
            assert int(host(err_a)[0]) == 0 and int(host(err_b)[0]) == 0
            a, b = host(ya), host(yb)
            assert np.isfinite(b).all(), f"{what} pipeline {p}: unwritten outputs"
            assert (a.view(np.uint32) == b.view(np.uint32)).all(), f"{what} pipeline {p}: differs from uw_run_pipeline"
            check_gemm(b[mi, ni], y_ref, a_ref, f"noalloc {what} pipeline {p}")
            del ws
