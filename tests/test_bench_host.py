"""Host-side checks of bench.py: the one-GPU guard, the byte accounting the roofline
uses, and the rule that measured traffic is dropped once the GEMM sources change."""
import json
import os
import subprocess
import sys

import numpy as np

import bench
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert p.returncode == 2
    msg = json.loads(p.stdout.strip().splitlines()[-1])
    assert msg["n_gpus"] == 2 and "one GPU" in msg["error"]


def test_byte_accounting_matches_the_library_sizes():
    import decode_gemm_amd as uw

    w = synth.gen_weight(synth.CONFIGS["tiny"], "w")
    blob = uw.encode(w)
    h = uw.inspect(blob)
    N, K, M = h.N, h.K, 4
    assert bench.direct_bytes(h) == uw.direct_plane_bytes(h)
    s = bench.section_bytes(h)
    # every section the blob holds, plus its header and alignment padding, is the blob
    assert sum(s.values()) <= blob.size < sum(s.values()) + 8 * 256 + 4096
    # direct palette: the prepared plane, X in bf16 and Y in fp32, nothing else
    assert bench.algorithmic_bytes(h, M, 3) == uw.direct_plane_bytes(h) + 2 * M * K + 4 * M * N
    # full decode: reads the whole blob's payload and writes bf16 W, then the GEMM reads it
    full = bench.algorithmic_bytes(h, M, 0)
    assert full == bench.decode_bytes(h, "full") + 2 * N * K + 2 * M * K + 4 * M * N
    assert bench.decode_bytes(h, "full") - bench.decode_bytes(h, "exp") == N * K + N * K  # sm in, 2 vs 1 B out
    # expand: reads the direct plane, writes bf16 W, then the plain GEMM reads it
    assert bench.decode_bytes(h, "expand") == uw.direct_plane_bytes(h) + 2 * N * K
    assert bench.algorithmic_bytes(h, M, 4) == bench.decode_bytes(h, "expand") + 2 * N * K + 2 * M * K + 4 * M * N
    assert uw.workspace_bytes(h, uw.PIPE_EXPAND) == 2 * N * K


def test_measured_traffic_needs_the_profiled_sources(tmp_path, monkeypatch):
    key = "direct pipeline, skinny rt4 u2 w4, M=64"
    f = tmp_path / "t.json"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.measured_traffic(key) is None  # no summary
    f.write_text(json.dumps({"sources_sha256": bench.gemm_sources_sha256(),
                             "kernels": {key: {"hbm_bytes_per_launch": 123456}}}))
    assert bench.measured_traffic(key) == 123456
    assert bench.measured_traffic("direct pipeline, skinny rt1 u4 w4, M=64") is None
    f.write_text(json.dumps({"sources_sha256": "0" * 64, "kernels": {key: {"hbm_bytes_per_launch": 123456}}}))
    assert bench.measured_traffic(key) is None  # kernel changed since the counters were taken
    assert np.isfinite(bench.HBM_PEAK_GBS)


def test_resident_and_fused_byte_accounting():
    import decode_gemm_amd as uw

    w = synth.gen_weight(synth.CONFIGS["tiny"], "w")
    blob = uw.encode(w)
    h = uw.inspect(blob)
    N, K, M = h.N, h.K, 8
    # B_res: the Huffman blob for the decode-first pipelines, the direct plane otherwise
    for p in (0, 1, 2):
        assert bench.resident_bytes(h, p, blob.size) == blob.size
    for p in (3, 4):
        assert bench.resident_bytes(h, p, blob.size) == uw.direct_plane_bytes(h)
    # the fused gate/up launch: two planes, X once, g and u in fp32, h in bf16
    assert bench.gate_up_bytes(h, h, M) == 2 * uw.direct_plane_bytes(h) + 2 * M * K + 10 * M * N


def test_plans_json_round_trip():
    import decode_gemm_amd as uw

    plans = {1: {"gate": {"pipeline": uw.PIPE_DIRECT, "variant": 5, "split_k": 1, "t_ms": 0.0186},
                 "down": {"pipeline": uw.PIPE_TRANSCODE, "variant": uw.variant_count() - 1, "split_k": 4, "t_ms": 0.02}}}
    j = json.loads(json.dumps(bench.plans_to_json(uw, plans)))
    assert j["1"]["gate"]["variant"] == uw.variant_name(5) and j["1"]["down"]["pipeline"] == "transcode"
    back = bench.plans_from_json(uw, j)
    for r in ("gate", "down"):
        for k in ("pipeline", "variant", "split_k"):
            assert back[1][r][k] == plans[1][r][k]
