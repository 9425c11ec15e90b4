"""CPU tests of libuw's host side: exports, header layout, encoder vs the oracle,
validation and error paths. No device call is made here."""
import ctypes
import os
import re

import numpy as np
import pytest

import decode_gemm_amd as uw
import oracle
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def setup_module():
    oracle.build(force=False)


def test_library_exports_every_declared_symbol():
    src = open(os.path.join(ROOT, "include", "uw.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = set(re.findall(r"\b(uw_[a-z_]+)\s*\(", src))
    assert len(names) >= 17
    lib = ctypes.CDLL(uw.LIB_PATH)
    missing = [n for n in sorted(names) if not hasattr(lib, n)]
    assert not missing, missing
    assert uw.version() == 1


def test_header_struct_is_256_bytes_and_matches_blob():
    assert ctypes.sizeof(uw.Header) == 256
    w = synth.gen_weight(synth.CONFIGS["tiny"], "w")
    blob = uw.encode(w, chunk=512)
    h = uw.inspect(blob)
    assert bytes(h) == blob[:256].tobytes()
    oh = oracle.header(blob)
    for k in ("N", "K", "chunk", "lmax", "n_pal", "n_chunks", "n_raw", "total_bits", "off_sm", "off_stream", "total_bytes"):
        assert getattr(h, k) == oh[k], k


def _cross(w, chunk, lmax):
    """Library blob -> oracle decoder; oracle blob -> library validation; equal costs."""
    lb = uw.encode(w, chunk=chunk, lmax=lmax)
    ob = oracle.encode(w, chunk=chunk, lmax=lmax)
    lh, oh = uw.inspect(lb), uw.inspect(ob)
    d = oracle.decode(lb)
    assert (d["w"] == w).all()
    # both code-length constructions are optimal: same stream length
    assert lh.total_bits == oh.total_bits
    assert list(lh.palette) == list(oh.palette) and lh.n_pal == oh.n_pal
    assert lh.n_raw == oh.n_raw and lh.total_bytes == oh.total_bytes
    # every section other than the Huffman lengths-dependent ones is identical
    for a, b in (("off_sm", "off_chunk"),):
        assert (lb[getattr(lh, a) : getattr(lh, b)] == ob[getattr(oh, a) : getattr(oh, b)]).all()
    if list(lh.code_len) == list(oh.code_len):
        assert (lb == ob).all()
    return lb


@pytest.mark.parametrize("chunk,lmax", [(64, 12), (256, 12), (1024, 12), (192, 7), (256, 15), (128, 4)])
def test_encoder_matches_oracle_tiny(chunk, lmax):
    w = synth.gen_weight(synth.CONFIGS["tiny"], "w")
    _cross(w, chunk, lmax)


def test_encoder_matches_oracle_edge_matrices():
    rng = np.random.default_rng(21)
    # all-equal: one symbol
    _cross(np.full((3, 192), 0x3C01, np.uint16), 128, 12)
    # all raw: 5 rare exponents per group
    e = rng.integers(100, 116, size=(5, 128)).astype(np.uint16)
    e[:, 5] = 200 + np.arange(5)
    e[:, 70] = 210 + np.arange(5)
    w = ((e << 7) | rng.integers(0, 128, size=e.shape).astype(np.uint16)).astype(np.uint16)
    b = _cross(w, 64, 12)
    assert uw.inspect(b).total_bits == 0
    # special values and a ragged last chunk
    w = synth.f32_to_bf16_bits(rng.standard_normal((9, 320), dtype=np.float32) * 0.02)
    w.reshape(-1)[rng.choice(w.size, 50, replace=False)] = np.array([0, 0x8000, 1, 0x7F80, 0xFF80, 0x7FC1, 0xFFFF], np.uint16)[np.arange(50) % 7]
    _cross(w, 1024, 12)
    # K = 4096 (two bitmap words per row) with raw groups in the second word
    e = rng.integers(110, 126, size=(4, 4096)).astype(np.uint16)
    e[1, 64 * 33 + 3] = 230
    e[3, 64 * 63] = 231
    w = ((e << 7) | rng.integers(0, 128, size=e.shape).astype(np.uint16)).astype(np.uint16)
    _cross(w, 256, 12)


@pytest.mark.slow
def test_encoder_matches_oracle_gate_shape():
    w = synth.gen_weight(synth.CONFIGS["gate"], "gate")
    lb = uw.encode(w)
    ob = oracle.encode(w, chunk=256)
    lh, oh = uw.inspect(lb), uw.inspect(ob)
    assert lh.total_bits == oh.total_bits and lh.n_raw == oh.n_raw
    assert (oracle.decode(lb, want=("w",))["w"] == w).all()
    # compressed size in line with the exponent law: about 1.34 bytes per weight
    assert 1.30 < lh.total_bytes / w.size < 1.37


def test_encode_error_paths():
    w = np.zeros((4, 128), np.uint16)
    with pytest.raises(uw.UwError) as e:
        uw.encode(np.zeros((4, 100), np.uint16))
    assert e.value.status == uw.ESHAPE
    with pytest.raises(uw.UwError) as e:
        uw.encode(w, chunk=100)
    assert e.value.status == uw.EINVAL
    with pytest.raises(uw.UwError) as e:
        uw.encode(w, lmax=16)
    assert e.value.status == uw.EINVAL
    # 16 used palette indices cannot be coded with lmax = 3
    rng = np.random.default_rng(0)
    w16 = ((rng.integers(100, 116, size=(2, 256)).astype(np.uint16)) << 7).astype(np.uint16)
    with pytest.raises(uw.UwError) as e:
        uw.encode(w16, lmax=3)
    assert e.value.status == uw.EINVAL
    need = ctypes.c_size_t(0)
    st = uw.lib.uw_encode(None, 4, 128, None, None, ctypes.byref(need))
    assert st == uw.EINVAL
    st = uw.lib.uw_encode(w.ctypes.data, 4, 128, None, None, ctypes.byref(need))
    assert st == uw.ENOSPACE and need.value > 256
    small = np.zeros(16, np.uint8)
    need2 = ctypes.c_size_t(16)
    assert uw.lib.uw_encode(w.ctypes.data, 4, 128, None, small.ctypes.data, ctypes.byref(need2)) == uw.ENOSPACE
    assert need2.value == need.value
    assert uw.lib.uw_last_error().decode() != ""
    assert uw.lib.uw_status_string(uw.EFORMAT).decode().startswith("UW_EFORMAT")
    assert uw.lib.uw_status_string(99).decode() == "unknown uw_status"


def _u32(blob, off, value):
    b = blob.copy()
    b[off : off + 4] = np.frombuffer(np.uint32(value).tobytes(), np.uint8)
    return b


def test_inspect_rejects_corrupt_blobs():
    w = synth.gen_weight(synth.CONFIGS["tiny"], "w")
    blob = uw.encode(w, chunk=256)
    h = uw.inspect(blob)

    def bad(b, status=uw.EFORMAT):
        with pytest.raises(uw.UwError) as e:
            uw.inspect(b)
        assert e.value.status == status

    bad(_u32(blob, 0, 0x12345678))                       # magic
    bad(_u32(blob, 4, 2))                                # version
    bad(blob[: h.total_bytes - 1])                        # truncated
    bad(blob[:100])                                       # shorter than a header
    bad(_u32(blob, 28, 16))                              # lmax out of range
    b = blob.copy(); b[56] = 1; b[57] = 1; b[58] = 1; bad(b)  # Kraft inequality violated
    b = blob.copy(); b[41] = b[40]; bad(b)                # duplicate palette entry
    oc = h.off_chunk
    bad(_u32(blob, oc + 4 * 3, int(np.frombuffer(blob[oc + 4 * 4 : oc + 4 * 5].tobytes(), "<u4")[0]) + 1))  # non-monotone
    bad(_u32(blob, oc, 1))                                # first offset not 0
    orb = h.off_rowbase
    bad(_u32(blob, orb + 4 * 10, 10**6))                  # row_base inconsistent with the bitmap
    b = blob.copy(); b[h.off_bitmap + 3] |= 0x80; bad(b)   # bitmap bit beyond the row's 4 groups
    bad(_u32(blob, 88, h.off_sm + 16))                    # section offsets off the layout
    with pytest.raises(uw.UwError) as e:
        uw.lib_inspect_null = uw.lib.uw_inspect(None, 0, None)
        uw._check(uw.lib_inspect_null)
    assert e.value.status == uw.EINVAL


def test_oracle_blobs_pass_library_validation():
    for name in ("tiny",):
        w = synth.gen_weight(synth.CONFIGS[name], "w")
        for chunk in (64, 320, 1024):
            uw.inspect(oracle.encode(w, chunk=chunk))


def test_workspace_bytes_follow_the_pipelines():
    w = synth.gen_weight(synth.CONFIGS["tiny"], "w")
    h = uw.inspect(uw.encode(w))
    n = w.size
    # preprocessing output per weight: 2 (full), 1 (exponent-only), 0.5 (transcode), 0 (direct)
    assert [uw.workspace_bytes(h, p) for p in range(5)] == [2 * n, n, n // 2, 0, 2 * n]
    with pytest.raises(uw.UwError):
        uw.workspace_bytes(h, 7)


def test_variants_table():
    n = uw.variant_count()
    assert n >= 3
    names = [uw.variant_name(v) for v in range(n)]
    assert all(names) and uw.variant_name(n) == ""
    assert any(uw.variant_supports(v, 4096, 4096, 1, uw.W_IDX) for v in range(n))
    assert any(uw.variant_supports(v, 4096, 4096, 4096, uw.W_IDX) for v in range(n))
    assert not uw.variant_supports(0, 4096, 100, 1, uw.W_IDX)


def test_dma_variant_takes_bf16_weights_within_32_bit_offsets():
    """The LDS-DMA 256x256 kernel streams bf16 operands only (no rebuild step), and it
    addresses X and W with 32-bit offsets: it reports no support for the compressed planes
    or for an operand of 4 GiB or more."""
    names = [uw.variant_name(v) for v in range(uw.variant_count())]
    v = names.index("dma 256x256")
    assert uw.variant_supports(v, 14336, 4096, 4096, uw.W_BF16)
    assert uw.variant_supports(v, 4096, 14336, 1, uw.W_BF16)
    for src in (uw.W_EXP, uw.W_IDX, uw.W_DIRECT):
        assert not uw.variant_supports(v, 14336, 4096, 4096, src)
    assert not uw.variant_supports(v, 1 << 18, 8192, 64, uw.W_BF16)   # W: 4 GiB of bf16
    assert not uw.variant_supports(v, 8192, 8192, 1 << 18, uw.W_BF16)  # X: 4 GiB of bf16
    assert not uw.variant_supports(v, 4096, 4096, 0, uw.W_BF16)


def test_one_hip_runtime_whatever_the_import_order():
    """Importing the binding before PyTorch must not load a second HIP runtime: libuw and
    the tensors it is given have to share PyTorch's (a second runtime finds no device)."""
    import subprocess
    import sys

    code = ("import decode_gemm_amd, torch, os\n"
            "m = open('/proc/%d/maps' % os.getpid()).read()\n"
            "print(len({l.split()[-1] for l in m.splitlines() if 'libamdhip64' in l}))\n")
    out = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True, timeout=300)
    assert out.returncode == 0, out.stderr
    assert out.stdout.strip() == "1", out.stdout


def test_mlp_stack_host_checks():
    """Workspace size of the stack forward and its shape / argument checks (host side,
    no device call: the checks come before any launch)."""
    w = synth.gen_weight(synth.CONFIGS["tiny"], "w")  # 512 x 256
    hg = uw.inspect(uw.encode(w))
    wd = np.ascontiguousarray(w.reshape(256, 512))
    hd = uw.inspect(uw.encode(wd))
    fake = 1 << 20
    good = uw.mlp_layers([(uw.proj(hg, fake, uw.PIPE_FULL), uw.proj(hg, fake, uw.PIPE_EXP),
                           uw.proj(hd, fake, uw.PIPE_TRANSCODE))])
    M = 7
    a = lambda v: (v + 255) // 256 * 256
    slot = a(2 * 512 * 256)  # the largest decode plane: full decode of a 512 x 256 matrix
    base = 2 * a(4 * M * 512) + a(2 * M * 512)
    assert uw.mlp_stack_workspace(good, M) == base + slot
    assert uw.mlp_stack_workspace(good, M, two_slots=True) == base + 2 * slot
    bad = uw.mlp_layers([(uw.proj(hg, fake, uw.PIPE_FULL), uw.proj(hg, fake, uw.PIPE_FULL),
                          uw.proj(hg, fake, uw.PIPE_FULL))])  # down must be 256 x 512
    with pytest.raises(uw.UwError) as e:
        uw.mlp_stack_workspace(bad, M)
    assert e.value.status == uw.ESHAPE
    nodirect = uw.mlp_layers([(uw.proj(hg, fake, uw.PIPE_DIRECT), uw.proj(hg, fake, uw.PIPE_FULL),
                               uw.proj(hd, fake, uw.PIPE_FULL))])
    with pytest.raises(uw.UwError) as e:
        uw.mlp_stack_forward(nodirect, M, fake, fake, fake, 1 << 30, stream=0)
    assert e.value.status == uw.EINVAL
    with pytest.raises(uw.UwError) as e:
        uw.mlp_stack_forward(good, M, fake, fake, fake, 16, stream=0)
    assert e.value.status == uw.ENOSPACE


def test_mlp_stack_schedule_options_host():
    """Slot count and decode order of the stack forward: workspace sizes, the slot range,
    a down-first order that would need a slot still held by a later GEMM (rejected before
    any launch), and the tuner's check of its starting plan (also before any launch)."""
    w = synth.gen_weight(synth.CONFIGS["tiny"], "w")  # 512 x 256
    hg = uw.inspect(uw.encode(w))
    hd = uw.inspect(uw.encode(np.ascontiguousarray(w.reshape(256, 512))))
    fake = 1 << 20
    hard = (uw.proj(hg, fake, uw.PIPE_FULL), uw.proj(hg, fake, uw.PIPE_EXP), uw.proj(hd, fake, uw.PIPE_TRANSCODE))
    layers = uw.mlp_layers([hard, hard])
    M = 3
    a = lambda v: (v + 255) // 256 * 256
    slot = a(2 * 512 * 256)
    base = 2 * a(4 * M * 512) + a(2 * M * 512)
    assert uw.mlp_stack_workspace_ex(layers, M, slots=3) == base + 3 * slot
    assert uw.mlp_stack_workspace_ex(layers, M, slots=0) == base + 2 * slot  # 0 = the default, 2
    assert uw.mlp_stack_workspace_ex(layers, M, slots=1) == uw.mlp_stack_workspace(layers, M)
    for bad in (9, -1):
        with pytest.raises(uw.UwError) as e:
            uw.mlp_stack_workspace_ex(layers, M, slots=bad)
        assert e.value.status == uw.EINVAL
    # down first: decode order down0, gate0, up0, ... with two slots, up0 would need the
    # slot of down0, which is freed only after up0's own GEMM
    with pytest.raises(uw.UwError) as e:
        uw.mlp_stack_forward_ex(layers, M, fake, fake, fake, 1 << 30, stream=0, decode_stream=fake, slots=2,
                                down_first=True)
    assert e.value.status == uw.EINVAL and "decode slots" in str(e.value)
    with pytest.raises(uw.UwError) as e:
        uw.mlp_stack_autotune(layers, M, fake, fake, fake, 64, stream=0)
    assert e.value.status == uw.EINVAL


def test_stream_pair_argument_checks():
    """uw_stream_pair_create rejects NULL outputs and an empty decode share before it
    touches the device."""
    P = ctypes.c_void_p
    g, d = P(), P()
    assert uw.lib.uw_stream_pair_create(8, None, ctypes.byref(d)) == uw.EINVAL
    assert uw.lib.uw_stream_pair_create(8, ctypes.byref(g), None) == uw.EINVAL
    with pytest.raises(uw.UwError) as e:
        uw.stream_pair_create(0)
    assert e.value.status == uw.EINVAL
    with pytest.raises(uw.UwError) as e:
        uw.stream_pair_create(-3)
    assert e.value.status == uw.EINVAL
    assert uw.lib.uw_stream_destroy(None) == uw.EINVAL
    assert uw.lib.uw_stream_cu_count(None, None) == uw.EINVAL


def test_split_count_rounds_to_whole_groups():
    """uw_split_count: an explicit split is rounded so every slice has the same whole number
    of 64-groups; out-of-range requests give 0."""
    names = [uw.variant_name(v) for v in range(uw.variant_count())]
    assert not any("vendor" in n for n in names)
    v = names.index("tiled 128x128")
    N, K = 4096, 14336  # 224 groups
    assert uw.split_count(v, N, K, 1024, 1) == 1
    assert uw.split_count(v, N, K, 1024, 3) == 3  # 75 groups per slice -> 3 slices
    assert uw.split_count(v, N, K, 1024, 5) == 5
    assert uw.split_count(v, N, K, 1024, 224) == 224
    assert uw.split_count(v, N, K, 1024, 225) == 0
    assert uw.split_count(v, N, K, 1024, -1) == 0
    assert uw.split_count(v, 256, 448, 64, 5) == 4  # 7 groups: 2 per slice -> 4 slices
    assert uw.split_count(v, 256, 448, 64, 0) >= 1
    assert uw.split_count(len(names), N, K, 1024, 1) == 0
    assert uw.split_count(v, N, 100, 1024, 1) == 0


def test_noalloc_entry_point_rejects_slots_beyond_its_scratch():
    """uw_run_pipeline_noalloc refuses, before any device call, a pipeline whose
    preprocessing slot is larger than the library's scratch array (bf16 weights of a
    8200 x 8192 matrix: 2 B/w > 128 MiB); a pipeline that needs no slot is not refused
    for size."""
    assert uw.noalloc_scratch_bytes() == 128 << 20
    w = np.full((8200, 8192), 0x3C00, np.uint16)
    h = uw.inspect(uw.encode(w))
    assert uw.workspace_bytes(h, uw.PIPE_FULL) > uw.noalloc_scratch_bytes()
    for p in (uw.PIPE_FULL, uw.PIPE_EXPAND):
        with pytest.raises(uw.UwError) as e:
            uw.run_pipeline_noalloc(p, h, 0x1000, 0x1000, 0x1000, 1, d_direct=0x1000, stream=0)
        assert e.value.status == uw.ENOSPACE
