"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each test targets a plausible mistake: swapped bf16 fields, a wrong palette order, a
wrong raw-row rule, non-optimal or over-long code lengths, a wrong canonical code
assignment, a wrong bit order, a dropped chunk offset, a transposed GEMM operand, a
double rounding in the SwiGLU glue.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
from scipy.special import erf, expit

import oracle
import synth


def setup_module():
    oracle.build(force=False)


# ---------------------------------------------------------------- bf16 fields (split)
def test_split_matches_value_semantics_exhaustive():
    """All 65536 bf16 patterns: the exponent byte, sign and mantissa the oracle splits
    out must agree with the value they encode (frexp on the float), and join must undo
    split. A swapped or shifted field fails here."""
    w = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    sm, e = oracle.split(w)
    assert (oracle.join(sm, e) == w).all()
    with np.errstate(invalid="ignore"):
        x = synth.bf16_bits_to_f32(w).astype(np.float64)
    finite_normal = np.isfinite(x) & (np.abs(x) >= 2.0**-126)
    m, ex = np.frexp(np.abs(x[finite_normal]))  # |x| = m * 2^ex, m in [0.5, 1)
    assert (e[finite_normal].astype(np.int64) == ex.astype(np.int64) - 1 + 127).all()
    mant = np.round((m * 2 - 1) * 128).astype(np.int64)
    assert (sm[finite_normal] & 0x7F == mant).all()
    assert ((sm[finite_normal] >> 7).astype(bool) == np.signbit(x[finite_normal])).all()
    # zero / subnormal: exponent byte 0; inf / nan: 255
    sub = np.isfinite(x) & (np.abs(x) < 2.0**-126)
    assert (e[sub] == 0).all()
    assert (e[~np.isfinite(x)] == 255).all()


# ---------------------------------------------------------------- palette
def test_palette_order_hand_case():
    counts = {100: 5, 101: 9, 102: 9, 103: 1, 104: 20, 105: 2, 106: 2, 107: 3, 108: 4,
              109: 6, 110: 7, 111: 8, 112: 10, 113: 11, 114: 12, 115: 13, 116: 14, 117: 1, 118: 2}
    e = np.concatenate([np.full(c, v, np.uint8) for v, c in counts.items()])
    np.random.default_rng(1).shuffle(e)
    pal, hist = oracle.palette(e)
    # by hand: count desc, then value asc
    expected = [104, 116, 115, 114, 113, 112, 101, 102, 111, 110, 109, 100, 108, 107, 105, 106]
    assert pal.tolist() == expected
    assert hist[104] == 20 and hist[103] == 1


def test_palette_fewer_than_16_distinct():
    e = np.array([7, 7, 3, 3, 3, 9], np.uint8)
    pal, _ = oracle.palette(e)
    assert pal.tolist() == [3, 7, 9]


# ---------------------------------------------------------------- raw 64-weight rows
def _matrix_with_exponents(e, seed=0):
    rng = np.random.default_rng(seed)
    sm = rng.integers(0, 256, size=e.shape, dtype=np.uint16)
    return ((sm >> 7) << 15 | (e.astype(np.uint16) << 7) | (sm & 0x7F)).astype(np.uint16)


def test_raw_group_rule_hand_case():
    """17 distinct exponents: 16 frequent ones and one rare (value 200). Only the 64-weight
    row groups holding a 200 are raw, whole group, one decision per group."""
    N, K = 3, 4096  # 64 groups per row -> bitmap needs two 32-bit words per row
    rng = np.random.default_rng(5)
    e = rng.integers(110, 126, size=(N, K)).astype(np.uint8)
    e[1, 130] = 200        # group (1, 2)
    e[1, 131] = 200        # same group again
    e[2, 64 * 40 + 7] = 200  # group (2, 40) -> word 1, bit 8
    w = _matrix_with_exponents(e)
    _, ex = oracle.split(w)
    pal, _ = oracle.palette(ex)
    assert 200 not in pal.tolist() and len(pal) == 16
    bitmap, row_base, raw = oracle.raw_groups(ex, pal)
    assert bitmap.shape == (3, 2)
    assert bitmap[0].tolist() == [0, 0]
    assert bitmap[1].tolist() == [1 << 2, 0]
    assert bitmap[2].tolist() == [0, 1 << 8]
    assert row_base.tolist() == [0, 0, 1, 2]
    assert (raw[0] == e[1, 128:192]).all()
    assert (raw[1] == e[2, 64 * 40 : 64 * 41]).all()
    blob = oracle.encode(w, chunk=256)
    h = oracle.header(blob)
    assert h["n_raw"] == 2
    # raw groups carry no symbols
    assert h["total_bits"] == sum(
        int(h["code_len"][list(pal).index(v)]) for v in e.reshape(-1)[_nonraw_mask(N, K, [(1, 2), (2, 40)])]
    )
    assert (oracle.decode(blob)["w"] == w).all()


def _nonraw_mask(N, K, raw_groups):
    m = np.ones((N, K), bool)
    for r, j in raw_groups:
        m[r, 64 * j : 64 * j + 64] = False
    return m.reshape(-1)


# ---------------------------------------------------------------- golden bitstream
def _hand_matrix(g):
    N, K = g["N"], g["K"]
    e = np.zeros(N * K, np.uint8)
    for v, (a, b) in g["exponents"].items():
        e[a:b] = int(v)
    sm = np.array([(37 * i) % 256 for i in range(N * K)], np.uint16)
    w = ((sm >> 7) << 15 | (e.astype(np.uint16) << 7) | (sm & 0x7F)).astype(np.uint16)
    return w.reshape(N, K), sm.astype(np.uint8)


def test_golden_hand_stream(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "hand_stream.json")))
    w, sm = _hand_matrix(g)
    blob = oracle.encode(w, chunk=g["chunk"])
    h = oracle.header(blob)
    assert h["palette"][: h["n_pal"]].tolist() == g["palette"]
    assert h["code_len"][: h["n_pal"]].tolist() == g["code_len"]
    assert oracle.canonical_codes(g["code_len"]).tolist() == g["codes"]
    assert h["total_bits"] == g["total_bits"]
    words = np.frombuffer(blob[h["off_stream"] : h["off_stream"] + 16].tobytes(), "<u4")
    assert [f"0x{v:08X}" for v in words] == g["stream_words"]
    offs = np.frombuffer(blob[h["off_chunk"] : h["off_chunk"] + 8].tobytes(), "<u4")
    assert offs.tolist() == g["chunk_offsets"]
    assert (blob[h["off_sm"] : h["off_sm"] + 64] == sm).all()
    assert (oracle.decode(blob)["w"] == w).all()


def test_golden_rfc1951_canonical(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "rfc1951_canonical.json")))
    codes = oracle.canonical_codes(g["lengths"])
    got = [format(int(c), f"0{l}b") for c, l in zip(codes, g["lengths"])]
    assert got == g["codes_binary"]


# ---------------------------------------------------------------- code lengths
def _all_length_vectors(n, lmax):
    return np.array(list(itertools.product(range(1, lmax + 1), repeat=n)), dtype=np.int64)


@pytest.mark.parametrize("n,lmax", [(2, 3), (3, 3), (4, 4), (5, 5), (6, 7), (6, 3)])
def test_code_lengths_brute_force_optimal(n, lmax):
    """Package-merge cost equals the minimum over every length vector with Kraft <= 1
    and every length <= lmax (exhaustive search)."""
    vecs = _all_length_vectors(n, lmax)
    kraft = (2.0 ** (-vecs)).sum(axis=1)
    ok = vecs[kraft <= 1.0 + 1e-12]
    rng = np.random.default_rng(n * 100 + lmax)
    for trial in range(40):
        if trial % 3 == 0:
            f = np.array([int(1.7**i) + 1 for i in range(n)])[rng.permutation(n)]  # skewed: lmax binds
        else:
            f = rng.integers(1, 1000, size=n)
        if (1 << lmax) < n:
            continue
        ln = oracle.code_lengths(f, lmax).astype(np.int64)
        assert ln.max() <= lmax and ln.min() >= 1
        assert abs((2.0 ** (-ln)).sum() - 1.0) < 1e-12  # Kraft equality: a full tree
        best = (ok * f).sum(axis=1).min()
        assert (ln * f).sum() == best


def test_code_lengths_degenerate():
    assert oracle.code_lengths([0, 0, 0], 12).tolist() == [0, 0, 0]
    assert oracle.code_lengths([0, 5, 0], 12).tolist() == [0, 1, 0]
    ln = oracle.code_lengths([3, 0, 3, 1], 12).tolist()
    assert ln[1] == 0 and sorted([ln[0], ln[2], ln[3]]) == [1, 2, 2]
    assert oracle.code_lengths([1] * 16, 4).tolist() == [4] * 16
    with pytest.raises(ValueError):
        oracle.code_lengths([1] * 16, 3)


def test_code_lengths_unlimited_equals_huffman():
    """With a generous limit, package-merge must reach the cost of plain Huffman merging
    (textbook two-smallest merge, computed here independently)."""
    import heapq

    rng = np.random.default_rng(3)
    for _ in range(50):
        n = int(rng.integers(2, 17))
        f = rng.integers(1, 10**6, size=n)
        h = [int(v) for v in f]
        heapq.heapify(h)
        cost = 0
        while len(h) > 1:
            a, b = heapq.heappop(h), heapq.heappop(h)
            cost += a + b
            heapq.heappush(h, a + b)
        ln = oracle.code_lengths(f, 15)
        assert int((ln.astype(np.int64) * f).sum()) == cost


# ---------------------------------------------------------------- entropy bound + law
def _closed_form_exponent_law(sigma):
    """P(bf16 exponent byte = E) for bf16_rne(N(0, sigma)): |x| rounds into binade E iff
    |x| in [2^(E-127)(1 - 2^-9), 2^(E-126)(1 - 2^-9))."""
    E = np.arange(1, 255)
    lo = 2.0 ** (E - 127) * (1 - 2.0**-9)
    hi = 2.0 ** (E - 126) * (1 - 2.0**-9)
    p = erf(hi / (sigma * math.sqrt(2))) - erf(lo / (sigma * math.sqrt(2)))
    return dict(zip(E.tolist(), p.tolist()))


def test_exponent_law_closed_form_and_entropy_bound():
    """The oracle's histogram/palette of synthetic N(0, 0.02) weights follows the closed
    form (synthetic stand-in for the post's 'top-16 cover >99%, ~2.6 bits'), and the
    mean code length lies in [H, H+1)."""
    cfg = synth.Config("law", 9, (("w", 2048, 2048),), 0.02, "normal", 0.0, 0.0, 0, (1,))
    w = synth.gen_weight(cfg, "w")
    _, e = oracle.split(w)
    pal, hist = oracle.palette(e)
    law = _closed_form_exponent_law(0.02)
    n = e.size
    H_cf = -sum(p * math.log2(p) for p in law.values() if p > 0)
    p_emp = hist[hist > 0] / n
    H_emp = float(-(p_emp * np.log2(p_emp)).sum())
    assert abs(H_emp - H_cf) < 0.01 and abs(H_cf - 2.545) < 0.002
    top16_cf = sorted(law.values(), reverse=True)[:16]
    assert sum(top16_cf) > 0.9999
    cov = hist[pal].sum() / n
    assert abs(cov - sum(top16_cf)) < 1e-4
    # the most probable exponents (well separated in probability) lead the palette
    ranked = sorted(law, key=lambda E: -law[E])
    assert pal[:8].tolist() == ranked[:8]
    # entropy bound of the Huffman code actually written
    blob = oracle.encode(w)
    h = oracle.header(blob)
    _, _, raw = oracle.raw_groups(e.reshape(w.shape), pal)
    nsym = n - 64 * len(raw)
    lbar = h["total_bits"] / nsym
    # H of the symbol distribution the code was built for
    freq = np.zeros(16)
    for i, v in enumerate(pal):
        freq[i] = hist[v]
    q = freq[freq > 0] / freq.sum()
    H = float(-(q * np.log2(q)).sum())
    assert H - 0.01 <= lbar < H + 1.0  # small slack: raw groups remove a few symbols from freq
    assert lbar >= 2.5


@pytest.mark.parametrize("name", ["tiny", "gate"])
def test_entropy_bound_on_configs(name):
    cfg = synth.CONFIGS[name]
    proj = cfg.shapes[0][0]
    w = synth.gen_weight(cfg, proj)
    blob = oracle.encode(w)
    h = oracle.header(blob)
    dec = oracle.decode(blob, want=("exp", "idx"))
    # symbol frequencies recounted from the decoded index plane, non-raw elements only
    N, K = w.shape
    bm = np.frombuffer(blob[h["off_bitmap"] : h["off_bitmap"] + 4 * N * h["bitmap_words"]].tobytes(), "<u4").reshape(N, -1)
    j = np.arange(K // 64)
    raw = (bm[:, j // 32] >> (j % 32)) & 1
    nonraw = np.repeat(raw == 0, 64, axis=1).reshape(-1)
    idx = np.empty(N * K, np.uint8)
    idx[0::2] = dec["idx"] & 15
    idx[1::2] = dec["idx"] >> 4
    f = np.bincount(idx[nonraw], minlength=16).astype(np.float64)
    q = f[f > 0] / f.sum()
    H = float(-(q * np.log2(q)).sum())
    lbar = h["total_bits"] / nonraw.sum()
    assert H <= lbar < H + 1
    ln = h["code_len"][: h["n_pal"]].astype(np.int64)
    assert abs((2.0 ** -ln[ln > 0]).sum() - 1.0) < 1e-12
    assert ln.max() <= 12


# ---------------------------------------------------------------- special structures
def test_uniform_alphabet_stream_equals_index_nibbles():
    """16 equally frequent symbols -> every length 4, code = index, so the Huffman stream
    is the palette-index sequence written 4 bits at a time, MSB first: the full decoder
    and the palette transcoder must agree on it."""
    N, K = 4, 256
    e = (np.arange(N * K) % 16 + 100).astype(np.uint8).reshape(N, K)
    rng = np.random.default_rng(2)
    e = e.reshape(-1)[rng.permutation(N * K)].reshape(N, K)
    w = _matrix_with_exponents(e)
    blob = oracle.encode(w, chunk=128)
    h = oracle.header(blob)
    assert h["code_len"].tolist() == [4] * 16
    assert h["palette"].tolist() == list(range(100, 116))
    words = np.frombuffer(blob[h["off_stream"] : h["off_stream"] + N * K // 2].tobytes(), "<u4")
    syms = np.array([(int(wd) >> (28 - 4 * t)) & 15 for wd in words for t in range(8)], np.uint8)
    assert (syms == (e.reshape(-1) - 100)).all()
    dec = oracle.decode(blob)
    assert (dec["idx"] & 15 == syms[0::2]).all() and (dec["idx"] >> 4 == syms[1::2]).all()
    assert (dec["w"] == w).all()


def test_all_raw_matrix_empty_stream():
    N, K = 5, 128
    rng = np.random.default_rng(4)
    e = rng.integers(100, 116, size=(N, K)).astype(np.uint8)
    e[:, 5] = 200 + np.arange(N)  # 5 rare values, one per row, first group
    e[:, 64 + 9] = 210 + np.arange(N)  # and in the second group
    # make the rare values rarer than all 16 common ones -> outside the palette
    w = _matrix_with_exponents(e)
    blob = oracle.encode(w, chunk=64)
    h = oracle.header(blob)
    assert h["n_raw"] == N * K // 64
    assert h["total_bits"] == 0
    offs = np.frombuffer(blob[h["off_chunk"] : h["off_chunk"] + 4 * (h["n_chunks"] + 1)].tobytes(), "<u4")
    assert (offs == 0).all()
    dec = oracle.decode(blob)
    assert (dec["w"] == w).all() and (dec["idx"] == 0).all()


def test_single_symbol_matrix():
    w = np.full((3, 192), 0x3C01, np.uint16)
    w[1, 7] = 0xBC7F  # same exponent, other sign/mantissa
    blob = oracle.encode(w, chunk=128)
    h = oracle.header(blob)
    assert h["n_pal"] == 1 and h["code_len"][0] == 1 and h["total_bits"] == w.size
    s = blob[h["off_stream"] : h["off_stream"] + h["bytes_stream"]]
    assert (s == 0).all()
    assert (oracle.decode(blob)["w"] == w).all()


def test_special_values_bit_exact():
    specials = np.array([0x0000, 0x8000, 0x0001, 0x807F, 0x0040, 0x7F80, 0xFF80, 0x7FC0, 0x7FA3, 0xFF81,
                         0x7F7F, 0xFF7F, 0x0080, 0x8080], np.uint16)
    rng = np.random.default_rng(7)
    w = synth.f32_to_bf16_bits(rng.standard_normal((8, 320), dtype=np.float32) * 0.02)
    flat = w.reshape(-1)
    pos = rng.choice(flat.size, size=200, replace=False)
    flat[pos] = specials[np.arange(200) % len(specials)]
    for chunk in (64, 192, 1024):
        blob = oracle.encode(w, chunk=chunk)
        assert (oracle.decode(blob)["w"] == w).all()


def test_partial_last_chunk_and_offsets():
    cfg = synth.CONFIGS["tiny"]
    w = synth.gen_weight(cfg, "w")[:37]  # 37*256 = 9472 elements, not a multiple of 1024
    blob = oracle.encode(w, chunk=1024)
    h = oracle.header(blob)
    assert h["n_chunks"] == 10
    offs = np.frombuffer(blob[h["off_chunk"] : h["off_chunk"] + 44].tobytes(), "<u4")
    assert offs[0] == 0 and offs[-1] == h["total_bits"] and (np.diff(offs.astype(np.int64)) >= 0).all()
    assert (oracle.decode(blob)["w"] == w).all()


def test_lmax_binds():
    cfg = synth.CONFIGS["tiny"]
    w = synth.gen_weight(cfg, "w")
    for lmax in (4, 6, 9, 15):
        blob = oracle.encode(w, lmax=lmax)
        h = oracle.header(blob)
        assert h["code_len"].max() <= lmax
        assert (oracle.decode(blob)["w"] == w).all()


def test_roundtrip_and_planes_tiny():
    cfg = synth.CONFIGS["tiny"]
    w = synth.gen_weight(cfg, "w")
    blob = oracle.encode(w)
    d = oracle.decode(blob)
    assert (d["w"] == w).all()
    sm, e = oracle.split(w)
    assert (d["exp"] == e).all()
    # palette plane: index of the exponent in the palette outside raw groups, else 0
    h = oracle.header(blob)
    pal = h["palette"][: h["n_pal"]].tolist()
    assert d["idx"].size == w.size // 2
    lo, hi = d["idx"] & 15, d["idx"] >> 4
    flat_e = e.reshape(-1)
    for i in range(0, w.size, 997):
        v = (lo if i % 2 == 0 else hi)[i // 2]
        if flat_e[i] in pal:
            grp = flat_e.reshape(-1, 64)[i // 64]
            if all(x in pal for x in grp):
                assert v == pal.index(flat_e[i])
                continue
        assert v == 0


def test_corrupt_blob_is_rejected():
    cfg = synth.CONFIGS["tiny"]
    w = synth.gen_weight(cfg, "w")
    blob = oracle.encode(w)
    h = oracle.header(blob)
    bad = blob.copy()
    bad[0] ^= 1
    assert oracle.decode_status(bad) == oracle.EFORMAT
    bad = blob.copy()
    o = h["off_chunk"] + 4 * 3
    bad[o] ^= 1  # chunk 3 now claims to start one bit off
    assert oracle.decode_status(bad) == oracle.EFORMAT
    assert oracle.decode_status(blob[: h["total_bytes"] - 1]) == oracle.EFORMAT
    assert oracle.encode_status(np.zeros((2, 100), np.uint16)) == oracle.ESHAPE


def test_sizes_follow_the_layout():
    cfg = synth.CONFIGS["tiny"]
    w = synth.gen_weight(cfg, "w")
    blob = oracle.encode(w, chunk=512)
    h = oracle.header(blob)
    N, K = w.shape

    def up(x, a):
        return (x + a - 1) // a * a

    o = 256
    assert h["off_sm"] == o
    o = up(o + N * K, 256); assert h["off_bitmap"] == o
    o = up(o + 4 * N * ((K + 2047) // 2048), 256); assert h["off_rowbase"] == o
    o = up(o + 4 * (N + 1), 256); assert h["off_raw"] == o
    o = up(o + 64 * h["n_raw"], 256); assert h["off_chunk"] == o
    o = up(o + 4 * (h["n_chunks"] + 1), 256); assert h["off_stream"] == o
    assert h["bytes_stream"] == up((h["total_bits"] + 7) // 8, 16) + 64
    assert h["total_bytes"] == blob.size == o + h["bytes_stream"]


# ---------------------------------------------------------------- GEMM
def test_gemm_one_hot_rows_select_weights_exactly():
    cfg = synth.CONFIGS["tiny"]
    w = synth.gen_weight(cfg, "w")
    N, K = w.shape
    ks = [0, 1, 63, 64, 200, 255]
    x = np.zeros((len(ks), K), np.uint16)
    for m, k in enumerate(ks):
        x[m, k] = 0x3F80  # 1.0
    y, a = oracle.gemm(x, w)
    wf = synth.bf16_bits_to_f32(w).astype(np.float64)
    for m, k in enumerate(ks):
        assert (y[m] == wf[:, k]).all()
        assert (a[m] == np.abs(wf[:, k])).all()


def test_gemm_small_integers_exact_and_not_transposed():
    rng = np.random.default_rng(11)
    M, N, K = 7, 13, 192
    xi = rng.integers(-8, 9, size=(M, K))
    wi = rng.integers(-8, 9, size=(N, K))
    x = synth.f32_to_bf16_bits(xi.astype(np.float32))
    w = synth.f32_to_bf16_bits(wi.astype(np.float32))
    y, a = oracle.gemm(x, w)
    assert (y == (xi @ wi.T).astype(np.float64)).all()
    assert (a == (np.abs(xi) @ np.abs(wi).T).astype(np.float64)).all()


def test_gemm_matches_numpy_float64():
    rng = np.random.default_rng(12)
    x = synth.f32_to_bf16_bits(rng.standard_normal((5, 320), dtype=np.float32))
    w = synth.f32_to_bf16_bits(rng.standard_normal((33, 320), dtype=np.float32))
    y, _ = oracle.gemm(x, w)
    ref = synth.bf16_bits_to_f32(x).astype(np.float64) @ synth.bf16_bits_to_f32(w).astype(np.float64).T
    assert np.allclose(y, ref, rtol=1e-12, atol=1e-12)
    mi = np.array([0, 4, 2]); ni = np.array([32, 0, 17])
    yp, ap = oracle.gemm_pairs(x, w, mi, ni)
    assert np.allclose(yp, ref[mi, ni], rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------- SwiGLU glue
def test_f64_to_bf16_agrees_with_single_rounding_from_float32():
    """For doubles that are exact float32 values, rounding double->bf16 once must equal
    the plain float32->bf16 round-to-nearest-even on the bit pattern."""
    rng = np.random.default_rng(13)
    v = np.concatenate([
        rng.standard_normal(4000).astype(np.float32) * np.float32(10.0) ** rng.integers(-30, 30, 4000).astype(np.float32),
        np.array([1.00390625, 1.01171875, -1.00390625, 3.0e38, 1e-39, -2e-40, 0.0, -0.0], np.float32),
    ]).astype(np.float32)
    v = v[np.isfinite(v)]
    got = np.array([oracle.f64_to_bf16(float(t)) for t in v], np.uint16)
    assert (got == synth.f32_to_bf16_bits(v)).all()
    assert oracle.f64_to_bf16(float("inf")) == 0x7F80
    assert oracle.f64_to_bf16(4e38) == 0x7F80


def test_swiglu_against_expit():
    rng = np.random.default_rng(14)
    g = rng.standard_normal(5000).astype(np.float32) * 3
    u = rng.standard_normal(5000).astype(np.float32) * 3
    h = oracle.swiglu(g, u)
    ref = g.astype(np.float64) * expit(g.astype(np.float64)) * u.astype(np.float64)
    hf = synth.bf16_bits_to_f32(h).astype(np.float64)
    # one bf16 rounding (8 significant bits): relative error <= 2^-8
    assert (np.abs(hf - ref) <= np.abs(ref) * 2.0**-8 + 1e-38).all()
    # and it is the nearest bf16: the neighbours one ulp away are not closer
    for i in range(0, 5000, 7):
        b = int(h[i])
        for nb in (b - 1, b + 1):
            if 0 <= nb < 0x10000 and (nb & 0x7F80) != 0x7F80 and (nb ^ b) < 0x8000:
                assert abs(float(synth.bf16_bits_to_f32(np.array([nb]))[0]) - ref[i]) >= abs(hf[i] - ref[i])
