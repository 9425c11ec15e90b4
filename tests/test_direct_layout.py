"""CPU checks of the test-side reader of the direct-palette plane (tests/direct_layout.py)
on a block built by hand from the format text, so that the GPU tests that read the
library's planes through it rest on something other than the library."""
import json
import os

import numpy as np

from tests import direct_layout as dl


def _hand_matrix(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "hand_stream.json")))
    e = np.zeros(64, np.uint16)
    for v, (a, b) in g["exponents"].items():
        e[a:b] = int(v)
    sm = np.array([(37 * i) % 256 for i in range(64)], np.uint16)
    w = ((sm >> 7) << 15 | (e << 7) | (sm & 0x7F)).astype(np.uint16)
    return w.reshape(1, 64)


def test_hand_block_bytes_and_rebuild(golden_dir):
    w = _hand_matrix(golden_dir)
    pal_sorted = [119, 120, 121, 122]
    d = dl.hand_block(w, pal_sorted)
    assert d.size == dl.plane_bytes(1, 64, 0) == 1536 + 64
    # by hand: value-sorted palette [119, 120, 121, 122]; weights 0..31 -> index 1,
    # 32..47 -> 2, 48..55 -> 0, 56..63 -> 3. Lane l = 16g (row 0) holds weights 16g..16g+15;
    # its two unit dwords pair weight b with b+4 in each byte.
    lanes = {0: [0x11] * 8, 16: [0x11] * 8, 32: [0x22] * 8, 48: [0x00] * 4 + [0x33] * 4}
    for l, exp in lanes.items():
        assert d[1024 + 8 * l: 1024 + 8 * l + 8].tolist() == exp
    # rows 1..15 of the tile do not exist: their bytes are zero
    assert not d[16 * 1: 16 * 16].any() and not d[1024 + 8: 1024 + 8 * 16].any()
    # weight 4 (sm 148: sign 1, mantissa 20) keeps its mantissa and weight 5's sign (sm 185: 1)
    assert d[4] == (20 << 1) | 1 and d[5] == (57 << 1) | 1 and d[0] == 0
    assert d[1536:1544].tolist() == [0] * 8
    assert (dl.rebuild(d, pal_sorted, 1, 64) == w).all()
    assert dl.zero_bytes_ok(d, 1, 64) == []
    assert not dl.raw_masks(d, 1, 64).any()


def test_rebuild_takes_raw_rows_from_the_side_table(golden_dir):
    """Mark row 0's group raw by hand: the reader must take its exponents from the side
    table and ignore the (zero) nibbles."""
    w = _hand_matrix(golden_dir).copy()
    w[0, 7] = (w[0, 7] & 0x807F) | (200 << 7)  # an exponent outside the palette
    pal_sorted = [119, 120, 121, 122]
    d = np.zeros(dl.plane_bytes(1, 64, 1), np.uint8)
    blk = dl.hand_block(_hand_matrix(golden_dir), pal_sorted)
    d[:1536] = blk[:1536]
    for g in range(4):  # a raw row keeps its sign/mantissa bytes; its nibbles are zero
        d[1024 + 8 * (16 * g): 1024 + 8 * (16 * g) + 8] = 0
    d[16 * 0 + 7] = ((int(w[0, 7]) & 0x7F) << 1) | (int(w[0, 6]) >> 15)
    d[16 * 0 + 6] = ((int(w[0, 6]) & 0x7F) << 1) | (int(w[0, 7]) >> 15)
    d[1536:1540] = np.frombuffer(np.uint32(1).tobytes(), np.uint8)  # mask: row 0 raw
    d[1536 + 64:] = ((w[0] >> 7) & 0xFF).astype(np.uint8)
    assert (dl.rebuild(d, pal_sorted, 1, 64) == w).all()
    assert dl.zero_bytes_ok(d, 1, 64) == []
    assert dl.raw_masks(d, 1, 64).tolist() == [[True]]
    # a raw row with a nonzero nibble, or padding that is not zero, is reported
    d2 = d.copy()
    d2[1024] = 1
    assert dl.zero_bytes_ok(d2, 1, 64)
    d3 = d.copy()
    d3[1536 + 9] = 1
    assert dl.zero_bytes_ok(d3, 1, 64)
