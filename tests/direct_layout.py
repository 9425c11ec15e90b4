"""Test-side reading of the library's direct-palette plane (the load-time form made by
uw_prepare_direct), written from the format text in include/uw.h.

The plane is a GPU operand layout, not a step of the method, so nothing in the oracle
builds it. These helpers only read a plane the library wrote and check it against what
the method fixes (the weights themselves and the raw-group rule): rebuild W from it,
and check the bytes the format says are zero.
"""
from __future__ import annotations

import numpy as np


def plane_bytes(N: int, K: int, n_raw: int) -> int:
    """1536 bytes per (16-row tile, 64-group) block, 8 meta bytes per block rounded up to
    64, then 64 exponent bytes per raw (row, group)."""
    T, G = (N + 15) // 16, K // 64
    return 1536 * T * G + (8 * T * G + 63) // 64 * 64 + 64 * n_raw


def _sections(plane: np.ndarray, N: int, K: int):
    """Blocks are stored group-major (block (t, j) at j*T + t), metas tile-major (at
    t*G + j); both are returned indexed [t][j]."""
    T, G = (N + 15) // 16, K // 64
    nb = 1536 * T * G
    blocks = plane[:nb].reshape(G, T, 1536).transpose(1, 0, 2)
    meta = plane[nb: nb + 8 * T * G].view("<u4").reshape(T, G, 2)
    pad = plane[nb + 8 * T * G: nb + (8 * T * G + 63) // 64 * 64]
    side = plane[nb + (8 * T * G + 63) // 64 * 64:].reshape(-1, 64)
    return T, G, blocks, meta, pad, side


def rebuild(plane: np.ndarray, pal_sorted, N: int, K: int) -> np.ndarray:
    """W [N][K] (bf16 bit patterns) from a direct plane. In block (t, j), lane l = 16g + r
    holds row 16t+r, weights 64j+16g .. +15: weight x takes its mantissa from bits 1..7 of
    its byte and its sign from bit 0 of the byte of weight x^1; its exponent is
    pal_sorted[nibble] (unit dword u of the lane: byte b holds unit weight b in the low
    nibble and b+4 in the high one), or, when bit r of the block's meta mask is set, the
    side-table entry meta.base + (raw rows below r) of the block."""
    plane = np.ascontiguousarray(plane, dtype=np.uint8)
    T, G, blocks, meta, _, side = _sections(plane, N, K)
    pal = np.zeros(16, np.uint16)
    pal[: len(pal_sorted)] = np.asarray(pal_sorted, np.uint16)
    r = np.arange(16)
    g = np.arange(4)
    lanes = (16 * g[None, :] + r[:, None])                      # [r][g]
    smb = blocks[:, :, 0:1024].reshape(T, G, 64, 16)[:, :, lanes, :].astype(np.uint16)  # [T][G][r][g][16]
    units = blocks[:, :, 1024:1536].reshape(T, G, 64, 2, 4)[:, :, lanes]                 # [T][G][r][g][2][4]
    nib = np.concatenate([units & 15, units >> 4], axis=-1).reshape(T, G, 16, 4, 16)     # weight order per unit
    e = pal[nib]
    mask = meta[:, :, 0].astype(np.uint64)
    base = meta[:, :, 1].astype(np.int64)
    rawbit = ((mask[:, :, None] >> r[None, None, :].astype(np.uint64)) & 1).astype(bool)  # [T][G][r]
    below = np.cumsum(rawbit, axis=2) - rawbit
    for t, j, rr in zip(*np.nonzero(rawbit)):
        ent = side[base[t, j] + below[t, j, rr]].astype(np.uint16)
        e[t, j, rr] = ent.reshape(4, 16)
    sign = (smb & 1)[..., np.arange(16) ^ 1]
    w = (sign << 15) | (e << 7) | (smb >> 1)                    # [T][G][r][g][16]
    out = w.transpose(0, 2, 1, 3, 4).reshape(T * 16, K)
    return out[:N].astype(np.uint16)


def zero_bytes_ok(plane: np.ndarray, N: int, K: int) -> list[str]:
    """The bytes the format fixes to zero: rows past N in the last tile, the index nibbles
    of raw rows, and the padding between the meta entries and the side table. Returns the
    list of violations (empty when the plane is well formed)."""
    plane = np.ascontiguousarray(plane, dtype=np.uint8)
    T, G, blocks, meta, pad, _ = _sections(plane, N, K)
    bad = []
    if pad.any():
        bad.append("meta padding not zero")
    lanes_of_row = lambda rr: [16 * g + rr for g in range(4)]
    for rr in range(16 - (T * 16 - N), 16) if T * 16 > N else []:
        for l in lanes_of_row(rr):
            if blocks[T - 1, :, 16 * l: 16 * l + 16].any() or blocks[T - 1, :, 1024 + 8 * l: 1024 + 8 * l + 8].any():
                bad.append(f"row {16 * (T - 1) + rr} past N not zero")
                break
        if (meta[T - 1, :, 0] >> rr & 1).any():
            bad.append(f"row {16 * (T - 1) + rr} past N marked raw")
    t_, j_ = np.nonzero(meta[:, :, 0])
    for t, j in zip(t_, j_):
        m = int(meta[t, j, 0])
        for rr in range(16):
            if m >> rr & 1:
                for l in lanes_of_row(rr):
                    if blocks[t, j, 1024 + 8 * l: 1024 + 8 * l + 8].any():
                        bad.append(f"raw row {16 * t + rr} group {j} has nonzero index nibbles")
    return bad


def raw_masks(plane: np.ndarray, N: int, K: int) -> np.ndarray:
    """bool [N][K/64]: the meta masks read back as (row, group) raw flags."""
    T, G, _, meta, _, _ = _sections(np.ascontiguousarray(plane, dtype=np.uint8), N, K)
    r = np.arange(16, dtype=np.uint64)
    bits = ((meta[:, :, 0].astype(np.uint64)[:, :, None] >> r[None, None, :]) & 1).astype(bool)  # [T][G][r]
    return bits.transpose(0, 2, 1).reshape(T * 16, G)[:N]


def hand_block(w: np.ndarray, pal_sorted) -> np.ndarray:
    """The expected plane of a one-row, 64-weight matrix with no raw group, byte by byte:
    one block (row 0 is lane r = 0 of each lane group g), then 64 meta bytes, all zero
    (an empty mask, side base 0). Used with the hand-derived fixture."""
    assert w.shape == (1, 64)
    out = np.zeros(1536 + 64, np.uint8)
    e = (w[0] >> 7) & 0xFF
    order = {int(v): i for i, v in enumerate(pal_sorted)}
    for x in range(64):
        g, xl = divmod(x, 16)
        l = 16 * g  # row 0
        mant = int(w[0, x]) & 0x7F
        psign = int(w[0, x ^ 1]) >> 15
        out[16 * l + xl] = (mant << 1) | psign
        unit, b = divmod(xl, 8)
        out[1024 + 8 * l + 4 * unit + (b % 4)] |= order[int(e[x])] << (0 if b < 4 else 4)
    return out
