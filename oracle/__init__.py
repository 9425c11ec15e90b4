"""CPU oracle for the Unweight weight format and for Y = X * W^T.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the bench's CPU-baseline
leg use it; the product library never imports, links or calls it. It shares no code
with the HIP library (see oracle.c for the method's steps and their sources in the
Unweight blog post).

Every function here is pinned by tests that do not re-use its own code: exhaustive
bf16 field round trips, a hand-worked bitstream fixture, the RFC 1951 canonical-code
example, brute-force optimal code lengths, the Kraft equality, the entropy bound, the
closed-form exponent law of the synthetic inputs, and exact GEMM special cases. No
function here is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "liboracle.so")
_SRC = os.path.join(_HERE, "oracle.c")

OK, EINVAL, ESHAPE, EFORMAT, ERANGE, ENOSPACE = 0, 1, 2, 3, 4, 5

# header byte offsets of the blob (format version 1)
HEADER_FIELDS = {
    "magic": (0, "<u4"), "version": (4, "<u4"), "N": (8, "<i8"), "K": (16, "<i8"),
    "chunk": (24, "<u4"), "lmax": (28, "<u4"), "n_pal": (32, "<u4"), "n_chunks": (36, "<u4"),
    "n_raw": (72, "<i8"), "total_bits": (80, "<u8"), "off_sm": (88, "<u8"),
    "off_bitmap": (96, "<u8"), "off_rowbase": (104, "<u8"), "off_raw": (112, "<u8"),
    "off_chunk": (120, "<u8"), "off_stream": (128, "<u8"), "bytes_stream": (136, "<u8"),
    "total_bytes": (144, "<u8"), "bitmap_words": (152, "<u4"),
}


def build(force: bool = True) -> str:
    """Compile oracle.c with gcc (plain C11, -O2, no intrinsics)."""
    if force or not os.path.exists(_SO) or os.path.getmtime(_SO) < os.path.getmtime(_SRC):
        tmp = _SO + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _SO)
    return _SO


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            build(force=False)
        lib = ctypes.CDLL(_SO)
        P = ctypes.c_void_p
        i64, u32, u64 = ctypes.c_int64, ctypes.c_uint32, ctypes.c_uint64
        lib.or_split.argtypes = [P, i64, P, P]
        lib.or_join.argtypes = [P, P, i64, P]
        lib.or_palette.argtypes = [P, i64, P, P]
        lib.or_palette.restype = ctypes.c_int
        lib.or_raw_groups.argtypes = [P, i64, i64, P, ctypes.c_int, P, P, P]
        lib.or_raw_groups.restype = i64
        lib.or_code_lengths.argtypes = [P, ctypes.c_int, ctypes.c_int, P]
        lib.or_code_lengths.restype = ctypes.c_int
        lib.or_canonical_codes.argtypes = [P, ctypes.c_int, P]
        lib.or_encode.argtypes = [P, i64, i64, u32, u32, P, ctypes.POINTER(u64)]
        lib.or_encode.restype = ctypes.c_int
        lib.or_decode.argtypes = [P, u64, P, P, P]
        lib.or_decode.restype = ctypes.c_int
        lib.or_gemm_pairs.argtypes = [P, i64, P, i64, i64, P, P, i64, P, P]
        lib.or_gemm.argtypes = [P, P, i64, i64, i64, P, P]
        lib.or_swiglu.argtypes = [P, P, i64, P]
        lib.or_f64_to_bf16.argtypes = [ctypes.c_double]
        lib.or_f64_to_bf16.restype = ctypes.c_uint16
        _lib = lib
    return _lib


def _p(a: np.ndarray | None):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def split(w: np.ndarray):
    w = np.ascontiguousarray(w, dtype=np.uint16)
    sm = np.empty(w.shape, np.uint8)
    e = np.empty(w.shape, np.uint8)
    _load().or_split(_p(w), w.size, _p(sm), _p(e))
    return sm, e


def join(sm: np.ndarray, e: np.ndarray) -> np.ndarray:
    sm = np.ascontiguousarray(sm, dtype=np.uint8)
    e = np.ascontiguousarray(e, dtype=np.uint8)
    w = np.empty(sm.shape, np.uint16)
    _load().or_join(_p(sm), _p(e), sm.size, _p(w))
    return w


def palette(e: np.ndarray):
    """Returns (palette uint8[n_pal], histogram uint64[256])."""
    e = np.ascontiguousarray(e, dtype=np.uint8)
    pal = np.zeros(16, np.uint8)
    hist = np.zeros(256, np.uint64)
    n = _load().or_palette(_p(e), e.size, _p(pal), _p(hist))
    return pal[:n].copy(), hist


def raw_groups(e: np.ndarray, pal: np.ndarray):
    """Returns (bitmap uint32[N, words], row_base uint32[N+1], raw_exp uint8[n_raw, 64])."""
    e = np.ascontiguousarray(e, dtype=np.uint8)
    N, K = e.shape
    words = (K + 2047) // 2048
    p16 = np.zeros(16, np.uint8)
    p16[: len(pal)] = pal
    bitmap = np.zeros((N, words), np.uint32)
    row_base = np.zeros(N + 1, np.uint32)
    lib = _load()
    n_raw = lib.or_raw_groups(_p(e), N, K, _p(p16), len(pal), _p(bitmap), _p(row_base), None)
    raw = np.zeros((max(n_raw, 1), 64), np.uint8)
    lib.or_raw_groups(_p(e), N, K, _p(p16), len(pal), None, None, _p(raw))
    return bitmap, row_base, raw[:n_raw]


def code_lengths(freq, lmax: int = 12) -> np.ndarray:
    f = np.ascontiguousarray(freq, dtype=np.uint64)
    ln = np.zeros(max(len(f), 1), np.uint8)
    rc = _load().or_code_lengths(_p(f), len(f), lmax, _p(ln))
    if rc != 0:
        raise ValueError("no prefix code with these lengths fits lmax")
    return ln[: len(f)]


def canonical_codes(lengths) -> np.ndarray:
    ln = np.ascontiguousarray(lengths, dtype=np.uint8)
    code = np.zeros(max(len(ln), 1), np.uint32)
    _load().or_canonical_codes(_p(ln), len(ln), _p(code))
    return code[: len(ln)]


def encode(w: np.ndarray, chunk: int = 1024, lmax: int = 12) -> np.ndarray:
    w = np.ascontiguousarray(w, dtype=np.uint16)
    N, K = w.shape
    lib = _load()
    need = ctypes.c_uint64(0)
    rc = lib.or_encode(_p(w), N, K, chunk, lmax, None, ctypes.byref(need))
    if rc != ENOSPACE:
        raise ValueError(f"or_encode failed with status {rc}")
    blob = np.zeros(need.value, np.uint8)
    rc = lib.or_encode(_p(w), N, K, chunk, lmax, _p(blob), ctypes.byref(need))
    if rc != OK:
        raise ValueError(f"or_encode failed with status {rc}")
    return blob


def encode_status(w: np.ndarray, chunk: int = 1024, lmax: int = 12) -> int:
    w = np.ascontiguousarray(w, dtype=np.uint16)
    need = ctypes.c_uint64(0)
    N, K = w.shape if w.ndim == 2 else (1, w.size)
    return _load().or_encode(_p(w), N, K, chunk, lmax, None, ctypes.byref(need))


def header(blob: np.ndarray) -> dict:
    b = np.ascontiguousarray(blob, dtype=np.uint8)
    h = {k: int(np.frombuffer(b[o : o + np.dtype(t).itemsize].tobytes(), dtype=t)[0]) for k, (o, t) in HEADER_FIELDS.items()}
    h["palette"] = b[40:56].copy()
    h["code_len"] = b[56:72].copy()
    return h


def decode(blob: np.ndarray, want=("w", "exp", "idx")):
    """Bit-serial decode. Returns a dict with the requested planes: 'w' (uint16 [N,K]),
    'exp' (uint8 [N,K]) and 'idx' (uint8 [N*K/2] nibble plane). Raises on a corrupt blob."""
    b = np.ascontiguousarray(blob, dtype=np.uint8)
    h = header(b)
    N, K = h["N"], h["K"]
    out = {}
    w = np.empty((N, K), np.uint16) if "w" in want else None
    e = np.empty((N, K), np.uint8) if "exp" in want else None
    i = np.empty(N * K // 2, np.uint8) if "idx" in want else None
    rc = _load().or_decode(_p(b), b.size, _p(w), _p(e), _p(i))
    if rc != OK:
        raise ValueError(f"or_decode failed with status {rc}")
    if w is not None:
        out["w"] = w
    if e is not None:
        out["exp"] = e
    if i is not None:
        out["idx"] = i
    return out


def decode_status(blob: np.ndarray) -> int:
    b = np.ascontiguousarray(blob, dtype=np.uint8)
    return _load().or_decode(_p(b), b.size, None, None, None)


def gemm(x: np.ndarray, w: np.ndarray):
    """Y = X * W^T in double on bf16 bit patterns; returns (Y, A) with A = sum |x*w|."""
    x = np.ascontiguousarray(x, dtype=np.uint16)
    w = np.ascontiguousarray(w, dtype=np.uint16)
    M, K = x.shape
    N, K2 = w.shape
    assert K == K2
    y = np.empty((M, N), np.float64)
    a = np.empty((M, N), np.float64)
    _load().or_gemm(_p(x), _p(w), M, N, K, _p(y), _p(a))
    return y, a


def gemm_pairs(x: np.ndarray, w: np.ndarray, m_idx, n_idx):
    """Y[m_idx[t], n_idx[t]] and A for a sample of output elements."""
    x = np.ascontiguousarray(x, dtype=np.uint16)
    w = np.ascontiguousarray(w, dtype=np.uint16)
    mi = np.ascontiguousarray(m_idx, dtype=np.int64)
    ni = np.ascontiguousarray(n_idx, dtype=np.int64)
    y = np.empty(mi.size, np.float64)
    a = np.empty(mi.size, np.float64)
    _load().or_gemm_pairs(_p(x), x.shape[1], _p(w), w.shape[1], x.shape[1], _p(mi), _p(ni), mi.size, _p(y), _p(a))
    return y, a


def swiglu(g: np.ndarray, u: np.ndarray) -> np.ndarray:
    g = np.ascontiguousarray(g, dtype=np.float32)
    u = np.ascontiguousarray(u, dtype=np.float32)
    h = np.empty(g.shape, np.uint16)
    _load().or_swiglu(_p(g), _p(u), g.size, _p(h))
    return h


def f64_to_bf16(x: float) -> int:
    return int(_load().or_f64_to_bf16(float(x)))
