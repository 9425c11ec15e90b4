"""Seeded synthetic inputs shared by the oracle tests, the GPU parity tests and the bench.

This module only draws random numbers and rounds them to bf16 bit patterns. It holds
none of the compression method's arithmetic (no palette, no raw-row rule, no Huffman
code, no GEMM), so both the CPU oracle and the HIP library can be fed from it without
sharing any of the method's code.

The workloads stand in for the trained Llama-3.1-8B MLP weights the Unweight blog post
measures on ("How weights compress" and "Bundles and results" sections): same shapes,
a Gaussian (or Student-t for the 70B-shaped layer) value law whose bf16 exponent
distribution is as skewed as the post describes, plus injected outliers that push a
few exponents outside the top-16 palette.
"""
from __future__ import annotations

import dataclasses

import numpy as np

__all__ = [
    "CONFIGS",
    "Config",
    "f32_to_bf16_bits",
    "bf16_bits_to_f32",
    "gen_weight",
    "gen_x",
    "gen_stack_sigmas",
    "weight_shapes",
]


@dataclasses.dataclass(frozen=True)
class Config:
    """One synthetic workload.

    cfg_id is the integer fed to the seed sequence; law is "normal" or "t4";
    outlier_frac is the fraction of single elements pushed by 2**(+/-outlier_k)
    (law "normal"), outlier_group_frac the fraction of 64-element row groups that
    receive one such element (law "t4").
    """

    name: str
    cfg_id: int
    shapes: tuple  # ((proj_name, N, K), ...)
    sigma: float
    law: str
    outlier_frac: float
    outlier_group_frac: float
    outlier_k: int
    Ms: tuple
    layers: int = 1


CONFIGS = {
    "tiny": Config("tiny", 1, (("w", 512, 256),), 0.02, "normal", 0.0005, 0.0, 12, (4,)),
    "gate": Config("gate", 2, (("gate", 14336, 4096),), 0.02, "normal", 0.0001, 0.0, 10, (1, 16, 64)),
    "down": Config("down", 3, (("down", 4096, 14336),), 0.015, "normal", 0.0001, 0.0, 10, (256, 1024, 4096)),
    "stack": Config(
        "stack",
        4,
        (("gate", 14336, 4096), ("up", 14336, 4096), ("down", 4096, 14336)),
        0.02,
        "normal",
        0.0,
        0.0,
        0,
        tuple(2**i for i in range(13)),
        layers=32,
    ),
    "70b": Config(
        "70b",
        5,
        (("gate", 28672, 8192), ("up", 28672, 8192), ("down", 8192, 28672)),
        0.01,
        "t4",
        0.0,
        0.01,
        12,
        (1, 64, 512, 2048),
    ),
}

_PROJ_ID = {"w": 0, "gate": 0, "up": 1, "down": 2}


def weight_shapes(cfg: Config):
    return {name: (n, k) for name, n, k in cfg.shapes}


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit pattern (uint16), round to nearest even on the bit pattern.

    NaN inputs are not produced by the generators, so no NaN quieting is done here.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    # u + 0x7FFF + lsb stays below 2^32 for every non-NaN pattern (the largest, -inf, is
    # 0xFF800000), so 32-bit arithmetic is exact here
    r = (u >> 16) & 1
    r += u
    r += 0x7FFF
    r >>= 16
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _shift_exponent(bits: np.ndarray, pos: np.ndarray, up: np.ndarray, k: int) -> None:
    """Multiply the selected bf16 elements by 2**(+k) or 2**(-k) by moving the exponent
    field. The field is kept inside [1, 254] so a finite normal value stays finite and
    normal (zero and subnormal inputs are not expected from a continuous law)."""
    w = bits[pos].astype(np.int32)
    e = (w >> 7) & 0xFF
    e2 = np.clip(np.where(up, e + k, e - k), 1, 254)
    bits[pos] = ((w & ~(0xFF << 7)) | (e2 << 7)).astype(np.uint16)


def gen_weight(cfg: Config, proj: str, layer: int = 0, sigma: float | None = None) -> np.ndarray:
    """Weight matrix W[N][K] as bf16 bit patterns (uint16), PyTorch Linear layout."""
    n, k = weight_shapes(cfg)[proj]
    rng = np.random.default_rng(np.random.SeedSequence([0, cfg.cfg_id, layer, _PROJ_ID[proj]]))
    s = cfg.sigma if sigma is None else sigma
    if cfg.law == "normal":
        w = rng.standard_normal((n, k), dtype=np.float32)
        w *= np.float32(s)
    elif cfg.law == "t4":
        w = (rng.standard_t(4, size=(n, k)) * s).astype(np.float32)
    else:
        raise ValueError(cfg.law)
    bits = f32_to_bf16_bits(w).reshape(-1)
    del w
    total = n * k
    if cfg.outlier_frac > 0:
        cnt = int(round(cfg.outlier_frac * total))
        pos = rng.choice(total, size=cnt, replace=False)
        up = rng.integers(0, 2, size=cnt).astype(bool)
        _shift_exponent(bits, pos, up, cfg.outlier_k)
    if cfg.outlier_group_frac > 0:
        groups = total // 64
        cnt = int(round(cfg.outlier_group_frac * groups))
        g = rng.choice(groups, size=cnt, replace=False)
        off = rng.integers(0, 64, size=cnt)
        up = rng.integers(0, 2, size=cnt).astype(bool)
        _shift_exponent(bits, g * 64 + off, up, cfg.outlier_k)
    return bits.reshape(n, k)


def gen_stack_sigmas(cfg: Config) -> np.ndarray:
    """Per-layer sigma of the 32-layer stack: 0.02 * U(0.8, 1.2), one draw per layer,
    shared by the layer's gate, up and down projections."""
    rng = np.random.default_rng(np.random.SeedSequence([0, cfg.cfg_id, 999]))
    return cfg.sigma * rng.uniform(0.8, 1.2, size=cfg.layers)


def gen_x(cfg: Config, M: int, K: int) -> np.ndarray:
    """Activations X[M][K] ~ N(0, 1) as bf16 bit patterns (uint16)."""
    rng = np.random.default_rng(np.random.SeedSequence([0, cfg.cfg_id, 1000 + M, K]))
    return f32_to_bf16_bits(rng.standard_normal((M, K), dtype=np.float32))
