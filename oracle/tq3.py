"""3-bit rotated KV cache: CPU oracle.  TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this module.  The HIP library never calls it, and it shares
no code, table or constant generator with the GPU path.

The qengine README's feature list names a 3-bit KV cache built from a
Walsh-Hadamard rotation followed by a Lloyd-Max scalar quantiser, and says no more.
Every detail below is a reading of that one line, chosen as the plainest that
works (each is also listed in the design notes):

* The rotation is the Walsh-Hadamard transform over the head dimension D, in
  Sylvester order and unnormalised: ``y = H_D x``.  ``H_D H_D = D I``, so the
  inverse is ``H_D / D``.
* Each cached (token, KV head) vector, K and V alike, keeps one float32 scale: the
  RMS of ``y``, ``s = sqrt(sum(y^2) / D)`` (equal to ``||x||``).  So ``y / s`` has
  unit mean square, the variance the quantiser is designed for.
* The quantiser is the 8-level Lloyd-Max (minimum mean-square error) quantiser of
  the unit normal distribution: the fixed point of Lloyd's two conditions
  (thresholds at midpoints of adjacent levels, levels at the centroids of their
  cells).  It is symmetric: levels ``+-M[0..3]`` and thresholds ``0, +-T[0..2]``.
* Codes are sign-magnitude: bits 0-1 hold the index m of the magnitude M[m]
  (ascending), bit 2 is 1 for a positive level.  ``t = y/s >= 0`` counts as
  positive, and ``m = #{k : |t| >= T[k]}``.  A zero vector (s = 0) takes t = 0.
* The codes of a vector are stored as D/8 little-endian 24-bit fields, 3 bytes
  each: field j holds elements 8j .. 8j+7, element 8j+i in bits 3i .. 3i+2.
* The decisions (codes and the stored scale) are made in float32, in a fixed order
  of operations, so that a GPU quantiser can match them bit for bit: the rotation
  by butterflies of stride 1, 2, 4, ..., D/2 (each ``(a + b, a - b)``); the sum of
  squares over consecutive groups of 8 elements, each group summed in order, then
  the group sums added in a pairwise tree (partner ``g ^ 1``, then ``g ^ 2``, ...);
  the scale by a correctly rounded square root; ``t`` by a correctly rounded
  division.  The codebook enters as float32 values: each M[m] and each T[k]
  (midpoint of the float64 levels) rounded to nearest.
* The dequantised vector is ``x^ = H_D (s * c) / D`` with ``c = +-M[m]``, in float64.

The cache is then attended exactly like the BF16 and INT8 caches: ``gather`` in
``paged_attention`` dequantises it densely.
"""
from __future__ import annotations

import functools
import math

import numpy as np
import scipy.linalg

LEVELS = 8


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> float32 (exact)."""
    b = np.ascontiguousarray(bits).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32)


# ---------------------------------------------------------------------------
# the codebook
# ---------------------------------------------------------------------------

def _phi(x: float) -> float:
    return 0.0 if math.isinf(x) else math.exp(-0.5 * x * x) / math.sqrt(2.0 * math.pi)


def _cdf(x: float) -> float:
    return 0.5 * (1.0 + math.erf(x / math.sqrt(2.0)))


@functools.lru_cache(maxsize=None)
def lloyd_max_normal(iters: int = 100000, tol: float = 1e-13):
    """The symmetric 8-level Lloyd-Max quantiser of N(0, 1), in float64.

    Lloyd's iteration on the positive half: thresholds are the midpoints of
    adjacent levels (the first one is 0, the last +inf), and each level moves to the
    centroid of its cell, ``E[X | a < X < b] = (phi(a) - phi(b)) / (Phi(b) - Phi(a))``.
    Starts from the evenly spaced levels 0.25, 0.75, 1.25, 2.0 and stops when no
    level moves by more than ``tol`` (about 200 steps; the float64 centroids stop
    improving near 3e-15).  Every float32 rounding of the result lies more than 0.02
    ulp from a rounding boundary, so any converged float64 iteration rounds the same.
    Returns ``(M [4] ascending, T [3])``.
    """
    half = LEVELS // 2
    m = [0.25, 0.75, 1.25, 2.0]
    for _ in range(iters):
        edges = [0.0] + [0.5 * (m[k] + m[k + 1]) for k in range(half - 1)] + [math.inf]
        new = [(_phi(edges[k]) - _phi(edges[k + 1])) / (_cdf(edges[k + 1]) - _cdf(edges[k]))
               for k in range(half)]
        moved = max(abs(a - b) for a, b in zip(new, m))
        m = new
        if moved <= tol:
            break
    M = np.array(m, dtype=np.float64)
    T = 0.5 * (M[:-1] + M[1:])
    M.flags.writeable = False
    T.flags.writeable = False
    return M, T


def codebook_f32():
    """The codebook as the quantiser uses it: float32 M [4] and T [3]."""
    M, T = lloyd_max_normal()
    return M.astype(np.float32), T.astype(np.float32)


# ---------------------------------------------------------------------------
# the quantiser (float32 decisions in a fixed order)
# ---------------------------------------------------------------------------

def fwht_f32(x: np.ndarray) -> np.ndarray:
    """Unnormalised Walsh-Hadamard transform along the last axis, in float32, by
    butterflies of stride 1, 2, ..., D/2: elements e (stride bit clear) and e + h
    become (x_e + x_{e+h}, x_e - x_{e+h})."""
    y = np.array(x, dtype=np.float32, copy=True)
    D = y.shape[-1]
    h = 1
    while h < D:
        v = y.reshape(y.shape[:-1] + (D // (2 * h), 2, h))
        a = v[..., 0, :].copy()
        b = v[..., 1, :].copy()
        v[..., 0, :] = a + b
        v[..., 1, :] = a - b
        h *= 2
    return y


def sum_squares_f32(y: np.ndarray) -> np.ndarray:
    """Sum of squares along the last axis in float32: groups of 8 consecutive
    elements summed in order (each square rounded, then added), then the group
    sums in a pairwise tree (g + (g ^ 1), then g + (g ^ 2), ...)."""
    y = np.asarray(y, dtype=np.float32)
    D = y.shape[-1]
    g = y.reshape(y.shape[:-1] + (D // 8, 8))
    s = g[..., 0] * g[..., 0]
    for i in range(1, 8):
        s = s + g[..., i] * g[..., i]
    n = D // 8
    idx = np.arange(n)
    step = 1
    while step < n:
        s = s + s[..., idx ^ step]
        step *= 2
    return s[..., 0]


def quantize_tq3(x_bits: np.ndarray, codebook=None):
    """Quantise bf16 vectors (uint16 bits) along the last axis.

    Returns ``(packed uint8 [..., 3D/8], scale float32 [...])``.
    """
    M, T = codebook_f32() if codebook is None else codebook
    x = bf16_to_f32(np.asarray(x_bits, dtype=np.uint16))
    D = x.shape[-1]
    y = fwht_f32(x)
    ss = sum_squares_f32(y)
    scale = np.sqrt(ss / np.float32(D)).astype(np.float32)
    with np.errstate(invalid="ignore", divide="ignore"):
        t = (y / scale[..., None]).astype(np.float32)
    t = np.where(scale[..., None] == 0, np.float32(0), t)
    sign = (t >= 0).astype(np.uint8)
    a = np.abs(t)
    mag = ((a >= T[0]).astype(np.uint8) + (a >= T[1]).astype(np.uint8) + (a >= T[2]).astype(np.uint8))
    codes = (mag | (sign << 2)).astype(np.uint8)
    return pack_codes(codes), scale


def pack_codes(codes: np.ndarray) -> np.ndarray:
    """3-bit codes [..., D] -> packed bytes [..., 3D/8]: field j (bytes 3j .. 3j+2,
    little-endian) holds element 8j+i in bits 3i .. 3i+2."""
    codes = np.asarray(codes, dtype=np.uint8)
    D = codes.shape[-1]
    c = codes.reshape(codes.shape[:-1] + (D // 8, 8)).astype(np.uint32)
    field = np.zeros(c.shape[:-1], dtype=np.uint32)
    for i in range(8):
        field |= c[..., i] << np.uint32(3 * i)
    out = np.stack([(field >> np.uint32(8 * k)) & np.uint32(0xFF) for k in range(3)], axis=-1)
    return out.astype(np.uint8).reshape(codes.shape[:-1] + (3 * D // 8,))


def unpack_codes(packed: np.ndarray) -> np.ndarray:
    """Packed bytes [..., 3D/8] -> 3-bit codes [..., D]."""
    packed = np.asarray(packed, dtype=np.uint8)
    n = packed.shape[-1] // 3
    b = packed.reshape(packed.shape[:-1] + (n, 3)).astype(np.uint32)
    field = b[..., 0] | (b[..., 1] << np.uint32(8)) | (b[..., 2] << np.uint32(16))
    codes = np.stack([(field >> np.uint32(3 * i)) & np.uint32(7) for i in range(8)], axis=-1)
    return codes.astype(np.uint8).reshape(packed.shape[:-1] + (8 * n,))


def dequantize_tq3(packed: np.ndarray, scale: np.ndarray, codebook=None) -> np.ndarray:
    """``x^ = H_D (s * c) / D`` in float64, with ``c = +-M[m]`` from the codes."""
    M, _ = codebook_f32() if codebook is None else codebook
    codes = unpack_codes(packed)
    D = codes.shape[-1]
    mag = M.astype(np.float64)[codes & 3]
    c = np.where((codes >> 2) & 1, mag, -mag)
    z = np.asarray(scale, dtype=np.float64)[..., None] * c
    H = scipy.linalg.hadamard(D).astype(np.float64)
    return (z @ H) / D          # H is symmetric
