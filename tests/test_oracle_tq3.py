"""Pins for the 3-bit rotated KV oracle (Walsh-Hadamard rotation + 8-level Lloyd-Max).

Each test ties the oracle to something other than itself: Max's published table,
quadrature of the normal density, the Hadamard matrix from scipy, closed forms,
brute force and symmetries.
"""
import math
import os

import numpy as np
import pytest
import scipy.integrate
import scipy.linalg

import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "lloyd_max_normal8.txt")


def _golden():
    out = {}
    for line in open(GOLDEN):
        line = line.strip()
        if line and not line.startswith("#"):
            k, *v = line.split()
            out[k] = np.array([float(x) for x in v])
    return out


def _bf16_bits(x):
    """float32 -> bf16 bits, round to nearest even."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def _phi(x):
    return math.exp(-0.5 * x * x) / math.sqrt(2 * math.pi)


def test_codebook_matches_max_table():
    g = _golden()
    M, T = O.lloyd_max_normal()
    assert np.allclose(M, g["levels"], atol=6e-4)
    assert np.allclose(np.concatenate([[0.0], T]), g["thresholds"], atol=6e-4)


def test_codebook_is_a_fixed_point_by_quadrature():
    """Levels are the centroids of their cells, and the distortion is Max's."""
    M, T = O.lloyd_max_normal()
    edges = [0.0] + list(T) + [math.inf]
    mse = 0.0
    for k in range(4):
        mass = scipy.integrate.quad(_phi, edges[k], edges[k + 1])[0]
        first = scipy.integrate.quad(lambda x: x * _phi(x), edges[k], edges[k + 1])[0]
        assert abs(first / mass - M[k]) < 1e-9
        mse += 2 * scipy.integrate.quad(lambda x: (x - M[k]) ** 2 * _phi(x), edges[k], edges[k + 1])[0]
    assert abs(mse - _golden()["mse"][0]) < 1e-4
    assert np.allclose(T, 0.5 * (M[:-1] + M[1:]), rtol=0, atol=0)


def test_codebook_f32_is_far_from_rounding_boundaries():
    """Any converged float64 iteration rounds to the same float32 codebook."""
    M, T = O.lloyd_max_normal()
    for v in list(M) + list(T):
        f = np.float32(v)
        ulp = float(np.spacing(f))
        assert abs(v - float(f)) < 0.49 * ulp
        assert 0.5 * ulp - abs(v - float(f)) > 0.01 * ulp


@pytest.mark.parametrize("D", [8, 64, 128])
def test_fwht_matches_hadamard_matrix(D):
    rng = np.random.default_rng(D)
    H = scipy.linalg.hadamard(D)
    xi = rng.integers(-50, 50, size=(7, D)).astype(np.float32)      # exact in float32
    assert np.array_equal(O.fwht_f32(xi), (xi.astype(np.int64) @ H.T).astype(np.float32))
    assert np.array_equal(O.fwht_f32(O.fwht_f32(xi)), D * xi)        # H H = D I
    xf = rng.standard_normal((5, D)).astype(np.float32)
    assert np.allclose(O.fwht_f32(xf), xf.astype(np.float64) @ H.T, rtol=1e-5, atol=1e-4)


def test_sum_squares_against_float64():
    rng = np.random.default_rng(1)
    yi = rng.integers(-100, 100, size=(4, 128)).astype(np.float32)
    assert np.array_equal(O.sum_squares_f32(yi), (yi.astype(np.int64) ** 2).sum(-1).astype(np.float32))
    yf = rng.standard_normal((9, 64)).astype(np.float32) * 10
    assert np.allclose(O.sum_squares_f32(yf), (yf.astype(np.float64) ** 2).sum(-1), rtol=1e-6)


@pytest.mark.parametrize("D", [64, 128])
def test_quantiser_against_brute_force(D):
    """Codes are the nearest of the 8 levels to y / rms(y), computed in float64 from
    the Hadamard matrix (elements within 1e-5 of a cell edge are skipped), and the
    scale is ||x||."""
    rng = np.random.default_rng(D + 3)
    bits = _bf16_bits(rng.standard_normal((300, D)).astype(np.float32) * rng.uniform(0.01, 10, (300, 1)))
    packed, scale = O.quantize_tq3(bits)
    codes = O.unpack_codes(packed)
    x = O.bf16_to_f64(bits)
    y = x @ scipy.linalg.hadamard(D).T
    rms = np.sqrt((y ** 2).mean(-1))
    assert np.allclose(scale, np.linalg.norm(x, axis=-1), rtol=1e-6)
    assert np.allclose(scale, rms, rtol=1e-6)
    t = y / rms[:, None]
    M, T = O.codebook_f32()
    lev = np.concatenate([-M[::-1], M]).astype(np.float64)           # ascending, 8 levels
    nearest = np.abs(t[..., None] - lev).argmin(-1)                  # 0..7
    brute = np.where(nearest >= 4, 4 + (nearest - 4), 3 - nearest)  # sign-magnitude
    edges = np.concatenate([-T[::-1], [0.0], T]).astype(np.float64)
    clear = np.abs(t[..., None] - edges).min(-1) > 1e-5
    assert clear.mean() > 0.99
    assert np.array_equal(codes[clear], brute[clear])


def test_zero_vector():
    packed, scale = O.quantize_tq3(np.zeros((2, 128), np.uint16))
    assert np.all(scale == 0)
    assert np.all(O.unpack_codes(packed) == 4)                      # t = 0: positive, magnitude 0
    assert np.all(O.dequantize_tq3(packed, scale) == 0)


@pytest.mark.parametrize("k", [0, 5, 127])
def test_spike_reconstructs_closed_form(k):
    """x = a e_k rotates to +-a in every coordinate, so |t| = 1 and every element
    takes the magnitude M[1] (T[0] < 1 < T[1]); dequantising gives M[1] a e_k."""
    a = np.float32(-3.5)
    x = np.zeros((1, 128), np.float32)
    x[0, k] = a
    packed, scale = O.quantize_tq3(_bf16_bits(x))
    assert np.all(O.unpack_codes(packed) & 3 == 1)
    M, _ = O.codebook_f32()
    expect = np.zeros(128)
    expect[k] = float(M[1]) * float(a)
    assert np.allclose(O.dequantize_tq3(packed, scale)[0], expect, atol=1e-6)


def test_sign_symmetry():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((50, 128)).astype(np.float32)
    pa, sa = O.quantize_tq3(_bf16_bits(x))
    pb, sb = O.quantize_tq3(_bf16_bits(-x))
    assert np.array_equal(sa, sb)
    assert np.array_equal(O.unpack_codes(pb), O.unpack_codes(pa) ^ 4)


def test_packed_codes_roundtrip_and_layout():
    rng = np.random.default_rng(6)
    codes = rng.integers(0, 8, size=(3, 5, 128)).astype(np.uint8)
    packed = O.pack_codes(codes)
    assert packed.shape == (3, 5, 48)
    assert np.array_equal(O.unpack_codes(packed), codes)
    # element 8j+i sits in bits 3i .. 3i+2 of the little-endian 24-bit field j
    one = np.zeros(128, np.uint8)
    one[8 * 3 + 5] = 6                                               # field 3, bits 15..17 = 0b110
    p = O.pack_codes(one)
    field = int(p[9]) | (int(p[10]) << 8) | (int(p[11]) << 16)
    assert field == 6 << 15
    assert p.sum() == p[9] + p[10] + p[11]


def test_gaussian_round_trip_distortion():
    """Rotated Gaussian vectors are Gaussian, so the relative error of the round
    trip is the quantiser's distortion, 0.0345 (Max's table), up to sampling."""
    rng = np.random.default_rng(7)
    bits = _bf16_bits(rng.standard_normal((3000, 128)).astype(np.float32))
    packed, scale = O.quantize_tq3(bits)
    x = O.bf16_to_f64(bits)
    err = ((O.dequantize_tq3(packed, scale) - x) ** 2).sum() / (x ** 2).sum()
    assert 0.031 < err < 0.037


def test_pool_write_and_gather():
    """A tq3 pool written through kv_write gathers to the dequantised vectors."""
    rng = np.random.default_rng(8)
    P, Hkv, D = 16, 2, 64
    pool = O.empty_pool(8, Hkv, P, D, "tq3")
    k = _bf16_bits(rng.standard_normal((20, Hkv, D)).astype(np.float32))
    v = _bf16_bits(rng.standard_normal((20, Hkv, D)).astype(np.float32))
    bt = np.array([[3, 1, 6, 0, 0, 0, 0, 0]], np.int32)
    O.kv_write(pool, k, v, np.array([0, 20]), np.array([20]), bt, P, "tq3")
    K, V = O.gather(pool, bt[0], 20, P, "tq3")
    kp, ks = O.quantize_tq3(k)
    vp, vs = O.quantize_tq3(v)
    assert np.array_equal(K, O.dequantize_tq3(kp, ks))
    assert np.array_equal(V, O.dequantize_tq3(vp, vs))
    assert np.all(np.isnan(pool["k_scale"][2]))                      # untouched pages keep poison
