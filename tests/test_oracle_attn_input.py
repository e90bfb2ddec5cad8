"""Pins for the attention-input oracle (RMSNorm + RoPE + KV write from fused qkv).

The checks come from outside the oracle's own code:
* hand-derived values (tests/golden/attn_input.txt);
* the exact float64 definitions of RMSNorm and of a rotation (complex product),
  which the bf16 chain must meet within one bf16 step;
* closed forms: a zero angle leaves the bits unchanged, a power-of-two scale of x
  leaves RMSNorm (eps 0) unchanged;
* a scalar re-implementation in plain Python loops, with its own bf16 rounding,
  that must agree bit for bit with the vectorised oracle.
"""
import math
import os
import struct

import numpy as np
import pytest

import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "attn_input.txt")


def bits_to_float(b):
    return struct.unpack("<f", struct.pack("<I", (int(b) & 0xFFFF) << 16))[0]


def float_to_bf16_scalar(x):
    """Round a float32 value to bf16 bits, nearest even, by integer arithmetic."""
    u = struct.unpack("<I", struct.pack("<f", float(np.float32(x))))[0]
    if (u & 0x7F800000) == 0x7F800000 and (u & 0x7FFFFF):
        return (u >> 16) | 0x40
    lsb = (u >> 16) & 1
    return ((u + 0x7FFF + lsb) >> 16) & 0xFFFF


def f32_bits_of(vals):
    return O.f32_to_bf16(np.asarray(vals, np.float32))


def rand_bits(rng, shape, scale=1.0):
    return O.f32_to_bf16((rng.standard_normal(shape) * scale).astype(np.float32))


# ---------------------------------------------------------------------------

def test_golden_values():
    for line in open(GOLDEN):
        line = line.split("#", 1)[0].strip()
        if not line:
            continue
        f = line.split()
        if f[0] == "rms":
            D, eps = int(f[1]), float(f[2])
            x = np.zeros(D, np.float32)
            xs = [float(t) for t in f[3].split(",")]
            x[:len(xs)] = xs
            want = np.zeros(D, np.uint16)
            ws = [int(t, 16) for t in f[4].split(",")]
            want[:len(ws)] = ws
            got = O.rms_norm_bf16(f32_bits_of(x), f32_bits_of(np.ones(D)), eps)
            assert np.array_equal(got, want), (got, want)
        elif f[0] == "rope":
            c, s = float(f[1]), float(f[2])
            a, b = (float(t) for t in f[3].split(","))
            want = [int(t, 16) for t in f[4].split(",")]
            got = O.rope_bf16(f32_bits_of([a, b]), np.float32([c]), np.float32([s]))
            assert list(got) == want, ([hex(v) for v in got], [hex(v) for v in want])


@pytest.mark.parametrize("D", [64, 128])
def test_rms_norm_within_one_bf16_step_of_exact(D):
    rng = np.random.default_rng(1)
    x = rand_bits(rng, (300, D), 3.0)
    w = O.f32_to_bf16((1 + 0.1 * rng.standard_normal(D)).astype(np.float32))
    eps = 1e-6
    got = O.bf16_to_f64(O.rms_norm_bf16(x, w, eps))
    xf = O.bf16_to_f64(x)
    exact = xf / np.sqrt((xf * xf).mean(axis=-1, keepdims=True) + eps) * O.bf16_to_f64(w)
    step = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(exact), 1e-30))) - 7)   # one bf16 step
    assert np.all(np.abs(got - exact) <= step * 1.0001)
    # and most elements are the exact value correctly rounded
    assert np.mean(O.rms_norm_bf16(x, w, eps) == O.f32_to_bf16(exact.astype(np.float32))) > 0.98


def test_rms_norm_power_of_two_scale_invariance():
    rng = np.random.default_rng(2)
    x = rand_bits(rng, (50, 128))
    w = rand_bits(rng, (128,))
    base = O.rms_norm_bf16(x, w, 0.0)
    for k in (-3, 5):
        xs = O.f32_to_bf16((O.bf16_to_f32(x) * np.float32(2.0 ** k)).astype(np.float32))
        assert np.array_equal(O.rms_norm_bf16(xs, w, 0.0), base)


def test_rope_zero_angle_is_identity():
    rng = np.random.default_rng(3)
    y = rand_bits(rng, (20, 4, 128))
    assert np.array_equal(O.rope_bf16(y, np.ones(64, np.float32), np.zeros(64, np.float32)), y)


def test_rope_is_a_rotation():
    """Against the complex product (a + ib)(c + is) in float64: within one bf16 step."""
    rng = np.random.default_rng(4)
    y = rand_bits(rng, (40, 64), 2.0)
    ang = rng.uniform(-10, 10, (40, 32))
    c, s = np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)
    got = O.bf16_to_f64(O.rope_bf16(y, c, s))
    yf = O.bf16_to_f64(y)
    z = (yf[:, :32] + 1j * yf[:, 32:]) * (c.astype(np.float64) + 1j * s.astype(np.float64))
    exact = np.concatenate([z.real, z.imag], axis=-1)
    step = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(exact), 1e-30))) - 7)
    assert np.all(np.abs(got - exact) <= np.maximum(step * 1.0001, 1e-6))


def brute_force_chain(qkv_bits, qw, kw, eps, table, cu_new, seq_lens, Hq, Hkv, D):
    """The documented chain with scalar float32 operations in plain loops."""
    f = np.float32
    T = qkv_bits.shape[0]
    heads = Hq + 2 * Hkv
    out_q = np.zeros((T, Hq, D), np.uint16)
    out_k = np.zeros((T, Hkv, D), np.uint16)
    out_v = np.zeros((T, Hkv, D), np.uint16)
    for s in range(len(seq_lens)):
        n = int(cu_new[s + 1] - cu_new[s])
        for i in range(n):
            t = int(cu_new[s]) + i
            pos = int(seq_lens[s]) - n + i
            for h in range(heads):
                x = [f(bits_to_float(qkv_bits[t, h * D + d])) for d in range(D)]
                if h >= Hq + Hkv:
                    out_v[t, h - Hq - Hkv] = [qkv_bits[t, h * D + d] for d in range(D)]
                    continue
                w = qw if h < Hq else kw
                groups = []
                for j in range(D // 8):
                    acc = f(x[8 * j] * x[8 * j])
                    for e in range(1, 8):
                        acc = f(acc + f(x[8 * j + e] * x[8 * j + e]))
                    groups.append(acc)
                m = len(groups) // 2
                while m >= 1:
                    groups = [f(groups[j] + groups[j ^ m]) for j in range(len(groups))]
                    m //= 2
                r = f(f(1.0) / f(math.sqrt(f(f(groups[0] / f(D)) + f(eps)))))
                y = [bits_to_float(float_to_bf16_scalar(f(f(x[d] * r) * f(bits_to_float(w[d])))))
                     for d in range(D)]
                half = D // 2
                rot = [0] * D
                for d in range(half):
                    c, sn = f(table[pos, d, 0]), f(table[pos, d, 1])
                    a, b = f(y[d]), f(y[d + half])
                    rot[d] = float_to_bf16_scalar(f(f(a * c) - f(b * sn)))
                    rot[d + half] = float_to_bf16_scalar(f(f(b * c) + f(a * sn)))
                if h < Hq:
                    out_q[t, h] = rot
                else:
                    out_k[t, h - Hq] = rot
    return out_q, out_k, out_v


def test_chain_matches_scalar_brute_force():
    rng = np.random.default_rng(5)
    Hq, Hkv, D = 4, 2, 16
    seq_lens = np.array([5, 3, 9], np.int64)
    cu_new = np.array([0, 2, 5, 6], np.int64)
    T = int(cu_new[-1])
    qkv = rand_bits(rng, (T, (Hq + 2 * Hkv) * D), 2.0)
    qw = O.f32_to_bf16((1 + 0.2 * rng.standard_normal(D)).astype(np.float32))
    kw = O.f32_to_bf16((1 + 0.2 * rng.standard_normal(D)).astype(np.float32))
    table = np.stack([np.cos(rng.uniform(-4, 4, (12, D // 2))), np.sin(rng.uniform(-4, 4, (12, D // 2)))],
                     axis=-1).astype(np.float32)
    got = O.attention_input(qkv, qw, kw, 1e-6, table, cu_new, seq_lens, Hq, Hkv, D)
    want = brute_force_chain(qkv, qw, kw, 1e-6, table, cu_new, seq_lens, Hq, Hkv, D)
    for g, w_, name in zip(got, want, ("q", "k", "v")):
        assert np.array_equal(g, w_), name


def test_positions_follow_the_kv_write_convention():
    seq, pos = O.token_positions(np.array([0, 2, 2, 5]), np.array([10, 4, 3]))
    assert list(seq) == [0, 0, 2, 2, 2] and list(pos) == [8, 9, 0, 1, 2]
