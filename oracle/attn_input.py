"""CPU oracle for the fused attention-input step.  TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this module.  The HIP library never calls it.  It shares no
code with the GPU path.

The TileInfer.jl performance page (section "Fused kernels, FlashAttention and
PagedAttention") lists, among the engine's fused kernels, one for the attention
inputs: q/k RMSNorm, RoPE and the KV-cache write straight from the fused q/k/v
projection, bit-identical to the chain of kernels it replaces (copies, two norms,
two RoPEs, one write).  This module is that chain, one op after another, each op
reading bf16 and writing bf16.  Inside an op the arithmetic is IEEE float32, with
every product and sum rounded on its own (no fused multiply-add), in the order
written below.  The page fixes the bf16 hand-offs; the float32 order inside an op
is this module's reading, and the HIP kernel follows the same one.

* RMSNorm of one head vector x (D elements), weight w (bf16, D), epsilon eps:
    sq_d  = x_d * x_d
    g_j   = sum of sq over d = 8j .. 8j+7, added left to right       (j < D/8)
    ss    = the D/8 group sums added pairwise: at each step, entry j
            takes g_j + g_(j xor m), for m = D/16, D/32, ..., 1; then entry 0
    r     = 1 / sqrt(ss / D + eps)      (correctly rounded sqrt and divide)
    y_d   = bf16( (x_d * r) * w_d )     (round to nearest even)
* RoPE, rotate-half pairing (i < D/2), with (c, s) = table[pos][i]:
    out_i       = bf16( a*c - b*s ),   a = y_i, b = y_(i+D/2)
    out_(i+D/2) = bf16( b*c + a*s )
  The cos/sin table is an input, as a model holds it.
* q heads: RMSNorm with q_norm_w, then RoPE -> q out.  k heads: RMSNorm with
  k_norm_w, then RoPE -> the cache.  v heads: copied.  The qkv row of a token is
  [Hq heads | Hkv heads | Hkv heads] x D.  Token i of sequence s sits at position
  seq_lens[s] - n_s + i, as in the KV write.
"""
from __future__ import annotations

import numpy as np

from .paged_attention import bf16_to_f32, kv_write

F32 = np.float32


def f32_to_bf16(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bits, round to nearest even (NaN stays a quiet NaN)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    nan = np.isnan(np.asarray(x, dtype=np.float32))
    out = rounded.astype(np.uint16)
    out = np.where(nan, ((u >> np.uint64(16)) | np.uint64(0x40)).astype(np.uint16), out)
    return out


def rms_norm_bf16(x_bits: np.ndarray, w_bits: np.ndarray, eps: float) -> np.ndarray:
    """RMSNorm over the last axis (D), bf16 in and out, the float32 order above."""
    x = bf16_to_f32(x_bits)
    D = x.shape[-1]
    assert D % 8 == 0 and (D // 8) & (D // 8 - 1) == 0, "D/8 must be a power of two"
    sq = (x * x).astype(F32)
    g = sq[..., 0::8].copy()
    for k in range(1, 8):                      # each group left to right
        g = (g + sq[..., k::8]).astype(F32)
    n = D // 8
    m = n // 2
    while m >= 1:                              # pairwise: g_j + g_(j xor m)
        idx = np.arange(n) ^ m
        g = (g + g[..., idx]).astype(F32)
        m //= 2
    ss = g[..., 0]
    mean = (ss / F32(D)).astype(F32)
    r = (F32(1.0) / np.sqrt((mean + F32(eps)).astype(F32))).astype(F32)
    w = bf16_to_f32(w_bits)
    y = ((x * r[..., None]).astype(F32) * w).astype(F32)
    return f32_to_bf16(y)


def rope_bf16(y_bits: np.ndarray, cos: np.ndarray, sin: np.ndarray) -> np.ndarray:
    """Rotate-half RoPE over the last axis: cos/sin broadcast against [..., D/2]."""
    y = bf16_to_f32(y_bits)
    h = y.shape[-1] // 2
    a, b = y[..., :h], y[..., h:]
    c = np.asarray(cos, dtype=F32)
    s = np.asarray(sin, dtype=F32)
    lo = ((a * c).astype(F32) - (b * s).astype(F32)).astype(F32)
    hi = ((b * c).astype(F32) + (a * s).astype(F32)).astype(F32)
    return f32_to_bf16(np.concatenate([lo, hi], axis=-1))


def token_positions(cu_new: np.ndarray, seq_lens: np.ndarray):
    """(sequence, position) of every new token: token i of s at seq_lens[s] - n_s + i."""
    cu_new = np.asarray(cu_new, dtype=np.int64)
    B = len(seq_lens)
    T = int(cu_new[B])
    tok_seq = np.repeat(np.arange(B), np.diff(cu_new))
    tok_i = np.arange(T) - cu_new[tok_seq]
    n_s = np.diff(cu_new)[tok_seq]
    return tok_seq, np.asarray(seq_lens, dtype=np.int64)[tok_seq] - n_s + tok_i


def attention_input(qkv_bits: np.ndarray, q_norm_w: np.ndarray, k_norm_w: np.ndarray, eps: float,
                    rope_table: np.ndarray, cu_new: np.ndarray, seq_lens: np.ndarray,
                    num_q_heads: int, num_kv_heads: int, head_dim: int):
    """The chain on every new token.

    qkv_bits [T, (Hq + 2 Hkv) * D] bf16 bits; rope_table [max_pos, D/2, 2] float32
    holding (cos, sin).  Returns (q_out, k, v) as bf16 bits [T, H, D].
    """
    T = qkv_bits.shape[0]
    Hq, Hkv, D = num_q_heads, num_kv_heads, head_dim
    x = qkv_bits.reshape(T, Hq + 2 * Hkv, D)
    _, pos = token_positions(cu_new, seq_lens)
    cs = np.asarray(rope_table, dtype=F32)[pos]                # [T, D/2, 2]
    cos, sin = cs[:, None, :, 0], cs[:, None, :, 1]
    q = rope_bf16(rms_norm_bf16(x[:, :Hq], q_norm_w, eps), cos, sin)
    k = rope_bf16(rms_norm_bf16(x[:, Hq:Hq + Hkv], k_norm_w, eps), cos, sin)
    v = x[:, Hq + Hkv:].copy()
    return q, k, v


def attention_input_to_pool(pool: dict, qkv_bits, q_norm_w, k_norm_w, eps, rope_table, cu_new,
                            seq_lens, block_table, num_q_heads, num_kv_heads, head_dim, page_size,
                            kv_dtype):
    """The chain, then the KV write of k and v into ``pool`` (in place).  Returns q_out."""
    q, k, v = attention_input(qkv_bits, q_norm_w, k_norm_w, eps, rope_table, cu_new, seq_lens,
                              num_q_heads, num_kv_heads, head_dim)
    kv_write(pool, k, v, cu_new, seq_lens, block_table, page_size, kv_dtype)
    return q
