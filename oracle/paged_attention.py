"""CPU float64 oracle for paged attention.  TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this module.  The HIP library never calls it.  It shares no
code with the GPU path.

This is the plain definition, written out.  The TileInfer.jl performance page
(section "Fused kernels, FlashAttention and PagedAttention") describes reference
attention ops this way: they gather the pages into dense K and V, then materialise
the scores.  Fused paged flash attention must reach the same result up to rounding
order.  So the oracle:

1. gathers each sequence's keys and values from the pool through its block table;
2. forms every visible score;
3. takes the softmax over them explicitly.

Nothing here is blocked, fused or reordered.  Query rows are independent, and the
oracle may process them in groups only to bound memory.

Readings where the pages are silent (each is also listed in the design notes):

* The softmax scale is ``1/sqrt(D)`` unless one is given.
* GQA uses contiguous groups: query head h reads KV head ``h // (Hq/Hkv)``.
* Query i of a sequence with ``n`` new tokens sits at position ``seq_len - n + i``.
  It sees keys ``j <= pos``.  With a window W > 0 it sees only ``pos - j < W``.
  The Qml-engine announcement lists attention sinks and a sliding window for
  gpt-oss-20b in its model table.
* A sink is one logit per query head, not multiplied by the softmax scale.  It takes
  part in the max and in the denominator only, and carries no value vector.
* INT8 K/V holds one float32 scale per cached (token, KV head) vector, equal to
  absmax/127.  The TileInfer page, section "INT8 KV cache", gives one scale per
  cached vector.  Codes are ``rint(x/scale)`` (ties to even), clamped to +-127.
  An all-zero vector has scale 0 and codes 0.
* Split-KV decode (same page and section as above) splits a sequence's keys into
  ranges ``[iS, (i+1)S)``.  Each split returns ``(o_i, lse_i)`` over its visible keys,
  or ``lse = -inf`` when it has none.  A separate combine merges the splits and
  adds the sink once.
"""
from __future__ import annotations

import math

import numpy as np

from . import tq3

NEG_INF = -math.inf


# ---------------------------------------------------------------------------
# value decoding
# ---------------------------------------------------------------------------

def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> float32 (exact: bf16 is the top half of f32)."""
    b = np.ascontiguousarray(bits).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32)


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    return bf16_to_f32(bits).astype(np.float64)


# ---------------------------------------------------------------------------
# a2: the INT8 quantiser (numpy float32, the precision the stored scale has)
# ---------------------------------------------------------------------------

def smoothing_factors(smooth) -> np.ndarray:
    """The per-channel factors an INT8 cache smooths keys by: for each given weight
    s > 0 (float32, a normal number), the largest power of two not above it,
    2^(e-1) where s = m * 2^e with 0.5 <= m < 1.  A power of two keeps k / s and
    q * s exact (a reading: the page names the key norm's weight as the smoothing,
    not how it is applied)."""
    s = np.asarray(smooth, dtype=np.float32)
    assert np.all(s > 0), "smoothing weights must be positive"
    _, e = np.frexp(s.astype(np.float64))
    return np.ldexp(1.0, e - 1).astype(np.float32)


def quantize_int8(x_bits: np.ndarray, smooth=None):
    """Quantise bf16 vectors along the last axis to int8 codes + one float32 scale.

    Follows the TileInfer page, section "INT8 KV cache": one Int8 scale for each
    cached vector.  The steps, all in IEEE float32:

    * with a per-channel ``smooth`` weight (float32 [D], all > 0), the vector
      quantised is ``x / s`` with s = ``smoothing_factors(smooth)`` (the same
      section smooths keys by the key norm's weight; a query then meets ``q * s``,
      leaving q.k unchanged);
    * ``scale = absmax / 127``;
    * ``code = clamp(rint(x / scale), -127, 127)``, where rint rounds ties to even;
    * an all-zero vector gets scale 0 and codes 0.

    Returns ``(codes int8 [..., D], scale float32 [...])``.
    """
    x = bf16_to_f32(x_bits)
    if smooth is not None:
        x = (x / smoothing_factors(smooth)).astype(np.float32)
    absmax = np.max(np.abs(x), axis=-1)
    scale = (absmax / np.float32(127.0)).astype(np.float32)
    safe = np.where(scale > 0, scale, np.float32(1.0)).astype(np.float32)
    q = np.rint(x / safe[..., None]).astype(np.float32)
    q = np.where(scale[..., None] > 0, q, np.float32(0.0))
    codes = np.clip(q, -127, 127).astype(np.int8)
    return codes, scale


def dequantize_int8(codes: np.ndarray, scale: np.ndarray, smooth=None) -> np.ndarray:
    """code * scale (* s per channel when smoothed, s = smoothing_factors(smooth)),
    exact in float64."""
    x = codes.astype(np.float64) * scale.astype(np.float64)[..., None]
    if smooth is not None:
        x = x * smoothing_factors(smooth).astype(np.float64)
    return x


# ---------------------------------------------------------------------------
# the page pool and a1/a2: writing new tokens
# ---------------------------------------------------------------------------

def empty_pool(num_pages: int, num_kv_heads: int, page_size: int, head_dim: int, kv_dtype: str,
               k_smooth=None):
    """A pool whose every slot is poison.

    BF16 slots hold NaN.  INT8 and 3-bit slots hold code 0 with a NaN scale.
    Layout: ``[num_pages, Hkv, P, D]``; scales ``[num_pages, Hkv, P]``.  A 3-bit
    ("tq3") pool holds packed codes ``[num_pages, Hkv, P, 3D/8]`` (see ``tq3``).  An
    INT8 pool may carry ``k_smooth`` (float32 [D]): its keys are stored smoothed by it.
    """
    shape = (num_pages, num_kv_heads, page_size, head_dim)
    if kv_dtype == "bf16":
        assert k_smooth is None, "key smoothing is an INT8 cache feature"
        return {"k": np.full(shape, 0x7FC0, np.uint16), "v": np.full(shape, 0x7FC0, np.uint16)}
    if kv_dtype == "tq3":
        assert k_smooth is None, "key smoothing is an INT8 cache feature"
        pshape = shape[:3] + (3 * head_dim // 8,)
        return {"k": np.zeros(pshape, np.uint8), "v": np.zeros(pshape, np.uint8),
                "k_scale": np.full(shape[:3], np.nan, np.float32),
                "v_scale": np.full(shape[:3], np.nan, np.float32)}
    pool = {"k": np.zeros(shape, np.int8), "v": np.zeros(shape, np.int8),
            "k_scale": np.full(shape[:3], np.nan, np.float32),
            "v_scale": np.full(shape[:3], np.nan, np.float32)}
    if k_smooth is not None:
        pool["k_smooth"] = np.asarray(k_smooth, dtype=np.float32).copy()
    return pool


def slot_of(block_table_row: np.ndarray, pos: int, page_size: int):
    """(page id, offset in page) of cached position ``pos``."""
    return int(block_table_row[pos // page_size]), pos % page_size


def kv_write(pool: dict, k_new: np.ndarray, v_new: np.ndarray, cu_new: np.ndarray,
             seq_lens: np.ndarray, block_table: np.ndarray, page_size: int, kv_dtype: str):
    """Append tokens to each sequence's pages.  Updates ``pool`` in place.

    Token i of sequence s (rows ``cu_new[s]..cu_new[s+1]`` of ``k_new``/``v_new``,
    bf16 bits ``[T, Hkv, D]``) goes to position ``seq_lens[s] - n_s + i``.  Here
    ``seq_lens`` counts the tokens after the append.  BF16 pools take a copy of the
    bits.  INT8 pools take the quantised codes and scales (keys divided by the
    pool's ``k_smooth`` first, when it has one), 3-bit pools the packed codes and
    scales of ``tq3.quantize_tq3``.  The TileInfer page
    (section "Fused kernels, ...") names the KV write as one of the engine's kernels.
    """
    B = len(seq_lens)
    cu_new = np.asarray(cu_new, dtype=np.int64)
    T = int(cu_new[B])
    tok_seq = np.repeat(np.arange(B), np.diff(cu_new))           # sequence of each new token
    tok_i = np.arange(T) - cu_new[tok_seq]                        # index within its sequence
    n_s = np.diff(cu_new)[tok_seq]
    pos = np.asarray(seq_lens, dtype=np.int64)[tok_seq] - n_s + tok_i
    pg = np.asarray(block_table, dtype=np.int64)[tok_seq, pos // page_size]
    off = pos % page_size
    if kv_dtype == "bf16":
        pool["k"][pg, :, off, :] = k_new[:T]
        pool["v"][pg, :, off, :] = v_new[:T]
    elif kv_dtype == "tq3":
        kc, ks = tq3.quantize_tq3(k_new[:T])
        vc, vs = tq3.quantize_tq3(v_new[:T])
        pool["k"][pg, :, off] = kc
        pool["v"][pg, :, off] = vc
        pool["k_scale"][pg, :, off] = ks
        pool["v_scale"][pg, :, off] = vs
    else:
        kc, ks = quantize_int8(k_new[:T], pool.get("k_smooth"))
        vc, vs = quantize_int8(v_new[:T])
        pool["k"][pg, :, off, :] = kc
        pool["v"][pg, :, off, :] = vc
        pool["k_scale"][pg, :, off] = ks
        pool["v_scale"][pg, :, off] = vs
    return pool


def gather(pool: dict, block_table_row: np.ndarray, n: int, page_size: int, kv_dtype: str):
    """Dense float64 K, V ``[n, Hkv, D]`` of one sequence's first n positions."""
    pages = np.asarray(block_table_row[: -(-n // page_size)], dtype=np.int64)
    pos = np.arange(n)
    pg = pages[pos // page_size]
    off = pos % page_size
    if kv_dtype == "bf16":
        K = bf16_to_f64(pool["k"][pg, :, off, :])
        V = bf16_to_f64(pool["v"][pg, :, off, :])
    elif kv_dtype == "tq3":
        K = tq3.dequantize_tq3(pool["k"][pg, :, off], pool["k_scale"][pg, :, off])
        V = tq3.dequantize_tq3(pool["v"][pg, :, off], pool["v_scale"][pg, :, off])
    else:
        K = dequantize_int8(pool["k"][pg, :, off, :], pool["k_scale"][pg, :, off], pool.get("k_smooth"))
        V = dequantize_int8(pool["v"][pg, :, off, :], pool["v_scale"][pg, :, off])
    return K, V


# ---------------------------------------------------------------------------
# attention, materialised
# ---------------------------------------------------------------------------

def visible_mask(pos: np.ndarray, n_keys: int, window: int) -> np.ndarray:
    """[rows, n_keys] bool: key j is visible to the query at ``pos`` if j <= pos and
    (window == 0 or pos - j < window)."""
    j = np.arange(n_keys)[None, :]
    p = np.asarray(pos)[:, None]
    m = j <= p
    if window > 0:
        m &= (p - j) < window
    return m


def attend(q: np.ndarray, pos: np.ndarray, K: np.ndarray, V: np.ndarray, params,
           key_range=None):
    """Materialised softmax attention for a set of query rows of one sequence.

    q: float64 ``[rows, Hq, D]``; pos: ``[rows]`` positions; K, V: float64
    ``[n_keys, Hkv, D]``.  Returns ``(out [rows, Hq, D], m [rows, Hq], l [rows, Hq])``.

    * ``m`` is the max over the visible scores.  The sink is left out of ``m`` here.
    * ``l`` is the sum of ``exp(x - m)`` over the visible keys.
    * ``out`` includes the sink in its denominator when ``params.sinks`` is set and
      ``key_range`` is None.

    ``key_range=(lo, hi)`` restricts the keys to ``[lo, hi)``, as one split does.
    Then no sink is added, rows with no visible key get ``m = -inf``, ``l = 0`` and
    ``out = 0``.
    """
    Hq, Hkv = params.num_q_heads, params.num_kv_heads
    G = Hq // Hkv
    rows, _, D = q.shape
    n_keys = K.shape[0]
    vis = visible_mask(pos, n_keys, params.window)
    if key_range is not None:
        lo, hi = key_range
        kr = np.zeros(n_keys, bool)
        kr[lo:hi] = True
        vis &= kr[None, :]
    out = np.zeros((rows, Hq, D))
    m_all = np.full((rows, Hq), NEG_INF)
    l_all = np.zeros((rows, Hq))
    use_sink = params.sinks is not None and key_range is None
    has = vis.any(axis=1)
    for h in range(Hq):
        g = h // G
        x = params.sm_scale * (q[:, h, :] @ K[:, g, :].T)          # [rows, n_keys]
        x = np.where(vis, x, NEG_INF)
        m = np.where(has, x.max(axis=1, initial=NEG_INF), NEG_INF)  # max over visible keys (-inf if none)
        M = np.maximum(m, float(params.sinks[h])) if use_sink else m
        Ms = np.where(np.isfinite(M), M, 0.0)
        p = np.where(vis, np.exp(x - Ms[:, None]), 0.0)            # exp(x_j - M)
        Z = p.sum(axis=1)
        if use_sink:
            Z = Z + np.exp(float(params.sinks[h]) - Ms)
        num = p @ V[:, g, :]
        out[:, h, :] = np.where((Z > 0)[:, None], num / np.where(Z > 0, Z, 1.0)[:, None], 0.0)
        ms = np.where(has, m, 0.0)
        m_all[:, h] = m
        l_all[:, h] = np.where(vis, np.exp(x - ms[:, None]), 0.0).sum(axis=1)
    return out, m_all, l_all


def _rows_of(q_bits, cu_q, s):
    return bf16_to_f64(q_bits[int(cu_q[s]):int(cu_q[s + 1])])


def paged_attention(q_bits: np.ndarray, cu_q: np.ndarray, pool: dict, block_table: np.ndarray,
                    seq_lens: np.ndarray, params, rows=None, max_rows_per_chunk=None):
    """Attention of every new query row (``[Tq, Hq, D]`` bf16 bits, offsets ``cu_q``)
    over its sequence's paged K/V.  Decode is the case ``q_len = 1``.

    ``rows`` (optional) lists global query-row indices to compute; the result then
    has one entry per listed row, in that order.  Returns float64.
    """
    Tq, Hq, D = q_bits.shape
    want = np.arange(Tq) if rows is None else np.asarray(rows, dtype=np.int64)
    out = np.zeros((len(want), Hq, D))
    seq_of = np.searchsorted(np.asarray(cu_q[1:]), want, side="right")
    if max_rows_per_chunk is None:
        max_rows_per_chunk = 1 << 30
    for s in np.unique(seq_of):
        s = int(s)
        idx = np.nonzero(seq_of == s)[0]
        n = int(seq_lens[s])
        qlen = int(cu_q[s + 1] - cu_q[s])
        K, V = gather(pool, block_table[s], n, params.page_size, params.kv_dtype)
        local = want[idx] - int(cu_q[s])
        budget = max(1, int(max_rows_per_chunk))
        for c in range(0, len(idx), budget):
            sel = idx[c:c + budget]
            lr = local[c:c + budget]
            qr = bf16_to_f64(q_bits[want[sel]])
            pos = n - qlen + lr
            o, _, _ = attend(qr, pos, K, V, params)
            out[sel] = o
    return out


# ---------------------------------------------------------------------------
# a3/a5 algebra: split partials and the combine
# ---------------------------------------------------------------------------

def split_partials(q_bits: np.ndarray, pool: dict, block_table: np.ndarray,
                   seq_lens: np.ndarray, params, split_keys: int, max_splits: int):
    """Per-split decode partials.  One query per sequence at ``pos = len - 1``.

    Split i of sequence b covers keys ``[i*S, min((i+1)*S, len))``.  It returns the
    normalised partial output ``o[b, h, i]`` and ``lse[b, h, i] = m + ln l`` over its
    visible keys.  A split with no visible key gets ``lse = -inf`` and ``o = 0``.
    Splits at or past ``ceil(len/S)`` are not defined for that sequence.  They are
    left as ``-inf`` and 0.
    """
    B, Hq, D = q_bits.shape
    o = np.zeros((B, Hq, max_splits, D))
    lse = np.full((B, Hq, max_splits), NEG_INF)
    for b in range(B):
        n = int(seq_lens[b])
        K, V = gather(pool, block_table[b], n, params.page_size, params.kv_dtype)
        qr = bf16_to_f64(q_bits[b:b + 1])
        pos = np.array([n - 1])
        for i in range(-(-n // split_keys)):
            oi, mi, li = attend(qr, pos, K, V, params, key_range=(i * split_keys, min((i + 1) * split_keys, n)))
            o[b, :, i, :] = oi[0]
            with np.errstate(divide="ignore"):
                lse[b, :, i] = np.where(li[0] > 0, mi[0] + np.log(np.where(li[0] > 0, li[0], 1.0)), NEG_INF)
    return o, lse


def combine(o_part: np.ndarray, lse_part: np.ndarray, seq_lens: np.ndarray, split_keys: int, sinks=None):
    """Merge split partials.  For each (b, h):

    * ``M = max(max_i lse_i, sink_h)``;
    * ``w_i = exp(lse_i - M)``;
    * ``out = sum_i w_i o_i / (sum_i w_i + exp(sink_h - M))``.

    The sink term appears only when sinks are given.  Only the ``ceil(len/S)``
    splits of each sequence are read.
    """
    B, Hq, _, D = o_part.shape
    out = np.zeros((B, Hq, D))
    for b in range(B):
        ns = -(-int(seq_lens[b]) // split_keys)
        L = lse_part[b, :, :ns]                       # [Hq, ns]
        M = L.max(axis=1)
        if sinks is not None:
            M = np.maximum(M, np.asarray(sinks, np.float64))
        safe = np.where(np.isfinite(M), M, 0.0)
        w = np.where(np.isfinite(L), np.exp(L - safe[:, None]), 0.0)
        Z = w.sum(axis=1)
        if sinks is not None:
            Z = Z + np.exp(np.asarray(sinks, np.float64) - safe)
        num = np.einsum("hs,hsd->hd", w, o_part[b, :, :ns, :])
        out[b] = np.where((Z > 0)[:, None], num / np.where(Z > 0, Z, 1.0)[:, None], 0.0)
    return out


def decode(q_bits: np.ndarray, pool: dict, block_table: np.ndarray, seq_lens: np.ndarray, params):
    """One query per sequence, at ``pos = len - 1``, attending over its whole visible
    cache; ``q_bits`` is ``[B, Hq, D]``.  Returns float64 ``[B, Hq, D]``."""
    B = q_bits.shape[0]
    cu = np.arange(B + 1, dtype=np.int64)
    return paged_attention(q_bits, cu, pool, block_table, seq_lens, params)
