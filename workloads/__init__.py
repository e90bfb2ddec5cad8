"""Seeded synthetic inputs for paged attention, shaped like the workloads of the
TileInfer.jl performance page (Qwen3-4B attention at 1k/8k/32k positions) and the
model table of the Qml-engine announcement (Llama-3.1-8B, Qwen3-30B-A3B,
gpt-oss-20b attention shapes).

This module holds no attention arithmetic: it draws random numbers, rounds them to
bfloat16 bit patterns, draws sequence lengths and assigns pool pages to sequences.
Writing tokens into pages, quantising, and attending are done separately by the
CPU oracle (``oracle/``) and by the HIP library; both consume what is built here.

Every array is numpy.  bfloat16 tensors are carried as ``uint16`` bit patterns.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

BF16_NAN = np.uint16(0x7FC0)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); return bit patterns."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    t = b >> np.uint32(16)
    t &= np.uint32(1)
    t += np.uint32(0x7FFF)
    t += b
    t >>= np.uint32(16)
    return t.astype(np.uint16)


_CHUNK = 1 << 22   # elements per independently seeded block (fixed, so draws do not depend on threads)


def normal_bf16(rng: np.random.Generator, shape, outlier_frac: float = 0.0,
                outlier_mag: float = 8.0) -> np.ndarray:
    """N(0,1) float32 draws rounded to bfloat16 bits.  With ``outlier_frac`` > 0 each
    element is independently replaced, with that probability, by +-outlier_mag
    (fair sign) before rounding (outlier_mag must be exact in bfloat16).

    The draw is split into fixed-size blocks, each with its own child seed taken
    from ``rng``, and the blocks are filled on a thread pool."""
    from concurrent.futures import ThreadPoolExecutor

    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16)
    nblk = max(1, -(-n // _CHUNK))
    seeds = rng.integers(0, 2**63 - 1, size=nblk)

    def fill(i):
        g = np.random.default_rng(int(seeds[i]))
        a, b = i * _CHUNK, min(n, (i + 1) * _CHUNK)
        x = g.standard_normal(size=b - a, dtype=np.float32)
        if outlier_frac > 0.0:
            hit = g.random(size=b - a, dtype=np.float32) < np.float32(outlier_frac)
            sign = np.where(g.random(size=b - a, dtype=np.float32) < 0.5, np.float32(-1), np.float32(1))
            x = np.where(hit, sign * np.float32(outlier_mag), x)
        out[a:b] = f32_to_bf16_bits(x)

    if nblk == 1:
        fill(0)
    else:
        with ThreadPoolExecutor(max_workers=min(8, nblk)) as ex:
            list(ex.map(fill, range(nblk)))
    return out.reshape(shape)


def uniform_int_lens(rng, n, lo, hi):
    """Integers drawn uniformly from [lo, hi], both ends included."""
    return rng.integers(lo, hi + 1, size=n).astype(np.int32)


def log_uniform_lens(rng, n, lo, hi):
    """round(exp(U(ln lo, ln hi))), clipped to [lo, hi]."""
    v = np.rint(np.exp(rng.uniform(math.log(lo), math.log(hi), size=n)))
    return np.clip(v, lo, hi).astype(np.int32)


def assign_pages(rng, lens, page_size, pool_pages: Optional[int] = None, slack_pages: int = 8):
    """Give every sequence ceil(len/P) pages of a shared pool, in a seeded random order.

    Returns (block_table [B, max_pages] int32, num_pages, spare_page).  Entries past a
    sequence's pages point at ``spare_page``, a page no sequence owns (its content is
    poison); with no spare page available they point at page 0.
    """
    lens = np.asarray(lens, dtype=np.int64)
    need = [int(-(-int(n) // page_size)) for n in lens]
    total = int(sum(need))
    num_pages = max(total + slack_pages, pool_pages or 0)
    perm = rng.permutation(num_pages).astype(np.int32)
    max_pages = max(1, max(need) if need else 1)
    spare = int(perm[total]) if total < num_pages else 0
    bt = np.full((len(lens), max_pages), spare, dtype=np.int32)
    off = 0
    for s, n in enumerate(need):
        bt[s, :n] = perm[off:off + n]
        off += n
    return bt, num_pages, spare


@dataclass
class AttnParams:
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    page_size: int = 16
    kv_dtype: str = "bf16"          # "bf16", "int8" or "tq3" (3-bit rotated)
    window: int = 0                 # 0 = full attention
    sm_scale: float = 0.0           # 0 -> 1/sqrt(head_dim)
    sinks: Optional[np.ndarray] = None  # float32 [num_q_heads] or None

    def __post_init__(self):
        if self.sm_scale == 0.0:
            self.sm_scale = 1.0 / math.sqrt(self.head_dim)


@dataclass
class PagedCase:
    """A batch of sequences whose K/V live in a paged pool.

    ``k_tok``/``v_tok`` hold every cached token of every sequence, sequence after
    sequence ([sum(seq_lens), Hkv, D] bf16 bits; offsets ``cu_tok``).  The last
    ``q_lens[s]`` tokens of sequence s are the new ones of this step; the others are
    the restored prefix.  ``q`` holds one query vector per new token
    ([sum(q_lens), Hq, D] bf16 bits, offsets ``cu_q``).
    """
    name: str
    p: AttnParams
    seq_lens: np.ndarray      # [B] int32, after this step's tokens are appended
    q_lens: np.ndarray        # [B] int32
    cu_q: np.ndarray          # [B+1] int32
    cu_tok: np.ndarray        # [B+1] int64
    block_table: np.ndarray   # [B, max_pages] int32
    num_pages: int
    spare_page: int
    k_tok: np.ndarray
    v_tok: np.ndarray
    q: np.ndarray
    split_keys: int = 256
    meta: dict = field(default_factory=dict)
    k_smooth: Optional[np.ndarray] = None   # INT8 pools: [D] float32 key smoothing, or None

    @property
    def batch(self) -> int:
        return int(self.seq_lens.shape[0])

    def prefix_lens(self) -> np.ndarray:
        return (self.seq_lens - self.q_lens).astype(np.int32)

    def token_slice(self, s: int, lo: int, hi: int):
        """Rows [lo, hi) of sequence s in k_tok/v_tok."""
        a = int(self.cu_tok[s])
        return slice(a + lo, a + hi)

    def new_tokens(self):
        """(k_new, v_new, cu_new) for the tokens this step appends."""
        ks, vs = [], []
        for s in range(self.batch):
            sl = self.token_slice(s, int(self.seq_lens[s] - self.q_lens[s]), int(self.seq_lens[s]))
            ks.append(self.k_tok[sl])
            vs.append(self.v_tok[sl])
        cu = np.zeros(self.batch + 1, dtype=np.int32)
        cu[1:] = np.cumsum(self.q_lens)
        return np.concatenate(ks), np.concatenate(vs), cu

    def prefix_tokens(self):
        """(k_old, v_old, cu_old) for the restored prefix of every sequence."""
        pl = self.prefix_lens()
        ks, vs = [], []
        for s in range(self.batch):
            sl = self.token_slice(s, 0, int(pl[s]))
            ks.append(self.k_tok[sl])
            vs.append(self.v_tok[sl])
        cu = np.zeros(self.batch + 1, dtype=np.int32)
        cu[1:] = np.cumsum(pl)
        return np.concatenate(ks), np.concatenate(vs), cu

    def max_splits(self) -> int:
        if self.split_keys <= 0:
            return 1
        return max(1, int(-(-int(self.seq_lens.max()) // self.split_keys)))


def _scale_bf16(bits: np.ndarray, factor) -> np.ndarray:
    """bf16 bits times a float32 factor (broadcast), rounded back to bf16."""
    x = (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)
    return f32_to_bf16_bits((x * np.asarray(factor, np.float32)).astype(np.float32))


def make_case(name, seed, p: AttnParams, seq_lens, q_lens, pool_pages=None,
              outlier_frac=0.0, split_keys=256, sink_seed_offset=1000, meta=None,
              key_weight=None, q_scale=1.0, k_ramp=None, v_mags=None) -> PagedCase:
    """Draw K/V for every token, queries for the new tokens, and a page assignment.

    ``key_weight`` (float32 [D], INT8 cases): keys are drawn as N(0,1) times this
    per-channel weight (the shape a key-norm weight gives them), and the pool
    smooths keys by it.

    Value ranges beyond N(0,1) logits and values:
    * ``q_scale``: queries times this factor (a power of two keeps them exact), so
      the logits have standard deviation ``q_scale`` (with the 1/sqrt(D) scale);
    * ``k_ramp``: the key at position j of a sequence of n tokens is multiplied
      by ``k_ramp ** (j / (n - 1))``, so key norms grow along the sequence and a
      row's maximum logit jumps as later keys arrive;
    * ``v_mags``: each token's value vectors are multiplied by one of these
      magnitudes, drawn uniformly per token."""
    rng = np.random.default_rng(seed)
    seq_lens = np.asarray(seq_lens, dtype=np.int32)
    q_lens = np.asarray(q_lens, dtype=np.int32)
    assert seq_lens.shape == q_lens.shape and np.all(q_lens <= seq_lens) and np.all(q_lens >= 0)
    bt, num_pages, spare = assign_pages(rng, seq_lens, p.page_size, pool_pages)
    cu_tok = np.zeros(len(seq_lens) + 1, dtype=np.int64)
    cu_tok[1:] = np.cumsum(seq_lens.astype(np.int64))
    T = int(cu_tok[-1])
    k_tok = normal_bf16(rng, (T, p.num_kv_heads, p.head_dim), outlier_frac)
    v_tok = normal_bf16(rng, (T, p.num_kv_heads, p.head_dim), outlier_frac)
    if key_weight is not None:
        kf = (k_tok.astype(np.uint32) << np.uint32(16)).view(np.float32)
        k_tok = f32_to_bf16_bits((kf * np.asarray(key_weight, np.float32)).astype(np.float32))
    cu_q = np.zeros(len(seq_lens) + 1, dtype=np.int32)
    cu_q[1:] = np.cumsum(q_lens)
    q = normal_bf16(rng, (int(cu_q[-1]), p.num_q_heads, p.head_dim))
    if q_scale != 1.0:
        q = _scale_bf16(q, q_scale)
    if k_ramp is not None:
        f = np.empty(T, np.float32)
        for s_, n in enumerate(seq_lens):
            j = np.arange(int(n), dtype=np.float64)
            f[cu_tok[s_]:cu_tok[s_ + 1]] = (float(k_ramp) ** (j / max(int(n) - 1, 1))).astype(np.float32)
        k_tok = _scale_bf16(k_tok, f[:, None, None])
    if v_mags is not None:
        mags = np.asarray(v_mags, np.float32)[rng.integers(0, len(v_mags), size=T)]
        v_tok = _scale_bf16(v_tok, mags[:, None, None])
    return PagedCase(name=name, p=p, seq_lens=seq_lens, q_lens=q_lens, cu_q=cu_q,
                     cu_tok=cu_tok, block_table=bt, num_pages=num_pages, spare_page=spare,
                     k_tok=k_tok, v_tok=v_tok, q=q, split_keys=split_keys, meta=meta or {},
                     k_smooth=None if key_weight is None else np.asarray(key_weight, np.float32))


def sinks_normal(seed, n):
    """One sink logit per query head, N(0,1) float32."""
    return np.random.default_rng(seed).standard_normal(n).astype(np.float32)


# ---------------------------------------------------------------------------
# The named workloads.  Each is a model's attention shape with the length mix the
# pages measure at; sizes are the full ones unless ``small`` asks for a scaled
# version the CPU oracle finishes in seconds.
# ---------------------------------------------------------------------------

def decode_1seq_ctx1024(seed=1, split_keys=64):
    """One sequence, 16 q / 8 KV heads, D 128, 1024 cached positions, its 64 pages
    drawn from a 256-page pool.  64-key splits: one sequence gives few waves, and
    16 splits per KV head (128 waves of 4 pages) take the decode kernel from 14.0 us
    at 256-key splits to 7.0 us, the combine from 4.5 to 3.7 us (one MI355X)."""
    p = AttnParams(16, 8, 128)
    return make_case("decode_1seq_ctx1024", seed, p, [1024], [1], pool_pages=256,
                     split_keys=split_keys)


def decode_batch32_ctx512_8192(seed=2, batch=32, lo=512, hi=8192, fixed_len=None, split_keys=256):
    """Qwen3-4B attention shape (32 q / 8 KV heads, D 128); batch 32, lengths
    U[512, 8192] (or all ``fixed_len``); 256-key splits unless ``split_keys`` says
    otherwise (the name then ends in ``_s<split_keys>``)."""
    rng = np.random.default_rng(seed + 7)
    lens = (np.full(batch, fixed_len, np.int32) if fixed_len
            else uniform_int_lens(rng, batch, lo, hi))
    p = AttnParams(32, 8, 128)
    name = f"decode_batch{batch}_ctx{fixed_len}" if fixed_len else f"decode_batch{batch}_ctx{lo}_{hi}"
    if split_keys != 256:
        name += f"_s{split_keys}"
    return make_case(name, seed, p, lens, np.ones(batch, np.int32), split_keys=split_keys)


def prefill_llama8b(seed=3, prompt=1024, prefix=0, kv_dtype="bf16"):
    """Llama-3.1-8B attention shape (32 q / 8 KV heads, D 128), causal; a fresh
    prompt, or ``prompt`` new tokens on a restored ``prefix``-token paged prefix.
    ``kv_dtype`` "int8": the same over an INT8 cache (raw K/V N(0,1) with 1%
    outliers at +-8, as the INT8 decode workload)."""
    p = AttnParams(32, 8, 128, kv_dtype=kv_dtype)
    name = f"prefill_causal_{prompt}" if prefix == 0 else f"prefill_chunk{prompt}_on_{prefix}"
    if kv_dtype != "bf16":
        name = name.replace("prefill_", f"prefill_{kv_dtype}_", 1)
    return make_case(name, seed, p, [prefix + prompt], [prompt], split_keys=0,
                     outlier_frac=0.0 if kv_dtype == "bf16" else 0.01)


def kv_write_prompt(kv_dtype="bf16", seed=12, prompt=8192):
    """The KV write of one ``prompt``-token prompt in the Llama-3.1-8B attention shape
    (8 KV heads, D 128), into a BF16, INT8 or 3-bit pool; raw K/V N(0,1) with 1%
    outliers at +-8 for the quantised pools."""
    p = AttnParams(32, 8, 128, kv_dtype=kv_dtype)
    return make_case(f"kv_write_{kv_dtype}_{prompt}", seed, p, [prompt], [prompt], split_keys=0,
                     outlier_frac=0.0 if kv_dtype == "bf16" else 0.01)


def key_norm_weight(seed: int, head_dim: int, n_large: int = 4, large: float = 8.0) -> np.ndarray:
    """A synthetic key-norm weight (float32 [D], > 0): 1 + |N(0, 0.3)| per channel,
    with ``n_large`` channels at ``large`` (the few large channels such weights have)."""
    rng = np.random.default_rng(seed)
    w = (1.0 + np.abs(0.3 * rng.standard_normal(head_dim))).astype(np.float32)
    w[rng.choice(head_dim, n_large, replace=False)] = large
    return (f32_to_bf16_bits(w).astype(np.uint32) << np.uint32(16)).view(np.float32)   # bf16 values


def decode_int8_qwen30b(seed=4, batch=8, ctx=32768, smooth=False):
    """Qwen3-30B-A3B attention shape (32 q / 4 KV heads, D 128), INT8 KV, batch 8 at
    32768 positions, 1024-key splits; raw K/V N(0,1) with 1% outliers at +-8.  ``smooth``: keys
    shaped by a synthetic key-norm weight and the pool smoothing keys by it."""
    p = AttnParams(32, 4, 128, kv_dtype="int8")
    name = f"decode_int8_batch{batch}_ctx{ctx}" + ("_smooth" if smooth else "")
    return make_case(name, seed, p, np.full(batch, ctx, np.int32), np.ones(batch, np.int32),
                     outlier_frac=0.01, split_keys=1024,
                     key_weight=key_norm_weight(seed + 50, 128) if smooth else None)


def decode_tq3_qwen30b(seed=4, batch=8, ctx=32768):
    """The INT8 decode shape above (32 q / 4 KV heads, D 128, batch 8 at 32768
    positions, N(0,1) with 1% outliers at +-8) on the 3-bit rotated cache."""
    p = AttnParams(32, 4, 128, kv_dtype="tq3")
    return make_case(f"decode_tq3_batch{batch}_ctx{ctx}", seed, p, np.full(batch, ctx, np.int32),
                     np.ones(batch, np.int32), outlier_frac=0.01, split_keys=256)


def mixed_gptoss(seed=5, layer="window", part="decode", batch=64, lo=128, hi=32768,
                 chunks=2, chunk_len=2048):
    """gpt-oss-20b attention shape (64 q / 8 KV heads, D 64, one sink logit per q
    head).  Window layers see the last 128 positions, full layers all of them.
    ``part`` = "decode": 64 sequences, lengths log-uniform in [128, 32768], 256-key
    splits for full layers and no split for window layers (a sequence sees at most
    128 keys there, and splits of the hidden prefix would only write lse = -inf);
    ``part`` = "prefill": fresh prompts of ``chunk_len`` tokens."""
    window = 128 if layer == "window" else 0
    p = AttnParams(64, 8, 64, window=window, sinks=sinks_normal(seed + 99, 64))
    if part == "decode":
        rng = np.random.default_rng(seed + 11)
        lens = log_uniform_lens(rng, batch, lo, hi)
        return make_case(f"mixed_{layer}_decode_b{batch}", seed, p, lens, np.ones(batch, np.int32),
                         split_keys=0 if window else 256)
    lens = np.full(chunks, chunk_len, np.int32)
    return make_case(f"mixed_{layer}_prefill_{chunks}x{chunk_len}", seed, p, lens, lens, split_keys=0)


def verify_qwen4b(seed=6, batch=1, tokens=16, ctx=1024, lo=None, hi=None):
    """A speculative-decoding verify step on the Qwen3-4B attention shape (32 q / 8
    KV heads, D 128): ``tokens`` new tokens per sequence (the last accepted token
    plus tokens-1 drafted ones) on a cached context of ``ctx`` positions, or of
    lengths U[lo, hi] when both are given."""
    p = AttnParams(32, 8, 128)
    if lo is not None and hi is not None:
        rng = np.random.default_rng(seed + 13)
        ctxs = uniform_int_lens(rng, batch, lo, hi)
        name = f"verify_{tokens}tok_batch{batch}_ctx{lo}_{hi}"
    else:
        ctxs = np.full(batch, ctx, np.int32)
        name = f"verify_{tokens}tok_batch{batch}_ctx{ctx}"
    q_lens = np.full(batch, tokens, np.int32)
    return make_case(name, seed, p, ctxs + q_lens, q_lens, split_keys=0)


def verify_qwen4b_int8(seed=6, batch=1, tokens=16, ctx=1024):
    """The verify step above over an INT8 cache (1% outliers at +-8)."""
    c = verify_qwen4b(seed, batch, tokens, ctx)
    p = AttnParams(32, 8, 128, kv_dtype="int8")
    return make_case(c.name.replace("verify_", "verify_int8_", 1), seed, p, c.seq_lens, c.q_lens,
                     split_keys=0, outlier_frac=0.01)


# ---------------------------------------------------------------------------
# Attention-input inputs: the fused q/k/v projection output of new tokens, the
# q/k RMSNorm weights and the rotary table a model holds.
# ---------------------------------------------------------------------------

def rope_table(max_pos: int, head_dim: int, theta: float) -> np.ndarray:
    """Rotary cos/sin table [max_pos, D/2, 2] float32, as a model holds it: the
    angle of position p and pair i is p * theta^(-2i/D), evaluated in float64 and
    rounded to float32 (Qwen3 uses theta = 1e6)."""
    i = np.arange(head_dim // 2, dtype=np.float64)
    inv = theta ** (-2.0 * i / head_dim)
    ang = np.arange(max_pos, dtype=np.float64)[:, None] * inv[None, :]
    return np.stack([np.cos(ang), np.sin(ang)], axis=-1).astype(np.float32)


@dataclass
class AttnInputCase:
    """New tokens' fused qkv rows over a paged pool (``case`` gives the sequences,
    the block table and the pool size; its own K/V draws are not used)."""
    name: str
    case: PagedCase
    qkv: np.ndarray          # bf16 bits [T_new, (Hq + 2 Hkv) * D]
    q_norm_w: np.ndarray     # bf16 bits [D]
    k_norm_w: np.ndarray     # bf16 bits [D]
    rope: np.ndarray         # float32 [max_pos, D/2, 2]
    eps: float


def attn_input_case(name, seed, p: AttnParams, seq_lens, new_lens, theta=1e6, eps=1e-6,
                    qkv_scale=1.0, smooth=False) -> AttnInputCase:
    """qkv ~ N(0, qkv_scale^2) rounded to bf16; norm weights 1 + 0.1 N(0,1) in bf16.
    ``smooth`` (INT8): the pool smooths keys by |k norm weight|."""
    case = make_case(name, seed, p, seq_lens, new_lens, split_keys=0)
    rng = np.random.default_rng(seed + 11)
    T = int(case.cu_q[-1])
    width = (p.num_q_heads + 2 * p.num_kv_heads) * p.head_dim
    qkv = normal_bf16(rng, (T, width)) if qkv_scale == 1.0 else _scaled_bf16(rng, (T, width), qkv_scale)
    q_w = _scaled_bf16(rng, (p.head_dim,), 0.1, offset=1.0)
    k_w = _scaled_bf16(rng, (p.head_dim,), 0.1, offset=1.0)
    if smooth:
        case.k_smooth = np.abs((k_w.astype(np.uint32) << np.uint32(16)).view(np.float32))
    return AttnInputCase(name, case, qkv, q_w, k_w,
                         rope_table(int(np.max(seq_lens)) + 1, p.head_dim, theta), eps)


def _scaled_bf16(rng, shape, scale, offset=0.0):
    x = (offset + scale * rng.standard_normal(shape)).astype(np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def attn_input_qwen4b(seed=8, prompt=8192, batch=1, prefix=0):
    """Qwen3-4B attention shape (32 q / 8 KV heads, D 128): ``batch`` sequences of
    ``prompt`` new tokens each on a ``prefix``-token prefix."""
    p = AttnParams(32, 8, 128)
    lens = np.full(batch, prefix + prompt, np.int32)
    name = f"attn_input_{batch}x{prompt}" + (f"_on_{prefix}" if prefix else "")
    return attn_input_case(name, seed, p, lens, np.full(batch, prompt, np.int32))

