"""Parity of the HIP path (through the C ABI) with the CPU float64 oracle.

Bars, from the target tolerances:
* BF16 KV: max-abs 1e-2 and rel-L2 5e-3 over each call's whole output.
* INT8 KV: max-abs 3e-2, graded against the oracle on the dequantised cache.
* 3-bit rotated KV: the BF16 bars, against the oracle on the dequantised cache (the
  GPU computes the same function in fp32, in the rotated domain).
* The INT8 and 3-bit quantisers and the BF16 KV write: bit-exact.

Every pool starts poisoned, with NaN in BF16 slots and NaN scales in INT8 ones,
so a read of an unwritten slot shows up as a non-finite output.
"""
import os

import numpy as np
import pytest
import torch

import oracle as O
import paged_flash_attention_amd as pfa
import workloads as W
from gpu_support import (BF16_TOL, INT8_TOL, GpuCase, assert_close, bits_of, dev_bf16, dev_i32, main_build_batch,
                         gpu_attn_input, oracle_attn_input, oracle_pool, pool_bits_equal, tol_of)

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(__file__)


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    pfa.lib()


def P(Hq, Hkv, D, window=0, sinks=False, kv="bf16", seed=0):
    return W.AttnParams(Hq, Hkv, D, kv_dtype=kv, window=window,
                        sinks=W.sinks_normal(seed + 31, Hq) if sinks else None)


# ---------------------------------------------------------------------------
# fused attention input (q/k RMSNorm + RoPE + KV write): bit for bit
# ---------------------------------------------------------------------------

ATTN_INPUT_CASES = [
    # (params, seq_lens, new_lens, qkv_scale)
    (dict(Hq=32, Hkv=8, D=128), [1, 40, 300], [1, 17, 300], 1.0),
    (dict(Hq=32, Hkv=8, D=128, kv="int8"), [5, 70, 33], [5, 3, 33], 1.0),
    (dict(Hq=64, Hkv=8, D=64), [2, 130, 17], [2, 130, 1], 4.0),
    (dict(Hq=16, Hkv=4, D=64, kv="int8"), [9, 1, 600], [9, 1, 64], 0.25),
    (dict(Hq=8, Hkv=8, D=128), [31, 16], [15, 16], 30.0),
]


@pytest.mark.parametrize("ci", range(len(ATTN_INPUT_CASES)))
def test_attn_input_bitwise(ci):
    prm, lens, new, scale = ATTN_INPUT_CASES[ci]
    ic = W.attn_input_case(f"ain{ci}", 180 + ci, P(seed=ci, **prm), lens, new, qkv_scale=scale)
    q, pool = gpu_attn_input(ic)
    q_ref, pool_ref = oracle_attn_input(ic)
    assert np.array_equal(q, q_ref), f"q_out differs in {np.sum(q != q_ref)} elements"
    assert pool_bits_equal(pool, pool_ref, ic.case.p.kv_dtype), "pool differs"


# ---------------------------------------------------------------------------
# kv_write
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("D", [64, 128])
def test_kv_write_bf16_bitwise(D):
    case = W.make_case("kvw", 1, P(8, 4, D), [1, 17, 40, 300], [1, 5, 40, 33])
    g = GpuCase(case)
    ref = oracle_pool(case)
    torch.cuda.synchronize()
    assert np.array_equal(bits_of(g.pool.k), ref["k"])
    assert np.array_equal(bits_of(g.pool.v), ref["v"])


def _golden_vectors(D):
    rows = []
    for line in open(os.path.join(HERE, "golden", "int8_quantiser.txt")):
        line = line.split("#", 1)[0].strip()
        if line:
            xs = [float(t) for t in line.split()[0].split(",")]
            v = np.zeros(D, np.float32)
            v[: len(xs)] = xs
            rows.append(v)
    return W.f32_to_bf16_bits(np.stack(rows))


@pytest.mark.parametrize("D", [64, 128])
def test_kv_write_int8_bitwise(D):
    case = W.make_case("kvw8", 2, P(8, 2, D, kv="int8"), [3, 30, 70], [3, 30, 9], outlier_frac=0.01)
    gold = _golden_vectors(D)                                 # ties, exact scales, a zero vector
    n = min(len(gold), case.k_tok.shape[0])
    case.k_tok[:n, 0] = gold[:n]
    case.v_tok[-n:, 1] = gold[:n]
    g = GpuCase(case)
    ref = oracle_pool(case)
    torch.cuda.synchronize()
    assert np.array_equal(g.pool.k.cpu().numpy(), ref["k"])
    assert np.array_equal(g.pool.v.cpu().numpy(), ref["v"])
    ks, vs = g.pool.k_scale.cpu().numpy(), g.pool.v_scale.cpu().numpy()
    assert np.array_equal(ks.view(np.uint32), ref["k_scale"].view(np.uint32))   # NaN poison included
    assert np.array_equal(vs.view(np.uint32), ref["v_scale"].view(np.uint32))


@pytest.mark.parametrize("D", [64, 128])
def test_kv_write_int8_smoothed_bitwise(D):
    """Keys smoothed per channel (quantised as k / s): codes and scales bit-exact."""
    w = W.key_norm_weight(90 + D, D)
    case = W.make_case("kvw8s", 3, P(8, 2, D, kv="int8"), [3, 30, 70], [3, 30, 9], outlier_frac=0.01,
                       key_weight=w)
    g = GpuCase(case)
    ref = oracle_pool(case)
    torch.cuda.synchronize()
    assert np.array_equal(g.pool.k.cpu().numpy(), ref["k"])
    assert np.array_equal(g.pool.v.cpu().numpy(), ref["v"])
    ks, vs = g.pool.k_scale.cpu().numpy(), g.pool.v_scale.cpu().numpy()
    assert np.array_equal(ks.view(np.uint32), ref["k_scale"].view(np.uint32))
    assert np.array_equal(vs.view(np.uint32), ref["v_scale"].view(np.uint32))


def test_attn_input_int8_smoothed_bitwise():
    ic = W.attn_input_case("ain_s", 186, P(32, 8, 128, kv="int8"), [9, 200, 40], [9, 100, 1], smooth=True)
    q, pool = gpu_attn_input(ic)
    q_ref, pool_ref = oracle_attn_input(ic)
    assert np.array_equal(q, q_ref)
    assert pool_bits_equal(pool, pool_ref, "int8")


SMOOTH_CASES = [
    (dict(Hq=32, Hkv=4, D=128, kv="int8"), [1, 33, 257, 2000], [256, 0]),
    (dict(Hq=16, Hkv=4, D=64, kv="int8", window=50, sinks=True), [7, 64, 300], [32, 0]),
]


@pytest.mark.parametrize("ci", range(len(SMOOTH_CASES)))
def test_decode_int8_smoothed(ci):
    """Decode over a key-smoothed INT8 cache meets the oracle on that cache.  Beside
    it, reported: the error against the BF16-cache oracle with and without smoothing,
    on keys shaped by a key-norm weight with large channels (smoothing must help)."""
    prm, lens, splits = SMOOTH_CASES[ci]
    w = W.key_norm_weight(95 + ci, prm["D"])
    kw = dict(outlier_frac=0.0, key_weight=w)
    case_s = W.make_case(f"sm{ci}", 190 + ci, P(seed=ci, **prm), lens, np.ones(len(lens), np.int32), **kw)
    g = GpuCase(case_s)
    ref = O.decode(case_s.q, oracle_pool(case_s), case_s.block_table, case_s.seq_lens, case_s.p)
    outs = {}
    for S in splits:
        outs[S] = g.decode(split_keys=S)
        assert_close(outs[S], ref, INT8_TOL, f"smoothed decode case {ci} S={S}")
    # the same keys in a BF16 cache and in an unsmoothed INT8 cache
    prm_bf = dict(prm, kv="bf16")
    case_bf = W.make_case(f"sm{ci}b", 190 + ci, P(seed=ci, **prm_bf), lens, np.ones(len(lens), np.int32), **kw)
    case_bf.k_smooth = None
    exact = O.decode(case_bf.q, oracle_pool(case_bf), case_bf.block_table, case_bf.seq_lens, case_bf.p)
    case_u = W.make_case(f"sm{ci}u", 190 + ci, P(seed=ci, **prm), lens, np.ones(len(lens), np.int32), **kw)
    case_u.k_smooth = None
    plain = GpuCase(case_u).decode(split_keys=splits[0])
    e_s = float(np.sqrt(np.mean((outs[splits[0]] - exact) ** 2)))
    e_u = float(np.sqrt(np.mean((plain - exact) ** 2)))
    print(f"rms error vs the BF16 cache: smoothed {e_s:.3e}, unsmoothed {e_u:.3e}", flush=True)
    assert e_s < e_u


# ---------------------------------------------------------------------------
# decode + combine
# ---------------------------------------------------------------------------

def _tq3_special_rows(D, n):
    """bf16 rows for the 3-bit encoder: a zero vector, spikes, signed zeros,
    large and tiny magnitudes, a constant row (one nonzero rotated coordinate)."""
    rows = np.zeros((n, D), np.float32)
    rows[1, 3] = 5.0
    rows[2, D - 1] = -0.75
    rows[3] = -0.0
    rows[3, 0] = 2.0
    rows[4] = np.linspace(-300, 300, D)
    rows[5] = 1e-30 * np.arange(D)
    rows[6] = 1.0
    rows[7, ::2] = 1.0
    rows[7, 1::2] = -1.0
    return W.f32_to_bf16_bits(rows[:n])


@pytest.mark.parametrize("D", [64, 128])
def test_kv_write_tq3_bitwise(D):
    """3-bit rotated KV write: packed codes and scales equal the oracle's, whole
    pool, poison included."""
    case = W.make_case("kvw3", 5, P(8, 2, D, kv="tq3"), [3, 30, 70], [3, 30, 9], outlier_frac=0.01)
    sp = _tq3_special_rows(D, 8)
    case.k_tok[:8, 0] = sp
    case.v_tok[-8:, 1] = sp
    g = GpuCase(case)
    ref = oracle_pool(case)
    torch.cuda.synchronize()
    assert pool_bits_equal(g.pool, ref, "tq3")


TQ3_DECODE_CASES = [
    # (params, lens, split_keys list): G = 8, 1, 2, 4 at D = 128 and 64, window and sinks
    (dict(Hq=32, Hkv=4, D=128, kv="tq3"), [1, 33, 257, 2000], [256, 0]),
    (dict(Hq=8, Hkv=8, D=128, kv="tq3", sinks=True), [1, 90, 16], [16, 0]),
    (dict(Hq=16, Hkv=8, D=128, kv="tq3"), [15, 16, 17, 1024], [64, 0]),
    (dict(Hq=16, Hkv=4, D=64, kv="tq3", window=50, sinks=True), [7, 64, 300], [32, 0]),
    (dict(Hq=64, Hkv=8, D=64, kv="tq3", window=128, sinks=True), [1, 128, 129, 700], [256, 0]),
    (dict(Hq=16, Hkv=8, D=64, kv="tq3"), list(np.random.default_rng(78).integers(1, 1500, 24)), [16]),
]


@pytest.mark.parametrize("ci", range(len(TQ3_DECODE_CASES)))
def test_decode_tq3(ci):
    prm, lens, splits = TQ3_DECODE_CASES[ci]
    case = W.make_case(f"dec3_{ci}", 140 + ci, P(seed=ci, **prm), lens, np.ones(len(lens), np.int32),
                       outlier_frac=0.01)
    g = GpuCase(case)
    pool = oracle_pool(case)
    assert pool_bits_equal(g.pool, pool, "tq3")
    ref = O.decode(case.q, pool, case.block_table, case.seq_lens, case.p)
    for S in splits:
        got = g.decode(split_keys=S)
        assert_close(got, ref, BF16_TOL, f"tq3 decode case {ci} S={S}")


DECODE_CASES = [
    # (params, lens, split_keys list)
    (dict(Hq=16, Hkv=8, D=128), [1, 15, 16, 17, 300, 1024], [0, 256, 16]),
    (dict(Hq=32, Hkv=8, D=128), [5, 511, 512, 513, 2049], [256, 64]),
    (dict(Hq=8, Hkv=8, D=64), [1, 2, 64, 333], [0, 32]),
    (dict(Hq=64, Hkv=8, D=64, window=128, sinks=True), [1, 100, 128, 129, 700, 3000], [0, 256]),
    (dict(Hq=32, Hkv=4, D=128, kv="int8"), [1, 33, 257, 2000], [256, 0]),
    (dict(Hq=16, Hkv=4, D=64, kv="int8", window=50, sinks=True), [7, 64, 300], [32, 0]),
    (dict(Hq=8, Hkv=8, D=128, kv="int8", sinks=True), [1, 90], [16]),
    (dict(Hq=16, Hkv=8, D=64, window=1), [1, 2, 17], [16, 0]),
]


@pytest.mark.parametrize("ci", range(len(DECODE_CASES)))
def test_decode_parity(ci):
    prm, lens, splits = DECODE_CASES[ci]
    case = W.make_case(f"dec{ci}", 100 + ci, P(seed=ci, **prm), lens, np.ones(len(lens), np.int32),
                       outlier_frac=0.01 if prm.get("kv") == "int8" else 0.0)
    g = GpuCase(case)
    ref = O.decode(case.q, oracle_pool(case), case.block_table, case.seq_lens, case.p)
    for S in splits:
        got = g.decode(split_keys=S)
        assert_close(got, ref, tol_of(case), f"decode case {ci} S={S}")


# Many 16-key splits: several times more workgroups than the device holds at once,
# ragged lengths, and a window that hides a prefix of splits.
_rng = np.random.default_rng(77)
MANY_SPLIT_CASES = [
    (dict(Hq=32, Hkv=8, D=128, window=100, sinks=True), list(_rng.integers(1, 1200, 40)), 16),
    (dict(Hq=32, Hkv=4, D=128, kv="int8"), list(_rng.integers(1, 2500, 30)), 16),
    (dict(Hq=64, Hkv=8, D=64, sinks=True), list(_rng.integers(1, 1500, 48)), 16),
]


@pytest.mark.parametrize("ci", range(len(MANY_SPLIT_CASES)))
def test_decode_many_splits(ci):
    prm, lens, S = MANY_SPLIT_CASES[ci]
    case = W.make_case(f"many{ci}", 150 + ci, P(seed=ci, **prm), lens, np.ones(len(lens), np.int32),
                       outlier_frac=0.01 if prm.get("kv") == "int8" else 0.0)
    g = GpuCase(case)
    ref = O.decode(case.q, oracle_pool(case), case.block_table, case.seq_lens, case.p)
    assert_close(g.decode(split_keys=S), ref, tol_of(case), f"many-split case {ci}")


def test_decode_batch_2048_short():
    """Many short sequences: far more rows than splits, one page or less each."""
    rng = np.random.default_rng(81)
    lens = list(rng.integers(1, 40, 2048))
    case = W.make_case("b2048", 161, P(8, 2, 128), lens, np.ones(2048, np.int32))
    g = GpuCase(case)
    ref = O.decode(case.q, oracle_pool(case), case.block_table, case.seq_lens, case.p)
    for S in (0, 16):
        assert_close(g.decode(split_keys=S), ref, BF16_TOL, f"batch 2048 S={S}")


def test_decode_batch_600():
    """A large batch of short windowed sequences with sinks."""
    rng = np.random.default_rng(78)
    lens = list(rng.integers(1, 300, 600))
    case = W.make_case("bigbatch", 160, P(8, 2, 64, window=90, sinks=True), lens, np.ones(600, np.int32))
    g = GpuCase(case)
    ref = O.decode(case.q, oracle_pool(case), case.block_table, case.seq_lens, case.p)
    assert_close(g.decode(split_keys=64), ref, BF16_TOL, "batch 600")


FUSED_CASES = [
    (dict(Hq=32, Hkv=8, D=128), [1, 15, 16, 17, 300, 1024, 2049], 256),
    (dict(Hq=64, Hkv=8, D=64, window=128, sinks=True), [1, 100, 129, 700, 3000], 64),
    (dict(Hq=32, Hkv=4, D=128, kv="int8", sinks=True), [1, 33, 257, 2000], 256),
    (dict(Hq=16, Hkv=8, D=64, window=1), [1, 2, 17], 16),
    (dict(Hq=32, Hkv=8, D=128, window=100, sinks=True), list(np.random.default_rng(79).integers(1, 1200, 40)), 16),
]


@pytest.mark.parametrize("ci", range(len(FUSED_CASES)))
def test_decode_fused_equals_decode_then_combine(ci):
    """The fused merge gives the same bits as decode + combine, on repeated calls
    over one counter array, which it leaves zero; and it meets the oracle."""
    prm, lens, S = FUSED_CASES[ci]
    case = W.make_case(f"fused{ci}", 170 + ci, P(seed=ci, **prm), lens, np.ones(len(lens), np.int32),
                       outlier_frac=0.01 if prm.get("kv") == "int8" else 0.0)
    g = GpuCase(case)
    ref = O.decode(case.q, oracle_pool(case), case.block_table, case.seq_lens, case.p)
    plain = g.decode(split_keys=S)
    outs, ctr = g.decode_fused(split_keys=S, calls=3)
    assert not ctr.any(), "counters not reset"
    for k, got in enumerate(outs):
        assert np.array_equal(got.view(np.uint32), plain.view(np.uint32)), f"fused call {k} differs from decode+combine"
    assert_close(outs[-1], ref, tol_of(case), f"fused case {ci}")


def test_decode_partials_match_oracle():
    prm = dict(Hq=32, Hkv=8, D=128, window=300, sinks=True)
    lens = [10, 256, 257, 900]
    case = W.make_case("parts", 7, P(**prm), lens, np.ones(4, np.int32))
    g = GpuCase(case)
    S = 256
    ms = pfa.decode_num_splits(max(lens), S)
    _, (op, lp) = g.decode(split_keys=S, keep_parts=True)
    o_ref, l_ref = O.split_partials(case.q, oracle_pool(case), case.block_table, case.seq_lens, case.p, S, ms)
    op, lp = op.cpu().numpy(), lp.cpu().numpy()
    for b, n in enumerate(lens):
        ns = -(-n // S)
        assert np.array_equal(np.isneginf(lp[b, :, :ns]), np.isneginf(l_ref[b, :, :ns]))
        fin = np.isfinite(l_ref[b, :, :ns])
        assert np.max(np.abs(lp[b, :, :ns][fin] - l_ref[b, :, :ns][fin])) < 1e-3
        assert_close(op[b, :, :ns][fin], o_ref[b, :, :ns][fin], BF16_TOL, f"o_part seq {b}")


def test_combine_on_oracle_partials():
    """Feed the oracle's partials (float32) to the GPU combine alone."""
    prm = dict(Hq=16, Hkv=4, D=64, window=40, sinks=True)
    lens = [3, 64, 65, 200]
    case = W.make_case("comb", 8, P(**prm), lens, np.ones(4, np.int32))
    S = 32
    ms = pfa.decode_num_splits(max(lens), S)
    o_ref, l_ref = O.split_partials(case.q, oracle_pool(case), case.block_table, case.seq_lens, case.p, S, ms)
    ref = O.combine(o_ref, l_ref, case.seq_lens, S, case.p.sinks)
    g = GpuCase(case, fill=False)
    out = torch.empty(4, 16, 64, device="cuda")
    pfa.paged_attn_combine(g.desc, torch.from_numpy(o_ref.astype(np.float32)).cuda(),
                           torch.from_numpy(l_ref.astype(np.float32)).cuda(), g.seq_lens, S, ms, out)
    torch.cuda.synchronize()
    np.testing.assert_allclose(out.cpu().numpy(), ref, rtol=0, atol=2e-6)


# ---------------------------------------------------------------------------
# prefill
# ---------------------------------------------------------------------------

PREFILL_CASES = [
    # (params, seq_lens, q_lens)
    (dict(Hq=32, Hkv=8, D=128), [1, 37, 130, 300], [1, 37, 130, 300]),
    (dict(Hq=32, Hkv=8, D=128), [330, 64, 1001], [130, 64, 1]),          # chunks on restored prefixes
    (dict(Hq=64, Hkv=8, D=64, window=128, sinks=True), [300, 517], [300, 200]),
    (dict(Hq=8, Hkv=8, D=128, sinks=True), [200], [200]),
    (dict(Hq=4, Hkv=2, D=64, window=7), [90, 33], [90, 20]),
    (dict(Hq=32, Hkv=2, D=64), [77], [77]),                              # G = 16
    (dict(Hq=32, Hkv=1, D=128, window=64), [150], [150]),                # G = 32
    (dict(Hq=32, Hkv=8, D=128), [63, 64, 65, 128, 255, 256, 257], [63, 64, 65, 128, 255, 256, 257]),  # tile edges
    (dict(Hq=16, Hkv=4, D=128, sinks=True), [100, 50, 200, 9], [10, 0, 64, 0]),  # sequences with no new tokens
    (dict(Hq=8, Hkv=4, D=64, window=1, sinks=True), [70, 33], [70, 5]),  # window 1: each row sees itself
    (dict(Hq=32, Hkv=8, D=128, window=100), [1037, 16], [37, 16]),       # prefix not page-aligned
]


@pytest.mark.parametrize("ci", range(len(PREFILL_CASES)))
def test_prefill_parity(ci):
    prm, lens, qlens = PREFILL_CASES[ci]
    case = W.make_case(f"pre{ci}", 200 + ci, P(seed=ci, **prm), lens, qlens, split_keys=0)
    g = GpuCase(case)
    ref = O.paged_attention(case.q, case.cu_q, oracle_pool(case), case.block_table, case.seq_lens, case.p)
    for split in (None, (64, -(-max(lens) // 64)), (256, -(-max(lens) // 256))):
        got = g.prefill(split=split)
        assert_close(got, ref, BF16_TOL, f"prefill case {ci} split={split}")


MAIN_BUILD_CASES = [ci for ci, c in enumerate(PREFILL_CASES) if main_build_batch(*c) is not None]


@pytest.mark.parametrize("ci", MAIN_BUILD_CASES)
def test_prefill_parity_on_the_256_row_build(ci):
    """The prefill cases whose build is not fixed by a short window, their sequences
    repeated until the unsplit chunk takes the 256-row (64-key tile) build."""
    prm, lens, qlens = PREFILL_CASES[ci]
    lens, qlens = main_build_batch(prm, lens, qlens)
    case = W.make_case(f"pre256_{ci}", 260 + ci, P(seed=ci, **prm), lens, qlens, split_keys=0)
    g = GpuCase(case)
    ref = O.paged_attention(case.q, case.cu_q, oracle_pool(case), case.block_table, case.seq_lens, case.p)
    assert_close(g.prefill(split=None), ref, BF16_TOL, f"prefill case {ci} on the 256-row build ({len(lens)} sequences)")


def test_prefill_split_choice():
    """The library splits a short chunk on a long prefix, not a long prompt."""
    d = pfa.AttnDesc(32, 8, 128)
    ms, sk = pfa.prefill_num_splits(d, 1, 130, 8322)
    assert ms > 1 and sk % 64 == 0 and ms * sk >= 8322
    assert pfa.prefill_num_splits(d, 1, 8192, 8192) == (1, 0)


VERIFY_CASES = [
    # (params, seq_lens, q_lens): 2-16 new tokens per sequence on cached contexts
    (dict(Hq=32, Hkv=8, D=128), [1040], [16]),                           # 16 tokens at 1,024 positions
    (dict(Hq=32, Hkv=8, D=128), [39, 1002, 300, 2], [2, 2, 2, 2]),       # ragged; a 2-token sequence
    (dict(Hq=64, Hkv=8, D=64, window=128, sinks=True), [709, 3009], [9, 9]),
    (dict(Hq=8, Hkv=8, D=128, sinks=True), [518, 777], [5, 16]),
    (dict(Hq=32, Hkv=2, D=64), [1500], [8]),                             # G = 16: 128 rows
]


@pytest.mark.parametrize("ci", range(len(VERIFY_CASES)))
def test_verify_parity(ci):
    prm, lens, qlens = VERIFY_CASES[ci]
    case = W.make_case(f"ver{ci}", 300 + ci, P(seed=40 + ci, **prm), lens, qlens, split_keys=0)
    g = GpuCase(case)
    ref = O.paged_attention(case.q, case.cu_q, oracle_pool(case), case.block_table, case.seq_lens, case.p)
    for split in ("auto", None, (64, -(-max(lens) // 64)), (320, -(-max(lens) // 320))):
        got = g.verify(split=split)
        assert_close(got, ref, BF16_TOL, f"verify case {ci} split={split} ({g.last_split})")


def test_verify_split_choice():
    d = pfa.AttnDesc(32, 8, 128)
    ms, sk = pfa.verify_num_splits(d, 1, 16, 1040)
    assert ms > 1 and sk % 64 == 0 and ms * sk >= 1040
    assert pfa.verify_num_splits(d, 64, 16, 32768) == (1, 0)


# ---------------------------------------------------------------------------
# invariants on the GPU
# ---------------------------------------------------------------------------

def _permuted(case: W.PagedCase, seed=0):
    perm = np.random.default_rng(seed).permutation(case.num_pages).astype(np.int32)
    return W.PagedCase(case.name + "_perm", case.p, case.seq_lens, case.q_lens, case.cu_q, case.cu_tok,
                       perm[case.block_table], case.num_pages, int(perm[case.spare_page]),
                       case.k_tok, case.v_tok, case.q, case.split_keys)


def test_page_permutation_is_bitwise_invariant():
    dcase = W.make_case("pp", 9, P(32, 8, 128, sinks=True), [100, 700], [1, 1])
    pcase = W.make_case("ppf", 10, P(32, 8, 128), [300, 90], [130, 90], split_keys=0)
    for case, run in ((dcase, lambda g: g.decode(256)), (pcase, lambda g: g.prefill())):
        a = run(GpuCase(case))
        b = run(GpuCase(_permuted(case)))
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_split_count_invariance():
    case = W.make_case("sc", 11, P(32, 8, 128, window=500, sinks=True), [17, 256, 1000, 1500],
                       np.ones(4, np.int32))
    g = GpuCase(case)
    ref = O.decode(case.q, oracle_pool(case), case.block_table, case.seq_lens, case.p)
    outs = [g.decode(S) for S in (0, 16, 64, 256, 1024)]
    for o in outs:
        assert_close(o, ref, BF16_TOL, "split invariance")
    for o in outs[1:]:
        assert np.max(np.abs(o - outs[0])) < 2e-3


def test_repeat_runs_are_bitwise_identical():
    case = W.make_case("det", 12, P(64, 8, 64, window=128, sinks=True), [400, 2100], [1, 1])
    g = GpuCase(case)
    a, b = g.decode(256), g.decode(256)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    pc = W.make_case("detp", 13, P(32, 8, 128), [700], [700], split_keys=0)
    gp = GpuCase(pc)
    a, b = gp.prefill(), gp.prefill()
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_decode_equals_last_prefill_row():
    p = P(32, 8, 128, window=100, sinks=True)
    pc = W.make_case("lastrow", 14, p, [333], [333], split_keys=0)
    gp = GpuCase(pc)
    pre = gp.prefill()
    dc = W.PagedCase("lastrow_d", p, pc.seq_lens, np.array([1], np.int32), np.array([0, 1], np.int32), pc.cu_tok,
                     pc.block_table, pc.num_pages, pc.spare_page, pc.k_tok, pc.v_tok, pc.q[-1:], 256)
    gd = GpuCase(dc)
    for S in (0, 256):
        dec = gd.decode(S)
        assert np.max(np.abs(dec[0] - pre[-1])) < 1e-2


# ---------------------------------------------------------------------------
# a decode step under HIP graph capture: every replay equals the eager step
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("kv,fused", [("bf16", False), ("int8", False), ("tq3", False),
                                      ("bf16", True), ("int8", True)])
def test_decode_step_replays_in_a_graph(kv, fused):
    """kv_write + split decode + combine (or the fused decode, whose last split per
    row merges and clears its counter) captured once and replayed four times, with
    eager work and synchronisations between the replays; each replay is bit-identical
    to the eager step (the calls record no memset nodes)."""
    case = W.make_case(f"graph_{kv}", 310, P(32, 8, 128, kv=kv, window=0), [100, 700, 1500, 33],
                       np.ones(4, np.int32), outlier_frac=0.01 if kv != "bf16" else 0.0)
    g = GpuCase(case)
    k, v, cu = case.new_tokens()
    kn, vn, cun = dev_bf16(k), dev_bf16(v), dev_i32(cu)
    B, Hq, D = case.batch, case.p.num_q_heads, case.p.head_dim
    max_len = int(case.seq_lens.max())
    S = 256
    ms = pfa.decode_num_splits(max_len, S)
    op = torch.zeros((B, Hq, ms, D), device="cuda")
    lp = torch.zeros((B, Hq, ms), device="cuda")
    out = torch.zeros((B, Hq, D), device="cuda")
    ctr = torch.zeros(B * case.p.num_kv_heads, dtype=torch.int32, device="cuda")

    def step():
        pfa.kv_write(g.desc, g.pool, kn, vn, cun, g.seq_lens, g.bt)
        if fused:
            pfa.paged_attn_decode_fused(g.desc, g.pool, g.q, g.bt, g.seq_lens, max_len, S, ms, op, lp, ctr, out)
            return
        pfa.paged_attn_decode(g.desc, g.pool, g.q, g.bt, g.seq_lens, max_len, S, ms, o_part=op, lse_part=lp)
        pfa.paged_attn_combine(g.desc, op, lp, g.seq_lens, S, ms, out)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):          # warm-up off the capture
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    ref = out.clone()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    scratch = torch.randn(1 << 20, device="cuda")
    for i in range(4):
        out.fill_(float("nan"))
        scratch.mul_(1.0001)               # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"replay {i} differs from the eager step"
        if fused:
            assert not ctr.any(), "the fused decode leaves its counters at zero"
    assert_close(ref.cpu().numpy(), O.decode(case.q, oracle_pool(case), case.block_table, case.seq_lens, case.p),
                 tol_of(case), f"graph step ({kv}, fused={fused})")
