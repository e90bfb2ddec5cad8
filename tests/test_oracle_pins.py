"""Pins for the CPU float64 oracle, against facts independent of its own code.

Each check comes from mathematics or from the pages' definitions:
* brute force over tiny inputs: pure-Python loops, math.fsum, explicit page walks
  and a separate bf16 decoder;
* closed forms;
* torch's CPU float64 scaled_dot_product_attention, with explicit masks;
* invariants;
* hand-derived quantiser values (tests/golden/).

The checks are chosen so that a plausible slip in the oracle fails at least one:
a dropped sink term, an off-by-one in the causal or window mask, a wrong GQA head
map, a transposed operand, a wrong page index.
"""
import math
import struct

import numpy as np
import pytest
import torch

import oracle as O
import workloads as W

pytestmark = []

GOLDEN = __import__("os").path.join(__import__("os").path.dirname(__file__), "golden")


# ---------------------------------------------------------------------------
# helpers that do not use the oracle
# ---------------------------------------------------------------------------

def bf16_bits_to_float(b: int) -> float:
    """Independent bf16 decoder: place the 16 bits on top of a float32 word."""
    return struct.unpack("<f", struct.pack("<I", (int(b) & 0xFFFF) << 16))[0]


def fill_pool(case, kv_dtype="bf16"):
    p = case.p
    pool = O.empty_pool(case.num_pages, p.num_kv_heads, p.page_size, p.head_dim, kv_dtype)
    kp, vp, cup = case.prefix_tokens()
    O.kv_write(pool, kp, vp, cup, case.prefix_lens(), case.block_table, p.page_size, kv_dtype)
    kn, vn, cun = case.new_tokens()
    O.kv_write(pool, kn, vn, cun, case.seq_lens, case.block_table, p.page_size, kv_dtype)
    return pool


def brute_force(case, pool):
    """Pure-Python attention over the pool: explicit page walk, math.fsum, math.exp."""
    p = case.p
    G = p.num_q_heads // p.num_kv_heads
    P = p.page_size
    out = []
    for s in range(case.batch):
        n = int(case.seq_lens[s])
        ql = int(case.q_lens[s])
        for i in range(ql):
            row = int(case.cu_q[s]) + i
            pos = n - ql + i
            orow = []
            for h in range(p.num_q_heads):
                g = h // G
                qv = [bf16_bits_to_float(x) for x in case.q[row, h]]
                xs, vs = [], []
                for j in range(n):
                    if j > pos:
                        continue
                    if p.window > 0 and pos - j >= p.window:
                        continue
                    page = int(case.block_table[s][j // P])
                    off = j % P
                    kv = [bf16_bits_to_float(x) for x in pool["k"][page, g, off]]
                    vv = [bf16_bits_to_float(x) for x in pool["v"][page, g, off]]
                    xs.append(p.sm_scale * math.fsum(a * b for a, b in zip(qv, kv)))
                    vs.append(vv)
                cand = list(xs)
                if p.sinks is not None:
                    cand.append(float(p.sinks[h]))
                M = max(cand)
                w = [math.exp(x - M) for x in xs]
                Z = math.fsum(w + ([math.exp(float(p.sinks[h]) - M)] if p.sinks is not None else []))
                orow.append([math.fsum(wj * vj[d] for wj, vj in zip(w, vs)) / Z for d in range(p.head_dim)])
            out.append(orow)
    return np.array(out)


def tiny_case(seed, lens, q_lens, Hq=4, Hkv=2, D=3, P=2, window=0, sinks=False):
    p = W.AttnParams(Hq, Hkv, D, page_size=P, window=window,
                     sinks=W.sinks_normal(seed + 5, Hq) if sinks else None)
    return W.make_case("tiny", seed, p, lens, q_lens)


# ---------------------------------------------------------------------------
# brute force
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("window,sinks", [(0, False), (2, False), (0, True), (3, True)])
def test_brute_force_prefill_and_decode(seed, window, sinks):
    rng = np.random.default_rng(seed)
    lens = [int(x) for x in rng.integers(1, 7, size=3)]
    q_lens = [int(rng.integers(1, n + 1)) for n in lens]
    case = tiny_case(seed, lens, q_lens, window=window, sinks=sinks)
    pool = fill_pool(case)
    got = O.paged_attention(case.q, case.cu_q, pool, case.block_table, case.seq_lens, case.p)
    ref = brute_force(case, pool)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-13)


def test_brute_force_gqa_groups_of_four():
    case = tiny_case(11, [5, 3], [2, 3], Hq=8, Hkv=2, D=4, P=2, sinks=True)
    pool = fill_pool(case)
    got = O.paged_attention(case.q, case.cu_q, pool, case.block_table, case.seq_lens, case.p)
    np.testing.assert_allclose(got, brute_force(case, pool), rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------------------------
# closed forms
# ---------------------------------------------------------------------------

def _dense_params(Hq=1, Hkv=1, D=4, window=0, sinks=None, scale=0.5):
    return W.AttnParams(Hq, Hkv, D, window=window, sm_scale=scale, sinks=sinks)


def test_single_key_gives_its_value():
    p = _dense_params()
    K = np.array([[[0.3, -1.0, 2.0, 0.5]]])
    V = np.array([[[1.5, -2.25, 0.0, 7.0]]])
    q = np.array([[[4.0, 1.0, -3.0, 2.0]]])
    out, _, _ = O.attend(q, np.array([0]), K, V, p)
    np.testing.assert_allclose(out[0, 0], V[0, 0], rtol=0, atol=1e-15)


def test_two_keys_logistic_weight():
    p = _dense_params(scale=0.5)
    q = np.array([[[1.0, 0.0, 0.0, 0.0]]])
    K = np.array([[[2.0, 9.0, 9.0, 9.0]], [[-1.0, 5.0, 5.0, 5.0]]])    # scores 1.0 and -0.5
    V = np.array([[[1.0, 0.0, 0.0, 0.0]], [[0.0, 1.0, 0.0, 0.0]]])
    out, _, _ = O.attend(q, np.array([1]), K, V, p)
    w1 = 1.0 / (1.0 + math.exp(-0.5 - 1.0))
    np.testing.assert_allclose(out[0, 0], [w1, 1.0 - w1, 0.0, 0.0], rtol=1e-14, atol=1e-15)


def test_constant_values_give_that_value():
    rng = np.random.default_rng(0)
    p = _dense_params(Hq=4, Hkv=2, D=8, scale=0.35)
    K = rng.standard_normal((40, 2, 8))
    V = np.broadcast_to(rng.standard_normal((1, 2, 8)), (40, 2, 8)).copy()
    q = rng.standard_normal((5, 4, 8)) * 3
    out, _, _ = O.attend(q, np.arange(35, 40), K, V, p)
    for h in range(4):
        np.testing.assert_allclose(out[:, h], np.broadcast_to(V[0, h // 2], (5, 8)), rtol=1e-13)


def test_zero_query_averages_visible_values():
    rng = np.random.default_rng(1)
    p = _dense_params(Hq=2, Hkv=1, D=6, window=5)
    K = rng.standard_normal((20, 1, 6))
    V = rng.standard_normal((20, 1, 6))
    q = np.zeros((3, 2, 6))
    pos = np.array([2, 10, 19])
    out, _, _ = O.attend(q, pos, K, V, p)
    for r, ps in enumerate(pos):
        lo = max(0, ps - 5 + 1)
        np.testing.assert_allclose(out[r, 0], V[lo:ps + 1, 0].mean(axis=0), rtol=1e-13)


def test_window_one_returns_own_value():
    rng = np.random.default_rng(2)
    p = _dense_params(Hq=2, Hkv=2, D=5, window=1)
    K = rng.standard_normal((9, 2, 5))
    V = rng.standard_normal((9, 2, 5))
    q = rng.standard_normal((9, 2, 5)) * 4
    out, _, _ = O.attend(q, np.arange(9), K, V, p)
    np.testing.assert_allclose(out, V, rtol=1e-14)


def test_one_key_with_sink():
    sink = 0.7
    p = _dense_params(sinks=np.array([sink], np.float32), scale=1.0)
    q = np.array([[[1.0, 1.0, 0.0, 0.0]]])
    K = np.array([[[0.25, 0.5, 3.0, 3.0]]])                          # x = 0.75
    V = np.array([[[2.0, -4.0, 1.0, 0.5]]])
    out, _, _ = O.attend(q, np.array([0]), K, V, p)
    s32 = float(np.float32(sink))
    w = 1.0 / (1.0 + math.exp(s32 - 0.75))
    np.testing.assert_allclose(out[0, 0], w * V[0, 0], rtol=1e-14)


def test_no_keys_gives_zero():
    """A row with no keys at all (an empty sequence) outputs 0, sink or not, and
    its split statistics are m = -inf, l = 0."""
    q = np.array([[[1.0, -2.0, 0.5, 3.0]]])
    K = np.zeros((0, 1, 4))
    V = np.zeros((0, 1, 4))
    for sinks in (None, np.array([0.3], np.float32)):
        out, m, l = O.attend(q, np.array([-1]), K, V, _dense_params(sinks=sinks, scale=1.0))
        assert np.array_equal(out, np.zeros((1, 1, 4)))
        assert np.isneginf(m).all() and np.array_equal(l, np.zeros((1, 1)))


def test_sink_at_minus_infinity_is_no_sink():
    case = tiny_case(3, [6, 4], [3, 1], sinks=True)
    pool = fill_pool(case)
    ref = O.paged_attention(case.q, case.cu_q, pool, case.block_table, case.seq_lens,
                            W.AttnParams(4, 2, 3, page_size=2, sinks=None))
    case.p.sinks = np.full(4, -np.inf, np.float32)
    got = O.paged_attention(case.q, case.cu_q, pool, case.block_table, case.seq_lens, case.p)
    np.testing.assert_array_equal(got, ref)


# ---------------------------------------------------------------------------
# torch CPU float64 SDPA, identity block table, explicit masks
# ---------------------------------------------------------------------------

def _sdpa_reference(case, pool_k_tok, pool_v_tok):
    """torch SDPA in float64 on dense per-sequence K/V.

    * GQA is expressed with repeat_interleave.
    * The additive mask is built here from positions.
    * A sink is an extra key with k = 0 and v = 0, whose bias equals the sink.
    """
    p = case.p
    G = p.num_q_heads // p.num_kv_heads
    outs = []
    for s in range(case.batch):
        n, ql = int(case.seq_lens[s]), int(case.q_lens[s])
        sl = case.token_slice(s, 0, n)
        K = torch.from_numpy(O.bf16_to_f64(pool_k_tok[sl])).permute(1, 0, 2)   # [Hkv, n, D]
        V = torch.from_numpy(O.bf16_to_f64(pool_v_tok[sl])).permute(1, 0, 2)
        K = K.repeat_interleave(G, dim=0)
        V = V.repeat_interleave(G, dim=0)
        Q = torch.from_numpy(O.bf16_to_f64(case.q[int(case.cu_q[s]):int(case.cu_q[s + 1])])).permute(1, 0, 2)
        bias = torch.full((ql, n), -math.inf, dtype=torch.float64)
        for i in range(ql):
            pos = n - ql + i
            lo = 0 if p.window == 0 else max(0, pos - p.window + 1)
            bias[i, lo:pos + 1] = 0.0
        bias = bias.unsqueeze(0).repeat(p.num_q_heads, 1, 1)
        if p.sinks is not None:
            K = torch.cat([K, torch.zeros(p.num_q_heads, 1, p.head_dim, dtype=torch.float64)], dim=1)
            V = torch.cat([V, torch.zeros(p.num_q_heads, 1, p.head_dim, dtype=torch.float64)], dim=1)
            sb = torch.tensor(p.sinks.astype(np.float64)).view(-1, 1, 1).expand(-1, ql, 1)
            bias = torch.cat([bias, sb], dim=2)
        o = torch.nn.functional.scaled_dot_product_attention(
            Q.contiguous(), K.contiguous(), V.contiguous(), attn_mask=bias, scale=p.sm_scale)
        outs.append(o.permute(1, 0, 2).numpy())
    return np.concatenate(outs)


@pytest.mark.parametrize("window,sinks", [(0, False), (7, False), (0, True), (16, True)])
def test_against_torch_sdpa_float64(window, sinks):
    p = W.AttnParams(8, 2, 16, page_size=4, window=window,
                     sinks=W.sinks_normal(9, 8) if sinks else None)
    case = W.make_case("sdpa", 21, p, [37, 12, 64], [37, 5, 1])
    pool = fill_pool(case)
    got = O.paged_attention(case.q, case.cu_q, pool, case.block_table, case.seq_lens, case.p)
    ref = _sdpa_reference(case, case.k_tok, case.v_tok)
    np.testing.assert_allclose(got, ref, rtol=1e-10, atol=1e-12)


def test_decode_shape_against_torch_sdpa():
    case = W.decode_1seq_ctx1024(seed=17)
    pool = fill_pool(case)
    got = O.decode(case.q, pool, case.block_table, case.seq_lens, case.p)
    ref = _sdpa_reference(case, case.k_tok, case.v_tok)
    np.testing.assert_allclose(got, ref, rtol=1e-10, atol=1e-12)


# ---------------------------------------------------------------------------
# invariants
# ---------------------------------------------------------------------------

def test_page_permutation_invariance():
    case = tiny_case(4, [9, 14, 3], [2, 14, 1], Hq=4, Hkv=2, D=5, P=4, sinks=True)
    pool = fill_pool(case)
    ref = O.paged_attention(case.q, case.cu_q, pool, case.block_table, case.seq_lens, case.p)
    perm = np.random.default_rng(0).permutation(case.num_pages)
    pool2 = {k: np.empty_like(v) for k, v in pool.items()}
    for k in pool:
        pool2[k][perm] = pool[k]
    bt2 = perm[case.block_table]
    got = O.paged_attention(case.q, case.cu_q, pool2, bt2, case.seq_lens, case.p)
    np.testing.assert_array_equal(got, ref)


@pytest.mark.parametrize("window,sinks", [(0, False), (0, True), (40, True), (100, False)])
def test_split_count_invariance(window, sinks):
    p = W.AttnParams(8, 2, 16, window=window, sinks=W.sinks_normal(2, 8) if sinks else None)
    case = W.make_case("split", 5, p, [1, 15, 16, 17, 255, 256, 257, 600], np.ones(8, np.int32))
    pool = fill_pool(case)
    ref = O.decode(case.q, pool, case.block_table, case.seq_lens, case.p)
    for S in (16, 64, 256, 1024):
        ms = -(-int(case.seq_lens.max()) // S)
        o, lse = O.split_partials(case.q, pool, case.block_table, case.seq_lens, case.p, S, ms)
        got = O.combine(o, lse, case.seq_lens, S, case.p.sinks)
        np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-14)


def test_split_lse_is_logsumexp_of_scores():
    """One split covering every key: lse = log sum_j exp(x_j), with x from fsum."""
    case = tiny_case(8, [7], [1], Hq=2, Hkv=1, D=4, P=2)
    pool = fill_pool(case)
    o, lse = O.split_partials(case.q, pool, case.block_table, case.seq_lens, case.p, 8, 1)
    for h in range(2):
        qv = [bf16_bits_to_float(x) for x in case.q[0, h]]
        xs = []
        for j in range(7):
            page, off = int(case.block_table[0][j // 2]), j % 2
            kv = [bf16_bits_to_float(x) for x in pool["k"][page, 0, off]]
            xs.append(case.p.sm_scale * math.fsum(a * b for a, b in zip(qv, kv)))
        M = max(xs)
        assert abs(lse[0, h, 0] - (M + math.log(math.fsum(math.exp(x - M) for x in xs)))) < 1e-13


def test_gqa_equals_mha_with_repeated_kv():
    p = W.AttnParams(8, 2, 8, window=5, sinks=W.sinks_normal(4, 8))
    case = W.make_case("gqa", 6, p, [30, 11], [4, 11])
    pool = fill_pool(case)
    got = O.paged_attention(case.q, case.cu_q, pool, case.block_table, case.seq_lens, case.p)
    pool_mha = {k: np.repeat(v, 4, axis=1) for k, v in pool.items()}
    p_mha = W.AttnParams(8, 8, 8, window=5, sinks=case.p.sinks)
    ref = O.paged_attention(case.q, case.cu_q, pool_mha, case.block_table, case.seq_lens, p_mha)
    np.testing.assert_array_equal(got, ref)
    # and a wrong head map (h % Hkv) would differ
    swapped = {k: v[:, ::-1].copy() for k, v in pool.items()}
    bad = O.paged_attention(case.q, case.cu_q, swapped, case.block_table, case.seq_lens, case.p)
    assert np.abs(bad - got).max() > 1e-3


def test_window_at_least_len_is_full():
    p = W.AttnParams(4, 2, 8)
    case = W.make_case("win", 7, p, [20, 33], [20, 1])
    pool = fill_pool(case)
    full = O.paged_attention(case.q, case.cu_q, pool, case.block_table, case.seq_lens, case.p)
    case.p.window = 33
    win = O.paged_attention(case.q, case.cu_q, pool, case.block_table, case.seq_lens, case.p)
    np.testing.assert_array_equal(full, win)


def test_decode_is_last_prefill_row_and_chunks_match_one_shot():
    p = W.AttnParams(4, 2, 8, window=9, sinks=W.sinks_normal(1, 4))
    one = W.make_case("pf", 8, p, [50], [50])
    pool = fill_pool(one)
    full = O.paged_attention(one.q, one.cu_q, pool, one.block_table, one.seq_lens, one.p)
    # the same tokens as a restored 37-token prefix + a 13-token chunk
    chunk = W.PagedCase("chunk", p, np.array([50], np.int32), np.array([13], np.int32),
                        np.array([0, 13], np.int32), one.cu_tok, one.block_table, one.num_pages,
                        one.spare_page, one.k_tok, one.v_tok, one.q[37:])
    got = O.paged_attention(chunk.q, chunk.cu_q, pool, chunk.block_table, chunk.seq_lens, p)
    # BLAS may block a different number of rows differently: agree to rounding.
    np.testing.assert_allclose(got, full[37:], rtol=1e-13, atol=1e-15)
    dec = O.decode(one.q[49:50], pool, one.block_table, one.seq_lens, p)
    np.testing.assert_allclose(dec[0], full[49], rtol=1e-13, atol=1e-15)


def test_rows_subset_matches_full():
    case = W.make_case("rows", 9, W.AttnParams(4, 2, 8), [40, 25], [40, 3])
    pool = fill_pool(case)
    full = O.paged_attention(case.q, case.cu_q, pool, case.block_table, case.seq_lens, case.p)
    rows = [0, 17, 39, 40, 42]
    sub = O.paged_attention(case.q, case.cu_q, pool, case.block_table, case.seq_lens, case.p, rows=rows,
                            max_rows_per_chunk=2)
    np.testing.assert_allclose(sub, full[rows], rtol=1e-13, atol=1e-15)


# ---------------------------------------------------------------------------
# kv_write placement
# ---------------------------------------------------------------------------

def test_kv_write_places_tokens_by_block_table():
    """Block table [[5, 2], [0, 4]], P = 4.  Sequence 0 holds 6 tokens and appends
    2, so its new tokens sit at positions 4 and 5: page 2, offsets 0 and 1.
    Sequence 1 appends 3 tokens to reach 3: page 0, offsets 0..2."""
    pool = O.empty_pool(6, 1, 4, 2, "bf16")
    bt = np.array([[5, 2], [0, 4]], np.int32)
    k = np.arange(10, dtype=np.uint16).reshape(5, 1, 2) + 0x3F80
    v = k + 0x100
    O.kv_write(pool, k, v, np.array([0, 2, 5]), np.array([6, 3]), bt, 4, "bf16")
    assert list(pool["k"][2, 0, 0]) == list(k[0, 0]) and list(pool["k"][2, 0, 1]) == list(k[1, 0])
    for i in range(3):
        assert list(pool["v"][0, 0, i]) == list(v[2 + i, 0])
    untouched = np.ones(6, bool)
    untouched[[0, 2]] = False
    assert np.all(pool["k"][untouched] == 0x7FC0)
    assert np.all(pool["k"][2, 0, 2:] == 0x7FC0) and np.all(pool["k"][0, 0, 3] == 0x7FC0)


# ---------------------------------------------------------------------------
# the INT8 quantiser
# ---------------------------------------------------------------------------

def _read_golden(name):
    rows = []
    with open(f"{GOLDEN}/{name}") as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                rows.append(line.split())
    return rows


def test_quantiser_golden_ties_and_values():
    for row in _read_golden("int8_quantiser.txt"):
        xs = [float(t) for t in row[0].split(",")]
        want_scale = float(row[1])
        want_codes = [int(t) for t in row[2].split(",")]
        bits = W.f32_to_bf16_bits(np.array([xs], np.float32))
        assert all(bf16_bits_to_float(b) == x for b, x in zip(bits[0], xs)), "fixture value not exact in bf16"
        codes, scale = O.quantize_int8(bits)
        assert float(scale[0]) == np.float32(want_scale)
        assert codes[0].tolist() == want_codes


def test_quantiser_bounds_and_argmax():
    rng = np.random.default_rng(3)
    bits = W.normal_bf16(rng, (2000, 64), outlier_frac=0.01)
    bits[7] = 0                                                    # a zero vector
    bits[8] = W.f32_to_bf16_bits(np.full(64, -3.0, np.float32))  # all equal, negative
    codes, scale = O.quantize_int8(bits)
    x = O.bf16_to_f64(bits)
    assert codes.dtype == np.int8 and codes.min() >= -127 and codes.max() <= 127
    assert scale[7] == 0 and np.all(codes[7] == 0)
    assert np.all(codes[8] == -127)
    nz = scale > 0
    am = np.argmax(np.abs(x), axis=1)
    assert np.all(np.abs(codes[np.arange(2000), am])[nz] == 127)
    err = np.abs(x - O.dequantize_int8(codes, scale))
    bound = scale.astype(np.float64)[:, None] * (0.5 + 2.0 ** -16)
    assert np.all(err <= bound)
    # scale is the float32 quotient absmax/127
    np.testing.assert_array_equal(scale, (np.abs(x).max(axis=1).astype(np.float32) / np.float32(127)))


# ---------------------------------------------------------------------------
# INT8 key smoothing (keys stored as k / s per channel; queries meet q * s)
# ---------------------------------------------------------------------------

def test_smoothing_factor_is_the_largest_power_of_two_not_above_the_weight():
    w = np.array([1.0, 1.5, 1.999, 2.0, 0.75, 0.5, 12.0, 8.0, 3e-30, 1e30], np.float32)
    want = np.array([2.0 ** math.floor(math.log2(float(x))) for x in w], np.float32)
    np.testing.assert_array_equal(O.smoothing_factors(w), want)
    f = O.smoothing_factors(w).astype(np.float64)
    assert np.all((f <= w) & (w < 2 * f))


def test_smoothing_by_ones_is_no_smoothing():
    rng = np.random.default_rng(21)
    bits = W.normal_bf16(rng, (300, 128), outlier_frac=0.01)
    c0, s0 = O.quantize_int8(bits)
    c1, s1 = O.quantize_int8(bits, np.ones(128, np.float32))
    assert np.array_equal(c0, c1) and np.array_equal(s0, s1)


def test_smoothing_by_a_power_of_two_divides_the_scale_only():
    rng = np.random.default_rng(22)
    bits = W.normal_bf16(rng, (300, 64))
    c0, s0 = O.quantize_int8(bits)
    c1, s1 = O.quantize_int8(bits, np.full(64, 4.0, np.float32))
    assert np.array_equal(c0, c1)
    assert np.array_equal(s1, (s0 / np.float32(4)).astype(np.float32))


def test_smoothed_dequantisation_bound():
    rng = np.random.default_rng(23)
    bits = W.normal_bf16(rng, (500, 64), outlier_frac=0.02)
    s = (0.2 + rng.random(64) * 5).astype(np.float32)
    codes, scale = O.quantize_int8(bits, s)
    x = O.bf16_to_f64(bits)
    err = np.abs(O.dequantize_int8(codes, scale, s) - x)
    bound = scale.astype(np.float64)[:, None] * s.astype(np.float64)[None, :] * (0.5 + 2.0 ** -15) \
        + np.abs(x) * 2.0 ** -22
    assert np.all(err <= bound)


def test_smoothed_attention_is_scaled_query_on_unsmoothed_codes():
    """q . (code * scale * s) = (q * s) . (code * scale): the smoothing vector sits on
    channels, so a brute force with the query scaled instead must agree.  s is the
    power of two at or below each given weight."""
    rng = np.random.default_rng(24)
    p = W.AttnParams(4, 2, 8, page_size=2, kv_dtype="int8")
    case = W.make_case("smooth", 24, p, [5, 3], [1, 1])
    s = (0.5 + rng.random(8) * 3).astype(np.float32)
    pool = O.empty_pool(case.num_pages, 2, 2, 8, "int8", k_smooth=s)
    k, v, cu = case.k_tok, case.v_tok, case.cu_tok
    O.kv_write(pool, k, v, cu, case.seq_lens, case.block_table, 2, "int8")
    got = O.decode(case.q, pool, case.block_table, case.seq_lens, p)
    for b in range(case.batch):
        n = int(case.seq_lens[b])
        for h in range(4):
            g = h // 2
            q = [bf16_bits_to_float(x) * 2.0 ** math.floor(math.log2(float(s[d])))
                 for d, x in enumerate(case.q[b, h])]
            xs, vs = [], []
            for j in range(n):
                pg, off = int(case.block_table[b][j // 2]), j % 2
                kc = pool["k"][pg, g, off].astype(np.float64) * float(pool["k_scale"][pg, g, off])
                vc = pool["v"][pg, g, off].astype(np.float64) * float(pool["v_scale"][pg, g, off])
                xs.append(p.sm_scale * math.fsum(qd * kd for qd, kd in zip(q, kc)))
                vs.append(vc)
            M = max(xs)
            w = [math.exp(x - M) for x in xs]
            Z = math.fsum(w)
            ref = [math.fsum(wj * vj[d] for wj, vj in zip(w, vs)) / Z for d in range(8)]
            np.testing.assert_allclose(got[b, h], ref, rtol=1e-12, atol=1e-13)


def test_smoothing_by_the_channel_weight_helps_outlier_channels():
    """Keys shaped like k_norm output (a unit-RMS vector times a per-channel weight with
    a few large channels) quantise with less error when smoothed by that weight."""
    rng = np.random.default_rng(25)
    w = np.ones(128, np.float32)
    w[[3, 77]] = 12.0
    base = rng.standard_normal((2000, 128)).astype(np.float32)
    bits = W.f32_to_bf16_bits((base * w).astype(np.float32))
    x = O.bf16_to_f64(bits)
    e0 = np.abs(O.dequantize_int8(*O.quantize_int8(bits)) - x)
    c1, s1 = O.quantize_int8(bits, w)
    e1 = np.abs(O.dequantize_int8(c1, s1, w) - x)
    others = np.ones(128, bool)
    others[[3, 77]] = False
    assert e1[:, others].mean() < 0.5 * e0[:, others].mean()
