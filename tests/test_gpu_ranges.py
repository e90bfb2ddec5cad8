"""Parity away from N(0,1) inputs: large logits, keys whose norms grow along the
sequence (a row's maximum jumps as later keys arrive, so the online softmax moves
its reference maximum mid-row), sliding windows longer than 512 keys, and INT8
value vectors from 1e-30 to 1e30 in magnitude.

Each case runs every kernel build that serves it (decode split and unsplit at
G = 4 and 8, prefill on the 64-key build and on the 32-key KV-split build, verify)
and is judged against the float64 oracle at the same bars as the N(0,1) suite:
BF16 KV max-abs 1e-2 and rel-L2 5e-3; INT8 KV max-abs 3e-2 on the dequantised
cache.  The value-magnitude cases scale the INT8 bar by the output's magnitude.
"""
import numpy as np
import pytest
import torch

import oracle as O
import paged_flash_attention_amd as pfa
import workloads as W
from gpu_support import BF16_TOL, INT8_TOL, GpuCase, assert_close, errors, oracle_pool, tol_of

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    pfa.lib()


def P(Hq, Hkv, D, window=0, sinks=False, kv="bf16", seed=0):
    return W.AttnParams(Hq, Hkv, D, kv_dtype=kv, window=window,
                        sinks=W.sinks_normal(seed + 51, Hq) if sinks else None)


# ---------------------------------------------------------------------------
# large logits: q scaled so that sm_scale * q.k has standard deviation 4, 8, 16;
# "ramp" cases also grow key norms 4x along each sequence
# ---------------------------------------------------------------------------

PREFILL_LOGIT_CASES = [
    # (id, params, seq_lens, q_lens, q_scale, k_ramp)
    ("llama_s4", dict(Hq=32, Hkv=8, D=128), [1024], [1024], 4.0, None),
    ("llama_s8", dict(Hq=32, Hkv=8, D=128), [1024], [1024], 8.0, None),
    ("llama_s16", dict(Hq=32, Hkv=8, D=128), [1024], [1024], 16.0, None),
    ("llama_ramp", dict(Hq=32, Hkv=8, D=128), [1500, 700], [1500, 200], 4.0, 4.0),
    ("gptoss_s8", dict(Hq=64, Hkv=8, D=64, sinks=True), [600, 333], [600, 333], 8.0, None),
    ("gptoss_s16_win", dict(Hq=64, Hkv=8, D=64, window=128, sinks=True), [600], [600], 16.0, None),
    ("gptoss_ramp", dict(Hq=64, Hkv=8, D=64, sinks=True), [900], [900], 4.0, 4.0),
]


@pytest.mark.parametrize("ci", range(len(PREFILL_LOGIT_CASES)), ids=[c[0] for c in PREFILL_LOGIT_CASES])
def test_prefill_large_logits(ci):
    name, prm, lens, qlens, qs, ramp = PREFILL_LOGIT_CASES[ci]
    case = W.make_case(f"pl_{name}", 400 + ci, P(seed=ci, **prm), lens, qlens, split_keys=0,
                       q_scale=qs, k_ramp=ramp)
    g = GpuCase(case)
    ref = O.paged_attention(case.q, case.cu_q, oracle_pool(case), case.block_table, case.seq_lens, case.p)
    n = max(lens)
    # unsplit on the 64-key build (the 32-key build when the window is short), then
    # two KV-split configurations on the 32-key build
    for split in (None, (64, -(-n // 64)), (256, -(-n // 256))):
        got = g.prefill(split=split)
        assert_close(got, ref, BF16_TOL, f"prefill {name} split={split}")


VERIFY_LOGIT_CASES = [
    ("s16", dict(Hq=32, Hkv=8, D=128), [1040, 520], [16, 9], 16.0, None),
    ("ramp", dict(Hq=32, Hkv=8, D=128), [2000, 64], [12, 3], 4.0, 4.0),
    ("gptoss_s8", dict(Hq=64, Hkv=8, D=64, window=128, sinks=True), [709], [9], 8.0, None),
]


@pytest.mark.parametrize("ci", range(len(VERIFY_LOGIT_CASES)), ids=[c[0] for c in VERIFY_LOGIT_CASES])
def test_verify_large_logits(ci):
    name, prm, lens, qlens, qs, ramp = VERIFY_LOGIT_CASES[ci]
    case = W.make_case(f"vl_{name}", 420 + ci, P(seed=ci, **prm), lens, qlens, split_keys=0,
                       q_scale=qs, k_ramp=ramp)
    g = GpuCase(case)
    ref = O.paged_attention(case.q, case.cu_q, oracle_pool(case), case.block_table, case.seq_lens, case.p)
    for split in ("auto", None, (64, -(-max(lens) // 64))):
        assert_close(g.verify(split=split), ref, BF16_TOL, f"verify {name} split={split}")


DECODE_LOGIT_CASES = [
    # (id, params, lens, q_scale, k_ramp); G = 4 and 8, BF16 and INT8 (plain and smoothed)
    ("bf16_g4_s4", dict(Hq=32, Hkv=8, D=128), [300, 1024, 2049], 4.0, None),
    ("bf16_g4_s16", dict(Hq=32, Hkv=8, D=128), [300, 1024, 2049], 16.0, None),
    ("bf16_g4_ramp", dict(Hq=32, Hkv=8, D=128), [700, 3000], 4.0, 4.0),
    ("bf16_g8_s8", dict(Hq=64, Hkv=8, D=64, sinks=True), [100, 1500], 8.0, None),
    ("bf16_g8_s16", dict(Hq=64, Hkv=8, D=64, window=128, sinks=True), [100, 1500], 16.0, None),
    ("bf16_g8_d128_s16", dict(Hq=64, Hkv=8, D=128), [257, 1200], 16.0, None),
    ("bf16_g8_ramp", dict(Hq=64, Hkv=8, D=64), [2500], 4.0, 4.0),
    ("int8_g8_s4", dict(Hq=32, Hkv=4, D=128, kv="int8"), [33, 1000, 2000], 4.0, None),
    ("int8_g8_s8", dict(Hq=32, Hkv=4, D=128, kv="int8"), [33, 1000, 2000], 8.0, None),
    ("int8_g8_s16", dict(Hq=32, Hkv=4, D=128, kv="int8", sinks=True), [33, 1000, 2000], 16.0, None),
    ("int8_g8_ramp", dict(Hq=32, Hkv=4, D=128, kv="int8"), [3000], 4.0, 4.0),
    ("int8_g4_s16", dict(Hq=16, Hkv=4, D=64, kv="int8", window=50), [7, 300], 16.0, None),
]


@pytest.mark.parametrize("ci", range(len(DECODE_LOGIT_CASES)), ids=[c[0] for c in DECODE_LOGIT_CASES])
@pytest.mark.parametrize("smooth", [False, True], ids=["plain", "smoothed"])
def test_decode_large_logits(ci, smooth):
    name, prm, lens, qs, ramp = DECODE_LOGIT_CASES[ci]
    if smooth and prm.get("kv") != "int8":
        pytest.skip("key smoothing is an INT8 cache option")
    kw = dict(q_scale=qs, k_ramp=ramp, outlier_frac=0.01 if prm.get("kv") == "int8" else 0.0)
    if smooth:
        kw["key_weight"] = W.key_norm_weight(440 + ci, prm["D"])
    case = W.make_case(f"dl_{name}", 440 + ci, P(seed=ci, **prm), lens, np.ones(len(lens), np.int32), **kw)
    g = GpuCase(case)
    ref = O.decode(case.q, oracle_pool(case), case.block_table, case.seq_lens, case.p)
    for S in (0, 256, 64):
        assert_close(g.decode(split_keys=S), ref, tol_of(case), f"decode {name} smooth={smooth} S={S}")


# ---------------------------------------------------------------------------
# sliding windows longer than 512 keys: the 64-key prefill build's window path
# (window start tiles skipped, partially visible tiles masked on both edges)
# ---------------------------------------------------------------------------

LONG_WINDOW_CASES = [
    # (id, params, seq_lens, q_lens): prefixes not aligned to a 64-key tile
    ("d128_g4_w700", dict(Hq=32, Hkv=8, D=128, window=700, sinks=True), [2500, 900], [2000, 900]),
    ("d64_g8_w1000", dict(Hq=64, Hkv=8, D=64, window=1000, sinks=True), [2200, 1337], [2200, 37]),
    ("d128_g4_w4096", dict(Hq=32, Hkv=8, D=128, window=4096), [3001], [3001]),
    ("d128_g1_w513", dict(Hq=8, Hkv=8, D=128, window=513), [1600], [1031]),
]


@pytest.mark.parametrize("ci", range(len(LONG_WINDOW_CASES)), ids=[c[0] for c in LONG_WINDOW_CASES])
def test_prefill_long_window(ci):
    name, prm, lens, qlens = LONG_WINDOW_CASES[ci]
    case = W.make_case(f"lw_{name}", 460 + ci, P(seed=ci, **prm), lens, qlens, split_keys=0)
    g = GpuCase(case)
    ref = O.paged_attention(case.q, case.cu_q, oracle_pool(case), case.block_table, case.seq_lens, case.p)
    for split in (None, "auto", (256, -(-max(lens) // 256))):
        assert_close(g.prefill(split=split), ref, BF16_TOL, f"long window {name} split={split}")


# ---------------------------------------------------------------------------
# INT8 value vectors far from unit magnitude, at G = 8 (the paired value path)
# ---------------------------------------------------------------------------

V_MAG_CASES = [
    ("1e-4", [1e-4]),
    ("1", [1.0]),
    ("1e3", [1e3]),
    ("1e4", [1e4]),
    ("mixed", [1e-4, 1.0, 1e3, 1e4]),
    # far ends of the bf16 range: the fp16 weights' exponent follows the value scales
    ("1e-30", [1e-30]),
    ("1e30", [1e30]),
]


V_MAG_SHAPES = [(32, 4, 128), (64, 8, 64)]   # G = 8 at D 128 (head-pair scores) and at D 64


@pytest.mark.parametrize("shape", V_MAG_SHAPES, ids=["d128", "d64"])
@pytest.mark.parametrize("ci", range(len(V_MAG_CASES)), ids=[c[0] for c in V_MAG_CASES])
def test_decode_int8_value_magnitudes(ci, shape):
    """G = 8, INT8 (32 q / 4 KV heads at D 128, 64 / 8 at D 64): the output meets 3e-2
    relative to its own magnitude (max |ref|), with no overflow or flush of the weights."""
    name, mags = V_MAG_CASES[ci]
    Hq, Hkv, D = shape
    case = W.make_case(f"vm_{name}_{D}", 480 + ci + D, P(Hq, Hkv, D, kv="int8", seed=ci), [40, 700, 2100],
                       [1, 1, 1], outlier_frac=0.01, v_mags=mags)
    g = GpuCase(case)
    ref = O.decode(case.q, oracle_pool(case), case.block_table, case.seq_lens, case.p)
    scale = float(np.max(np.abs(ref)))
    for S in (0, 256):
        got = g.decode(split_keys=S)
        assert np.all(np.isfinite(got)), f"value magnitudes {name} S={S}: non-finite output"
        max_abs, rel = errors(got, ref)
        print(f"value magnitudes {name} D={D} S={S}: max_abs/scale={max_abs / scale:.3e} rel_l2={rel:.3e}",
              flush=True)
        assert max_abs <= INT8_TOL["max_abs"] * scale
        # per sequence, against its own magnitude (the mixed case spans 8 decades)
        for b in range(case.batch):
            sb = float(np.max(np.abs(ref[b])))
            assert np.max(np.abs(got[b] - ref[b])) <= INT8_TOL["max_abs"] * sb, f"sequence {b}"


# ---------------------------------------------------------------------------
# INT8 query magnitudes: the INT8 kernels take q in fp16 after a per-head power-
# of-two scale; heads far apart in magnitude, a zero head, and elements far below
# their head's largest (fp16 subnormals after the scale) must not matter
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("G", [8, 4, 1])
def test_decode_int8_query_magnitudes(G):
    Hkv = 4 if G == 8 else 2
    Hq = G * Hkv
    case = W.make_case(f"qm_g{G}", 490 + G, P(Hq, Hkv, 128, kv="int8", seed=G), [77, 1500, 2048],
                       [1, 1, 1], outlier_frac=0.01)
    x = (case.q.astype(np.uint32) << np.uint32(16)).view(np.float32).copy()   # [B, Hq, D]
    exps = np.array([4, -24, 0, -7, 2, -15, 1, -3] * 4)[:Hq].astype(np.float32)
    x *= np.exp2(exps)[None, :, None]
    x[:, 1] = 0.0                                   # a head that is all zero
    x[:, 0, ::17] *= np.float32(2.0 ** -40)         # elements far below their head's largest
    case.q = (x.view(np.uint32) >> np.uint32(16)).astype(np.uint16)   # power-of-two scaling: exact in bf16
    g = GpuCase(case)
    ref = O.decode(case.q, oracle_pool(case), case.block_table, case.seq_lens, case.p)
    for S in (0, 256):
        assert_close(g.decode(split_keys=S), ref, INT8_TOL, f"int8 query magnitudes G={G} S={S}")
