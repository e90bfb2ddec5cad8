"""Prefill and verify over an INT8 cache (TileInfer.jl Performance, section "INT8
KV cache": prefill runs over the INT8 cache too; Qml-engine announcement: a turn
is prefilled on a restored cache).  The GPU attends over the dequantised cache
(codes x per-vector scales, and per-channel smoothing when the pool has it); the
oracle gathers that same cache in float64.  Bar: max-abs 3e-2 (INT8 KV).

Cases: fresh prompts and chunked turns on restored prefixes, tile edges, GQA
1..32, sliding windows short and long, sinks, sequences with no new tokens, key
smoothing, large logits and keys growing along the sequence; each on the
unsplit 64-key build and on the 32-key KV-split build; verify steps of 2..16
tokens; and at full size, the 130-token chunk on an 8192-token restored prefix.
"""
import numpy as np
import pytest
import torch

import oracle as O
import paged_flash_attention_amd as pfa
import workloads as W
from gpu_support import INT8_TOL, GpuCase, assert_close, main_build_batch, oracle_pool

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    pfa.lib()


def P(Hq, Hkv, D, window=0, sinks=False, seed=0):
    return W.AttnParams(Hq, Hkv, D, kv_dtype="int8", window=window,
                        sinks=W.sinks_normal(seed + 77, Hq) if sinks else None)


INT8_PREFILL_CASES = [
    # (id, params, seq_lens, q_lens, extra make_case args)
    ("fresh_d128_g4", dict(Hq=32, Hkv=8, D=128), [300, 37], [300, 37], {}),
    ("chunk_on_prefix", dict(Hq=32, Hkv=8, D=128), [1500, 64, 1001], [130, 64, 1], {}),
    ("tile_edges", dict(Hq=32, Hkv=8, D=128), [63, 64, 65, 128, 257], [63, 64, 65, 128, 257], {}),
    ("gptoss_window", dict(Hq=64, Hkv=8, D=64, window=128, sinks=True), [517, 300], [200, 300], {}),
    ("gptoss_full", dict(Hq=64, Hkv=8, D=64, sinks=True), [700], [700], {}),
    ("long_window", dict(Hq=32, Hkv=8, D=128, window=700, sinks=True), [2000], [1500], {}),
    ("g1", dict(Hq=8, Hkv=8, D=128, sinks=True), [200], [200], {}),
    ("g16", dict(Hq=32, Hkv=2, D=64), [77], [77], {}),
    ("g32_window", dict(Hq=32, Hkv=1, D=128, window=64), [150], [150], {}),
    ("empty_chunks", dict(Hq=16, Hkv=4, D=128, sinks=True), [100, 50, 200, 9], [10, 0, 64, 0], {}),
    ("window1", dict(Hq=8, Hkv=4, D=64, window=1, sinks=True), [70, 33], [70, 5], {}),
    ("smoothed", dict(Hq=32, Hkv=8, D=128), [600, 90], [400, 90], dict(key_weight="w")),
    ("logits16", dict(Hq=32, Hkv=8, D=128), [700], [700], dict(q_scale=16.0)),
    ("ramp", dict(Hq=64, Hkv=8, D=64, sinks=True), [900], [900], dict(q_scale=4.0, k_ramp=4.0)),
    ("v_range", dict(Hq=32, Hkv=8, D=128), [500], [200], dict(v_mags=[1e-4, 1.0, 1e3])),
]


def _case(name, seed, prm, lens, qlens, extra):
    kw = dict(outlier_frac=0.01, split_keys=0)
    for k, v in extra.items():
        kw[k] = W.key_norm_weight(seed, prm["D"]) if v == "w" else v
    return W.make_case(name, seed, P(seed=seed, **prm), lens, qlens, **kw)


@pytest.mark.parametrize("ci", range(len(INT8_PREFILL_CASES)), ids=[c[0] for c in INT8_PREFILL_CASES])
def test_int8_prefill_parity(ci):
    name, prm, lens, qlens, extra = INT8_PREFILL_CASES[ci]
    case = _case(f"i8p_{name}", 800 + ci, prm, lens, qlens, extra)
    g = GpuCase(case)
    ref = O.paged_attention(case.q, case.cu_q, oracle_pool(case), case.block_table, case.seq_lens, case.p)
    n = max(lens)
    scale = max(1.0, float(np.max(np.abs(ref)))) if "v_mags" in extra else 1.0
    tol = dict(INT8_TOL, max_abs=INT8_TOL["max_abs"] * scale)
    for split in (None, (64, -(-n // 64)), (256, -(-n // 256))):
        got = g.prefill(split=split)
        assert_close(got, ref, tol, f"int8 prefill {name} split={split}")


I8_MAIN_BUILD = [ci for ci, c in enumerate(INT8_PREFILL_CASES) if main_build_batch(c[1], c[2], c[3]) is not None]


@pytest.mark.parametrize("ci", I8_MAIN_BUILD, ids=[INT8_PREFILL_CASES[ci][0] for ci in I8_MAIN_BUILD])
def test_int8_prefill_parity_on_the_256_row_build(ci):
    """As above, the sequences repeated until the unsplit chunk takes the 256-row build."""
    name, prm, lens, qlens, extra = INT8_PREFILL_CASES[ci]
    lens, qlens = main_build_batch(prm, lens, qlens)
    case = _case(f"i8p256_{name}", 860 + ci, prm, lens, qlens, extra)
    g = GpuCase(case)
    ref = O.paged_attention(case.q, case.cu_q, oracle_pool(case), case.block_table, case.seq_lens, case.p)
    scale = max(1.0, float(np.max(np.abs(ref)))) if "v_mags" in extra else 1.0
    tol = dict(INT8_TOL, max_abs=INT8_TOL["max_abs"] * scale)
    assert_close(g.prefill(split=None), ref, tol, f"int8 prefill {name} on the 256-row build ({len(lens)} sequences)")


INT8_VERIFY_CASES = [
    ("16_on_1024", dict(Hq=32, Hkv=8, D=128), [1040], [16], {}),
    ("ragged_2", dict(Hq=32, Hkv=8, D=128), [39, 1002, 300, 2], [2, 2, 2, 2], {}),
    ("gptoss", dict(Hq=64, Hkv=8, D=64, window=128, sinks=True), [709, 3009], [9, 9], {}),
    ("smoothed_logits8", dict(Hq=32, Hkv=4, D=128), [1500, 77], [8, 5], dict(key_weight="w", q_scale=8.0)),
]


@pytest.mark.parametrize("ci", range(len(INT8_VERIFY_CASES)), ids=[c[0] for c in INT8_VERIFY_CASES])
def test_int8_verify_parity(ci):
    name, prm, lens, qlens, extra = INT8_VERIFY_CASES[ci]
    case = _case(f"i8v_{name}", 830 + ci, prm, lens, qlens, extra)
    g = GpuCase(case)
    ref = O.paged_attention(case.q, case.cu_q, oracle_pool(case), case.block_table, case.seq_lens, case.p)
    for split in ("auto", None, (64, -(-max(lens) // 64))):
        assert_close(g.verify(split=split), ref, INT8_TOL, f"int8 verify {name} split={split}")


@pytest.mark.slow
def test_int8_chunk130_on_8192_sampled():
    """Full size: 130 new tokens on an 8192-token restored INT8 prefix (Llama-3.1-8B
    attention shape), the library's split choice; every output row checked."""
    p = W.AttnParams(32, 8, 128, kv_dtype="int8")
    case = W.make_case("i8_chunk130", 860, p, [8322], [130], split_keys=0, outlier_frac=0.01)
    g = GpuCase(case)
    got = g.prefill(split="auto")
    assert g.last_split[1] > 1
    ref = O.paged_attention(case.q, case.cu_q, oracle_pool(case), case.block_table, case.seq_lens, case.p)
    assert_close(got, ref, INT8_TOL, "int8 chunk 130 on 8192")
