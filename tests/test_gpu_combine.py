"""The combine kernel (LSE merge of split partials, TileInfer.jl performance page,
"Fused kernels, FlashAttention and PagedAttention") at split counts on both sides
of each launch depth: rows of up to 8, 16, 32, 64 and 128 splits are loaded at
once, longer ones through the chunked merge; and with (row, head) items on both
sides of the launch's slice threshold (a wave per 64-element slice of D, or per
whole row).

The partials are synthetic and seeded: lse values spread over several units, a
leading run of -inf splits per sequence (the splits a window hides, whose o rows
decode never writes: NaN here, so a kernel that read one would show it), -inf
splits in the middle with zero rows (splits no query row of a chunk sees), rows
that are -inf throughout, sinks, and ragged split counts.  Rows past a sequence's
split count are NaN as well.

* Against the oracle's combine, to the atol of the combine test on oracle partials.
* The one-shot merge and the chunked merge give the same bits on the same
  partials (the chunked one is reached by laying them out with more than 128
  splits per row).
"""
import numpy as np
import pytest
import torch

import oracle as O
import paged_flash_attention_amd as pfa

pytestmark = pytest.mark.gpu

S = 16          # split size in keys (one page)
Hq, Hkv = 8, 2
ATOL = 2e-6


def partials(seed, B, ms, D, lens, hidden, sinks):
    """o, lse for the oracle (hidden rows 0) and for the GPU (hidden and unused rows NaN)."""
    rng = np.random.default_rng(seed)
    o = rng.standard_normal((B, Hq, ms, D)).astype(np.float32)
    lse = (rng.standard_normal((B, Hq, ms)) * 2.0 + rng.uniform(-4, 4, (B, Hq, 1))).astype(np.float32)
    o_gpu = o.copy()
    lse_gpu = lse.copy()
    for b in range(B):
        ns = -(-int(lens[b]) // S)
        h = min(hidden[b], ns)
        lse[b, :, :h] = -np.inf
        o[b, :, :h] = 0.0
        if ns - h > 3:                                  # a -inf split in the middle, o written as 0
            i = int(rng.integers(h + 1, ns - 1))
            lse[b, 1, i] = -np.inf
            o[b, 1, i] = 0.0
        lse_gpu[b, :, :ns] = lse[b, :, :ns]
        o_gpu[b, :, :ns] = o[b, :, :ns]
        o_gpu[b, :, :h] = np.nan
        lse_gpu[b, :, ns:] = np.nan
        o_gpu[b, :, ns:] = np.nan
    return o, lse, o_gpu, lse_gpu


def gpu_combine(o_gpu, lse_gpu, lens, ms, D, sinks):
    B = o_gpu.shape[0]
    desc = pfa.AttnDesc(Hq, Hkv, D, sinks=None if sinks is None else torch.from_numpy(sinks).cuda())
    out = torch.full((B, Hq, D), float("nan"), device="cuda")
    pfa.paged_attn_combine(desc, torch.from_numpy(np.ascontiguousarray(o_gpu)).cuda(),
                           torch.from_numpy(np.ascontiguousarray(lse_gpu)).cuda(),
                           torch.tensor(lens, dtype=torch.int32, device="cuda"), S, ms, out)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def case_of(ms):
    """Sequence lengths and leading hidden split counts for max_splits = ms."""
    full = ms * S
    lens = [full, full - 7, 1, max(1, full // 2 + 3), full, full]
    hidden = [0, min(ms - 1, 30), 0, min(ms // 4, 70), min(ms - 1, 70), ms]   # the last row: all -inf
    return np.array(lens, np.int32), hidden


SPLITS = [1, 2, 8, 9, 16, 17, 32, 33, 64, 65, 100, 128, 129, 300]


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("ms", SPLITS)
def test_combine_split_counts_against_oracle(ms, D):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lens, hidden = case_of(ms)
    for with_sinks in (False, True):
        sinks = (np.random.default_rng(ms).standard_normal(Hq) * 2).astype(np.float32) if with_sinks else None
        o, lse, o_gpu, lse_gpu = partials(1000 + ms + D, len(lens), ms, D, lens, hidden, sinks)
        ref = O.combine(o.astype(np.float64), lse.astype(np.float64), lens, S, sinks)
        got = gpu_combine(o_gpu, lse_gpu, lens, ms, D, sinks)
        assert np.isfinite(got).all(), f"ms={ms} D={D} sinks={with_sinks}"
        np.testing.assert_allclose(got, ref, rtol=0, atol=ATOL, err_msg=f"ms={ms} D={D} sinks={with_sinks}")


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("ns_max", [9, 64, 100, 128])
def test_one_shot_and_chunked_merge_give_the_same_bits(ns_max, D):
    """Rows of at most ns_max splits, laid out with max_splits = ns_max (one-shot
    merge) and with max_splits = 200 (chunked merge)."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lens, hidden = case_of(ns_max)
    sinks = (np.random.default_rng(7).standard_normal(Hq) * 2).astype(np.float32)
    _, _, o_gpu, lse_gpu = partials(2000 + ns_max + D, len(lens), ns_max, D, lens, hidden, sinks)
    wide = 200
    o_w = np.full((len(lens), Hq, wide, D), np.nan, np.float32)
    l_w = np.full((len(lens), Hq, wide), np.nan, np.float32)
    o_w[:, :, :ns_max] = o_gpu
    l_w[:, :, :ns_max] = lse_gpu
    short = gpu_combine(o_gpu, lse_gpu, lens, ns_max, D, sinks)
    chunked = gpu_combine(o_w, l_w, lens, wide, D, sinks)
    assert np.array_equal(short.view(np.uint32), chunked.view(np.uint32))


@pytest.mark.parametrize("ms", [9, 33, 64])
def test_whole_row_waves_for_many_rows(ms):
    """1030 rows x 8 heads = 8240 (row, head) items at D = 128: past the launch's
    slice threshold, so one wave takes a whole row (2 elements per lane).  Against
    the oracle, and bit-equal to the chunked merge on the same partials (laid out
    with 129 splits per row)."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    D, B = 128, 1030
    rng = np.random.default_rng(3000 + ms)
    lens = rng.integers(1, ms * S + 1, B).astype(np.int32)
    hidden = list(rng.integers(0, 3, B) * (ms // 4))
    sinks = (rng.standard_normal(Hq) * 2).astype(np.float32)
    o, lse, o_gpu, lse_gpu = partials(4000 + ms, B, ms, D, lens, hidden, sinks)
    ref = O.combine(o.astype(np.float64), lse.astype(np.float64), lens, S, sinks)
    got = gpu_combine(o_gpu, lse_gpu, lens, ms, D, sinks)
    assert np.isfinite(got).all()
    np.testing.assert_allclose(got, ref, rtol=0, atol=ATOL)
    wide = 129
    o_w = np.full((B, Hq, wide, D), np.nan, np.float32)
    l_w = np.full((B, Hq, wide), np.nan, np.float32)
    o_w[:, :, :ms] = o_gpu
    l_w[:, :, :ms] = lse_gpu
    chunked = gpu_combine(o_w, l_w, lens, wide, D, sinks)
    assert np.array_equal(got.view(np.uint32), chunked.view(np.uint32))
