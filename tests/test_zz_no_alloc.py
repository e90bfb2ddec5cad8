"""pfa_paged_attn_decode_static (decode + combine with the split partials in the
library's own device array, allocating nothing) against the existing entry
points, pfa_paged_attn_decode + pfa_paged_attn_combine, and against the oracle.
Two static calls in a row, the second on a smaller input: the array keeps the
first call's partials, which the second must not read."""
import numpy as np
import pytest
import torch

import oracle as O
import paged_flash_attention_amd as pfa
import workloads as W
from gpu_support import GpuCase, assert_close, oracle_pool, tol_of

pytestmark = pytest.mark.gpu


def _case(name, seed, prm, lens, kv="bf16", window=0, sinks=False):
    p = W.AttnParams(*prm, kv_dtype=kv, window=window, sinks=W.sinks_normal(seed, prm[0]) if sinks else None)
    return W.make_case(name, seed, p, lens, np.ones(len(lens), np.int32),
                       outlier_frac=0.01 if kv == "int8" else 0.0)


@pytest.mark.parametrize("kv", ["bf16", "int8"])
def test_static_decode_equals_decode_then_combine(kv):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    big = _case(f"st_big_{kv}", 501, (32, 8, 128), [8000, 1500, 4097, 33, 6000, 700], kv=kv)
    small = _case(f"st_small_{kv}", 502, (32, 8, 128), [300, 17], kv=kv, window=200, sinks=True)
    S = 256
    runs = []
    for case in (big, small):
        g = GpuCase(case)
        plain = g.decode(split_keys=S)          # the existing entry points, caller buffers
        out = torch.full((case.batch, case.p.num_q_heads, case.p.head_dim), float("nan"), device="cuda")
        runs.append((case, g, plain, out))
    # the two static calls back to back: the second reads a smaller part of the array
    for case, g, _, out in runs:
        pfa.paged_attn_decode_static(g.desc, g.pool, g.q, g.bt, g.seq_lens, int(case.seq_lens.max()), S, out)
    torch.cuda.synchronize()
    for case, g, plain, out in runs:
        got = out.cpu().numpy()
        assert np.array_equal(got.view(np.uint32), plain.view(np.uint32)), f"{case.name}: differs from decode+combine"
        ref = O.decode(case.q, oracle_pool(case), case.block_table, case.seq_lens, case.p)
        assert_close(got, ref, tol_of(case), f"{case.name} static")


def test_static_decode_unsplit_and_too_large():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    case = _case("st_unsplit", 503, (64, 8, 64), [129, 2000], window=128, sinks=True)
    g = GpuCase(case)
    plain = g.decode(split_keys=0)
    out = torch.full((case.batch, 64, 64), float("nan"), device="cuda")
    pfa.paged_attn_decode_static(g.desc, g.pool, g.q, g.bt, g.seq_lens, 2000, 0, out)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy().view(np.uint32), plain.view(np.uint32))
    # partials beyond the array: refused, nothing launched, out untouched
    out.fill_(7.0)
    with pytest.raises(pfa.PfaError) as e:
        pfa.paged_attn_decode_static(g.desc, g.pool, g.q, g.bt, g.seq_lens, 2000 * 64, 16, out)
    assert e.value.status == 4
    torch.cuda.synchronize()
    assert bool(torch.all(out == 7.0))
