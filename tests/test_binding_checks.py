"""The Python binding rejects inconsistent tensors before anything is launched:
pool dtypes against the descriptor's kv_dtype, pool and scale shapes against
(Hkv, P, D), q / out / partial-buffer shapes against the batch, the heads and
max_splits, and the batch of block_table against seq_lens and cu arrays.  These
checks run on host tensors (no GPU): the shape and dtype checks come before the
device check, so each error names the offending tensor."""
import pytest
import torch

import paged_flash_attention_amd as pfa

B, HQ, HKV, D, P, NPAGES, STRIDE = 3, 8, 2, 64, 16, 20, 5


def desc(kv="bf16", **kw):
    return pfa.AttnDesc(HQ, HKV, D, P, kv, **kw)


def pool(kv="bf16", hkv=HKV, d=D, scales=True):
    if kv == "bf16":
        k = torch.zeros(NPAGES, hkv, P, d, dtype=torch.bfloat16)
        return pfa.KVPool(k, k.clone())
    dt = torch.int8 if kv == "int8" else torch.uint8
    last = d if kv == "int8" else 3 * d // 8
    k = torch.zeros(NPAGES, hkv, P, last, dtype=dt)
    s = torch.zeros(NPAGES, hkv, P) if scales else None
    return pfa.KVPool(k, k.clone(), s, None if s is None else s.clone())


def i32(*shape):
    return torch.zeros(*shape, dtype=torch.int32)


def bt():
    return i32(B, STRIDE)


def raises(match, fn, *a, **kw):
    with pytest.raises((ValueError, TypeError)) as e:
        fn(*a, **kw)
    msg = str(e.value)
    assert match in msg, msg
    assert "device tensor" not in msg, msg


def test_pool_dtype_must_match_kv_dtype():
    k = torch.zeros(4, HKV, D, dtype=torch.bfloat16)
    raises("k_pool", pfa.kv_write, desc("bf16"), pool("int8"), k, k, i32(B + 1), i32(B), bt())
    raises("k_pool", pfa.kv_write, desc("int8"), pool("bf16"), k, k, i32(B + 1), i32(B), bt())
    raises("k_pool", pfa.kv_write, desc("tq3"), pool("int8"), k, k, i32(B + 1), i32(B), bt())


def test_pool_shape_must_match_the_descriptor():
    k = torch.zeros(4, HKV, D, dtype=torch.bfloat16)
    raises("k_pool", pfa.kv_write, desc(), pool(hkv=HKV * 2), k, k, i32(B + 1), i32(B), bt())
    raises("k_pool", pfa.kv_write, desc(), pool(d=128), k, k, i32(B + 1), i32(B), bt())
    raises("k_scale", pfa.kv_write, desc("int8"), pool("int8", scales=False), k, k, i32(B + 1), i32(B), bt())
    p = pool()
    p.v = torch.zeros(NPAGES + 1, HKV, P, D, dtype=torch.bfloat16)
    raises("v_pool", pfa.kv_write, desc(), p, k, k, i32(B + 1), i32(B), bt())
    p = pool("bf16")
    p.k_smooth = torch.ones(D)
    raises("k_smooth", pfa.kv_write, desc(), p, k, k, i32(B + 1), i32(B), bt())


def test_kv_write_shapes():
    k = torch.zeros(4, HKV, D, dtype=torch.bfloat16)
    raises("k_new", pfa.kv_write, desc(), pool(), torch.zeros(4, HKV + 1, D, dtype=torch.bfloat16), k,
           i32(B + 1), i32(B), bt())
    raises("v_new", pfa.kv_write, desc(), pool(), k, torch.zeros(5, HKV, D, dtype=torch.bfloat16),
           i32(B + 1), i32(B), bt())
    raises("cu_new", pfa.kv_write, desc(), pool(), k, k, i32(B), i32(B), bt())
    raises("seq_lens", pfa.kv_write, desc(), pool(), k, k, i32(B + 1), i32(B + 1), bt())


def test_decode_shapes():
    q = torch.zeros(B, HQ, D, dtype=torch.bfloat16)
    ms = 4
    op, lp = torch.zeros(B, HQ, ms, D), torch.zeros(B, HQ, ms)
    raises("q", pfa.paged_attn_decode, desc(), pool(), torch.zeros(B + 1, HQ, D, dtype=torch.bfloat16), bt(),
           i32(B), 64, 16, ms, op, lp)
    raises("seq_lens", pfa.paged_attn_decode, desc(), pool(), q, bt(), i32(B - 1), 64, 16, ms, op, lp)
    raises("o_part", pfa.paged_attn_decode, desc(), pool(), q, bt(), i32(B), 64, 16, ms,
           torch.zeros(B, HQ, ms - 1, D), lp)
    raises("lse_part", pfa.paged_attn_decode, desc(), pool(), q, bt(), i32(B), 64, 16, ms, op,
           torch.zeros(B, HQ, ms + 1))
    raises("o_part is required", pfa.paged_attn_decode, desc(), pool(), q, bt(), i32(B), 64, 16, ms, None, lp)
    raises("out is required", pfa.paged_attn_decode, desc(), pool(), q, bt(), i32(B), 64, 0, 1)
    raises("out", pfa.paged_attn_decode, desc(), pool(), q, bt(), i32(B), 64, 0, 1, out=torch.zeros(B, HQ, 2 * D))
    raises("q", pfa.paged_attn_decode, desc(), pool(), q.float(), bt(), i32(B), 64, 0, 1, out=torch.zeros(B, HQ, D))


def test_decode_fused_counters():
    q = torch.zeros(B, HQ, D, dtype=torch.bfloat16)
    ms = 4
    op, lp, out = torch.zeros(B, HQ, ms, D), torch.zeros(B, HQ, ms), torch.zeros(B, HQ, D)
    raises("counters", pfa.paged_attn_decode_fused, desc(), pool(), q, bt(), i32(B), 64, 16, ms, op, lp,
           i32(B * HKV - 1), out)
    raises("out", pfa.paged_attn_decode_fused, desc(), pool(), q, bt(), i32(B), 64, 16, ms, op, lp,
           i32(B * HKV), None)


def test_combine_shapes():
    ms = 3
    raises("o_part", pfa.paged_attn_combine, desc(), torch.zeros(B, HQ, ms, D + 1), torch.zeros(B, HQ, ms),
           i32(B), 16, ms, torch.zeros(B, HQ, D))
    raises("lse_part", pfa.paged_attn_combine, desc(), torch.zeros(B, HQ, ms, D), torch.zeros(B, HQ, 1),
           i32(B), 16, ms, torch.zeros(B, HQ, D))
    raises("out", pfa.paged_attn_combine, desc(), torch.zeros(B, HQ, ms, D), torch.zeros(B, HQ, ms),
           i32(B), 16, ms, torch.zeros(B, HQ + 1, D))


@pytest.mark.parametrize("fn", [pfa.paged_attn_prefill, pfa.paged_attn_verify], ids=["prefill", "verify"])
def test_chunk_shapes(fn):
    T = 10
    q = torch.zeros(T, HQ, D, dtype=torch.bfloat16)
    out = torch.zeros(T, HQ, D)
    raises("cu_q", fn, desc(), pool(), q, i32(B), bt(), i32(B), 16, out)
    raises("out", fn, desc(), pool(), q, i32(B + 1), bt(), i32(B), 16, torch.zeros(T + 1, HQ, D))
    raises("q", fn, desc(), pool(), torch.zeros(T, HQ, D // 2, dtype=torch.bfloat16), i32(B + 1), bt(), i32(B),
           16, out)
    raises("o_part is required", fn, desc(), pool(), q, i32(B + 1), bt(), i32(B), 16, out,
           split_keys=64, max_splits=2, lse_part=torch.zeros(T, HQ, 2))
    raises("lse_part", fn, desc(), pool(), q, i32(B + 1), bt(), i32(B), 16, out,
           split_keys=64, max_splits=2, o_part=torch.zeros(T, HQ, 2, D), lse_part=torch.zeros(T, HQ, 3))
    raises("seq_lens", fn, desc(), pool(), q, i32(B + 1), bt(), i32(B + 2), 16, out)


def test_attn_input_shapes():
    T = 6
    width = (HQ + 2 * HKV) * D
    w = torch.ones(D, dtype=torch.bfloat16)
    rope = torch.zeros(100, D // 2, 2)
    qkv = torch.zeros(T, width, dtype=torch.bfloat16)
    q_out = torch.zeros(T, HQ, D, dtype=torch.bfloat16)
    raises("qkv", pfa.attn_input, desc(), pool(), w, w, rope, 1e-6, torch.zeros(T, width - D, dtype=torch.bfloat16),
           i32(B + 1), i32(B), bt(), q_out)
    raises("q_out", pfa.attn_input, desc(), pool(), w, w, rope, 1e-6, qkv, i32(B + 1), i32(B), bt(),
           torch.zeros(T + 1, HQ, D, dtype=torch.bfloat16))
    raises("rope_cos_sin", pfa.attn_input, desc(), pool(), w, w, torch.zeros(100, D, 2), 1e-6, qkv, i32(B + 1),
           i32(B), bt(), q_out)
    raises("k_norm_weight", pfa.attn_input, desc(), pool(), w, torch.ones(D + 1, dtype=torch.bfloat16), rope, 1e-6,
           qkv, i32(B + 1), i32(B), bt(), q_out)
