"""Parity at the full workload sizes, in the launch configuration the benchmark
times.  Outputs are compared whole where the oracle is quick.  For the long
prefills the oracle computes sampled query rows one by one: the first and last
rows of the chunk plus seeded random ones.

Workloads:
* decode, 1 sequence at 1024 positions (16 q / 8 KV heads, D 128): split and unsplit;
* batched decode, Qwen3-4B attention (32/8, D 128), batch 32, lengths U[512, 8192];
* causal prefill, Llama-3.1-8B attention (32/8, D 128): 1024, 8192 and 32768
  tokens, and 130 new tokens on a restored 8192-token prefix;
* one sequence decoding at 131072 positions (the longest context here);
* INT8-KV decode, Qwen3-30B-A3B attention (32/4, D 128), batch 8 at 32768 positions,
  and the same shape on the 3-bit rotated cache (pool bit-exact, then decode);
* gpt-oss-20b attention (64/8, D 64, sinks), window-128 and full layers: batch-64
  decode with lengths log-uniform in [128, 32768], and two 2048-token prefills;
* verify steps on Qwen3-4B attention: 16 tokens at 1,024 positions (one sequence),
  and 8 tokens per sequence on batch 32 with contexts U[512, 8192].
"""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from gpu_support import BF16_TOL, GpuCase, assert_close, oracle_pool, pool_bits_equal, tol_of

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _decode_check(case, splits=(256,)):
    print(f"[full] {case.name}: B={case.batch} max_len={int(case.seq_lens.max())}", flush=True)
    g = GpuCase(case)
    ref = O.decode(case.q, oracle_pool(case), case.block_table, case.seq_lens, case.p)
    for S in splits:
        assert_close(g.decode(S), ref, tol_of(case), f"{case.name} S={S}")


def _prefill_check(case, sample=None, seed=0, verify=False):
    print(f"[full] {case.name}: q_tokens={int(case.cu_q[-1])}", flush=True)
    g = GpuCase(case)
    got = g.verify() if verify else g.prefill()
    Tq = int(case.cu_q[-1])
    if sample is None or sample >= Tq:
        rows = np.arange(Tq)
    else:
        rng = np.random.default_rng(seed)
        ends = []
        for s in range(case.batch):
            a, b = int(case.cu_q[s]), int(case.cu_q[s + 1])
            ends += list(range(a, min(a + 16, b))) + list(range(max(a, b - 16), b))
        rows = np.unique(np.concatenate([np.array(ends, np.int64),
                                         rng.choice(Tq, size=sample, replace=False)]))
    ref = O.paged_attention(case.q, case.cu_q, oracle_pool(case), case.block_table, case.seq_lens,
                            case.p, rows=rows, max_rows_per_chunk=64)
    assert_close(got[rows], ref, BF16_TOL, f"{case.name} ({len(rows)} rows)")


def test_decode_1seq_ctx1024():
    _decode_check(W.decode_1seq_ctx1024(), splits=(0, 64, 256))


def test_decode_batch32_ctx512_8192():
    _decode_check(W.decode_batch32_ctx512_8192())


def test_decode_batch32_ctx8192():
    """256-key splits (the workload's), and 1024-key splits (the bench's target-sweep line)."""
    _decode_check(W.decode_batch32_ctx512_8192(fixed_len=8192), splits=(256, 1024))


def test_prefill_causal_1024():
    _prefill_check(W.prefill_llama8b(prompt=1024))


def test_prefill_causal_8192_sampled():
    _prefill_check(W.prefill_llama8b(prompt=8192), sample=224)


def test_prefill_chunk130_on_8192():
    _prefill_check(W.prefill_llama8b(prompt=130, prefix=8192))


def test_decode_1seq_ctx131072():
    """The longest context here: one sequence at 131072 positions (32 q / 8 KV heads,
    D 128), as 512 splits of 256 keys and unsplit (one wave per KV head)."""
    case = W.make_case("decode_1seq_ctx131072", 201, W.AttnParams(32, 8, 128), [131072], [1])
    _decode_check(case, splits=(256, 0))


def test_prefill_causal_32768_sampled():
    """A 32768-token causal prompt (Llama-3.1-8B attention), sampled rows."""
    _prefill_check(W.prefill_llama8b(prompt=32768), sample=256, seed=5)


def test_decode_int8_batch8_ctx32768():
    _decode_check(W.decode_int8_qwen30b())


def test_decode_tq3_batch8_ctx32768():
    """The whole batch runs on the GPU; the oracle (whose fp32 rotation takes about a
    minute for all 8 x 32768 x 4 vectors) checks sequences 0 and 5: their pages bit
    for bit, then their decode outputs."""
    case = W.decode_tq3_qwen30b()
    seqs = [0, 5]
    print(f"[full] {case.name}: B={case.batch} max_len={int(case.seq_lens.max())}, oracle on {seqs}", flush=True)
    g = GpuCase(case)
    got = g.decode(256)
    p = case.p
    pool = O.empty_pool(case.num_pages, p.num_kv_heads, p.page_size, p.head_dim, "tq3")
    bt = case.block_table[seqs]
    lens = case.seq_lens[seqs]
    k = np.concatenate([case.k_tok[case.token_slice(s, 0, int(case.seq_lens[s]))] for s in seqs])
    v = np.concatenate([case.v_tok[case.token_slice(s, 0, int(case.seq_lens[s]))] for s in seqs])
    cu = np.concatenate([[0], np.cumsum(lens)])
    O.kv_write(pool, k, v, cu, lens, bt, p.page_size, "tq3")
    pages = np.unique(np.concatenate([bt[i, : -(-int(lens[i]) // p.page_size)] for i in range(len(seqs))]))
    for name in ("k", "v"):
        assert np.array_equal(getattr(g.pool, name).cpu().numpy()[pages], pool[name][pages]), name
        sc = getattr(g.pool, name + "_scale").cpu().numpy()[pages]
        assert np.array_equal(sc.view(np.uint32), pool[name + "_scale"][pages].view(np.uint32)), name
    ref = O.decode(case.q[seqs], pool, bt, lens, p)
    assert_close(got[seqs], ref, BF16_TOL, f"{case.name} S=256, sequences {seqs}")


@pytest.mark.parametrize("layer", ["window", "full"])
def test_mixed_gptoss_decode(layer):
    # the window layer is benchmarked unsplit
    _decode_check(W.mixed_gptoss(layer=layer, part="decode"), splits=(256, 0) if layer == "window" else (256,))


@pytest.mark.parametrize("layer", ["window", "full"])
def test_mixed_gptoss_prefill(layer):
    _prefill_check(W.mixed_gptoss(layer=layer, part="prefill"), sample=256)


def test_verify_16tok_ctx1024():
    _prefill_check(W.verify_qwen4b(), verify=True)


def test_verify_8tok_batch32_ctx512_8192():
    _prefill_check(W.verify_qwen4b(batch=32, tokens=8, lo=512, hi=8192), verify=True)


def test_attn_input_prompt_8192_bitwise():
    """Fused attention input for an 8192-token prompt (Qwen3-4B shape), bit for bit."""
    from gpu_support import gpu_attn_input, oracle_attn_input, pool_bits_equal
    ic = W.attn_input_qwen4b()
    print(f"[full] {ic.name}", flush=True)
    q, pool = gpu_attn_input(ic)
    q_ref, pool_ref = oracle_attn_input(ic)
    assert np.array_equal(q, q_ref), f"q_out differs in {np.sum(q != q_ref)} elements"
    assert pool_bits_equal(pool, pool_ref, "bf16")


def test_attn_input_decode_batch32_int8_bitwise():
    """One new token for each of 32 sequences at 4096 positions, INT8 pool."""
    from gpu_support import gpu_attn_input, oracle_attn_input, pool_bits_equal
    ic = W.attn_input_case("attn_input_32x1_int8", 9, W.AttnParams(32, 8, 128, kv_dtype="int8"),
                           np.full(32, 4096, np.int32), np.ones(32, np.int32))
    q, pool = gpu_attn_input(ic)
    q_ref, pool_ref = oracle_attn_input(ic)
    assert np.array_equal(q, q_ref)
    assert pool_bits_equal(pool, pool_ref, "int8")

