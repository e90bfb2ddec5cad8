"""A seeded random sweep of mixed configurations against the CPU float64 oracle.

The hand-picked parity cases pin each feature on its own; this sweep draws
configurations that combine them (operation, head dim, GQA group, KV dtype, window,
sinks, ragged lengths, split size) to catch interactions those cases miss.  Each
case is drawn from its own seed, so a failure names a reproducible configuration.
The draws stay inside the library's documented limits and sizes the oracle finishes
in about a second.  Draws 30 and on also put prefill and verify on INT8 caches.
"""
import numpy as np
import pytest
import torch

import oracle as O
import paged_flash_attention_amd as pfa
import workloads as W
from gpu_support import BF16_TOL, GpuCase, assert_close, oracle_pool, pool_bits_equal, tol_of

pytestmark = pytest.mark.gpu

N_CASES = 60
OPS = ("decode", "decode", "fused", "prefill", "verify")
INT8_PREFILL_FROM = 30     # draws from here on also put prefill and verify on an INT8 cache


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    pfa.lib()


def draw(i):
    """Configuration i of the sweep: (op, params dict, seq_lens, q_lens, split choice)."""
    rng = np.random.default_rng(5000 + i)
    op = OPS[i % len(OPS)]
    D = int(rng.choice([64, 128]))
    if op in ("prefill", "verify"):
        kv = "bf16"
        G = int(rng.choice([1, 2, 4, 8, 16, 32]))
        if i >= INT8_PREFILL_FROM:
            kv = str(rng.choice(["bf16", "int8"]))
    else:
        kv = str(rng.choice(["bf16", "int8", "tq3"] if op == "decode" else ["bf16", "int8"]))
        G = int(rng.choice([1, 2, 4, 8]))
    Hkv = int(rng.choice([h for h in (1, 2, 4, 8) if h * G <= 64]))
    window = int(rng.integers(1, 400)) if rng.random() < 0.4 else 0
    sinks = bool(rng.random() < 0.5)
    batch = int(rng.integers(1, 9))
    # lengths: a mix of short, page-edge and long ones
    lens = rng.integers(1, 2000, batch)
    edge = rng.random(batch) < 0.3
    lens[edge] = 16 * rng.integers(1, 64, int(edge.sum())) + rng.integers(-1, 2, int(edge.sum()))
    lens = np.maximum(lens, 1)
    if op in ("decode", "fused"):
        qlens = np.ones(batch, np.int64)
        split = int(rng.choice([0, 16, 32, 64, 256, 1024])) if op == "decode" else int(rng.choice([16, 64, 256]))
    elif op == "prefill":
        lens = np.minimum(lens, 1200)
        qlens = np.array([int(rng.integers(0, min(int(n), 300) + 1)) for n in lens])
        if qlens.max() == 0:
            qlens[0] = lens[0]
        split = str(rng.choice(["auto", "none", "split"]))
    else:
        qlens = np.array([int(rng.integers(2, 17)) for _ in lens])
        lens = np.maximum(lens, qlens)
        split = str(rng.choice(["auto", "none", "split"]))
    prm = dict(Hq=Hkv * G, Hkv=Hkv, D=D, kv=kv, window=window, sinks=sinks)
    return op, prm, [int(x) for x in lens], [int(x) for x in qlens], split


def _name(i):
    op, prm, lens, qlens, split = draw(i)
    return (f"{i}-{op}-{prm['kv']}-D{prm['D']}-G{prm['Hq'] // prm['Hkv']}-Hkv{prm['Hkv']}"
            f"-w{prm['window']}-s{int(prm['sinks'])}-b{len(lens)}-{split}")


@pytest.mark.parametrize("i", range(N_CASES), ids=_name)
def test_random_config(i):
    op, prm, lens, qlens, split = draw(i)
    print(f"case {_name(i)} lens={lens} qlens={qlens}", flush=True)
    p = W.AttnParams(prm["Hq"], prm["Hkv"], prm["D"], kv_dtype=prm["kv"], window=prm["window"],
                     sinks=W.sinks_normal(7000 + i, prm["Hq"]) if prm["sinks"] else None)
    case = W.make_case(f"rnd{i}", 6000 + i, p, lens, qlens, split_keys=0,
                       outlier_frac=0.01 if prm["kv"] != "bf16" else 0.0)
    g = GpuCase(case)
    pool = oracle_pool(case)
    if prm["kv"] != "bf16":
        assert pool_bits_equal(g.pool, pool, prm["kv"]), "quantised pool differs"
    ref = O.paged_attention(case.q, case.cu_q, pool, case.block_table, case.seq_lens, case.p)
    tol = tol_of(case)
    if op == "decode":
        got = g.decode(split_keys=split)
        assert_close(got.reshape(ref.shape), ref, tol, f"decode S={split}")
    elif op == "fused":
        outs, ctr = g.decode_fused(split_keys=split)
        assert np.all(ctr == 0), "fused decode left a counter non-zero"
        for k, got in enumerate(outs):
            assert_close(got.reshape(ref.shape), ref, tol, f"fused decode S={split} call {k}")
    else:
        max_len = max(lens)
        sp = {"auto": "auto", "none": None, "split": (64, -(-max_len // 64))}[split]
        got = g.prefill(split=sp) if op == "prefill" else g.verify(split=sp)
        assert_close(got, ref, tol, f"{op} split={split}")
