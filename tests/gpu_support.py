"""Helpers for the GPU parity tests: the device-side setup of a case (from
workloads.device: move it to the device, fill a GPU pool with the library's own
kv_write, run decode/combine/prefill through the C ABI), and the oracle's pool
filled the same way on the CPU.  No test lives here."""
from __future__ import annotations

import numpy as np
import torch

import oracle as O
import paged_flash_attention_amd as pfa
import workloads as W
from workloads.device import (GpuCase, bits_of, desc_of, dev_bf16, dev_i32, gpu_attn_input,  # noqa: F401
                              poisoned_pool)

BF16_TOL = dict(max_abs=1e-2, rel_l2=5e-3)
INT8_TOL = dict(max_abs=3e-2, rel_l2=None)


def oracle_pool(case: W.PagedCase) -> dict:
    p = case.p
    pool = O.empty_pool(case.num_pages, p.num_kv_heads, p.page_size, p.head_dim, p.kv_dtype,
                        k_smooth=case.k_smooth)
    k, v, cu = case.prefix_tokens()
    O.kv_write(pool, k, v, cu, case.prefix_lens(), case.block_table, p.page_size, p.kv_dtype)
    k, v, cu = case.new_tokens()
    O.kv_write(pool, k, v, cu, case.seq_lens, case.block_table, p.page_size, p.kv_dtype)
    return pool


def errors(got: np.ndarray, ref: np.ndarray):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    d = got - ref
    max_abs = float(np.max(np.abs(d))) if d.size else 0.0
    rel = float(np.linalg.norm(d) / max(np.linalg.norm(ref), 1e-300)) if d.size else 0.0
    return max_abs, rel


def assert_close(got, ref, tol, what=""):
    assert np.all(np.isfinite(got)), f"{what}: non-finite values in GPU output"
    max_abs, rel = errors(got, ref)
    msg = f"{what}: max_abs={max_abs:.3e} rel_l2={rel:.3e} tol={tol}"
    print(msg, flush=True)
    assert max_abs <= tol["max_abs"], msg
    if tol.get("rel_l2") is not None:
        assert rel <= tol["rel_l2"], msg


def tol_of(case):
    return INT8_TOL if case.p.kv_dtype == "int8" else BF16_TOL


def oracle_attn_input(ic: W.AttnInputCase):
    """The oracle chain on an empty (poisoned) pool.  Returns (q_out bits, pool dict)."""
    c = ic.case
    p = c.p
    pool = O.empty_pool(c.num_pages, p.num_kv_heads, p.page_size, p.head_dim, p.kv_dtype,
                        k_smooth=c.k_smooth)
    q = O.attention_input_to_pool(pool, ic.qkv, ic.q_norm_w, ic.k_norm_w, ic.eps, ic.rope, c.cu_q,
                                  c.seq_lens, c.block_table, p.num_q_heads, p.num_kv_heads, p.head_dim,
                                  p.page_size, p.kv_dtype)
    return q, pool


def pool_bits_equal(gpu_pool: pfa.KVPool, ref: dict, kv_dtype: str):
    """Whole-pool comparison, bit for bit (poison included)."""
    if kv_dtype == "bf16":
        return (np.array_equal(bits_of(gpu_pool.k), ref["k"]) and
                np.array_equal(bits_of(gpu_pool.v), ref["v"]))
    f32 = lambda t: t.cpu().numpy().view(np.uint32)
    return (np.array_equal(gpu_pool.k.cpu().numpy(), ref["k"]) and
            np.array_equal(gpu_pool.v.cpu().numpy(), ref["v"]) and
            np.array_equal(f32(gpu_pool.k_scale), ref["k_scale"].view(np.uint32)) and
            np.array_equal(f32(gpu_pool.v_scale), ref["v_scale"].view(np.uint32)))


def main_build_batch(prm: dict, lens: list, qlens: list):
    """The case's sequences repeated until an unsplit prefill of them has at least
    256 of the 256-row build's query tiles (batch x KV heads x ceil(max_q_len /
    (256 / G))): smaller unsplit chunks run on the 128-row build, so this is how a
    small case reaches the 256-row one.  None for windows of at most 512 keys,
    which always take the 128-row build."""
    if 0 < prm.get("window", 0) <= 512:
        return None
    G = prm["Hq"] // prm["Hkv"]
    tiles = prm["Hkv"] * -(-max(qlens) // (256 // G))
    k = max(1, -(-256 // (len(lens) * tiles)))
    return lens * k, qlens * k

