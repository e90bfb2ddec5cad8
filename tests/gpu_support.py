"""Helpers for the GPU parity tests: move a seeded case to the device, fill a GPU
pool with the library's own kv_write, run decode/combine/prefill through the
C ABI, and fill the oracle's pool the same way on the CPU.  No test lives here."""
from __future__ import annotations

import numpy as np
import torch

import oracle as O
import paged_flash_attention_amd as pfa
import workloads as W

BF16_TOL = dict(max_abs=1e-2, rel_l2=5e-3)
INT8_TOL = dict(max_abs=3e-2, rel_l2=None)


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def dev_i32(x) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.int32)).cuda()


def bits_of(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def desc_of(p: W.AttnParams) -> pfa.AttnDesc:
    sinks = None if p.sinks is None else torch.from_numpy(np.asarray(p.sinks, np.float32)).cuda()
    return pfa.AttnDesc(p.num_q_heads, p.num_kv_heads, p.head_dim, p.page_size, p.kv_dtype,
                        p.window, p.sm_scale, sinks)


def poisoned_pool(case: W.PagedCase) -> pfa.KVPool:
    p = case.p
    shape = (case.num_pages, p.num_kv_heads, p.page_size, p.head_dim)
    if p.kv_dtype == "bf16":
        k = torch.full(shape, float("nan"), dtype=torch.bfloat16, device="cuda")
        return pfa.KVPool(k, k.clone())
    if p.kv_dtype == "tq3":
        k = torch.zeros(shape[:3] + (3 * p.head_dim // 8,), dtype=torch.uint8, device="cuda")
        s = torch.full(shape[:3], float("nan"), dtype=torch.float32, device="cuda")
        return pfa.KVPool(k, k.clone(), s, s.clone())
    k = torch.zeros(shape, dtype=torch.int8, device="cuda")
    s = torch.full(shape[:3], float("nan"), dtype=torch.float32, device="cuda")
    sm = None if case.k_smooth is None else torch.from_numpy(np.asarray(case.k_smooth, np.float32)).cuda()
    return pfa.KVPool(k, k.clone(), s, s.clone(), sm)


class GpuCase:
    """Device copies of a case's inputs, and the pool filled by the GPU kv_write."""

    def __init__(self, case: W.PagedCase, fill=True):
        self.case = case
        self.desc = desc_of(case.p)
        self.bt = dev_i32(case.block_table)
        self.seq_lens = dev_i32(case.seq_lens)
        self.q = dev_bf16(case.q)
        self.cu_q = dev_i32(case.cu_q)
        self.pool = poisoned_pool(case)
        if fill:
            self.write_prefix()
            self.write_new()

    def write_prefix(self):
        k, v, cu = self.case.prefix_tokens()
        if k.shape[0]:
            pfa.kv_write(self.desc, self.pool, dev_bf16(k), dev_bf16(v), dev_i32(cu),
                         dev_i32(self.case.prefix_lens()), self.bt)

    def write_new(self):
        k, v, cu = self.case.new_tokens()
        if k.shape[0]:
            pfa.kv_write(self.desc, self.pool, dev_bf16(k), dev_bf16(v), dev_i32(cu), self.seq_lens, self.bt)

    def decode(self, split_keys=256, max_splits=None, keep_parts=False):
        c = self.case
        B, Hq, D = c.batch, c.p.num_q_heads, c.p.head_dim
        max_len = int(c.seq_lens.max())
        if max_splits is None:
            max_splits = 1 if split_keys == 0 else pfa.decode_num_splits(max_len, split_keys)
        out = torch.full((B, Hq, D), float("nan"), device="cuda")
        if max_splits == 1:
            pfa.paged_attn_decode(self.desc, self.pool, self.q, self.bt, self.seq_lens, max_len, 0, 1, out=out)
            parts = None
        else:
            op = torch.full((B, Hq, max_splits, D), float("nan"), device="cuda")
            lp = torch.full((B, Hq, max_splits), float("nan"), device="cuda")
            pfa.paged_attn_decode(self.desc, self.pool, self.q, self.bt, self.seq_lens, max_len,
                                  split_keys, max_splits, o_part=op, lse_part=lp)
            pfa.paged_attn_combine(self.desc, op, lp, self.seq_lens, split_keys, max_splits, out)
            parts = (op, lp)
        torch.cuda.synchronize()
        if keep_parts:
            return out.cpu().numpy(), parts
        return out.cpu().numpy()

    def decode_fused(self, split_keys=256, calls=2):
        """pfa_paged_attn_decode_fused, `calls` times on one counter array (the later
        calls check that each call leaves the counters zero).  Returns (out, counters)."""
        c = self.case
        B, Hq, D = c.batch, c.p.num_q_heads, c.p.head_dim
        max_len = int(c.seq_lens.max())
        ms = pfa.decode_num_splits(max_len, split_keys)
        ctr = torch.zeros(B * c.p.num_kv_heads, dtype=torch.int32, device="cuda")
        outs = []
        for _ in range(calls):
            out = torch.full((B, Hq, D), float("nan"), device="cuda")
            op = torch.full((B, Hq, ms, D), float("nan"), device="cuda")
            lp = torch.full((B, Hq, ms), float("nan"), device="cuda")
            pfa.paged_attn_decode_fused(self.desc, self.pool, self.q, self.bt, self.seq_lens, max_len,
                                        split_keys, ms, op, lp, ctr, out)
            outs.append(out)
        torch.cuda.synchronize()
        return [o.cpu().numpy() for o in outs], ctr.cpu().numpy()

    def prefill(self, split="auto"):
        """split: "auto" (the library's choice), None (unsplit) or (split_keys, max_splits)."""
        c = self.case
        Tq, Hq, D = int(c.cu_q[-1]), c.p.num_q_heads, c.p.head_dim
        max_q, max_len = int(c.q_lens.max()), int(c.seq_lens.max())
        if split == "auto":
            ms, sk = pfa.prefill_num_splits(self.desc, c.batch, max_q, max_len)
        elif split is None:
            ms, sk = 1, 0
        else:
            sk, ms = split
        out = torch.full((Tq, Hq, D), float("nan"), device="cuda")
        op = lp = None
        if ms > 1:
            op = torch.full((Tq, Hq, ms, D), float("nan"), device="cuda")
            lp = torch.full((Tq, Hq, ms), float("nan"), device="cuda")
        pfa.paged_attn_prefill(self.desc, self.pool, self.q, self.cu_q, self.bt, self.seq_lens, max_q, out,
                               max_seq_len=max_len, split_keys=sk, max_splits=ms, o_part=op, lse_part=lp)
        torch.cuda.synchronize()
        self.last_split = (sk, ms)
        return out.cpu().numpy()


    def verify(self, split="auto"):
        """A verify step over the case's new tokens (<= 16 per sequence); split as in prefill()."""
        c = self.case
        Tq, Hq, D = int(c.cu_q[-1]), c.p.num_q_heads, c.p.head_dim
        max_q, max_len = int(c.q_lens.max()), int(c.seq_lens.max())
        if split == "auto":
            ms, sk = pfa.verify_num_splits(self.desc, c.batch, max_q, max_len)
        elif split is None:
            ms, sk = 1, 0
        else:
            sk, ms = split
        out = torch.full((Tq, Hq, D), float("nan"), device="cuda")
        op = lp = None
        if ms > 1:
            op = torch.full((Tq, Hq, ms, D), float("nan"), device="cuda")
            lp = torch.full((Tq, Hq, ms), float("nan"), device="cuda")
        pfa.paged_attn_verify(self.desc, self.pool, self.q, self.cu_q, self.bt, self.seq_lens, max_q, out,
                              max_seq_len=max_len, split_keys=sk, max_splits=ms, o_part=op, lse_part=lp)
        torch.cuda.synchronize()
        self.last_split = (sk, ms)
        return out.cpu().numpy()


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


def gpu_attn_input(ic: W.AttnInputCase):
    """pfa_attn_input on a poisoned pool.  Returns (q_out bits, pool)."""
    c = ic.case
    p = c.p
    T = int(c.cu_q[-1])
    pool = poisoned_pool(c)
    q_out = torch.empty((T, p.num_q_heads, p.head_dim), dtype=torch.bfloat16, device="cuda")
    pfa.attn_input(desc_of(p), pool, dev_bf16(ic.q_norm_w), dev_bf16(ic.k_norm_w),
                   torch.from_numpy(ic.rope).cuda(), ic.eps, dev_bf16(ic.qkv), dev_i32(c.cu_q),
                   dev_i32(c.seq_lens), dev_i32(c.block_table), q_out)
    torch.cuda.synchronize()
    return bits_of(q_out), pool


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
