"""Device-side setup of a seeded case for the HIP library: copy its arrays to the
GPU, build the library's descriptors, fill a poisoned pool with the library's own
kv_write, and run the library's entry points on it.  Used by the GPU tests and by
the benchmark.  It holds no attention arithmetic and never touches the CPU oracle.
"""
from __future__ import annotations

import numpy as np
import torch

import paged_flash_attention_amd as pfa

from . import AttnInputCase, AttnParams, PagedCase


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def dev_i32(x) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.int32)).cuda()


def bits_of(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def desc_of(p: AttnParams) -> pfa.AttnDesc:
    sinks = None if p.sinks is None else torch.from_numpy(np.asarray(p.sinks, np.float32)).cuda()
    return pfa.AttnDesc(p.num_q_heads, p.num_kv_heads, p.head_dim, p.page_size, p.kv_dtype,
                        p.window, p.sm_scale, sinks)


def poisoned_pool(case: PagedCase) -> pfa.KVPool:
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

    def __init__(self, case: PagedCase, fill=True):
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


def gpu_attn_input(ic: AttnInputCase):
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
