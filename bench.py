"""Benchmark of the paged flash attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

The default workload is batched decode with Qwen3-4B attention: 32 q / 8 KV heads,
D 128, batch 32, lengths U[512, 8192], 16-token pages, 256-key splits.  One step
is the whole decode hot path for one batch:
  1. kv_write of the batch's new token;
  2. split-KV paged decode;
  3. combine.
Inputs sit in HBM before the timed region starts.  Every step reads one of several
identical pool copies in rotation, about 2 GiB in total, so the reads come from HBM
rather than the 256 MB MALL.

Exactly one JSON line is printed on stdout.  Its fields:
* value: the step's algorithmic bytes / step time, in GB/s.  The bytes are the
  visible K/V, q, out, the block-table entries, and the new tokens written.
* roofline: the decode kernel alone, with its average launch time measured by HIP
  events on its stream, against the 8 TB/s HBM peak.
* cpu_baseline: the CPU float64 oracle on the same workload.
* workloads: the other headline workloads of the same hot path, each with its own
  metric: prefill TFLOP/s, INT8 decode, and the gpt-oss mixed batch.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
ROTATE_BYTES = 2 << 30         # pool copies rotated across steps


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ---------------------------------------------------------------------------
# algorithmic work
# ---------------------------------------------------------------------------

def visible_keys(lens, window):
    lens = np.asarray(lens, np.int64)
    return np.minimum(lens, window) if window > 0 else lens


def kv_bytes_per_key_head(p) -> int:
    """Cached bytes of one key and its value for one KV head: bf16 elements, or int8
    codes + two fp32 scales, or 3-bit planes (3D/8 bytes) + two fp32 scales."""
    if p.kv_dtype == "int8":
        return 2 * p.head_dim + 8
    if p.kv_dtype == "tq3":
        return 2 * (3 * p.head_dim // 8 + 4)
    return 2 * p.head_dim * 2


def decode_bytes(case) -> int:
    """Visible K/V (+ scales for INT8 and 3-bit) + q + out + block-table entries of the decode."""
    p = case.p
    vis = visible_keys(case.seq_lens, p.window)
    per_key = p.num_kv_heads * kv_bytes_per_key_head(p)
    kv = int(vis.sum()) * per_key
    q = case.batch * p.num_q_heads * p.head_dim * 2
    out = case.batch * p.num_q_heads * p.head_dim * 4
    lens = np.asarray(case.seq_lens, np.int64)
    lo = np.maximum(0, lens - p.window) if p.window > 0 else np.zeros_like(lens)
    bt = int(((lens - 1) // p.page_size - lo // p.page_size + 1).sum()) * 4
    return kv + q + out + bt


def verify_bytes(case) -> int:
    """Bytes a verify step (or any chunk) must move at least: every visible K/V byte
    once per (sequence, KV head), the chunk's q and fp32 out, the block-table entries."""
    p = case.p
    vis = visible_keys(case.seq_lens, p.window)
    kv = int(vis.sum()) * p.num_kv_heads * kv_bytes_per_key_head(p)
    T = int(case.q_lens.sum())
    return kv + T * p.num_q_heads * p.head_dim * (2 + 4) + int((np.asarray(case.seq_lens) + 15).sum() // 16) * 4


def kv_write_bytes(case) -> int:
    p = case.p
    T = int(case.q_lens.sum())
    rd = T * p.num_kv_heads * p.head_dim * 2 * 2
    wr = T * p.num_kv_heads * kv_bytes_per_key_head(p)
    return rd + wr


def prefill_flops(case) -> float:
    """4*D*Hq per visible (query, key) pair: only causal/window-visible pairs count."""
    p = case.p
    total = 0
    for s in range(case.batch):
        n, ql = int(case.seq_lens[s]), int(case.q_lens[s])
        pos = np.arange(n - ql, n, dtype=np.int64)
        vis = pos + 1
        if p.window > 0:
            vis = np.minimum(vis, p.window)
        total += int(vis.sum())
    return 4.0 * p.head_dim * p.num_q_heads * total


def src_digest(*names) -> str:
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "paged_flash_attention_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str, digest: str):
    """HBM bytes per launch from a committed rocprofv3 counter summary, if it was
    taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f).get(kernel)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("src_digest") != digest:
        return None
    return rec.get("bytes_per_launch")


# ---------------------------------------------------------------------------
# GPU legs
# ---------------------------------------------------------------------------

class Timer:
    """HIP events around single kernels on the current stream.  Disabled, it records
    nothing: a multi-kernel step's timed region runs without them, since each event
    record between two kernels adds a gap of its own (about 12 us per headline
    decode step: 145.4 vs 133.6 us), and the kernels are timed in a pass of their own."""
    def __init__(self, torch):
        self.torch = torch
        self.pairs = {}
        self.enabled = True

    def mark(self, name):
        if not self.enabled:
            return None
        e0 = self.torch.cuda.Event(enable_timing=True)
        e0.record()
        return e0

    def close(self, name, e0):
        if e0 is None:
            return
        e1 = self.torch.cuda.Event(enable_timing=True)
        e1.record()
        self.pairs.setdefault(name, []).append((e0, e1))

    def mean_ms(self, name):
        ps = self.pairs.get(name, [])
        return sum(a.elapsed_time(b) for a, b in ps) / max(1, len(ps))

    def reset(self):
        self.pairs = {}


def setup_case(case, torch, pfa, gs, copies_for_bytes=ROTATE_BYTES):
    g = gs.GpuCase(case)
    pool_bytes = sum(t.numel() * t.element_size() for t in (g.pool.k, g.pool.v, g.pool.k_scale, g.pool.v_scale)
                     if t is not None)
    n_copies = max(1, min(16, int(math.ceil(copies_for_bytes / max(pool_bytes, 1)))))
    pools = [g.pool] + [pfa.KVPool(*(None if t is None else t.clone() for t in
                                     (g.pool.k, g.pool.v, g.pool.k_scale, g.pool.v_scale)))
                        for _ in range(n_copies - 1)]
    k, v, cu = case.new_tokens()
    new = (gs.dev_bf16(k), gs.dev_bf16(v), gs.dev_i32(cu))
    torch.cuda.synchronize()
    return g, pools, new


def run_decode(case, torch, pfa, gs, steps, warmup, fused=False):
    """Decode steps: kv_write + split decode + combine, or with fused=True kv_write +
    pfa_paged_attn_decode_fused (the combine merged into the split kernel).  The timed
    region runs `steps` bare steps (the step time); a second pass of `steps` more
    steps, each kernel between HIP events, gives the kernels' own durations."""
    g, pools, (kn, vn, cun) = setup_case(case, torch, pfa, gs)
    p = case.p
    B, Hq, D = case.batch, p.num_q_heads, p.head_dim
    max_len = int(case.seq_lens.max())
    S = case.split_keys
    ms = pfa.decode_num_splits(max_len, S) if S > 0 else 1   # S = 0: unsplit, no combine
    op = torch.empty((B, Hq, ms, D), device="cuda")
    lp = torch.empty((B, Hq, ms), device="cuda")
    out = torch.empty((B, Hq, D), device="cuda")
    ctr = torch.zeros(B * p.num_kv_heads, dtype=torch.int32, device="cuda")
    tm = Timer(torch)

    def step(i):
        pool = pools[i % len(pools)]
        pfa.kv_write(g.desc, pool, kn, vn, cun, g.seq_lens, g.bt)
        e = tm.mark("decode")
        if fused:
            pfa.paged_attn_decode_fused(g.desc, pool, g.q, g.bt, g.seq_lens, max_len, S, ms, op, lp, ctr, out)
            tm.close("decode", e)
            return
        if S == 0:
            pfa.paged_attn_decode(g.desc, pool, g.q, g.bt, g.seq_lens, max_len, 0, 1, out=out)
            tm.close("decode", e)
            return
        pfa.paged_attn_decode(g.desc, pool, g.q, g.bt, g.seq_lens, max_len, S, ms, o_part=op, lse_part=lp)
        tm.close("decode", e)
        e = tm.mark("combine")
        pfa.paged_attn_combine(g.desc, op, lp, g.seq_lens, S, ms, out)
        tm.close("combine", e)

    tm.enabled = False
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for i in range(steps):
        step(warmup + i)
    t1.record()
    torch.cuda.synchronize()
    step_ms = t0.elapsed_time(t1) / steps
    tm.enabled = True
    for i in range(steps):
        step(warmup + steps + i)
    torch.cuda.synchronize()
    dec_ms = tm.mean_ms("decode")
    r = dict(step_ms=step_ms, decode_ms=dec_ms, pool_copies=len(pools),
             decode_bytes=decode_bytes(case), step_bytes=decode_bytes(case) + kv_write_bytes(case),
             partial_bytes=int(B * Hq * ms * (D + 1) * 4))
    if not fused and S > 0:
        cms = tm.mean_ms("combine")
        cb = combine_bytes(case)
        r.update(combine_us=round(cms * 1e3, 2), combine_bytes=cb,
                 combine_gbs=round(cb / (cms * 1e-3) / 1e9, 1))
    return r


def combine_bytes(case) -> int:
    """The combine's algorithmic bytes: per (sequence, q head), the lse and o row of
    each split its length covers, read once, and the fp32 output row written."""
    p = case.p
    S = case.split_keys
    ns = (np.asarray(case.seq_lens, np.int64) + S - 1) // S
    return int(ns.sum()) * p.num_q_heads * (p.head_dim + 1) * 4 + case.batch * p.num_q_heads * p.head_dim * 4


def run_kv_write(case, torch, pfa, gs, steps, warmup):
    """KV writes of the case's new tokens alone, each into the next of a set of poisoned
    pools and from the next of a set of input copies (together >= 1 GiB, so the 256 MB
    MALL serves neither side)."""
    g = gs.GpuCase(case, fill=False)
    k, v, cu = case.new_tokens()
    per_call = sum(t.numel() * t.element_size() for t in (g.pool.k, g.pool.v, g.pool.k_scale, g.pool.v_scale)
                   if t is not None) + 2 * k.size * 2
    n = max(2, min(16, int(math.ceil((1 << 30) / per_call))))
    pools = [g.pool] + [pfa.KVPool(*(None if t is None else t.clone() for t in
                                     (g.pool.k, g.pool.v, g.pool.k_scale, g.pool.v_scale)))
                        for _ in range(n - 1)]
    ins = [(gs.dev_bf16(k), gs.dev_bf16(v)) for _ in range(n)]
    cun = gs.dev_i32(cu)
    tm = Timer(torch)

    def step(i):
        kn, vn = ins[i % n]
        e = tm.mark("kv_write")
        pfa.kv_write(g.desc, pools[i % n], kn, vn, cun, g.seq_lens, g.bt)
        tm.close("kv_write", e)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    tm.reset()
    for i in range(steps):
        step(warmup + i)
    torch.cuda.synchronize()
    ms = tm.mean_ms("kv_write")
    return dict(step_ms=ms, kv_write_ms=ms, kv_write_bytes=kv_write_bytes(case), copies=n)


def attn_input_bytes(ic) -> int:
    """Algorithmic HBM bytes of one fused attention-input launch: the qkv rows, the
    RoPE table row of each token, q out, and k/v (codes + scales for INT8) in."""
    c = ic.case
    p = c.p
    T = int(c.cu_q[-1])
    D, Hq, Hkv = p.head_dim, p.num_q_heads, p.num_kv_heads
    kv = 2 * Hkv * (D * (1 if p.kv_dtype == "int8" else 2) + (4 if p.kv_dtype == "int8" else 0))
    return T * ((Hq + 2 * Hkv) * D * 2 + (D // 2) * 8 + Hq * D * 2 + kv)


def run_attn_input(ic, torch, pfa, gs, steps, warmup):
    """Fused attention-input launches over rotating qkv copies (>= 1 GiB in all when
    the rows are large, so the 256 MB MALL does not serve them)."""
    c = ic.case
    p = c.p
    T = int(c.cu_q[-1])
    desc = gs.desc_of(p)
    pool = gs.poisoned_pool(c)
    qkv0 = gs.dev_bf16(ic.qkv)
    copies = max(1, min(8, -(-(1 << 30) // max(1, qkv0.numel() * 2))))
    qkvs = [qkv0] + [qkv0.clone() for _ in range(copies - 1)]
    qw, kw = gs.dev_bf16(ic.q_norm_w), gs.dev_bf16(ic.k_norm_w)
    rope = torch.from_numpy(ic.rope).cuda()
    cu, sl, bt = gs.dev_i32(c.cu_q), gs.dev_i32(c.seq_lens), gs.dev_i32(c.block_table)
    q_out = torch.empty((T, p.num_q_heads, p.head_dim), dtype=torch.bfloat16, device="cuda")
    tm = Timer(torch)

    def step(i):
        e = tm.mark("attn_input")
        pfa.attn_input(desc, pool, qw, kw, rope, ic.eps, qkvs[i % len(qkvs)], cu, sl, bt, q_out)
        tm.close("attn_input", e)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    tm.reset()
    for i in range(steps):
        step(warmup + i)
    torch.cuda.synchronize()
    ms = tm.mean_ms("attn_input")
    return dict(step_ms=ms, attn_input_ms=ms, bytes=attn_input_bytes(ic), copies=len(qkvs))


def run_prefill(case, torch, pfa, gs, steps, warmup, verify=False):
    """Prefill steps (kv_write + prefill), or with verify=True verify steps (kv_write
    + pfa_paged_attn_verify), on the library's split choice.  Steps rotate over pool
    copies (about 2 GiB in all, at most 16), so a short chunk on a long prefix reads
    its prefix from HBM rather than from the 256 MB MALL.  The timed region runs
    `steps` bare steps; a second pass of `steps` more, the attention kernel(s)
    between HIP events, gives their own duration."""
    g, pools, (kn, vn, cun) = setup_case(case, torch, pfa, gs)
    p = case.p
    Tq = int(case.cu_q[-1])
    out = torch.empty((Tq, p.num_q_heads, p.head_dim), device="cuda")
    max_q, max_len = int(case.q_lens.max()), int(case.seq_lens.max())
    ms, sk = (pfa.verify_num_splits if verify else pfa.prefill_num_splits)(g.desc, case.batch, max_q, max_len)
    attn = pfa.paged_attn_verify if verify else pfa.paged_attn_prefill
    op = lp = None
    if ms > 1:
        op = torch.empty((Tq, p.num_q_heads, ms, p.head_dim), device="cuda")
        lp = torch.empty((Tq, p.num_q_heads, ms), device="cuda")
    tm = Timer(torch)

    def step(i):
        pool = pools[i % len(pools)]
        pfa.kv_write(g.desc, pool, kn, vn, cun, g.seq_lens, g.bt)
        e = tm.mark("prefill")
        attn(g.desc, pool, g.q, g.cu_q, g.bt, g.seq_lens, max_q, out, max_seq_len=max_len,
             split_keys=sk, max_splits=ms, o_part=op, lse_part=lp)
        tm.close("prefill", e)

    tm.enabled = False
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for i in range(steps):
        step(warmup + i)
    t1.record()
    torch.cuda.synchronize()
    tm.enabled = True
    for i in range(steps):
        step(warmup + steps + i)
    torch.cuda.synchronize()
    return dict(step_ms=t0.elapsed_time(t1) / steps, prefill_ms=tm.mean_ms("prefill"),
                flops=prefill_flops(case), split_keys=sk, max_splits=ms, kv_bytes=verify_bytes(case),
                pool_copies=len(pools))


def run_verify_graph(case, torch, pfa, gs, steps, warmup):
    """The verify step (kv_write + pfa_paged_attn_verify on the library's split, with
    its combine) captured once in a HIP graph and replayed: the step as a serving loop
    that replays graphs runs it, without host launch gaps."""
    g, _, (kn, vn, cun) = setup_case(case, torch, pfa, gs, copies_for_bytes=0)
    p = case.p
    Tq = int(case.cu_q[-1])
    out = torch.empty((Tq, p.num_q_heads, p.head_dim), device="cuda")
    max_q, max_len = int(case.q_lens.max()), int(case.seq_lens.max())
    ms, sk = pfa.verify_num_splits(g.desc, case.batch, max_q, max_len)
    op = lp = None
    if ms > 1:
        op = torch.empty((Tq, p.num_q_heads, ms, p.head_dim), device="cuda")
        lp = torch.empty((Tq, p.num_q_heads, ms), device="cuda")

    def step():
        pfa.kv_write(g.desc, g.pool, kn, vn, cun, g.seq_lens, g.bt)
        pfa.paged_attn_verify(g.desc, g.pool, g.q, g.cu_q, g.bt, g.seq_lens, max_q, out,
                              max_seq_len=max_len, split_keys=sk, max_splits=ms, o_part=op, lse_part=lp)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for _ in range(warmup):
        graph.replay()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(steps):
        graph.replay()
    t1.record()
    torch.cuda.synchronize()
    return dict(step_ms=t0.elapsed_time(t1) / steps, split_keys=sk, max_splits=ms, kv_bytes=verify_bytes(case))


def run_decode_graph(case, torch, pfa, gs, steps, warmup, fused=False):
    """The decode step (kv_write + split decode + combine, or with fused=True kv_write +
    the fused decode) captured once in a HIP graph and replayed: the step without host
    launch gaps, which dominate a one-sequence step.  One pool (its 16 MB stay in the
    MALL between replays)."""
    g, _, (kn, vn, cun) = setup_case(case, torch, pfa, gs, copies_for_bytes=0)
    p = case.p
    B, Hq, D = case.batch, p.num_q_heads, p.head_dim
    max_len = int(case.seq_lens.max())
    S = case.split_keys
    ms = pfa.decode_num_splits(max_len, S)
    op = torch.empty((B, Hq, ms, D), device="cuda")
    lp = torch.empty((B, Hq, ms), device="cuda")
    out = torch.empty((B, Hq, D), device="cuda")
    ctr = torch.zeros(B * p.num_kv_heads, dtype=torch.int32, device="cuda")

    def step():
        pfa.kv_write(g.desc, g.pool, kn, vn, cun, g.seq_lens, g.bt)
        if fused:
            pfa.paged_attn_decode_fused(g.desc, g.pool, g.q, g.bt, g.seq_lens, max_len, S, ms, op, lp, ctr, out)
            return
        pfa.paged_attn_decode(g.desc, g.pool, g.q, g.bt, g.seq_lens, max_len, S, ms, o_part=op, lse_part=lp)
        pfa.paged_attn_combine(g.desc, op, lp, g.seq_lens, S, ms, out)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for _ in range(warmup):
        graph.replay()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(steps):
        graph.replay()
    t1.record()
    torch.cuda.synchronize()
    return dict(step_ms=t0.elapsed_time(t1) / steps, split_keys=S, max_splits=ms, decode_bytes=decode_bytes(case))


# ---------------------------------------------------------------------------
# CPU baseline: the oracle as it stands
# ---------------------------------------------------------------------------

def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline_decode(case, min_s=10.0, budget_s=25.0):
    import oracle as O
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        cores = 1
    p = case.p
    pool = O.empty_pool(case.num_pages, p.num_kv_heads, p.page_size, p.head_dim, p.kv_dtype)
    k, v, cu = case.prefix_tokens()
    O.kv_write(pool, k, v, cu, case.prefix_lens(), case.block_table, p.page_size, p.kv_dtype)
    kn, vn, cun = case.new_tokens()
    # timed: the oracle's own step (kv_write of the new tokens + decode), sequence
    # by sequence; whole passes over the batch repeat until min_s has passed, and a
    # pass stops early once budget_s is spent (at least one sequence).  Rewriting a
    # token into its own slot is idempotent, so every pass is the same work.
    t_start = time.perf_counter()
    seqs, passes = 0, 0
    nbytes = 0
    import copy

    def bytes_of(n):
        sub = copy.copy(case)
        sub.seq_lens = case.seq_lens[:n]
        sub.q_lens = case.q_lens[:n]
        return decode_bytes(sub) + kv_write_bytes(sub)

    while True:
        done = 0
        for s in range(case.batch):
            sl = slice(int(cun[s]), int(cun[s + 1]))
            O.kv_write(pool, kn[sl], vn[sl], np.array([0, sl.stop - sl.start]), case.seq_lens[s:s + 1],
                       case.block_table[s:s + 1], p.page_size, p.kv_dtype)
            O.decode(case.q[s:s + 1], pool, case.block_table[s:s + 1], case.seq_lens[s:s + 1], p)
            done += 1
            if time.perf_counter() - t_start > budget_s:
                break
        seqs += done
        nbytes += bytes_of(done)
        passes += 1
        if done < case.batch or time.perf_counter() - t_start >= min_s:
            break
    elapsed = time.perf_counter() - t_start
    return dict(value=round(nbytes / elapsed / 1e9, 4), unit="GB/s", cores=int(cores), kind="oracle",
                cpu_count=os.cpu_count(), affinity=len(os.sched_getaffinity(0)), cpu_model=cpu_model(),
                sample=f"{seqs} sequence-steps ({passes} pass(es) over the {case.batch} sequences of the same "
                       f"batch; kv_write of the new token + materialised-softmax decode, float64 numpy), "
                       f"{elapsed:.1f} s")


# ---------------------------------------------------------------------------

def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="decode_batch32_ctx512_8192")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true", help="skip the other headline workloads")
    ap.add_argument("--copy-probe", type=int, default=0,
                    help="only run N plain 1 GiB device copies (counter calibration) and exit")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(sharding is described in the design notes, not run).", file=sys.stderr)
        sys.exit(2)

    import torch
    import paged_flash_attention_amd as pfa
    import workloads as W
    import workloads.device as gs

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    pfa.lib()

    if args.copy_probe:
        a = torch.empty(1 << 28, dtype=torch.float32, device="cuda")   # 1 GiB
        b = torch.empty_like(a)
        a.fill_(1.0)
        torch.cuda.synchronize()
        for _ in range(args.copy_probe):
            b.copy_(a)
        torch.cuda.synchronize()
        log(f"copy probe: {args.copy_probe} x 1 GiB device copies")
        return

    builders = {
        "decode_batch32_ctx512_8192": lambda: W.decode_batch32_ctx512_8192(),
        "decode_batch32_ctx8192": lambda: W.decode_batch32_ctx512_8192(fixed_len=8192),
        "decode_batch32_ctx8192_s1024": lambda: W.decode_batch32_ctx512_8192(fixed_len=8192, split_keys=1024),
        "decode_batch32_ctx512_8192_fused": lambda: W.decode_batch32_ctx512_8192(),
        "decode_1seq_ctx1024": lambda: W.decode_1seq_ctx1024(),
        "decode_1seq_ctx1024_graph": lambda: W.decode_1seq_ctx1024(),
        "decode_1seq_ctx1024_fused": lambda: W.decode_1seq_ctx1024(),
        "decode_1seq_ctx1024_fused_graph": lambda: W.decode_1seq_ctx1024(),
        "decode_int8_batch8_ctx32768": lambda: W.decode_int8_qwen30b(),
        "decode_int8_batch8_ctx32768_smooth": lambda: W.decode_int8_qwen30b(smooth=True),
        "decode_tq3_batch8_ctx32768": lambda: W.decode_tq3_qwen30b(),
        "kv_write_bf16_8192": lambda: W.kv_write_prompt("bf16"),
        "kv_write_int8_8192": lambda: W.kv_write_prompt("int8"),
        "kv_write_tq3_8192": lambda: W.kv_write_prompt("tq3"),
        "mixed_full_decode_b64": lambda: W.mixed_gptoss(layer="full", part="decode"),
        "mixed_window_decode_b64": lambda: W.mixed_gptoss(layer="window", part="decode"),
        "prefill_causal_8192": lambda: W.prefill_llama8b(prompt=8192),
        "prefill_causal_1024": lambda: W.prefill_llama8b(prompt=1024),
        "prefill_chunk130_on_8192": lambda: W.prefill_llama8b(prompt=130, prefix=8192),
        "prefill_int8_causal_8192": lambda: W.prefill_llama8b(prompt=8192, kv_dtype="int8"),
        "prefill_int8_causal_1024": lambda: W.prefill_llama8b(prompt=1024, kv_dtype="int8"),
        "prefill_int8_chunk130_on_8192": lambda: W.prefill_llama8b(prompt=130, prefix=8192, kv_dtype="int8"),
        "verify_int8_16tok_batch1_ctx1024": lambda: W.verify_qwen4b_int8(),
        "mixed_full_prefill_2x2048": lambda: W.mixed_gptoss(layer="full", part="prefill"),
        "mixed_window_prefill_2x2048": lambda: W.mixed_gptoss(layer="window", part="prefill"),
        "attn_input_1x8192": lambda: W.attn_input_qwen4b(),
        "attn_input_32x1_on_4096": lambda: W.attn_input_qwen4b(prompt=1, batch=32, prefix=4095),
        "verify_16tok_batch1_ctx1024": lambda: W.verify_qwen4b(),
        "verify_16tok_batch1_ctx1024_graph": lambda: W.verify_qwen4b(),
        "verify_8tok_batch32_ctx512_8192": lambda: W.verify_qwen4b(batch=32, tokens=8, lo=512, hi=8192),
    }
    if args.workload not in builders:
        print(f"unknown workload {args.workload}; choose from {sorted(builders)}", file=sys.stderr)
        sys.exit(2)

    def measure(name, steps, warmup):
        case = builders[name]()
        log(f"[bench] {name}: building + timing {steps} steps")
        if name.startswith("attn_input"):
            r = run_attn_input(case, torch, pfa, gs, steps, warmup)
            gbs = r["bytes"] / (r["attn_input_ms"] * 1e-3) / 1e9
            r.update(metric="attn input GB/s", kernel_gbs=round(gbs, 1), frac_of_hbm_peak=round(gbs / HBM_PEAK_GBS, 4))
            return case, r
        if name.startswith("kv_write"):
            r = run_kv_write(case, torch, pfa, gs, steps, warmup)
            gbs = r["kv_write_bytes"] / (r["kv_write_ms"] * 1e-3) / 1e9
            r.update(metric="kv write GB/s", kernel_gbs=round(gbs, 1), frac_of_hbm_peak=round(gbs / HBM_PEAK_GBS, 4))
            return case, r
        if name.startswith("decode") and name.endswith("_graph"):
            r = run_decode_graph(case, torch, pfa, gs, steps, warmup, fused="_fused" in name)
            r.update(metric="decode step us (graph replay)")
            return case, r
        if name.endswith("_graph"):
            r = run_verify_graph(case, torch, pfa, gs, steps, warmup)
            r.update(metric="verify step us (graph replay)")
            return case, r
        if name.startswith("verify"):
            r = run_prefill(case, torch, pfa, gs, steps, warmup, verify=True)
            tf = r["flops"] / (r["prefill_ms"] * 1e-3) / 1e12
            gbs = r["kv_bytes"] / (r["prefill_ms"] * 1e-3) / 1e9
            r.update(metric="verify attn GB/s", kernel_tflops=round(tf, 2), kernel_gbs=round(gbs, 1),
                     frac_of_mfma_peak=round(tf / BF16_PEAK_TFLOPS, 4), frac_of_hbm_peak=round(gbs / HBM_PEAK_GBS, 4))
        elif name.startswith("prefill") or name.endswith("prefill_2x2048"):
            r = run_prefill(case, torch, pfa, gs, steps, warmup)
            tf = r["flops"] / (r["prefill_ms"] * 1e-3) / 1e12
            r.update(metric="prefill attn TFLOP/s", kernel_tflops=round(tf, 2),
                     frac_of_mfma_peak=round(tf / BF16_PEAK_TFLOPS, 4))
        else:
            r = run_decode(case, torch, pfa, gs, steps, warmup, fused=name.endswith("_fused"))
            gbs = r["decode_bytes"] / (r["decode_ms"] * 1e-3) / 1e9
            r.update(metric="decode attn GB/s", kernel_gbs=round(gbs, 1),
                     decode_us=round(r["decode_ms"] * 1e3, 2), frac_of_hbm_peak=round(gbs / HBM_PEAK_GBS, 4))
        return case, r

    case, r = measure(args.workload, args.steps, args.warmup)
    is_prefill = "prefill_ms" in r or args.workload.endswith("_graph")
    is_attn_input = args.workload.startswith("attn_input")
    is_kv_write = args.workload.startswith("kv_write")
    if is_kv_write:
        value = r["kernel_gbs"]
        unit, metric = "GB/s", "kv write GB/s (HBM)"
        roof = dict(bound="hbm", achieved=r["kernel_gbs"], peak=HBM_PEAK_GBS, unit="GB/s",
                    frac=r["frac_of_hbm_peak"], traffic=None)
    elif is_attn_input:
        value = r["kernel_gbs"]
        unit, metric = "GB/s", "attn input GB/s (HBM)"
        roof = dict(bound="hbm", achieved=r["kernel_gbs"], peak=HBM_PEAK_GBS, unit="GB/s",
                    frac=r["frac_of_hbm_peak"], traffic=None)
        case = case.case
    elif args.workload.endswith("_graph"):
        value = r.get("kv_bytes", r.get("decode_bytes", 0)) / (r["step_ms"] * 1e-3) / 1e9
        unit = "GB/s"
        metric = "decode step GB/s (graph replay)" if args.workload.startswith("decode") else \
            "verify step GB/s (HBM, graph replay)"
        roof = dict(bound="hbm", achieved=round(value, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                    frac=round(value / HBM_PEAK_GBS, 4), traffic=None)
    elif args.workload.startswith("verify"):
        value = r["kv_bytes"] / (r["step_ms"] * 1e-3) / 1e9
        unit, metric = "GB/s", "verify attn GB/s (HBM)"
        roof = dict(bound="hbm", achieved=r["kernel_gbs"], peak=HBM_PEAK_GBS, unit="GB/s",
                    frac=r["frac_of_hbm_peak"], traffic=None)
    elif is_prefill:
        value = r["flops"] / (r["step_ms"] * 1e-3) / 1e12
        unit, metric = "TFLOP/s", "prefill attn TFLOP/s"
        roof = dict(bound="mfma", achieved=r["kernel_tflops"], peak=BF16_PEAK_TFLOPS, unit="TFLOP/s",
                    frac=r["frac_of_mfma_peak"], traffic=None)
    else:
        value = r["step_bytes"] / (r["step_ms"] * 1e-3) / 1e9
        unit, metric = "GB/s", "decode attn GB/s (HBM)"
        kernel = "decode_kernel"
        traffic = measured_traffic(f"{kernel}:{args.workload}",
                                   src_digest("decode.hip", "pfa_device.h", "group_reduce.h", "merge_splits.h"))
        roof = dict(bound="hbm", achieved=r["kernel_gbs"], peak=HBM_PEAK_GBS, unit="GB/s",
                    frac=r["frac_of_hbm_peak"], traffic=traffic)

    extra = {}
    if not args.no_extra and args.workload == "decode_batch32_ctx512_8192":
        for name, st in (("decode_1seq_ctx1024", 100), ("decode_1seq_ctx1024_graph", 200),
                         ("decode_1seq_ctx1024_fused", 100), ("decode_1seq_ctx1024_fused_graph", 200),
                         ("decode_batch32_ctx512_8192_fused", 50),
                         ("decode_batch32_ctx8192", 30), ("decode_batch32_ctx8192_s1024", 30),
                         ("decode_int8_batch8_ctx32768", 30), ("decode_int8_batch8_ctx32768_smooth", 30),
                         ("decode_tq3_batch8_ctx32768", 30),
                         ("kv_write_bf16_8192", 40), ("kv_write_int8_8192", 40), ("kv_write_tq3_8192", 40),
                         ("mixed_full_decode_b64", 30), ("mixed_window_decode_b64", 50),
                         ("prefill_causal_8192", 30), ("prefill_causal_1024", 50),
                         ("prefill_int8_causal_8192", 20), ("prefill_int8_causal_1024", 50),
                         ("prefill_int8_chunk130_on_8192", 20), ("verify_int8_16tok_batch1_ctx1024", 50),
                         ("prefill_chunk130_on_8192", 20), ("mixed_full_prefill_2x2048", 20),
                         ("mixed_window_prefill_2x2048", 30),
                         ("verify_16tok_batch1_ctx1024", 50), ("verify_16tok_batch1_ctx1024_graph", 200),
                         ("verify_8tok_batch32_ctx512_8192", 30),
                         ("attn_input_1x8192", 30), ("attn_input_32x1_on_4096", 50)):
            try:
                # the long MFMA-bound prompt gets a longer warmup: its first ~10 launches
                # on a cold device run through a clock transient (up to ~20% slower)
                _, rr = measure(name, st, 20 if name == "prefill_causal_8192" else 3)
                if name.startswith("attn_input"):
                    extra[name] = dict(us=round(rr["attn_input_ms"] * 1e3, 2), gbs=rr["kernel_gbs"],
                                       frac_of_hbm_peak=rr["frac_of_hbm_peak"])
                elif name.endswith("_graph"):
                    extra[name] = dict(step_us=round(rr["step_ms"] * 1e3, 2),
                                       split=f"{rr['split_keys']}x{rr['max_splits']}")
                elif name.startswith("kv_write"):
                    extra[name] = dict(us=round(rr["kv_write_ms"] * 1e3, 2), gbs=rr["kernel_gbs"],
                                       frac_of_hbm_peak=rr["frac_of_hbm_peak"])
                elif name.startswith("verify"):
                    extra[name] = dict(us=round(rr["prefill_ms"] * 1e3, 2), gbs=rr["kernel_gbs"],
                                       frac_of_hbm_peak=rr["frac_of_hbm_peak"], tflops=rr["kernel_tflops"],
                                       split=f"{rr['split_keys']}x{rr['max_splits']}")
                elif "prefill_ms" in rr:
                    extra[name] = dict(us=round(rr["prefill_ms"] * 1e3, 1), tflops=rr["kernel_tflops"],
                                       frac_of_mfma_peak=rr["frac_of_mfma_peak"])
                else:
                    extra[name] = dict(us=rr["decode_us"], gbs=rr["kernel_gbs"],
                                       frac_of_hbm_peak=rr["frac_of_hbm_peak"],
                                       step_us=round(rr["step_ms"] * 1e3, 2))
                    if rr.get("combine_us") is not None:
                        extra[name]["combine_us"] = rr["combine_us"]
            except Exception as e:   # report, never hide
                extra[name] = dict(error=str(e)[:200])
            torch.cuda.empty_cache()

    cpu = None
    if not args.no_cpu_baseline and not is_prefill and not is_attn_input and not is_kv_write:
        log("[bench] cpu baseline (oracle)")
        cpu = cpu_baseline_decode(case)

    p = case.p
    line = {
        "metric": metric, "value": round(value, 2), "unit": unit, "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(r["step_ms"], 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": {"bf16": "bf16", "int8": "int8", "tq3": "fp32"}[p.kv_dtype], "data": "synthetic",
        "config": {"workload": case.name, "batch": case.batch, "q_heads": p.num_q_heads,
                   "kv_heads": p.num_kv_heads, "head_dim": p.head_dim, "page_size": p.page_size,
                   "split_keys": r.get("split_keys", case.split_keys if not is_prefill else None),
                   "max_seq_len": int(case.seq_lens.max()), "window": p.window,
                   "sinks": p.sinks is not None, "parallelism": "single GPU"},
        "roofline": roof,
        "cpu_baseline": cpu,
        "detail": {k: v for k, v in r.items() if isinstance(v, (int, float, str))},
        "workloads": extra,
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
