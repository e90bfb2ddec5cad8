"""Barrier audit of the prefill kernels and of the INT8 decode at G = 8.  Their direct HBM -> LDS tile loads are
issued as inline asm, which the compiler does not track, so the waits before a
tile is read (each wave waits for its own loads of that tile, then one barrier)
are placed by hand.  libpfa_debug.so is the same source built with
PFA_PREFILL_AUDIT=1 (and the device-side bounds checks, which change no
arithmetic): every ring step waits for all of the wave's loads and then for all
waves, before and after each refill.  If a hand-placed wait were too
short, the normal build would read a stage before its tile landed and its bits
would differ from the audit build's; here they must be equal, on both kernel
builds (64-key unsplit, 32-key split) and on verify steps.

The INT8 decode at G = 8 loads each page's K and V tiles and scales straight into
a 2-stage LDS ring the same way, one page ahead; the audit build (PFA_DECODE_AUDIT=1)
waits for all of them before every page."""
import numpy as np
import pytest
import torch

import paged_flash_attention_amd as pfa
import workloads as W
from gpu_support import GpuCase

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def audit_lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    pfa.lib()
    return pfa.load_library(pfa.DEBUG_LIB_PATH)


AUDIT_CASES = [
    # (params, seq_lens, q_lens, runs)
    (dict(Hq=32, Hkv=8, D=128), [1100, 300], [1100, 300], ("prefill", "split")),
    (dict(Hq=32, Hkv=8, D=128, window=700, sinks=True), [2000, 517], [1500, 517], ("prefill", "split")),
    (dict(Hq=64, Hkv=8, D=64, sinks=True), [777, 64], [777, 1], ("prefill", "split")),
    (dict(Hq=64, Hkv=8, D=64, window=128, sinks=True), [900], [900], ("prefill",)),
    (dict(Hq=32, Hkv=8, D=128), [1040, 2000, 17], [16, 9, 2], ("verify",)),
]


@pytest.mark.parametrize("ci", range(len(AUDIT_CASES)))
def test_prefill_bits_equal_the_barrier_audit_build(ci, audit_lib):
    prm, lens, qlens, runs = AUDIT_CASES[ci]
    p = W.AttnParams(prm["Hq"], prm["Hkv"], prm["D"], window=prm.get("window", 0),
                     sinks=W.sinks_normal(700 + ci, prm["Hq"]) if prm.get("sinks") else None)
    case = W.make_case(f"audit{ci}", 700 + ci, p, lens, qlens, split_keys=0)
    g = GpuCase(case)
    n = max(lens)

    def run(kind):
        if kind == "prefill":
            return g.prefill(split=None)
        if kind == "split":
            return g.prefill(split=(128, -(-n // 128)))
        return g.verify(split="auto")

    for kind in runs:
        normal = run(kind)
        prev = pfa.use_library(audit_lib)
        try:
            audited = run(kind)
        finally:
            pfa.use_library(prev)
        assert np.all(np.isfinite(normal))
        assert np.array_equal(normal.view(np.uint32), audited.view(np.uint32)), \
            f"case {ci} {kind}: {np.sum(normal != audited)} outputs differ from the audit build"


DECODE_AUDIT_CASES = [
    # (params, seq_lens, split_keys): INT8, G = 8
    (dict(Hq=32, Hkv=4, D=128), [33, 1000, 4100], (0, 256, 64)),
    (dict(Hq=32, Hkv=4, D=128, window=300, sinks=True), [2049, 16, 700], (0, 256)),
    (dict(Hq=64, Hkv=8, D=64, sinks=True), [1500, 17], (0, 128)),
]


@pytest.mark.parametrize("ci", range(len(DECODE_AUDIT_CASES)))
@pytest.mark.parametrize("smooth", [False, True], ids=["plain", "smoothed"])
def test_int8_decode_bits_equal_the_audit_build(ci, smooth, audit_lib):
    prm, lens, splits = DECODE_AUDIT_CASES[ci]
    p = W.AttnParams(prm["Hq"], prm["Hkv"], prm["D"], kv_dtype="int8", window=prm.get("window", 0),
                     sinks=W.sinks_normal(720 + ci, prm["Hq"]) if prm.get("sinks") else None)
    kw = dict(key_weight=W.key_norm_weight(730 + ci, prm["D"])) if smooth else {}
    case = W.make_case(f"daudit{ci}", 720 + ci, p, lens, np.ones(len(lens), np.int32), outlier_frac=0.01, **kw)
    g = GpuCase(case)
    def run(S, fused):
        return g.decode_fused(split_keys=S, calls=1)[0][0] if fused else g.decode(split_keys=S)

    for S in splits:
        for fused in (False, True):
            if fused and S == 0:
                continue
            normal = run(S, fused)
            prev = pfa.use_library(audit_lib)
            try:
                audited = run(S, fused)
            finally:
                pfa.use_library(prev)
            assert np.array_equal(normal.view(np.uint32), audited.view(np.uint32)), \
                f"case {ci} S={S} fused={fused}: {np.sum(normal != audited)} outputs differ from the audit build"
