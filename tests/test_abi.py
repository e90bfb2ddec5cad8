"""The C-ABI library on a machine without a GPU.

These tests check that libpfa.so loads and exports every symbol include/pfa.h
declares.  They also check that host-side validation returns the documented
status codes without launching anything.  Every call here fails before any HIP
call is made.
"""
import ctypes
import os
import re

import pytest

import paged_flash_attention_amd as pfa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pfa.h")

OK, NULL, SHAPE, UNSUP, WORKSPACE, HIP = 0, 1, 2, 3, 4, 5
FAKE = ctypes.c_void_p(0x1000)   # never dereferenced: validation fails first


def header_symbols():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\*?(pfa_\w+)\s*\(", text, re.M)))


def test_library_exports_every_declared_symbol():
    L = pfa.lib()
    syms = header_symbols()
    assert set(syms) == set(pfa.EXPORTS), syms
    for s in syms:
        assert hasattr(L, s), s


def test_debug_build_exports_the_same_symbols_and_bounds_query():
    """libpfa_debug.so (barrier audit + device-side bounds checks) exports the same
    ABI.  pfa_bounds_errors: NULL flags -> PFA_ERR_NULL in both builds; the normal
    build does not check and returns PFA_ERR_UNSUPPORTED with flags 0, before any
    HIP call."""
    D = pfa.load_library(pfa.DEBUG_LIB_PATH)
    for s in header_symbols():
        assert hasattr(D, s), s
    assert D.pfa_bounds_errors(None) == NULL
    L = pfa.lib()
    assert L.pfa_bounds_errors(None) == NULL
    f = ctypes.c_uint32(7)
    assert L.pfa_bounds_errors(ctypes.byref(f)) == UNSUP
    assert f.value == 0
    with pytest.raises(pfa.PfaError, match="UNSUPPORTED"):
        pfa.bounds_errors()


def test_status_strings_and_splits():
    L = pfa.lib()
    for st in range(6):
        assert L.pfa_status_string(st)
    assert L.pfa_status_string(99) == b"unknown status"
    assert pfa.decode_num_splits(8192, 256) == 32
    assert pfa.decode_num_splits(8193, 256) == 33
    assert pfa.decode_num_splits(1, 256) == 1
    assert pfa.decode_num_splits(100, 0) == 0
    assert L.pfa_last_hip_error() == 0


def test_decode_workspace_bytes():
    L = pfa.lib()
    d = desc()
    assert L.pfa_decode_workspace_bytes(ctypes.byref(d), 32, 33) == 32 * 32 * 33 * 129 * 4
    assert L.pfa_decode_workspace_bytes(ctypes.byref(d), 32, 1) == 0        # unsplit: no buffers
    assert L.pfa_decode_workspace_bytes(ctypes.byref(d), 0, 33) == 0
    assert L.pfa_decode_workspace_bytes(None, 32, 33) == 0
    assert L.pfa_decode_workspace_bytes(ctypes.byref(desc(head_dim=96)), 32, 33) == 0
    assert pfa.decode_workspace_bytes(pfa.AttnDesc(64, 8, 64), 64, 128) == 64 * 64 * 128 * 65 * 4


def test_decode_static_rejects_partials_beyond_its_array():
    """pfa_paged_attn_decode_static: partials larger than PFA_STATIC_SCRATCH_BYTES
    return PFA_ERR_WORKSPACE before any HIP call (no GPU needed)."""
    L = pfa.lib()
    d, p = desc(), pool()
    call = lambda B, ml, S, out=FAKE: L.pfa_paged_attn_decode_static(
        ctypes.byref(d), ctypes.byref(p), FAKE, FAKE, 4096, FAKE, B, ml, S, out, None)
    # 64 x 32 heads x 128 splits x 129 x 4 B = 135 MB > 32 MiB
    assert call(64, 32768, 256) == WORKSPACE
    assert pfa.STATIC_SCRATCH_BYTES == 32 << 20
    assert call(8, 1024, -16) == SHAPE
    assert call(-1, 1024, 256) == SHAPE


def desc(**kw):
    d = dict(num_q_heads=32, num_kv_heads=8, head_dim=128, page_size=16, kv_dtype=0, window=0,
             sm_scale=0.088, sinks=None)
    d.update(kw)
    return pfa.CAttnDesc(**d)


def pool(**kw):
    p = dict(k_pool=FAKE.value, v_pool=FAKE.value, k_scale=None, v_scale=None, num_pages=64, k_smooth=None)
    p.update(kw)
    return pfa.CKvPool(**p)


def kvw(d, p, **kw):
    a = dict(k=FAKE, v=FAKE, cu=FAKE, sl=FAKE, bt=FAKE, stride=8, batch=2, T=2)
    a.update(kw)
    return pfa.lib().pfa_kv_write(ctypes.byref(d) if d is not None else None,
                                  ctypes.byref(p) if p is not None else None,
                                  a["k"], a["v"], a["cu"], a["sl"], a["bt"], a["stride"], a["batch"], a["T"], None)


def test_key_smoothing_is_int8_only():
    assert kvw(desc(), pool(k_smooth=FAKE.value)) == UNSUP
    assert dec(desc(), pool(k_smooth=FAKE.value)) == UNSUP


def test_kv_write_validation():
    assert kvw(None, pool()) == NULL
    assert kvw(desc(), None) == NULL
    assert kvw(desc(num_q_heads=30), pool()) == SHAPE          # Hq % Hkv
    assert kvw(desc(head_dim=96), pool()) == UNSUP
    assert kvw(desc(page_size=32), pool()) == UNSUP
    assert kvw(desc(kv_dtype=7), pool()) == UNSUP
    assert kvw(desc(window=-1), pool()) == SHAPE
    assert kvw(desc(kv_dtype=1), pool()) == NULL               # INT8 without scale pools
    assert kvw(desc(), pool(num_pages=0)) == SHAPE
    assert kvw(desc(), pool(), k=None) == NULL
    assert kvw(desc(), pool(), stride=0) == SHAPE
    assert kvw(desc(), pool(), T=-1) == SHAPE
    assert kvw(desc(), pool(), batch=0) == SHAPE                # tokens but no sequences
    assert kvw(desc(), pool(), T=0, k=None) == OK              # nothing to do, nothing launched
    assert kvw(desc(num_q_heads=65535 * 2, num_kv_heads=65535), pool(), T=2**31 - 1) == SHAPE   # grid too large


def ain(d, p, prm=True, **kw):
    a = dict(qkv=FAKE, cu=FAKE, sl=FAKE, bt=FAKE, stride=8, batch=2, T=2, q=FAKE,
             qw=FAKE.value, kw=FAKE.value, rope=FAKE.value, maxpos=64, eps=1e-6)
    a.update(kw)
    pr = pfa.CAttnInputParams(a["qw"], a["kw"], a["rope"], a["maxpos"], a["eps"]) if prm else None
    return pfa.lib().pfa_attn_input(ctypes.byref(d), ctypes.byref(p), ctypes.byref(pr) if pr else None,
                                    a["qkv"], a["cu"], a["sl"], a["bt"], a["stride"], a["batch"], a["T"],
                                    a["q"], None)


def test_attn_input_validation():
    assert ain(desc(), pool(), prm=False) == NULL
    assert ain(desc(), pool(), qw=None) == NULL
    assert ain(desc(), pool(), rope=None) == NULL
    assert ain(desc(), pool(), q=None) == NULL
    assert ain(desc(), pool(), maxpos=0) == SHAPE
    assert ain(desc(), pool(), eps=-1.0) == SHAPE
    assert ain(desc(), pool(), eps=float("nan")) == SHAPE
    assert ain(desc(head_dim=96), pool()) == UNSUP
    assert ain(desc(kv_dtype=1), pool()) == NULL                # INT8 without scale pools
    assert ain(desc(), pool(), batch=0) == SHAPE
    assert ain(desc(), pool(), T=0, qkv=None) == OK


def dec(d, p, **kw):
    a = dict(q=FAKE, bt=FAKE, stride=64, sl=FAKE, batch=4, max_len=1024, S=256, ms=4,
             op=FAKE, lp=FAKE, out=FAKE)
    a.update(kw)
    return pfa.lib().pfa_paged_attn_decode(ctypes.byref(d), ctypes.byref(p), a["q"], a["bt"], a["stride"],
                                           a["sl"], a["batch"], a["max_len"], a["S"], a["ms"],
                                           a["op"], a["lp"], a["out"], None)


def test_decode_validation():
    assert dec(desc(num_q_heads=48, num_kv_heads=3), pool()) == UNSUP   # G = 16
    assert dec(desc(), pool(), S=100) == SHAPE                           # not a multiple of P
    assert dec(desc(), pool(), S=0) == SHAPE
    assert dec(desc(), pool(), ms=3) == WORKSPACE                        # 1024/256 = 4 splits
    assert dec(desc(), pool(), max_len=64 * 16 + 1) == SHAPE              # beyond the block table
    assert dec(desc(), pool(), op=None) == NULL
    assert dec(desc(), pool(), lp=None) == NULL
    assert dec(desc(), pool(), ms=1, out=None) == NULL
    assert dec(desc(), pool(), q=None) == NULL
    assert dec(desc(), pool(), ms=0) == SHAPE
    assert dec(desc(), pool(), batch=-1) == SHAPE
    assert dec(desc(), pool(), batch=0, q=None) == OK


def test_scale_must_be_positive_and_finite():
    """The kernels take the softmax maximum before the scale: a scale <= 0, inf or
    NaN is refused by decode (plain, fused, static), prefill and verify, before any
    launch."""
    for bad in (0.0, -0.088, float("inf"), float("nan")):
        assert dec(desc(sm_scale=bad), pool()) == SHAPE
        assert decf(desc(sm_scale=bad), pool()) == SHAPE
        assert pre(desc(sm_scale=bad), pool()) == SHAPE
        assert ver(desc(sm_scale=bad), pool()) == SHAPE
        L = pfa.lib()
        d, p = desc(sm_scale=bad), pool()
        assert L.pfa_paged_attn_decode_static(ctypes.byref(d), ctypes.byref(p), FAKE, FAKE, 4096, FAKE,
                                              4, 1024, 256, FAKE, None) == SHAPE
    # the KV write and the combine do not use it
    assert kvw(desc(sm_scale=0.0), pool(), T=0, batch=0) == OK
    assert comb(desc(sm_scale=0.0), batch=0, out=None) == OK


def decf(d, p, **kw):
    a = dict(q=FAKE, bt=FAKE, stride=64, sl=FAKE, batch=4, max_len=1024, S=256, ms=4,
             op=FAKE, lp=FAKE, ctr=FAKE, out=FAKE)
    a.update(kw)
    return pfa.lib().pfa_paged_attn_decode_fused(ctypes.byref(d), ctypes.byref(p), a["q"], a["bt"], a["stride"],
                                                 a["sl"], a["batch"], a["max_len"], a["S"], a["ms"],
                                                 a["op"], a["lp"], a["ctr"], a["out"], None)


def test_decode_fused_validation():
    assert decf(desc(), pool(), ctr=None) == NULL
    assert decf(desc(), pool(), out=None) == NULL
    assert decf(desc(), pool(), op=None) == NULL
    assert decf(desc(), pool(), ms=3) == WORKSPACE
    assert decf(desc(), pool(), S=100) == SHAPE
    assert decf(desc(num_q_heads=48, num_kv_heads=3), pool()) == UNSUP
    assert decf(desc(), pool(), batch=0, q=None, ctr=None) == OK


def comb(d, **kw):
    a = dict(op=FAKE, lp=FAKE, sl=FAKE, batch=4, S=256, ms=4, out=FAKE)
    a.update(kw)
    return pfa.lib().pfa_paged_attn_combine(ctypes.byref(d), a["op"], a["lp"], a["sl"], a["batch"],
                                            a["S"], a["ms"], a["out"], None)


def test_combine_validation():
    assert comb(desc(), out=None) == NULL
    assert comb(desc(), S=8) == SHAPE
    assert comb(desc(), ms=0) == SHAPE
    assert comb(desc(head_dim=80)) == UNSUP
    assert comb(desc(), batch=0, out=None) == OK


def pre(d, p, **kw):
    a = dict(q=FAKE, cu=FAKE, bt=FAKE, stride=64, sl=FAKE, batch=1, mq=1024, ml=1024, S=0, ms=1,
             op=None, lp=None, out=FAKE)
    a.update(kw)
    return pfa.lib().pfa_paged_attn_prefill(ctypes.byref(d), ctypes.byref(p), a["q"], a["cu"], a["bt"],
                                            a["stride"], a["sl"], a["batch"], a["mq"], a["ml"], a["S"],
                                            a["ms"], a["op"], a["lp"], a["out"], None)


def test_prefill_validation():
    assert pre(desc(kv_dtype=1), pool()) == NULL                             # INT8 pool without scales
    assert pre(desc(num_q_heads=64 * 3, num_kv_heads=3), pool()) == UNSUP   # G = 64
    assert pre(desc(), pool(), cu=None) == NULL
    assert pre(desc(), pool(), out=None) == NULL
    assert pre(desc(), pool(), mq=-1) == SHAPE
    assert pre(desc(), pool(), ml=512) == SHAPE                              # max_seq_len < max_q_len
    assert pre(desc(), pool(), ml=64 * 16 + 1, mq=10) == SHAPE               # beyond the block table
    assert pre(desc(), pool(), S=100, ms=11) == SHAPE                        # not a multiple of 64
    assert pre(desc(), pool(), S=128, ms=7) == WORKSPACE                     # 1024/128 = 8 ranges
    assert pre(desc(), pool(), S=128, ms=8) == NULL                          # no partial buffers
    assert pre(desc(), pool(), mq=0, q=None) == OK


def test_prefill_split_choice_host_only():
    L = pfa.lib()
    sk = ctypes.c_int32(-1)
    assert L.pfa_prefill_num_splits(ctypes.byref(desc()), 1, 8192, 8192, 256, ctypes.byref(sk)) == 1
    assert sk.value == 0
    ms = L.pfa_prefill_num_splits(ctypes.byref(desc()), 1, 130, 8322, 256, ctypes.byref(sk))
    assert ms > 1 and sk.value % 64 == 0 and ms * sk.value >= 8322 and sk.value >= 256


def test_binding_refuses_host_tensors():
    import torch
    d = pfa.AttnDesc(4, 2, 64)
    p = pfa.KVPool(torch.zeros(4, 2, 16, 64, dtype=torch.bfloat16), torch.zeros(4, 2, 16, 64, dtype=torch.bfloat16))
    with pytest.raises(ValueError):
        p.c()
    with pytest.raises(ValueError):
        pfa.paged_attn_combine(d, torch.zeros(1), torch.zeros(1), torch.zeros(1, dtype=torch.int32), 16, 1,
                               torch.zeros(1))


def ver(d, p, **kw):
    a = dict(q=FAKE, cu=FAKE, bt=FAKE, stride=64, sl=FAKE, batch=1, mq=16, ml=1024, S=0, ms=1,
             op=None, lp=None, out=FAKE)
    a.update(kw)
    return pfa.lib().pfa_paged_attn_verify(ctypes.byref(d), ctypes.byref(p), a["q"], a["cu"], a["bt"],
                                           a["stride"], a["sl"], a["batch"], a["mq"], a["ml"], a["S"],
                                           a["ms"], a["op"], a["lp"], a["out"], None)


def test_verify_validation():
    assert ver(desc(), pool(), mq=17) == SHAPE                               # more than 16 tokens
    assert ver(desc(kv_dtype=1), pool()) == NULL                             # INT8 pool without scales
    assert ver(desc(), pool(), out=None) == NULL
    assert ver(desc(), pool(), S=96, ms=11) == SHAPE                         # not a multiple of 64
    assert ver(desc(), pool(), S=64, ms=15) == WORKSPACE                     # 1024/64 = 16 ranges
    assert ver(desc(), pool(), S=64, ms=16) == NULL                          # no partial buffers
    assert ver(desc(), pool(), mq=0, q=None) == OK


def test_verify_split_choice_host_only():
    L = pfa.lib()
    sk = ctypes.c_int32(-1)
    # one sequence, 16 tokens on 1024 positions: 64-key ranges spread it over the chip
    ms = L.pfa_verify_num_splits(ctypes.byref(desc()), 1, 16, 1040, 256, ctypes.byref(sk))
    assert ms > 1 and sk.value % 64 == 0 and sk.value >= 64 and ms * sk.value >= 1040
    # enough sequences fill the chip unsplit
    assert L.pfa_verify_num_splits(ctypes.byref(desc()), 64, 16, 32768, 256, ctypes.byref(sk)) == 1
    assert sk.value == 0


def test_tq3_codebook_matches_the_oracle():
    """The library computes the 3-bit codebook itself (host code, no GPU); it must
    round to the oracle's float32 codebook exactly."""
    import numpy as np
    import oracle as O
    m, t = pfa.tq3_codebook()
    M, T = O.codebook_f32()
    assert np.array_equal(np.array(m, np.float32), M)
    assert np.array_equal(np.array(t, np.float32), T)
    assert pfa.lib().pfa_tq3_codebook(None, None) == NULL


def test_tq3_pool_validation():
    tq = dict(k_scale=FAKE.value, v_scale=FAKE.value)
    assert kvw(desc(kv_dtype=2), pool()) == NULL                           # 3-bit pool without scales
    assert dec(desc(kv_dtype=2), pool()) == NULL
    assert kvw(desc(kv_dtype=2), pool(k_smooth=FAKE.value, **tq)) == UNSUP  # smoothing is INT8-only
    assert pre(desc(kv_dtype=2), pool(**tq)) == UNSUP                      # prefill: BF16 or INT8
    assert ver(desc(kv_dtype=2), pool(**tq)) == UNSUP
    assert ain(desc(kv_dtype=2), pool(**tq)) == UNSUP
    assert decf(desc(kv_dtype=2), pool(**tq)) == UNSUP                     # no fused merge
    assert dec(desc(kv_dtype=2, num_q_heads=48, num_kv_heads=3), pool(**tq)) == UNSUP   # G = 16
    assert dec(desc(kv_dtype=2), pool(**tq), batch=0) == OK                # nothing launched
    assert kvw(desc(kv_dtype=2), pool(**tq), T=0, k=None) == OK


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    """With no built library the binding raises; there is no fallback path."""
    monkeypatch.setattr(pfa, "LIB_PATH", str(tmp_path / "libpfa.so"))
    monkeypatch.setattr(pfa, "_lib", None)
    with pytest.raises(RuntimeError, match="missing"):
        pfa.lib()
    with pytest.raises(RuntimeError, match="missing"):
        pfa.decode_num_splits(1024, 256)
