"""Python binding of libpfa.so, the paged flash attention C ABI in include/pfa.h.

This module only marshals arguments.  It checks tensor dtypes, devices and
contiguity, packs the descriptor structs, and passes raw device pointers and the
current HIP stream to the C entry points, which have the same names.  Every step
of the computation runs in the HIP kernels.  If the library is missing this
module raises; it never falls back to another implementation.
"""
from __future__ import annotations

import ctypes
import math
import os
from dataclasses import dataclass
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpfa.so")

PFA_OK = 0
STATUS_NAMES = {0: "PFA_OK", 1: "PFA_ERR_NULL", 2: "PFA_ERR_SHAPE", 3: "PFA_ERR_UNSUPPORTED",
                4: "PFA_ERR_WORKSPACE", 5: "PFA_ERR_HIP"}
KV_DTYPES = {"bf16": 0, "int8": 1, "tq3": 2}

# every symbol include/pfa.h declares
EXPORTS = ("pfa_kv_write", "pfa_attn_input", "pfa_paged_attn_decode", "pfa_paged_attn_decode_fused",
           "pfa_paged_attn_decode_static", "pfa_paged_attn_combine",
           "pfa_paged_attn_prefill", "pfa_paged_attn_verify", "pfa_decode_num_splits",
           "pfa_decode_workspace_bytes",
           "pfa_prefill_num_splits", "pfa_verify_num_splits", "pfa_tq3_codebook", "pfa_bounds_errors",
           "pfa_status_string", "pfa_last_hip_error")

# pfa_bounds_errors bits (debug build)
BOUNDS_PAGE, BOUNDS_SEQ_LEN, BOUNDS_Q_LEN = 1, 2, 4


class PfaError(RuntimeError):
    def __init__(self, fn: str, status: int, message: str, hip_error: int = 0):
        extra = f" (hipError {hip_error})" if status == 5 else ""
        super().__init__(f"{fn}: {STATUS_NAMES.get(status, status)}: {message}{extra}")
        self.status = status
        self.hip_error = hip_error


class CAttnDesc(ctypes.Structure):
    _fields_ = [("num_q_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("page_size", ctypes.c_int32),
                ("kv_dtype", ctypes.c_int32), ("window", ctypes.c_int32),
                ("sm_scale", ctypes.c_float), ("sinks", ctypes.c_void_p)]


class CAttnInputParams(ctypes.Structure):
    _fields_ = [("q_norm_weight", ctypes.c_void_p), ("k_norm_weight", ctypes.c_void_p),
                ("rope_cos_sin", ctypes.c_void_p), ("rope_max_pos", ctypes.c_int32),
                ("eps", ctypes.c_float)]


class CKvPool(ctypes.Structure):
    _fields_ = [("k_pool", ctypes.c_void_p), ("v_pool", ctypes.c_void_p),
                ("k_scale", ctypes.c_void_p), ("v_scale", ctypes.c_void_p),
                ("num_pages", ctypes.c_int32), ("k_smooth", ctypes.c_void_p)]


# debug build: prefill barrier audit + device-side bounds checks (tests, debugging)
DEBUG_LIB_PATH = os.path.join(_HERE, "libpfa_debug.so")

_lib = None


def lib() -> ctypes.CDLL:
    """Load libpfa.so (built in-tree) and declare its signatures."""
    global _lib
    if _lib is None:
        _lib = load_library(LIB_PATH)
    return _lib


def use_library(L: Optional[ctypes.CDLL]) -> Optional[ctypes.CDLL]:
    """Route the entry points below through another loaded build (e.g. the debug
    build, from load_library(DEBUG_LIB_PATH)); None restores libpfa.so.  Returns
    the build used before."""
    global _lib
    prev = _lib
    _lib = L
    return prev


def load_library(path: str) -> ctypes.CDLL:
    """Load a build of the library and declare its signatures."""
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m paged_flash_attention_amd.build`")
    L = ctypes.CDLL(path)
    P, I, F, V = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_void_p
    D, PL = ctypes.POINTER(CAttnDesc), ctypes.POINTER(CKvPool)
    sig = {
        "pfa_kv_write": [D, PL, P, P, P, P, P, I, I, I, V],
        "pfa_attn_input": [D, PL, ctypes.POINTER(CAttnInputParams), P, P, P, P, I, I, I, P, V],
        "pfa_paged_attn_decode": [D, PL, P, P, I, P, I, I, I, I, P, P, P, V],
        "pfa_paged_attn_decode_fused": [D, PL, P, P, I, P, I, I, I, I, P, P, P, P, V],
        "pfa_paged_attn_decode_static": [D, PL, P, P, I, P, I, I, I, P, V],
        "pfa_paged_attn_combine": [D, P, P, P, I, I, I, P, V],
        "pfa_paged_attn_prefill": [D, PL, P, P, P, I, P, I, I, I, I, I, P, P, P, V],
        "pfa_paged_attn_verify": [D, PL, P, P, P, I, P, I, I, I, I, I, P, P, P, V],
    }
    for name, args in sig.items():
        fn = getattr(L, name)
        fn.argtypes = args
        fn.restype = ctypes.c_int
    L.pfa_decode_num_splits.argtypes = [I, I]
    L.pfa_decode_num_splits.restype = ctypes.c_int32
    L.pfa_decode_workspace_bytes.argtypes = [D, I, I]
    L.pfa_decode_workspace_bytes.restype = ctypes.c_size_t
    L.pfa_prefill_num_splits.argtypes = [D, I, I, I, I, ctypes.POINTER(ctypes.c_int32)]
    L.pfa_prefill_num_splits.restype = ctypes.c_int32
    L.pfa_verify_num_splits.argtypes = [D, I, I, I, I, ctypes.POINTER(ctypes.c_int32)]
    L.pfa_verify_num_splits.restype = ctypes.c_int32
    L.pfa_tq3_codebook.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.POINTER(ctypes.c_float)]
    L.pfa_tq3_codebook.restype = ctypes.c_int
    L.pfa_bounds_errors.argtypes = [ctypes.POINTER(ctypes.c_uint32)]
    L.pfa_bounds_errors.restype = ctypes.c_int
    L.pfa_status_string.argtypes = [ctypes.c_int]
    L.pfa_status_string.restype = ctypes.c_char_p
    L.pfa_last_hip_error.argtypes = []
    L.pfa_last_hip_error.restype = ctypes.c_int32
    return L


def _check(fn: str, status: int):
    if status != PFA_OK:
        L = lib()
        raise PfaError(fn, status, L.pfa_status_string(status).decode(), L.pfa_last_hip_error())


# ---------------------------------------------------------------------------
# descriptors
# ---------------------------------------------------------------------------

@dataclass
class AttnDesc:
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    page_size: int = 16
    kv_dtype: str = "bf16"
    window: int = 0
    sm_scale: Optional[float] = None
    sinks: Optional[torch.Tensor] = None      # device float32 [num_q_heads]

    def c(self) -> CAttnDesc:
        if self.sinks is not None:
            _dev(self.sinks, torch.float32, "sinks")
            if self.sinks.numel() != self.num_q_heads:
                raise ValueError("sinks must have num_q_heads entries")
        scale = self.sm_scale if self.sm_scale is not None else 1.0 / math.sqrt(self.head_dim)
        return CAttnDesc(self.num_q_heads, self.num_kv_heads, self.head_dim, self.page_size,
                         KV_DTYPES[self.kv_dtype], self.window, scale,
                         self.sinks.data_ptr() if self.sinks is not None else None)


@dataclass
class KVPool:
    """k/v: [num_pages, Hkv, P, D] (bf16 or int8), or uint8 packed codes [num_pages, Hkv, P, 3D/8]
    for the 3-bit rotated format; scales [num_pages, Hkv, P] fp32 for INT8 and 3-bit pools.
    k_smooth: optional [D] fp32 key smoothing of an INT8 pool (keys stored as k / s)."""
    k: torch.Tensor
    v: torch.Tensor
    k_scale: Optional[torch.Tensor] = None
    v_scale: Optional[torch.Tensor] = None
    k_smooth: Optional[torch.Tensor] = None

    @property
    def num_pages(self) -> int:
        return int(self.k.shape[0])

    def c(self) -> CKvPool:
        dt = self.k.dtype
        if dt not in (torch.bfloat16, torch.int8, torch.uint8) or self.v.dtype != dt:
            raise TypeError("pool tensors must both be bfloat16, both int8 or both uint8 (3-bit codes)")
        _dev(self.k, dt, "k_pool")
        _dev(self.v, dt, "v_pool")
        ks = vs = None
        if dt != torch.bfloat16:
            if self.k_scale is None or self.v_scale is None:
                raise ValueError("an INT8 or 3-bit pool needs k_scale and v_scale")
            ks = _dev(self.k_scale, torch.float32, "k_scale").data_ptr()
            vs = _dev(self.v_scale, torch.float32, "v_scale").data_ptr()
        sm = None
        if self.k_smooth is not None:
            sm = _dev(self.k_smooth, torch.float32, "k_smooth").data_ptr()
        return CKvPool(self.k.data_ptr(), self.v.data_ptr(), ks, vs, self.num_pages, sm)


def _dev(t: Optional[torch.Tensor], dtype, name: str):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _expect(t: Optional[torch.Tensor], shape, dtype, name: str, optional: bool = False):
    """Check a tensor's dtype and shape (None in ``shape`` matches any size).  The
    device and contiguity checks follow when its pointer is taken (``_ptr``); both
    raise before anything is launched."""
    if t is None:
        if optional:
            return None
        raise ValueError(f"{name} is required")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    sh = t.shape
    ok = len(sh) == len(shape)
    if ok:
        for n, w in zip(sh, shape):
            if w is not None and n != w:
                ok = False
                break
    if not ok:
        want = "(" + ", ".join("*" if w is None else str(int(w)) for w in shape) + ")"
        raise ValueError(f"{name} must have shape {want}, got {tuple(sh)}")
    return t


def _check_pool(desc: "AttnDesc", pool: "KVPool"):
    """The pool's tensors against the descriptor: dtype of kv_dtype, shape
    [num_pages, Hkv, P, D] (3-bit codes: 3D/8 bytes), scales [num_pages, Hkv, P]."""
    want = {"bf16": torch.bfloat16, "int8": torch.int8, "tq3": torch.uint8}.get(desc.kv_dtype)
    if want is None:
        raise ValueError(f"unknown kv_dtype {desc.kv_dtype!r}")
    last = 3 * desc.head_dim // 8 if desc.kv_dtype == "tq3" else desc.head_dim
    shape = (None, desc.num_kv_heads, desc.page_size, last)
    _expect(pool.k, shape, want, "k_pool")
    _expect(pool.v, tuple(pool.k.shape), want, "v_pool")
    if desc.kv_dtype != "bf16":
        sshape = tuple(pool.k.shape[:3])
        _expect(pool.k_scale, sshape, torch.float32, "k_scale")
        _expect(pool.v_scale, sshape, torch.float32, "v_scale")
    if pool.k_smooth is not None:
        if desc.kv_dtype != "int8":
            raise ValueError("k_smooth is an INT8 pool option")
        _expect(pool.k_smooth, (desc.head_dim,), torch.float32, "k_smooth")


def _check_table(block_table, seq_lens, name="seq_lens"):
    _expect(block_table, (None, None), torch.int32, "block_table")
    batch = int(block_table.shape[0])
    _expect(seq_lens, (batch,), torch.int32, name)
    return batch


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"a {tuple(t.shape)} {t.dtype} argument must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"a {tuple(t.shape)} {t.dtype} argument must be contiguous")
    return t.data_ptr()


_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(stream, ref: torch.Tensor):
    """The stream to enqueue on: `stream` (a torch stream or a raw hipStream_t), or
    torch's current stream on ref's device."""
    if stream is None:
        if _raw_stream is not None:
            return ctypes.c_void_p(_raw_stream(ref.device.index))
        stream = torch.cuda.current_stream(ref.device)
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


# ---------------------------------------------------------------------------
# entry points (same names as the C ABI, without the pfa_ prefix)
# ---------------------------------------------------------------------------

def kv_write(desc: AttnDesc, pool: KVPool, k_new, v_new, cu_new, seq_lens, block_table, stream=None):
    """Append k_new/v_new [T, Hkv, D] bf16 to their sequences' pages (pfa_kv_write)."""
    _check_pool(desc, pool)
    batch = _check_table(block_table, seq_lens)
    _expect(k_new, (None, desc.num_kv_heads, desc.head_dim), torch.bfloat16, "k_new")
    _expect(v_new, tuple(k_new.shape), torch.bfloat16, "v_new")
    _expect(cu_new, (batch + 1,), torch.int32, "cu_new")
    st = lib().pfa_kv_write(ctypes.byref(desc.c()), ctypes.byref(pool.c()), _ptr(k_new), _ptr(v_new),
                            _ptr(cu_new), _ptr(seq_lens), _ptr(block_table), int(block_table.shape[1]),
                            batch, int(k_new.shape[0]), _stream(stream, k_new))
    _check("pfa_kv_write", st)


def attn_input(desc: AttnDesc, pool: KVPool, q_norm_weight, k_norm_weight, rope_cos_sin, eps: float,
               qkv, cu_new, seq_lens, block_table, q_out, stream=None):
    """Fused q/k RMSNorm + RoPE + KV write from qkv [T, (Hq + 2 Hkv) * D] bf16.
    rope_cos_sin [max_pos, D/2, 2] fp32; writes q_out [T, Hq, D] bf16 and the pool."""
    D = desc.head_dim
    _check_pool(desc, pool)
    batch = _check_table(block_table, seq_lens)
    _expect(qkv, (None, (desc.num_q_heads + 2 * desc.num_kv_heads) * D), torch.bfloat16, "qkv")
    _expect(q_norm_weight, (D,), torch.bfloat16, "q_norm_weight")
    _expect(k_norm_weight, (D,), torch.bfloat16, "k_norm_weight")
    _expect(rope_cos_sin, (None, D // 2, 2), torch.float32, "rope_cos_sin")
    _expect(q_out, (qkv.shape[0], desc.num_q_heads, D), torch.bfloat16, "q_out")
    _expect(cu_new, (batch + 1,), torch.int32, "cu_new")
    prm = CAttnInputParams(_ptr(q_norm_weight), _ptr(k_norm_weight), _ptr(rope_cos_sin),
                           int(rope_cos_sin.shape[0]), float(eps))
    st = lib().pfa_attn_input(ctypes.byref(desc.c()), ctypes.byref(pool.c()), ctypes.byref(prm), _ptr(qkv),
                              _ptr(cu_new), _ptr(seq_lens), _ptr(block_table), int(block_table.shape[1]),
                              int(seq_lens.numel()), int(qkv.shape[0]), _ptr(q_out), _stream(stream, qkv))
    _check("pfa_attn_input", st)


def tq3_codebook():
    """The 3-bit format's codebook as the library computes it: (magnitudes [4], thresholds [3])."""
    m = (ctypes.c_float * 4)()
    t = (ctypes.c_float * 3)()
    _check("pfa_tq3_codebook", lib().pfa_tq3_codebook(m, t))
    return list(m), list(t)


def decode_workspace_bytes(desc: AttnDesc, batch: int, max_splits: int) -> int:
    """Bytes of o_part + lse_part for a split decode (0 when unsplit)."""
    return int(lib().pfa_decode_workspace_bytes(ctypes.byref(desc.c()), int(batch), int(max_splits)))


def _check_decode(desc, pool, q, block_table, seq_lens, max_splits, o_part, lse_part, out,
                  need_out: bool, need_parts: bool) -> int:
    Hq, D = desc.num_q_heads, desc.head_dim
    _check_pool(desc, pool)
    batch = _check_table(block_table, seq_lens)
    _expect(q, (batch, Hq, D), torch.bfloat16, "q")
    _expect(o_part, (batch, Hq, max_splits, D), torch.float32, "o_part", optional=not need_parts)
    _expect(lse_part, (batch, Hq, max_splits), torch.float32, "lse_part", optional=not need_parts)
    _expect(out, (batch, Hq, D), torch.float32, "out", optional=not need_out)
    return batch


def decode_num_splits(max_seq_len: int, split_keys: int) -> int:
    return int(lib().pfa_decode_num_splits(int(max_seq_len), int(split_keys)))


def paged_attn_decode(desc: AttnDesc, pool: KVPool, q, block_table, seq_lens, max_seq_len: int,
                      split_keys: int, max_splits: int, o_part=None, lse_part=None, out=None,
                      stream=None):
    """Split-KV decode partials, or the final output when max_splits == 1."""
    _check_decode(desc, pool, q, block_table, seq_lens, max_splits, o_part, lse_part, out,
                  need_out=max_splits == 1, need_parts=max_splits > 1)
    st = lib().pfa_paged_attn_decode(ctypes.byref(desc.c()), ctypes.byref(pool.c()), _ptr(q),
                                     _ptr(block_table), int(block_table.shape[1]), _ptr(seq_lens),
                                     int(q.shape[0]), int(max_seq_len), int(split_keys), int(max_splits),
                                     _ptr(o_part), _ptr(lse_part), _ptr(out), _stream(stream, q))
    _check("pfa_paged_attn_decode", st)


def paged_attn_decode_fused(desc: AttnDesc, pool: KVPool, q, block_table, seq_lens, max_seq_len: int,
                            split_keys: int, max_splits: int, o_part, lse_part, counters, out, stream=None):
    """Split-KV decode with the combine fused in: out [B, Hq, D] fp32 is written by
    the last split of each (sequence, KV head).  counters [B * Hkv] int32 must be
    zero and are left zero."""
    batch = _check_decode(desc, pool, q, block_table, seq_lens, max_splits, o_part, lse_part, out,
                          need_out=True, need_parts=max_splits > 1)
    _expect(counters, (batch * desc.num_kv_heads,), torch.int32, "counters", optional=max_splits == 1)
    st = lib().pfa_paged_attn_decode_fused(ctypes.byref(desc.c()), ctypes.byref(pool.c()), _ptr(q),
                                           _ptr(block_table), int(block_table.shape[1]), _ptr(seq_lens),
                                           int(q.shape[0]), int(max_seq_len), int(split_keys), int(max_splits),
                                           _ptr(o_part), _ptr(lse_part), _ptr(counters), _ptr(out),
                                           _stream(stream, q))
    _check("pfa_paged_attn_decode_fused", st)


STATIC_SCRATCH_BYTES = 32 << 20   # PFA_STATIC_SCRATCH_BYTES


def paged_attn_decode_static(desc: AttnDesc, pool: KVPool, q, block_table, seq_lens, max_seq_len: int,
                             split_keys: int, out, stream=None):
    """Decode + combine with the split partials in the library's own device array
    (pfa_paged_attn_decode_static): nothing is allocated.  out [B, Hq, D] fp32."""
    _check_decode(desc, pool, q, block_table, seq_lens, 1, None, None, out, need_out=True, need_parts=False)
    st = lib().pfa_paged_attn_decode_static(ctypes.byref(desc.c()), ctypes.byref(pool.c()), _ptr(q),
                                            _ptr(block_table), int(block_table.shape[1]), _ptr(seq_lens),
                                            int(q.shape[0]), int(max_seq_len), int(split_keys), _ptr(out),
                                            _stream(stream, q))
    _check("pfa_paged_attn_decode_static", st)


def paged_attn_combine(desc: AttnDesc, o_part, lse_part, seq_lens, split_keys: int, max_splits: int,
                       out, stream=None):
    """Merge split partials into out [B, Hq, D] fp32."""
    Hq, D = desc.num_q_heads, desc.head_dim
    _expect(seq_lens, (None,), torch.int32, "seq_lens")
    batch = int(seq_lens.shape[0])
    _expect(o_part, (batch, Hq, max_splits, D), torch.float32, "o_part")
    _expect(lse_part, (batch, Hq, max_splits), torch.float32, "lse_part")
    _expect(out, (batch, Hq, D), torch.float32, "out")
    st = lib().pfa_paged_attn_combine(ctypes.byref(desc.c()), _ptr(o_part), _ptr(lse_part),
                                      _ptr(seq_lens), int(seq_lens.numel()), int(split_keys),
                                      int(max_splits), _ptr(out), _stream(stream, out))
    _check("pfa_paged_attn_combine", st)


def _check_chunk(desc, pool, q, cu_q, block_table, seq_lens, out, max_splits, o_part, lse_part):
    Hq, D = desc.num_q_heads, desc.head_dim
    _check_pool(desc, pool)
    batch = _check_table(block_table, seq_lens)
    _expect(cu_q, (batch + 1,), torch.int32, "cu_q")
    _expect(q, (None, Hq, D), torch.bfloat16, "q")
    T = int(q.shape[0])
    _expect(out, (T, Hq, D), torch.float32, "out")
    _expect(o_part, (T, Hq, max_splits, D), torch.float32, "o_part", optional=max_splits == 1)
    _expect(lse_part, (T, Hq, max_splits), torch.float32, "lse_part", optional=max_splits == 1)


def prefill_num_splits(desc: AttnDesc, batch: int, max_q_len: int, max_seq_len: int, num_cus: int = 256):
    """(max_splits, split_keys) the library suggests for a prefill of this shape."""
    sk = ctypes.c_int32(0)
    ms = lib().pfa_prefill_num_splits(ctypes.byref(desc.c()), int(batch), int(max_q_len), int(max_seq_len),
                                      int(num_cus), ctypes.byref(sk))
    return int(ms), int(sk.value)


def paged_attn_prefill(desc: AttnDesc, pool: KVPool, q, cu_q, block_table, seq_lens, max_q_len: int,
                       out, max_seq_len: Optional[int] = None, split_keys: int = 0, max_splits: int = 1,
                       o_part=None, lse_part=None, stream=None):
    """Causal prefill of the new tokens q [Tq, Hq, D] bf16 into out [Tq, Hq, D] fp32.
    With max_splits > 1 the key range is split (o_part [Tq, Hq, max_splits, D] and
    lse_part [Tq, Hq, max_splits] fp32 are the caller's workspace)."""
    _check_chunk(desc, pool, q, cu_q, block_table, seq_lens, out, max_splits, o_part, lse_part)
    if max_seq_len is None:
        max_seq_len = int(block_table.shape[1]) * desc.page_size
    st = lib().pfa_paged_attn_prefill(ctypes.byref(desc.c()), ctypes.byref(pool.c()), _ptr(q),
                                      _ptr(cu_q), _ptr(block_table), int(block_table.shape[1]),
                                      _ptr(seq_lens), int(seq_lens.numel()), int(max_q_len),
                                      int(max_seq_len), int(split_keys), int(max_splits),
                                      _ptr(o_part), _ptr(lse_part), _ptr(out), _stream(stream, q))
    _check("pfa_paged_attn_prefill", st)


def verify_num_splits(desc: AttnDesc, batch: int, max_q_len: int, max_seq_len: int, num_cus: int = 256):
    """(max_splits, split_keys) the library suggests for a verify step of this shape."""
    sk = ctypes.c_int32(0)
    ms = lib().pfa_verify_num_splits(ctypes.byref(desc.c()), int(batch), int(max_q_len), int(max_seq_len),
                                     int(num_cus), ctypes.byref(sk))
    return int(ms), int(sk.value)


def paged_attn_verify(desc: AttnDesc, pool: KVPool, q, cu_q, block_table, seq_lens, max_q_len: int,
                      out, max_seq_len: Optional[int] = None, split_keys: int = 0, max_splits: int = 1,
                      o_part=None, lse_part=None, stream=None):
    """Verify step: 2-16 new tokens per sequence, q [Tq, Hq, D] bf16 -> out [Tq, Hq, D]
    fp32, the same result as paged_attn_prefill for that chunk (see pfa.h)."""
    _check_chunk(desc, pool, q, cu_q, block_table, seq_lens, out, max_splits, o_part, lse_part)
    if max_seq_len is None:
        max_seq_len = int(block_table.shape[1]) * desc.page_size
    st = lib().pfa_paged_attn_verify(ctypes.byref(desc.c()), ctypes.byref(pool.c()), _ptr(q),
                                     _ptr(cu_q), _ptr(block_table), int(block_table.shape[1]),
                                     _ptr(seq_lens), int(seq_lens.numel()), int(max_q_len),
                                     int(max_seq_len), int(split_keys), int(max_splits),
                                     _ptr(o_part), _ptr(lse_part), _ptr(out), _stream(stream, q))
    _check("pfa_paged_attn_verify", st)


def bounds_errors() -> int:
    """The PFA_BOUNDS_* bits the kernels of the loaded build reported on the current
    device since the last call (then cleared); synchronises the device.  Raises
    PfaError (PFA_ERR_UNSUPPORTED) on the normal build, which does not check."""
    flags = ctypes.c_uint32(0)
    _check("pfa_bounds_errors", lib().pfa_bounds_errors(ctypes.byref(flags)))
    return int(flags.value)


__all__ = ["AttnDesc", "KVPool", "PfaError", "EXPORTS", "lib", "kv_write", "bounds_errors",
           "DEBUG_LIB_PATH", "load_library", "use_library", "attn_input", "decode_num_splits",
           "decode_workspace_bytes",
           "tq3_codebook", "paged_attn_decode_static", "STATIC_SCRATCH_BYTES",
           "prefill_num_splits", "verify_num_splits", "paged_attn_decode", "paged_attn_decode_fused",
           "paged_attn_combine",
           "paged_attn_prefill", "paged_attn_verify"]
