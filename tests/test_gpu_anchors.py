"""Order-free anchors for the two bit-exact paths whose oracle fixes an fp32
summation order (the 3-bit encoder and the fused attention input).  The oracle
reproduces one rounding order (groups of 8, then a pairwise tree), which the
pages do not state; these tests check the GPU outputs against float64
definitions that have no order at all:

* 3-bit rotated KV (qengine README feature list: a Walsh-Hadamard rotation and a
  Lloyd-Max quantiser): each code is the float64-nearest of the 8 levels to
  t = y / rms(y), y = H x (scipy's Hadamard matrix), wherever t is more than 1e-5
  from a cell edge; the scale is ||x|| to 1e-6.
* Fused attention input (TileInfer.jl Performance, "Fused kernels,
  FlashAttention and PagedAttention": bit-identical to the chain of ops): q and
  k equal the float64 chain -- RMSNorm, round to bf16, RoPE, round to bf16 -- to
  within one bf16 step of the result plus the step a hand-off rounding can carry
  through the rotation, and are exactly that correctly rounded value on at least
  98% of the elements.  v is copied bit for bit.
"""
import numpy as np
import pytest
import scipy.linalg
import torch

import paged_flash_attention_amd as pfa
import workloads as W
from gpu_support import GpuCase, bits_of, gpu_attn_input

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    pfa.lib()


def f64(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def bf16_round64(x):
    """float64 -> nearest bfloat16 value, ties to even, in one rounding."""
    m, e = np.frexp(np.asarray(x, np.float64))
    return np.ldexp(np.rint(m * 256.0), e - 8)


def bf16_step(x):
    return 2.0 ** (np.floor(np.log2(np.maximum(np.abs(x), 1e-38))) - 7)


def slots(case, h_count):
    """(page, offset) of every new token, in token order."""
    out = []
    for s in range(case.batch):
        n, ql = int(case.seq_lens[s]), int(case.q_lens[s])
        for pos in range(n - ql, n):
            out.append((int(case.block_table[s][pos // case.p.page_size]), pos % case.p.page_size))
    return out


# ---------------------------------------------------------------------------
# fused attention input
# ---------------------------------------------------------------------------

ANCHOR_INPUT_CASES = [
    (dict(Hq=32, Hkv=8, D=128), [300, 41], [300, 17], 1.0),
    (dict(Hq=64, Hkv=8, D=64), [200, 9], [200, 9], 30.0),
    (dict(Hq=16, Hkv=4, D=128), [128], [64], 0.25),
]


def chain64(x, w, eps, co, si):
    """The chain in float64: RMSNorm, bf16, RoPE (rotate-half), bf16.  Returns the
    result and the bound of one step plus what a hand-off rounding carries."""
    D = x.shape[-1]
    h = D // 2
    yx = x / np.sqrt((x * x).mean(-1, keepdims=True) + eps) * w
    y = bf16_round64(yx)
    out = np.concatenate([y[..., :h] * co - y[..., h:] * si, y[..., h:] * co + y[..., :h] * si], -1)
    sy = bf16_step(yx)
    carry = np.concatenate([np.abs(co) * sy[..., :h] + np.abs(si) * sy[..., h:],
                            np.abs(co) * sy[..., h:] + np.abs(si) * sy[..., :h]], -1)
    return bf16_round64(out), (bf16_step(out) + carry) * 1.0001


@pytest.mark.parametrize("ci", range(len(ANCHOR_INPUT_CASES)))
def test_attn_input_against_float64_chain(ci):
    prm, lens, new, scale = ANCHOR_INPUT_CASES[ci]
    p = W.AttnParams(prm["Hq"], prm["Hkv"], prm["D"])
    ic = W.attn_input_case(f"anc{ci}", 620 + ci, p, lens, new, qkv_scale=scale)
    c = ic.case
    D, Hq, Hkv = p.head_dim, p.num_q_heads, p.num_kv_heads
    q_bits, pool = gpu_attn_input(ic)
    T = int(c.cu_q[-1])
    x = f64(ic.qkv).reshape(T, Hq + 2 * Hkv, D)
    pos = np.concatenate([np.arange(int(c.seq_lens[s]) - int(c.q_lens[s]), int(c.seq_lens[s]))
                          for s in range(c.batch)])
    cs = ic.rope[pos].astype(np.float64)
    co, si = cs[..., 0][:, None, :], cs[..., 1][:, None, :]
    kb, vb = bits_of(pool.k), bits_of(pool.v)
    sl = slots(c, Hkv)
    k_got = f64(np.stack([kb[pg, :, off] for pg, off in sl]))
    v_got = np.stack([vb[pg, :, off] for pg, off in sl])
    for name, got, xs, w in (("q", f64(q_bits).reshape(T, Hq, D), x[:, :Hq], f64(ic.q_norm_w)),
                             ("k", k_got, x[:, Hq:Hq + Hkv], f64(ic.k_norm_w))):
        exact, bound = chain64(xs, w, ic.eps, co, si)
        d = np.abs(got - exact)
        assert np.all(d <= bound), f"{name}: {np.sum(d > bound)} elements beyond the bound"
        eq = float(np.mean(got == exact))
        print(f"case {ci} {name}: {eq:.6f} of elements equal the correctly rounded float64 chain", flush=True)
        assert eq >= 0.98
    v_in = np.asarray(ic.qkv).reshape(T, Hq + 2 * Hkv, D)[:, Hq + Hkv:]
    assert np.array_equal(v_got, v_in)


# ---------------------------------------------------------------------------
# 3-bit rotated KV write
# ---------------------------------------------------------------------------

def unpack3(packed, D):
    """[..., 3D/8] bytes -> [..., D] codes: field j (3 bytes, little endian) holds
    elements 8j..8j+7, element 8j+i in bits 3i..3i+2."""
    b = packed.astype(np.uint32).reshape(*packed.shape[:-1], D // 8, 3)
    field = b[..., 0] | (b[..., 1] << 8) | (b[..., 2] << 16)
    return np.stack([(field >> (3 * i)) & 7 for i in range(8)], -1).reshape(*packed.shape[:-1], D)


def lloyd_max_levels64():
    """The 4 positive levels of the 8-level Lloyd-Max quantiser of N(0,1), float64
    (Lloyd's iteration with scipy's normal pdf/cdf)."""
    from scipy.stats import norm
    m = np.array([0.25, 0.75, 1.25, 2.0])
    for _ in range(10000):
        e = np.concatenate([[0.0], (m[:-1] + m[1:]) / 2, [np.inf]])
        n = (norm.pdf(e[:-1]) - norm.pdf(e[1:])) / (norm.cdf(e[1:]) - norm.cdf(e[:-1]))
        if np.max(np.abs(n - m)) < 1e-15:
            break
        m = n
    return n


@pytest.mark.parametrize("D", [64, 128])
def test_tq3_codes_are_the_float64_nearest_level(D):
    p = W.AttnParams(8, 2, D, kv_dtype="tq3")
    case = W.make_case("anc3", 640 + D, p, [200, 77, 300], [200, 77, 150], outlier_frac=0.01)
    g = GpuCase(case)
    torch.cuda.synchronize()
    kp, ks = g.pool.k.cpu().numpy(), g.pool.k_scale.cpu().numpy()
    sl = slots(case, p.num_kv_heads)
    codes = unpack3(np.stack([kp[pg, :, off] for pg, off in sl]), D)        # [T, Hkv, D]
    scale = np.stack([ks[pg, :, off] for pg, off in sl]).astype(np.float64)
    k_new, _, _ = case.new_tokens()
    x = f64(k_new)                                                          # [T, Hkv, D]
    y = x @ scipy.linalg.hadamard(D).T.astype(np.float64)
    rms = np.sqrt((y * y).mean(-1))
    assert np.allclose(scale, np.linalg.norm(x, axis=-1), rtol=1e-6)
    t = y / rms[..., None]
    M = lloyd_max_levels64()
    lev = np.concatenate([-M[::-1], M])                                     # ascending
    nearest = np.abs(t[..., None] - lev).argmin(-1)
    want = np.where(nearest >= 4, 4 + (nearest - 4), 3 - nearest)          # sign-magnitude
    edges = np.concatenate([-((M[1:] + M[:-1]) / 2)[::-1], [0.0], (M[1:] + M[:-1]) / 2])
    clear = np.abs(t[..., None] - edges).min(-1) > 1e-5
    print(f"D={D}: {clear.mean():.5f} of elements clear of a cell edge", flush=True)
    assert clear.mean() > 0.99
    assert np.array_equal(codes[clear], want[clear])
