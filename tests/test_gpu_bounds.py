"""Device-side bounds checks of the debug build (libpfa_debug.so, PFA_BOUNDS_CHECK=1).

The kernels of every build clamp block-table entries and lengths, so a broken
device-side contract gives wrong numbers and never an access outside the pool or
the block table.  The debug build also reports each violation as a PFA_BOUNDS_*
bit in a device error word, read (and cleared) by pfa_bounds_errors.

* Valid inputs: every entry point runs with no bit set, and decode/prefill give
  the same bits as the normal build.
* Broken inputs (each turned into an error by the kernels' own checks): block-table
  entries past the pool and below 0, a length past the block-table row, a length
  below the chunk's new-token count (and 0), and a length past the splits a decode
  call covers.  Each sets its bit; outputs are not judged.
"""
import numpy as np
import pytest
import torch

import paged_flash_attention_amd as pfa
import workloads as W
from gpu_support import GpuCase, gpu_attn_input

pytestmark = pytest.mark.gpu

PAGE, SEQ_LEN, Q_LEN = pfa.BOUNDS_PAGE, pfa.BOUNDS_SEQ_LEN, pfa.BOUNDS_Q_LEN


@pytest.fixture(scope="module")
def debug_lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    pfa.lib()
    return pfa.load_library(pfa.DEBUG_LIB_PATH)


class use_debug:
    def __init__(self, L):
        self.L = L

    def __enter__(self):
        self.prev = pfa.use_library(self.L)
        pfa.bounds_errors()              # start from a clear word
        return self

    def __exit__(self, *exc):
        pfa.use_library(self.prev)


def params(kv="bf16", Hq=32, Hkv=8, D=128, window=0):
    return W.AttnParams(Hq, Hkv, D, kv_dtype=kv, window=window)


def test_valid_inputs_set_no_bit_and_match_the_normal_build(debug_lib):
    dec = {kv: W.make_case(f"bd_{kv}", 900 + i, params(kv, Hkv=4 if kv != "bf16" else 8),
                           [40, 777, 2049], [1, 1, 1], outlier_frac=0.01)
           for i, kv in enumerate(("bf16", "int8", "tq3"))}
    pre = W.make_case("bp", 905, params(), [300, 1500], [300, 130], split_keys=0)
    ver = W.make_case("bv", 906, params(), [1040, 77], [16, 5], split_keys=0)
    ic = W.attn_input_case("bi", 907, params(), [300, 41], [300, 17])
    normal = {}
    for kv, c in dec.items():
        normal[kv] = [GpuCase(c).decode(split_keys=S) for S in (0, 256)]
    normal_pre = [GpuCase(pre).prefill(split=s) for s in (None, "auto")]
    with use_debug(debug_lib):
        for kv, c in dec.items():
            g = GpuCase(c)                                     # kv_write through the debug build
            for S, ref in zip((0, 256), normal[kv]):
                got = g.decode(split_keys=S)
                assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), f"{kv} S={S}"
        g = GpuCase(pre)
        for s, ref in zip((None, "auto"), normal_pre):
            assert np.array_equal(g.prefill(split=s).view(np.uint32), ref.view(np.uint32)), f"prefill {s}"
        GpuCase(ver).verify(split="auto")
        gpu_attn_input(ic)
        assert pfa.bounds_errors() == 0


def test_block_table_entries_outside_the_pool(debug_lib):
    for kv in ("bf16", "int8", "tq3"):
        dc = W.make_case(f"bpd_{kv}", 910, params(kv, Hkv=4), [700, 300], [1, 1], outlier_frac=0.01)
        pc = W.make_case(f"bpp_{kv}", 911, params(kv, Hkv=4), [700, 300], [130, 1], split_keys=0,
                         outlier_frac=0.01)
        for c, ops in ((dc, ("decode", "decode_split", "kv_write")),
                       (pc, () if kv == "tq3" else ("prefill", "prefill_split"))):
            g = GpuCase(c)
            npages = g.pool.k.shape[0]
            with use_debug(debug_lib):
                g.bt[0, 3] = npages + 5              # inside sequence 0's prefix
                g.bt[1, 18] = -3                     # sequence 1's last page (its new token)
                for op in ops:
                    if op == "decode":
                        g.decode(split_keys=0)
                    elif op == "decode_split":
                        g.decode(split_keys=256)
                    elif op == "kv_write":
                        g.write_new()
                    elif op == "prefill":
                        g.prefill(split=None)
                    else:
                        g.prefill(split=(128, 6))
                    assert pfa.bounds_errors() & PAGE, f"{kv} {op}"


def test_lengths_outside_the_contract(debug_lib):
    dc = W.make_case("bld", 920, params(), [700, 300], [1, 1])
    pc = W.make_case("blp", 921, params(), [700, 300], [130, 1], split_keys=0)
    gd, gp = GpuCase(dc), GpuCase(pc)
    bt_cap = gd.bt.shape[1] * 16
    with use_debug(debug_lib):
        for g in (gd, gp):
            g.seq_lens[1] = bt_cap + 40              # past its block-table row
        gd.decode(split_keys=0)
        assert pfa.bounds_errors() & SEQ_LEN, "decode"
        gp.prefill(split=None)
        assert pfa.bounds_errors() & SEQ_LEN, "prefill"
        gd.write_new()
        assert pfa.bounds_errors() & SEQ_LEN, "kv_write"

        gp.seq_lens.copy_(torch.tensor([100, 300], dtype=torch.int32))   # 100 < the 130 new tokens
        gp.prefill(split=None)
        assert pfa.bounds_errors() & Q_LEN, "prefill, length below the chunk"
        gp.prefill(split=(128, 6))
        assert pfa.bounds_errors() & Q_LEN, "prefill split, length below the chunk"
        gp.write_new()
        assert pfa.bounds_errors() & Q_LEN, "kv_write, length below the chunk"
        gp.seq_lens.copy_(torch.tensor([0, 300], dtype=torch.int32))     # no pages at all
        gp.prefill(split=None)
        assert pfa.bounds_errors() & Q_LEN, "prefill, length 0"

        # a decode call told max_seq_len 512 (two 256-key splits) over a 700-key sequence
        gd.seq_lens.copy_(torch.tensor([700, 300], dtype=torch.int32))
        op = torch.zeros((2, 32, 2, 128), device="cuda")
        lp = torch.zeros((2, 32, 2), device="cuda")
        pfa.paged_attn_decode(gd.desc, gd.pool, gd.q, gd.bt, gd.seq_lens, 512, 256, 2, o_part=op, lse_part=lp)
        assert pfa.bounds_errors() == SEQ_LEN, "decode splits short of the length"
