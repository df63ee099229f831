"""CPU: bench.py's algorithmic byte and flop counts against closed forms of the
workloads (q, each cached row once, block-table entries, seq_lens, out, lse;
2 * (576 + 512) flops per visible (query row, key)). These are the figures the
roofline fractions divide by."""
import types

import numpy as np
import pytest

import bench
import mla_inputs as mi


def fake_inputs(name):
    wl = mi.WORKLOADS[name]
    lens = mi.draw_seq_lens(wl, np.random.default_rng(wl.seed))
    return types.SimpleNamespace(wl=wl, seq_lens=np.asarray(lens, dtype=np.int32))


@pytest.mark.parametrize("name,row_bytes", [("b128_h16_L4096_bf16", 1152), ("b128_h16_L4096_fp8", 576)])
def test_fixed_length_workloads(name, row_bytes):
    inp = fake_inputs(name)
    B, H, L, bs = 128, 16, 4096, 64
    kv = B * L * row_bytes
    expected = kv + B * (L // bs) * 4 + B * 4 + B * H * (576 * 2 + 512 * 2 + 4)
    assert bench.algorithmic_bytes(inp) == expected
    assert bench.algorithmic_flops(inp) == 2 * H * 1088 * B * L == 18_253_611_008


def test_the_kernel_test_shape_numbers():
    # 128 sequences of 4096 tokens, 16 heads: 604.0 MB of bf16 cache rows and
    # 608.5 MB in all; half the cache bytes with fp8
    assert bench.algorithmic_bytes(fake_inputs("b128_h16_L4096_bf16")) == 608_477_696
    assert bench.algorithmic_bytes(fake_inputs("b128_h16_L4096_fp8")) == 306_487_808


def test_causal_query_blocks_count_each_token_once():
    # s_q = 4, causal: query token i of a sequence of L tokens sees L - 3 + i keys
    inp = fake_inputs("b32_sq4_h128_L512_16k_fp8")
    lens = inp.seq_lens.astype(np.int64)
    vis = sum(int(np.clip(lens - 4 + 1 + i, 0, None).sum()) for i in range(4))
    assert bench.algorithmic_flops(inp) == 2 * 128 * 1088 * vis
    assert vis == 4 * int(lens.sum()) - 6 * len(lens)   # all lengths >= 4


def test_decode_kernel_names_follow_the_row_groups():
    assert bench.decode_kernel_name(16) == "mla_decode_narrow"
    assert bench.decode_kernel_name(17) == "mla_decode_wide"
    assert bench.decode_kernel_name(64) == "mla_decode_wide"
    assert bench.decode_kernel_name(65) == "mla_decode_wide128"
    assert bench.decode_kernel_name(512) == "mla_decode_wide128"
