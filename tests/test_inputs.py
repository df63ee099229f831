"""The seeded input generator (CPU only)."""
import numpy as np
import pytest

import mla_inputs as mi


def test_bf16_rounding_is_nearest_even():
    one = np.float32(1.0)
    ulp = np.float32(2.0 ** -7)        # bf16 spacing in [1, 2)
    x = np.array([one, one + ulp / 2, one + 3 * ulp / 2, one + ulp / 4, one + 3 * ulp / 4,
                  -(one + ulp / 2)], dtype=np.float32)
    got = mi.f32_to_bf16_bits(x)
    want = np.array([0x3F80, 0x3F80, 0x3F82, 0x3F80, 0x3F81, 0xBF80], dtype=np.uint16)
    np.testing.assert_array_equal(got, want)


def test_fp8_quantiser_saturates_and_rounds():
    x = np.array([0.0, 1.0, 448.0, 1000.0, -1000.0, 1.0625, 1.1875, 2.0 ** -9, 2.0 ** -11],
                 dtype=np.float32)
    got = mi.f32_to_e4m3fn_codes(x)
    # 1.0625 is halfway between 1.0 (0x38) and 1.125 (0x39): ties to even -> 0x38
    # 1.1875 is halfway between 1.125 (0x39) and 1.25 (0x3A): ties to even -> 0x3A
    want = np.array([0x00, 0x38, 0x7E, 0x7E, 0xFE, 0x38, 0x3A, 0x01, 0x00], dtype=np.uint8)
    np.testing.assert_array_equal(got, want)


@pytest.mark.parametrize("name", ["tiny", "tiny_fp8"])
def test_block_table_is_a_permutation_and_tails_are_poisoned(name):
    wl = mi.WORKLOADS[name]
    inp = mi.make_inputs(wl)
    bs = wl.block_size
    bt = inp.block_table
    used = bt[bt >= 0]
    assert len(np.unique(used)) == len(used)                 # no page shared
    assert used.max() < inp.num_blocks
    for b, L in enumerate(inp.seq_lens):
        n = (int(L) + bs - 1) // bs
        assert (bt[b, :n] >= 0).all() and (bt[b, n:] == -1).all()
        tail = int(L) - (n - 1) * bs
        last = inp.kv[bt[b, n - 1]]
        nan = mi.BF16_NAN if wl.kv_dtype == "bf16" else mi.FP8_NAN
        assert (last[tail:] == nan).all()
        assert not (last[:tail] == nan).all(axis=1).any()
    spare = np.setdiff1d(np.arange(inp.num_blocks), used)
    assert len(spare) == wl.spare_pages


def test_fp8_scale_is_amax_over_448():
    wl = mi.WORKLOADS["tiny_fp8"]
    inp = mi.make_inputs(wl)
    assert inp.kv_scale == float(np.float32(inp.kv_scale))
    # the largest magnitude code is 448 (0x7E/0xFE) exactly once the scale is amax/448
    valid = inp.kv[inp.kv != mi.FP8_NAN]
    assert ((valid & 0x7F) == 0x7E).any()
    assert not ((valid & 0x7F) == 0x7F).any()


def test_same_seed_same_inputs():
    a = mi.make_inputs(mi.WORKLOADS["tiny"])
    b = mi.make_inputs(mi.WORKLOADS["tiny"])
    np.testing.assert_array_equal(a.q_bits, b.q_bits)
    np.testing.assert_array_equal(a.kv, b.kv)
    np.testing.assert_array_equal(a.block_table, b.block_table)


def test_length_distributions():
    rng = np.random.default_rng(0)
    L = mi.draw_seq_lens(mi.WORKLOADS["b32_sq4_h128_L512_16k_fp8"], rng)
    assert L.min() >= 512 and L.max() <= 16384 and L.shape == (32,)
    L = mi.draw_seq_lens(mi.WORKLOADS["b64_h128_L1k2k_bs128_bf16"], rng)
    assert L.min() >= 1000 and L.max() <= 2048 and L.shape == (64,)
