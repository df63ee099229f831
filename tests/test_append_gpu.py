"""GPU: writing new rows into the paged cache (mla_kv_append) against the
oracle's encoder, byte for byte, and a decode over the appended cache."""
import numpy as np
import pytest
import torch

import mla_inputs as mi
from oracle import mla_oracle as orc

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mla():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mla_paged_decode_04_amd as m
    m.library()
    return m


def rows_with_edge_values(rng, n, scale, fp8):
    x = rng.standard_normal((n, 576)).astype(np.float32)
    x[0, :64] *= 1e-3 * scale          # fp8 subnormals after division by the scale
    x[1, :64] *= 1e3 * scale           # beyond 448 * scale: saturates
    x[2, :8] = np.array([0.0, -0.0, 448.0, -448.0, 1e30, -1e30, 3.0, -3.0]) * scale
    if fp8:
        x[3, :2] = np.nan
    return orc.round_bf16(x)


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("bs", [64, 128])
def test_kv_append_is_bit_exact(mla, kv_dtype, bs):
    rng = np.random.default_rng(11 if kv_dtype == "bf16" else 12)
    nb, n = 7, 300
    scale = 1.0 if kv_dtype == "bf16" else 0.0213
    rows = rows_with_edge_values(rng, n, scale, kv_dtype == "fp8")
    slots = rng.permutation(nb * bs)[:n].astype(np.int32)
    slots[5] = -1
    slots[9] = nb * bs + 3            # out of range: no write
    dt = np.uint16 if kv_dtype == "bf16" else np.uint8
    kv0 = rng.integers(0, 1 << (16 if kv_dtype == "bf16" else 8), size=(nb, bs, 576)).astype(dt)
    ref = orc.kv_append(kv0, rows, slots, scale, kv_dtype)

    dev = torch.device("cuda:0")
    tdt = torch.bfloat16 if kv_dtype == "bf16" else torch.float8_e4m3fn
    kv = torch.from_numpy(kv0.view(np.int16) if kv_dtype == "bf16" else kv0).to(dev).view(tdt)
    r = torch.from_numpy(rows.view(np.int16)).to(dev).view(torch.bfloat16)
    s = torch.from_numpy(slots).to(dev)
    mla.mla_kv_append(r, s, kv, scale)
    torch.cuda.synchronize()
    got = kv.view(torch.int16 if kv_dtype == "bf16" else torch.uint8).cpu().numpy().view(dt)
    if kv_dtype == "bf16":
        np.testing.assert_array_equal(got, ref)
    else:
        np.testing.assert_array_equal(got, ref)


def test_kv_append_fp8_every_code_and_tie(mla):
    """Every positive e4m3fn value, every midpoint between neighbouring values
    (exact ties: the even mantissa wins), the bf16 values just below and above
    each midpoint, values past 448 (saturation), both signs; scale 1, so the
    row values reach the encoder unchanged. Byte for byte against the oracle."""
    pos = orc.E4M3FN_TABLE[:0x7F].astype(np.float32)              # 0 .. 448
    mid_bits = orc.round_bf16((pos[:-1] + pos[1:]) / np.float32(2))   # exact in bf16
    vals = np.concatenate([orc.round_bf16(pos), mid_bits, mid_bits - 1, mid_bits + 1,
                           orc.round_bf16(np.float32([464.0, 480.0, 1e4, 2.0 ** -10, 3 * 2.0 ** -11]))])
    vals = np.concatenate([vals, vals | np.uint16(0x8000)]).astype(np.uint16)
    n_rows = -(-len(vals) // 576)
    rows = np.zeros((n_rows, 576), dtype=np.uint16)
    rows.flat[:len(vals)] = vals
    slots = np.arange(n_rows, dtype=np.int32)
    kv0 = np.zeros((1, 64, 576), dtype=np.uint8)
    ref = orc.kv_append(kv0, rows, slots, 1.0, "fp8")
    dev = torch.device("cuda:0")
    kv = torch.from_numpy(kv0).to(dev).view(torch.float8_e4m3fn)
    r = torch.from_numpy(rows.view(np.int16)).to(dev).view(torch.bfloat16)
    mla.mla_kv_append(r, torch.from_numpy(slots).to(dev), kv, 1.0)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(kv.view(torch.uint8).cpu().numpy(), ref)


@pytest.mark.parametrize("name", ["tiny", "tiny_fp8"])
def test_append_last_token_then_decode(mla, name):
    # rebuild each sequence's newest cached row through the append kernel
    wl = mi.WORKLOADS[name]
    inp = mi.make_inputs(wl)
    rng = np.random.default_rng(3)
    B, bs = wl.batch, wl.block_size
    new_rows = orc.round_bf16(rng.standard_normal((B, 576)).astype(np.float32))
    slots = np.array([inp.block_table[b, (inp.seq_lens[b] - 1) // bs] * bs + (inp.seq_lens[b] - 1) % bs
                      for b in range(B)], dtype=np.int32)
    scale = inp.kv_scale
    ref_kv = orc.kv_append(inp.kv, new_rows, slots, scale, wl.kv_dtype)

    dev = torch.device("cuda:0")
    if wl.kv_dtype == "bf16":
        kv = torch.from_numpy(inp.kv.view(np.int16)).to(dev).view(torch.bfloat16)
    else:
        kv = torch.from_numpy(inp.kv).to(dev).view(torch.float8_e4m3fn)
    mla.mla_kv_append(torch.from_numpy(new_rows.view(np.int16)).to(dev).view(torch.bfloat16),
                      torch.from_numpy(slots).to(dev), kv, scale)
    q = torch.from_numpy(inp.q_bits.view(np.int16)).to(dev).view(torch.bfloat16)
    bt = torch.from_numpy(inp.block_table).to(dev)
    sl = torch.from_numpy(inp.seq_lens).to(dev)
    out, lse = mla.mla_decode(q, kv, bt, sl, wl.softmax_scale, scale, causal=wl.causal)
    torch.cuda.synchronize()
    got_kv = kv.view(torch.int16 if wl.kv_dtype == "bf16" else torch.uint8).cpu().numpy()
    np.testing.assert_array_equal(got_kv.view(ref_kv.dtype), ref_kv)
    ro, rl = orc.mla_decode(inp.q_bits, ref_kv, inp.block_table, inp.seq_lens, wl.s_q,
                            wl.softmax_scale, scale, wl.kv_dtype, wl.causal)
    o = out.float().cpu().double().numpy()
    tol = 5e-3 if wl.kv_dtype == "bf16" else 1e-2
    assert orc.rel_fro(o, ro) <= tol
    assert np.abs(lse.cpu().double().numpy() - rl).max() <= 1e-3


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
def test_kv_append_beyond_4gib(mla, kv_dtype):
    # slots above the 4 GiB offset of a cache of about 4.3 GB: the row address
    # needs 64-bit arithmetic. The written region against the oracle's encoder
    # on a compact copy of it, byte for byte.
    rng = np.random.default_rng(13 if kv_dtype == "bf16" else 14)
    bs, nb, n = 64, 7, 300
    row_bytes = 576 * (2 if kv_dtype == "bf16" else 1)
    base_page = (2 ** 32) // (bs * row_bytes) + 1
    scale = 1.0 if kv_dtype == "bf16" else 0.0213
    rows = rows_with_edge_values(rng, n, scale, kv_dtype == "fp8")
    slots = rng.permutation(nb * bs)[:n].astype(np.int32)
    dt = np.uint16 if kv_dtype == "bf16" else np.uint8
    kv0 = rng.integers(0, 1 << (16 if kv_dtype == "bf16" else 8), size=(nb, bs, 576)).astype(dt)
    ref = orc.kv_append(kv0, rows, slots, scale, kv_dtype)

    dev = torch.device("cuda:0")
    tdt = torch.bfloat16 if kv_dtype == "bf16" else torch.float8_e4m3fn
    big = torch.empty((base_page + nb, bs, 576), dtype=tdt, device=dev)
    assert big.numel() * big.element_size() > 2 ** 32
    big[base_page:] = torch.from_numpy(kv0.view(np.int16) if kv_dtype == "bf16" else kv0).to(dev).view(tdt)
    r = torch.from_numpy(rows.view(np.int16)).to(dev).view(torch.bfloat16)
    s = torch.from_numpy(slots + base_page * bs).to(dev)
    mla.mla_kv_append(r, s, big, scale)
    torch.cuda.synchronize()
    got = big[base_page:].view(torch.int16 if kv_dtype == "bf16" else torch.uint8).cpu().numpy().view(dt)
    np.testing.assert_array_equal(got, ref)
