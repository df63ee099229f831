"""GPU: the absorbed projections (mla_absorb_q / mla_absorb_out) against the
float64 oracle. bf16 results: relative Frobenius error <= 5e-3 (about twice
the bf16 rounding of the output); the copied rotary part is bit-exact."""
import numpy as np
import pytest
import torch

from oracle import mla_oracle as orc

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mla():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mla_paged_decode_04_amd as m
    m.library()
    return m


def bf16(rng, shape, scale=1.0):
    return orc.round_bf16((rng.standard_normal(shape) * scale).astype(np.float32))


def dev(bits):
    return torch.from_numpy(bits.view(np.int16)).to("cuda:0").view(torch.bfloat16)


# From 241 tokens on, d = 128 takes the ring kernels: 256 / H workgroups per
# head, each over a run of 16-token tiles. 600 tokens at H = 128 give each
# workgroup 19 tiles (the last one ragged), so the LDS rings (8 and 5 slots)
# wrap twice or more; 2100 tokens at H = 2 give 2 tiles per workgroup. Other
# shapes take the streaming or weight-stationary kernels.
@pytest.mark.parametrize("T,H,d", [(128, 16, 128), (64, 128, 128), (37, 3, 64), (1, 1, 32), (2100, 2, 128),
                                   (256, 1, 128), (1000, 5, 128), (600, 128, 128)])
def test_absorb_q(mla, T, H, d):
    rng = np.random.default_rng(T * 1000 + H)
    qn, pe, w = bf16(rng, (T, H, d)), bf16(rng, (T, H, 64)), bf16(rng, (H, d, 512), d ** -0.5)
    out = mla.mla_absorb_q(dev(qn), dev(pe), dev(w))
    torch.cuda.synchronize()
    got = out.float().cpu().double().numpy()
    ref = orc.absorb_q(qn, pe, w)
    assert orc.rel_fro(got[..., :512], ref[..., :512]) <= 5e-3
    np.testing.assert_array_equal(got[..., 512:], ref[..., 512:])


@pytest.mark.parametrize("T,H,dv", [(128, 16, 128), (64, 128, 128), (37, 3, 64), (5, 2, 192),
                                    (4200, 2, 128), (4200, 3, 64), (256, 1, 128), (1000, 5, 128),
                                    (600, 128, 128)])
def test_absorb_out(mla, T, H, dv):
    rng = np.random.default_rng(T * 1000 + H + 7)
    o, w = bf16(rng, (T, H, 512)), bf16(rng, (H, 512, dv), 512 ** -0.5)
    out = mla.mla_absorb_out(dev(o), dev(w))
    torch.cuda.synchronize()
    assert orc.rel_fro(out.float().cpu().double().numpy(), orc.absorb_out(o, w)) <= 5e-3


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
def test_absorbed_decode_chain(mla, kv_dtype):
    # q_nope . W_UK (+ q_pe) -> paged MQA decode -> o . W_UV, against the same
    # chain in float64 with q rounded to bf16 where the GPU path stores it
    import mla_inputs as mi
    wl = mi.WORKLOADS["tiny" if kv_dtype == "bf16" else "tiny_fp8"]
    inp = mi.make_inputs(wl)
    rng = np.random.default_rng(31)
    B, H, d, dv = wl.batch, wl.heads, 128, 128
    qn, pe = bf16(rng, (B, H, d)), bf16(rng, (B, H, 64))
    w_uk, w_uv = bf16(rng, (H, d, 512), d ** -0.5), bf16(rng, (H, 512, dv), 512 ** -0.5)
    q = mla.mla_absorb_q(dev(qn), dev(pe), dev(w_uk))
    if kv_dtype == "bf16":
        kv = torch.from_numpy(inp.kv.view(np.int16)).to("cuda:0").view(torch.bfloat16)
    else:
        kv = torch.from_numpy(inp.kv).to("cuda:0").view(torch.float8_e4m3fn)
    bt = torch.from_numpy(inp.block_table).to("cuda:0")
    sl = torch.from_numpy(inp.seq_lens).to("cuda:0")
    o, _ = mla.mla_decode(q.view(B, 1, H, 576), kv, bt, sl, wl.softmax_scale, inp.kv_scale)
    out = mla.mla_absorb_out(o.view(B, H, 512), dev(w_uv))
    torch.cuda.synchronize()

    q_ref = orc.round_bf16(orc.absorb_q(qn, pe, w_uk).astype(np.float32)).reshape(B, 1, H, 576)
    o_ref, _ = orc.mla_decode(q_ref, inp.kv, inp.block_table, inp.seq_lens, 1, wl.softmax_scale,
                              inp.kv_scale, wl.kv_dtype, True)
    ref = np.einsum("thn,hnv->thv", o_ref.reshape(B, H, 512), orc.bf16_bits_to_f64(w_uv))
    assert orc.rel_fro(out.float().cpu().double().numpy(), ref) <= 1e-2


def test_absorb_beyond_4gib(mla):
    # 33000 tokens x 128 heads: q (576 wide) is 4.9 GB and o 4.3 GB, so
    # element offsets pass 2^32 bytes; 9 token ranges per head, the last one
    # ragged. Sampled rows against the oracle (the full products take the
    # oracle minutes): the first, middle and last tokens of several ranges,
    # over several heads.
    T, H, d = 33000, 128, 128
    assert T * H * 576 * 2 > 2 ** 32 and T * H * 512 * 2 > 2 ** 32
    g = torch.Generator(device="cuda:0")
    g.manual_seed(4242)
    qn = torch.randn((T, H, d), device="cuda:0", generator=g).bfloat16()
    pe = torch.randn((T, H, 64), device="cuda:0", generator=g).bfloat16()
    w_uk = (torch.randn((H, d, 512), device="cuda:0", generator=g) * d ** -0.5).bfloat16()
    o = torch.randn((T, H, 512), device="cuda:0", generator=g).bfloat16()
    w_uv = (torch.randn((H, 512, d), device="cuda:0", generator=g) * 512 ** -0.5).bfloat16()
    q = mla.mla_absorb_q(qn, pe, w_uk)
    y = mla.mla_absorb_out(o, w_uv)
    torch.cuda.synchronize()
    toks = torch.tensor([0, 1, 15, 16, 4095, 4096, 16383, 16400, 29999, 32767, 32768, 32990, 32999])
    heads = torch.tensor([0, 1, 63, 64, 127])
    tt, hh = torch.meshgrid(toks, heads, indexing="ij")
    tt, hh = tt.reshape(-1), hh.reshape(-1)
    bits = lambda x: x.cpu().view(torch.int16).numpy()   # noqa: E731
    w_uk_b, w_uv_b = bits(w_uk), bits(w_uv)
    got_q = q[tt, hh].float().cpu().double().numpy()
    got_y = y[tt, hh].float().cpu().double().numpy()
    ref_q = np.stack([orc.absorb_q(bits(qn[t:t + 1, h:h + 1]), bits(pe[t:t + 1, h:h + 1]),
                                   w_uk_b[h:h + 1])[0, 0] for t, h in zip(tt.tolist(), hh.tolist())])
    ref_y = np.stack([orc.absorb_out(bits(o[t:t + 1, h:h + 1]), w_uv_b[h:h + 1])[0, 0]
                      for t, h in zip(tt.tolist(), hh.tolist())])
    assert orc.rel_fro(got_q[:, :512], ref_q[:, :512]) <= 5e-3
    np.testing.assert_array_equal(got_q[:, 512:], ref_q[:, 512:])
    assert orc.rel_fro(got_y, ref_y) <= 5e-3
    # every sampled row individually as well (a misplaced row would be off by ~1)
    for i in range(len(tt)):
        assert orc.rel_fro(got_q[i, :512], ref_q[i, :512]) <= 1e-2
        assert orc.rel_fro(got_y[i], ref_y[i]) <= 1e-2
