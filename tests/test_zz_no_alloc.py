"""mla_decode_noalloc (the fixed device scratch array instead of a caller
workspace) against mla_decode, through the C ABI, at the parity bar: two
calls in a row, the second with a smaller input. The first description needs
more than the array's 64 MiB under the regular workspace bound, so the
no-alloc plan uses fewer partial slots; the second fits and must give the
same bits as mla_decode."""
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


def _dev(inp):
    dev = torch.device("cuda:0")
    q = torch.from_numpy(inp.q_bits.view(np.int16)).to(dev).view(torch.bfloat16)
    if inp.wl.kv_dtype == "bf16":
        kv = torch.from_numpy(inp.kv.view(np.int16)).to(dev).view(torch.bfloat16)
    else:
        kv = torch.from_numpy(inp.kv).to(dev).view(torch.float8_e4m3fn)
    return q, kv, torch.from_numpy(inp.block_table).to(dev), torch.from_numpy(inp.seq_lens).to(dev)


def _both(mla, inp):
    wl = inp.wl
    q, kv, bt, sl = _dev(inp)
    shape = (wl.batch, wl.s_q, wl.heads)
    o1 = torch.full(shape + (512,), float("nan"), dtype=torch.bfloat16, device=q.device)
    l1 = torch.full(shape, float("nan"), dtype=torch.float32, device=q.device)
    o2, l2 = torch.full_like(o1, float("nan")), torch.full_like(l1, float("nan"))
    mla.mla_decode(q, kv, bt, sl, wl.softmax_scale, inp.kv_scale, causal=wl.causal, out=o1, lse=l1)
    mla.mla_decode_noalloc(q, kv, bt, sl, wl.softmax_scale, o2, l2, kv_scale=inp.kv_scale,
                           causal=wl.causal)
    torch.cuda.synchronize()
    f = lambda t: t.float().cpu().double().numpy()   # noqa: E731
    return f(o1), f(l1), f(o2), f(l2)


def _check(o_ref_call, l_ref_call, o, l, dtype, tag):
    tol = 5e-3 if dtype == "bf16" else 1e-2
    assert np.isfinite(o).all(), tag
    fin = np.isfinite(l_ref_call)
    assert (np.isneginf(l) == ~fin).all(), tag
    err = orc.rel_fro(o, o_ref_call)
    rows = float(orc.rel_fro_rows(o, o_ref_call).max())
    lerr = float(np.abs(l[fin] - l_ref_call[fin]).max()) if fin.any() else 0.0
    print(f"[{tag}] noalloc vs mla_decode: rel_fro={err:.3e} max_row={rows:.3e} max|dlse|={lerr:.3e}",
          flush=True)
    assert err <= tol and rows <= 2 * tol and lerr <= 1e-3, tag


def test_noalloc_matches_mla_decode_two_calls(mla):
    lib = mla.library()
    assert lib.mla_decode_noalloc_scratch_bytes() == 64 * 1024 * 1024
    # 1) 128 heads x 4 query tokens, long contexts: the regular workspace bound
    #    exceeds 64 MiB, so the no-alloc plan takes longer chunks
    big = mi.Workload("noalloc_big", 6, 4, 128, 64, "fp8", "fixed", (9000, 700, 16000, 3000, 12000, 64),
                      seed=83)
    desc = mla.make_desc(6, 128, 64, 1, 250, 1, True)
    assert mla.workspace_size(4, desc) > 64 * 1024 * 1024
    inp = mi.make_inputs(big)
    o1, l1, o2, l2 = _both(mla, inp)
    _check(o1, l1, o2, l2, "fp8", "big")
    ro, rl, va = orc.mla_decode(inp.q_bits, inp.kv, inp.block_table, inp.seq_lens, 4, big.softmax_scale,
                                inp.kv_scale, "fp8", True, with_abs=True)
    assert orc.rel_fro(o2, ro) <= 1e-2 and np.abs(l2[np.isfinite(rl)] - rl[np.isfinite(rl)]).max() <= 1e-3
    # 2) a smaller input right after: the regular layout fits, the plan is the
    #    same as mla_decode's and so are the results, bit for bit
    small = mi.Workload("noalloc_small", 3, 1, 16, 64, "bf16", "fixed", (4096, 333, 1), seed=84)
    inp = mi.make_inputs(small)
    o1, l1, o2, l2 = _both(mla, inp)
    _check(o1, l1, o2, l2, "bf16", "small")
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)
    ro, rl = orc.mla_decode(inp.q_bits, inp.kv, inp.block_table, inp.seq_lens, 1, small.softmax_scale,
                            inp.kv_scale, "bf16", True)
    assert orc.rel_fro(o2, ro) <= 5e-3


def test_noalloc_rejects_what_does_not_fit(mla):
    # a forced split whose partials cannot fit 64 MiB: refused before any launch
    wl = mi.Workload("noalloc_forced", 2, 4, 128, 64, "bf16", "fixed", (16000, 16000), seed=85)
    inp = mi.make_inputs(wl)
    q, kv, bt, sl = _dev(inp)
    out = torch.zeros((2, 4, 128, 512), dtype=torch.bfloat16, device=q.device)
    with pytest.raises(mla.MlaError) as e:
        mla.mla_decode_noalloc(q, kv, bt, sl, wl.softmax_scale, out, None, split_keys=64)
    assert e.value.status == 3
