"""GPU: library calls captured in a HIP graph (torch.cuda.CUDAGraph) and
replayed.

The entry points only launch kernels on the caller's stream: no allocation,
no memset, no synchronisation, and the planner runs on the device from the
seq_lens the buffer holds at run time. A captured call must therefore give
the eager call's bytes on every replay, for whatever the captured buffers
hold when it replays (new q and cache contents, shorter sequences). Each
replay here follows eager work of the test's own (buffer refills, a reduction
over a large tensor, a synchronisation), and every replay is checked.
"""
import numpy as np
import pytest
import torch

import mla_inputs as mi

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mla():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mla_paged_decode_04_amd as m
    m.library()   # raises if the HIP library is missing: no fallback
    return m


def to_device(inp):
    dev = torch.device("cuda:0")
    q = torch.from_numpy(inp.q_bits.view(np.int16)).to(dev).view(torch.bfloat16)
    if inp.wl.kv_dtype == "bf16":
        kv = torch.from_numpy(inp.kv.view(np.int16)).to(dev).view(torch.bfloat16)
    else:
        kv = torch.from_numpy(inp.kv).to(dev).view(torch.float8_e4m3fn)
    bt = torch.from_numpy(inp.block_table).to(dev)
    sl = torch.from_numpy(inp.seq_lens).to(dev)
    return q, kv, bt, sl


def eager_work(dev):
    """Unrelated device work between replays (a multi-block reduction)."""
    x = torch.ones(1 << 24, dtype=torch.float32, device=dev)
    assert float(x.sum()) == float(1 << 24)


# (tag, batch, s_q, heads, block size, cache, lengths): the narrow (16-row),
# 64-row and both 128-row kernels, each with splits and a combine
DECODE_CASES = [
    ("narrow_bf16", 6, 1, 16, 64, "bf16", (3000, 64, 1200, 37, 2500, 700)),
    ("wide_fp8", 4, 4, 16, 64, "fp8", (2100, 300, 1500, 64)),
    ("wide128_bf16", 3, 1, 128, 128, "bf16", (1900, 640, 1300)),
    ("wide128_fp8_sq2", 3, 2, 64, 64, "fp8", (2600, 129, 1800)),
]


@pytest.mark.parametrize("entry", ["mla_decode", "mla_decode_noalloc"])
@pytest.mark.parametrize("case", DECODE_CASES, ids=[c[0] for c in DECODE_CASES])
def test_decode_graph_replays_match_eager(mla, case, entry):
    tag, B, s_q, H, bs, dtype, lens = case
    dev = torch.device("cuda:0")
    wl = mi.Workload(tag, B, s_q, H, bs, dtype, "fixed", lens, seed=91)
    a, b = mi.make_inputs(wl, seed=91), mi.make_inputs(wl, seed=92)
    assert a.kv.shape == b.kv.shape and a.block_table.shape == b.block_table.shape
    assert a.kv_scale == b.kv_scale or dtype == "fp8"
    da, db = to_device(a), to_device(b)
    # shorter sequences on a's cache: the captured planner must re-plan
    short = torch.from_numpy(np.maximum(a.seq_lens // 3, s_q).astype(np.int32)).to(dev)

    def call(q, kv, bt, sl, kv_scale, out, lse, ws):
        if entry == "mla_decode":
            mla.mla_decode(q, kv, bt, sl, wl.softmax_scale, kv_scale, out=out, lse=lse, workspace=ws)
        else:
            mla.mla_decode_noalloc(q, kv, bt, sl, wl.softmax_scale, out, lse, kv_scale=kv_scale)

    def new_out():
        return (torch.full((B, s_q, H, 512), float("nan"), dtype=torch.bfloat16, device=dev),
                torch.full((B, s_q, H), float("nan"), dtype=torch.float32, device=dev))

    desc = mla.make_desc(B, H, bs, a.kv.shape[0], a.block_table.shape[1], 0 if dtype == "bf16" else 1,
                         True)
    wsize = mla.workspace_size(s_q, desc)
    # eager references, each on buffers of its own
    refs = {}
    for name, (q, kv, bt, sl), scale in (("a", da, a.kv_scale), ("b", db, b.kv_scale),
                                         ("a_short", (da[0], da[1], da[2], short), a.kv_scale)):
        out, lse = new_out()
        ws = torch.empty(wsize, dtype=torch.uint8, device=dev)
        call(q, kv, bt, sl, scale, out, lse, ws)
        torch.cuda.synchronize()
        refs[name] = (out.clone(), lse.clone())
    assert not torch.equal(refs["a"][0], refs["b"][0])
    assert not torch.equal(refs["a"][0], refs["a_short"][0])

    # captured buffers (a's contents first); kv_scale is a launch argument,
    # so the graph keeps a's (b's cache is quantised with its own scale and
    # is only replayed when the two agree)
    gq, gkv, gbt, gsl = (t.clone() for t in da)
    gout, glse = new_out()
    gws = torch.empty(wsize, dtype=torch.uint8, device=dev)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(2):
            call(gq, gkv, gbt, gsl, a.kv_scale, gout, glse, gws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(gq, gkv, gbt, gsl, a.kv_scale, gout, glse, gws)
    torch.cuda.synchronize()

    plan = ["a", "a_short", "a", "a_short"]
    if a.kv_scale == b.kv_scale:
        plan[2:2] = ["b"]
    for r, src in enumerate(plan):
        q, kv, bt, sl = {"a": da, "b": db, "a_short": (da[0], da[1], da[2], short)}[src]
        for dst, s in zip((gq, gkv, gbt, gsl), (q, kv, bt, sl)):
            dst.copy_(s)
        gout.fill_(float("nan"))
        glse.fill_(float("nan"))
        eager_work(dev)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ro, rl = refs[src]
        assert torch.equal(gout, ro), f"{tag} {entry}: replay {r} ({src}) out differs from the eager call"
        assert torch.equal(glse, rl), f"{tag} {entry}: replay {r} ({src}) lse differs from the eager call"


# one decode layer: absorb_q -> kv_append of the new token -> decode -> absorb_out
LAYER_CASES = [("bf16", 16), ("fp8", 16), ("fp8", 128)]


@pytest.mark.parametrize("dtype,H", LAYER_CASES, ids=[f"{d}_h{h}" for d, h in LAYER_CASES])
def test_layer_chain_graph_replays_match_eager(mla, dtype, H):
    dev = torch.device("cuda:0")
    B, s_q, bs, d = 5, 1, 64, 128
    lens = (900, 64, 2200, 130, 1500)
    wl = mi.Workload(f"layer_{dtype}_{H}", B, s_q, H, bs, dtype, "fixed", lens, seed=93)
    inp = mi.make_inputs(wl, seed=93)
    _, kv0, bt, sl = to_device(inp)
    T = B * s_q
    gen = torch.Generator(device="cpu").manual_seed(94)

    def randn(*shape, scale=1.0):
        return (torch.randn(*shape, generator=gen) * scale).to(torch.bfloat16).to(dev)

    q_nope = [randn(T, H, d), randn(T, H, d)]
    q_pe = randn(T, H, 64)
    w_uk = randn(H, d, 512, scale=d ** -0.5)
    w_uv = randn(H, 512, d, scale=512 ** -0.5)
    rows = randn(T, 576)
    # the new token of sequence b sits at position len - 1
    last = inp.seq_lens.astype(np.int64) - 1
    slots = torch.from_numpy((inp.block_table[np.arange(B), last // bs].astype(np.int64) * bs
                              + last % bs).astype(np.int32)).to(dev)
    desc = mla.make_desc(B, H, bs, inp.kv.shape[0], inp.block_table.shape[1],
                         0 if dtype == "bf16" else 1, True)
    wsize = mla.workspace_size(s_q, desc)

    def layer(qn, kv, q, out, lse, ws, y):
        mla.mla_absorb_q(qn, q_pe, w_uk, out=q)
        mla.mla_kv_append(rows, slots, kv, kv_scale=inp.kv_scale)
        mla.mla_decode(q.view(B, s_q, H, 576), kv, bt, sl, wl.softmax_scale, inp.kv_scale,
                       out=out, lse=lse, workspace=ws)
        mla.mla_absorb_out(out.view(T, H, 512), w_uv, out=y)

    def buffers():
        return (kv0.clone(), torch.empty(T, H, 576, dtype=torch.bfloat16, device=dev),
                torch.empty(B, s_q, H, 512, dtype=torch.bfloat16, device=dev),
                torch.empty(B, s_q, H, dtype=torch.float32, device=dev),
                torch.empty(wsize, dtype=torch.uint8, device=dev),
                torch.empty(T, H, d, dtype=torch.bfloat16, device=dev))

    refs = []
    for qn in q_nope:
        kv, q, out, lse, ws, y = buffers()
        layer(qn, kv, q, out, lse, ws, y)
        torch.cuda.synchronize()
        refs.append((kv, y, lse))
    assert not torch.equal(refs[0][1], refs[1][1])
    assert not torch.equal(refs[0][0], kv0), "the append wrote nothing"

    gqn = q_nope[0].clone()
    gkv, gq, gout, glse, gws, gy = buffers()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        layer(gqn, gkv, gq, gout, glse, gws, gy)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        layer(gqn, gkv, gq, gout, glse, gws, gy)
    torch.cuda.synchronize()

    for r, which in enumerate((0, 1, 0, 1)):
        gqn.copy_(q_nope[which])
        gkv.copy_(kv0)
        gy.fill_(float("nan"))
        glse.fill_(float("nan"))
        eager_work(dev)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        kv_ref, y_ref, lse_ref = refs[which]
        assert torch.equal(gkv.view(torch.uint8), kv_ref.view(torch.uint8)), f"replay {r}: cache differs"
        assert torch.equal(glse, lse_ref), f"replay {r}: lse differs from the eager layer"
        assert torch.equal(gy, y_ref), f"replay {r}: projected output differs from the eager layer"
