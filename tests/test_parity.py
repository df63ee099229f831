"""GPU parity: the HIP path (through the C ABI) against the float64 oracle.

Tolerances, all checked on every case:
  * the stated bar over the whole output: bf16 cache -- relative Frobenius
    error of out <= 5e-3 and max |lse - ref| <= 1e-3; fp8 cache -- relative
    Frobenius error of out <= 1e-2 (lse is held to 1e-3 as well: both sides
    use the same dequantised values);
  * every row (b, i, h) on its own: relative error <= twice the stated bar;
  * every element: |out - ref| <= 2^-8 |ref| + 2^-7 a + 2^-10 max_row(a),
    where a = sum_t w_t |v_t| / sum_t w_t is the softmax-weighted mean of |v|
    for that element (the oracle's ``attend_abs``). The terms: rounding the
    result to bf16 (at most 2^-8 relative); rounding the weights p_t to bf16
    before the PV product (at most 2^-8 of a) plus fp32 accumulation over up
    to 16K keys (under 2^-10 of a) and the fp32 score sums; fp16 split
    partials keep 11 bits relative to their row's largest value (under
    2^-11 of max_row(a) each, doubled for slack);
  * the page's own kernel-test metric, cos_diff < 1e-4.
Outputs are prefilled with NaN so an unwritten element fails.
"""
import math

import numpy as np
import pytest
import torch

import mla_inputs as mi
from oracle import mla_oracle as orc

pytestmark = pytest.mark.gpu

TOL = {"bf16": (5e-3, 1e-3), "fp8": (1e-2, 1e-3)}


def have_gpu():
    return torch.cuda.is_available()


@pytest.fixture(scope="module")
def mla():
    if not have_gpu():
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


def run_gpu(mla, inp, split_keys=0, dev_inputs=None):
    q, kv, bt, sl = dev_inputs or to_device(inp)
    wl = inp.wl
    out = torch.full((wl.batch, wl.s_q, wl.heads, 512), float("nan"), dtype=torch.bfloat16,
                     device=q.device)
    lse = torch.full((wl.batch, wl.s_q, wl.heads), float("nan"), dtype=torch.float32,
                     device=q.device)
    mla.mla_decode(q, kv, bt, sl, wl.softmax_scale, inp.kv_scale, causal=wl.causal, out=out,
                   lse=lse, split_keys=split_keys)
    torch.cuda.synchronize()
    return out.float().cpu().double().numpy(), lse.cpu().double().numpy()


class OracleResult(tuple):
    """(out, lse) from the oracle, with the weighted mean |v| of every output
    element attached as ``.vabs`` (used by the elementwise bound)."""

    def __new__(cls, out, lse, vabs):
        r = super().__new__(cls, (out, lse))
        r.vabs = vabs
        return r


def run_oracle(inp, block_table=None, **kw):
    wl = inp.wl
    args = dict(s_q=wl.s_q, softmax_scale=wl.softmax_scale, kv_scale=inp.kv_scale,
                kv_dtype=wl.kv_dtype, causal=wl.causal)
    args.update(kw)
    bt = inp.block_table if block_table is None else block_table
    o, l, a = orc.mla_decode(inp.q_bits, inp.kv, bt, inp.seq_lens, with_abs=True, **args)
    return OracleResult(o, l, a)


ROW_FACTOR = 2.0                                   # per-row bar = 2 x the stated bar
ELEM_RTOL, ELEM_VTOL, ELEM_ROWTOL = 2.0 ** -8, 2.0 ** -7, 2.0 ** -10


def elementwise_excess(o, ro, vabs):
    """max over elements of |o - ref| / bound (> 1 means the bound is broken)."""
    bound = ELEM_RTOL * np.abs(ro) + ELEM_VTOL * vabs + ELEM_ROWTOL * vabs.max(axis=-1, keepdims=True)
    err = np.abs(o - ro)
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.where(bound > 0, err / bound, np.where(err > 0, np.inf, 0.0))
    return float(q.max()) if q.size else 0.0


def assert_parity(o, l, ro, rl, dtype, tag="", vabs=None):
    # the elementwise bound needs the oracle's weighted |v| of every element:
    # a call without it is a mistake in the test, not a case to skip
    assert vabs is not None, f"{tag}: assert_parity needs vabs (run_oracle(...).vabs)"
    tol_o, tol_l = TOL[dtype]
    assert np.isfinite(o).all(), f"{tag}: non-finite or unwritten output"
    fin = np.isfinite(rl)
    assert (np.isneginf(l) == ~fin).all(), f"{tag}: -inf lse pattern differs"
    # rows that see no key: exact zeros
    assert (o[~fin] == 0).all()
    err = orc.rel_fro(o, ro)
    rows = orc.rel_fro_rows(o, ro)
    row_max = float(rows.max()) if rows.size else 0.0
    lerr = float(np.abs(l[fin] - rl[fin]).max()) if fin.any() else 0.0
    cd = orc.cos_diff(o, ro)
    ex = elementwise_excess(o, ro, vabs)
    print(f"[{tag}] rel_fro={err:.3e} max_row={row_max:.3e} elem/bound={ex:.3f} "
          f"max|dlse|={lerr:.3e} cos_diff={cd:.3e}", flush=True)
    assert err <= tol_o, f"{tag}: rel Frobenius {err} > {tol_o}"
    if rows.size:
        worst = np.unravel_index(int(np.argmax(rows)), rows.shape)
        assert row_max <= ROW_FACTOR * tol_o, f"{tag}: row {worst} rel error {row_max} > {ROW_FACTOR * tol_o}"
    assert ex <= 1.0, f"{tag}: elementwise error {ex:.3f} x its bound"
    assert lerr <= tol_l, f"{tag}: lse error {lerr} > {tol_l}"
    if fin.any():
        assert cd < 1e-4, f"{tag}: cos_diff {cd}"


# ---------------------------------------------------------------------------
# the workloads at their full sizes
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("name", list(mi.WORKLOADS))
def test_workload_full_size(mla, name):
    wl = mi.WORKLOADS[name]
    print(f"workload {name}", flush=True)
    inp = mi.make_inputs(wl)
    o, l = run_gpu(mla, inp)
    r = run_oracle(inp)
    ro, rl = r
    assert_parity(o, l, ro, rl, wl.kv_dtype, name, vabs=r.vabs)


# ---------------------------------------------------------------------------
# split-KV: forced chunking agrees with the oracle and with the unsplit run
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("name,split", [("tiny", 64), ("tiny_fp8", 128),
                                        ("b128_h16_L4096_bf16", 448),
                                        ("b64_h128_L1k2k_bs128_bf16", 192)])
def test_forced_split(mla, name, split):
    wl = mi.WORKLOADS[name]
    if wl.batch > 16:
        wl = mi.shrink(wl, 16)
    inp = mi.make_inputs(wl)
    dev = to_device(inp)
    o1, l1 = run_gpu(mla, inp, split_keys=0, dev_inputs=dev)
    o2, l2 = run_gpu(mla, inp, split_keys=split, dev_inputs=dev)
    r = run_oracle(inp)
    ro, rl = r
    assert_parity(o2, l2, ro, rl, wl.kv_dtype, f"{name} split={split}", vabs=r.vabs)
    # split and unsplit runs agree with each other to bf16 rounding
    assert orc.rel_fro(o2, o1) <= 5e-3
    assert np.abs(l2 - l1).max() <= 1e-4


# ---------------------------------------------------------------------------
# edge cases
# ---------------------------------------------------------------------------

EDGE = [
    # (tag, B, s_q, H, bs, dtype, lens)
    ("empty_and_one", 3, 1, 16, 64, "bf16", (0, 1, 2)),
    ("ragged_tails", 4, 1, 16, 64, "bf16", (63, 64, 65, 127)),
    ("sq_longer_than_seq", 2, 4, 16, 64, "bf16", (2, 5)),
    ("one_head", 3, 1, 1, 64, "bf16", (100, 7, 300)),
    ("heads_24", 2, 1, 24, 128, "fp8", (129, 500)),
    ("heads_32_sq2", 2, 2, 32, 64, "bf16", (70, 1000)),
    ("heads_64", 2, 1, 64, 128, "bf16", (333, 1200)),
    ("heads_128_sq16", 1, 16, 128, 64, "fp8", (700,)),
    ("non_causal_sq3", 2, 3, 16, 64, "bf16", (10, 90)),
    ("bs128_fp8_short", 3, 1, 16, 128, "fp8", (1, 128, 129)),
    # query blocks up to the decode threshold of 512 tokens: many row groups,
    # per-row causal limits, tokens that see no key when s_q > L
    ("sq64_h16", 2, 64, 16, 64, "bf16", (64, 700)),
    ("sq512_h1", 2, 512, 1, 64, "bf16", (512, 1300)),
    ("sq300_h3_fp8", 3, 300, 3, 128, "fp8", (100, 300, 900)),
    ("sq128_h128_fp8", 1, 128, 128, 64, "fp8", (1000,)),
    # 128-row items that are only partly filled: 96 rows (three waves of 32)
    # and 80 rows (two and a half)
    ("heads_96", 2, 1, 96, 64, "bf16", (500, 1000)),
    ("sq5_h16_fp8", 2, 5, 16, 128, "fp8", (40, 2000)),
]


@pytest.mark.parametrize("case", EDGE, ids=[e[0] for e in EDGE])
def test_edge_cases(mla, case):
    tag, B, s_q, H, bs, dtype, lens = case
    causal = not tag.startswith("non_causal")
    wl = mi.Workload(tag, B, s_q, H, bs, dtype, "fixed", lens, causal=causal, seed=77)
    inp = mi.make_inputs(wl)
    o, l = run_gpu(mla, inp)
    r = run_oracle(inp)
    ro, rl = r
    assert_parity(o, l, ro, rl, dtype, tag, vabs=r.vabs)


def random_cases(n, seed=2026):
    """Seeded random descriptions across all three decode kernels: head counts
    from 1 to 128 (one, two or several row groups), s_q up to 8, both block
    sizes and caches, causal or not, lengths from 0 (no key) up to ~2500 with
    ragged last pages and tiles, automatic or forced splits."""
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        H = int(rng.choice([1, 3, 8, 16, 20, 32, 64, 100, 128]))
        s_q = int(rng.choice([1, 1, 2, 3, 4, 8]))
        bs = int(rng.choice([64, 128]))
        dtype = str(rng.choice(["bf16", "fp8"]))
        B = int(rng.integers(1, 6))
        lens = tuple(int(rng.integers(0, 10)) if rng.random() < 0.15 else int(rng.integers(10, 2500))
                     for _ in range(B))
        split = int(rng.choice([0, 0, 64, 320]))
        causal = bool(rng.random() < 0.8)
        tag = f"r{i}_B{B}_sq{s_q}_H{H}_bs{bs}_{dtype}_split{split}" + ("" if causal else "_nc")
        cases.append((tag, B, s_q, H, bs, dtype, lens, split, causal))
    return cases


RANDOM = random_cases(16)


@pytest.mark.parametrize("case", RANDOM, ids=[c[0] for c in RANDOM])
def test_random_descriptions(mla, case):
    tag, B, s_q, H, bs, dtype, lens, split, causal = case
    wl = mi.Workload(tag, B, s_q, H, bs, dtype, "fixed", lens, causal=causal, seed=B * 1000 + H)
    inp = mi.make_inputs(wl)
    o, l = run_gpu(mla, inp, split_keys=split)
    r = run_oracle(inp)
    ro, rl = r
    assert_parity(o, l, ro, rl, dtype, tag, vabs=r.vabs)


# Score jumps: a key aligned with one query row lifts that row's running max by
# far more than any ordinary tile does, after some tiles have been accumulated
# (and again later), so the kernels must rescale what they already summed.
JUMPS = [
    # (tag, B, s_q, H, bs, dtype, lens, spikes as (position, strength))
    ("jump_h16_bf16", 2, 1, 16, 64, "bf16", (1500, 700), ((200, 3.0), (650, 6.0))),
    ("jump_h16_fp8", 2, 1, 16, 64, "fp8", (1500, 700), ((200, 3.0), (650, 6.0))),
    ("jump_h128_bf16", 2, 1, 128, 128, "bf16", (1500, 700), ((200, 3.0), (650, 6.0))),
    ("jump_h128_sq4_fp8", 2, 4, 128, 64, "fp8", (3000, 700), ((100, 3.0), (600, 6.0))),
    ("jump_first_key_huge", 2, 1, 16, 64, "bf16", (900, 300), ((0, 6.0), (250, 3.0))),
]


def plant_spikes(inp, spikes):
    """Overwrite cache rows with strength * sign(q) of head 0 of the last query
    token: that row's score jumps by strength * softmax_scale * sum|q|."""
    wl = inp.wl
    q = inp.q_bits.astype(np.uint32) << 16
    q = q.view(np.float32)
    for b in range(wl.batch):
        sign = np.where(q[b, wl.s_q - 1, 0] < 0, -1.0, 1.0).astype(np.float32)
        for t, strength in spikes:
            if t >= inp.seq_lens[b] - wl.s_q + 1:
                continue
            page, slot = inp.block_table[b, t // wl.block_size], t % wl.block_size
            if wl.kv_dtype == "bf16":
                inp.kv[page, slot] = mi.f32_to_bf16_bits(strength * sign)
            else:
                inp.kv[page, slot] = mi.f32_to_e4m3fn_codes(strength * sign / np.float32(inp.kv_scale))
    return inp


@pytest.mark.parametrize("case", JUMPS, ids=[e[0] for e in JUMPS])
@pytest.mark.parametrize("split", [0, 192])
def test_score_jumps_rescale(mla, case, split):
    tag, B, s_q, H, bs, dtype, lens, spikes = case
    wl = mi.Workload(tag, B, s_q, H, bs, dtype, "fixed", lens, seed=91)
    inp = plant_spikes(mi.make_inputs(wl), spikes)
    o, l = run_gpu(mla, inp, split_keys=split)
    r = run_oracle(inp)
    ro, rl = r
    # the planted rows dominate: head 0 of the last token is (nearly) the spike row
    assert np.abs(rl[:, s_q - 1, 0]).max() > 100.0
    assert_parity(o, l, ro, rl, dtype, f"{tag} split={split}", vabs=r.vabs)


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("shift", [40, -40])
def test_split_partials_at_extreme_magnitudes(mla, dtype, shift):
    """128-row items keep split partials as fp16 with a per-row power-of-two
    scale. Values scaled by 2^40 (past fp16's range) or 2^-40 (below its
    normal range) must come through at the usual tolerance: kv_scale times
    2^shift and softmax_scale times 2^-shift leave every score unchanged and
    scale the exact output by 2^shift."""
    wl = mi.Workload(f"mag{shift}_{dtype}", 2, 1, 128, 64, dtype, "fixed", (700, 1500), seed=23)
    inp = mi.make_inputs(wl)
    q, kv, bt, sl = to_device(inp)
    kv_scale = float(inp.kv_scale) * 2.0 ** shift
    sm = wl.softmax_scale * 2.0 ** -shift
    out = torch.full((wl.batch, 1, 128, 512), float("nan"), dtype=torch.bfloat16, device=q.device)
    lse = torch.full((wl.batch, 1, 128), float("nan"), dtype=torch.float32, device=q.device)
    mla.mla_decode(q, kv, bt, sl, sm, kv_scale, out=out, lse=lse, split_keys=128)
    torch.cuda.synchronize()
    o, l = out.float().cpu().double().numpy(), lse.cpu().double().numpy()
    ro, rl, va = orc.mla_decode(inp.q_bits, inp.kv, inp.block_table, inp.seq_lens, 1, sm, kv_scale,
                                dtype, True, with_abs=True)
    assert np.abs(ro).max() > 2.0 ** (shift - 8) and np.abs(ro).max() < 2.0 ** (shift + 8)
    # compare at unit scale (exact: a power of two); every bound is relative
    unit = 2.0 ** -shift
    assert_parity(o * unit, l, ro * unit, rl, dtype, f"magnitude 2^{shift} {dtype}", vabs=va * unit)


def test_page_permutation_is_bit_identical_on_gpu(mla):
    wl = mi.shrink(mi.WORKLOADS["b64_h128_L1k2k_bs128_bf16"], 6)
    inp = mi.make_inputs(wl)
    o1, l1 = run_gpu(mla, inp)
    o2, l2 = run_gpu(mla, mi.permute_pages(inp, seed=5))
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)


def test_repeat_calls_are_deterministic(mla):
    wl = mi.shrink(mi.WORKLOADS["b32_sq4_h128_L512_16k_fp8"], 4)
    inp = mi.make_inputs(wl)
    dev = to_device(inp)
    a = run_gpu(mla, inp, dev_inputs=dev)
    b = run_gpu(mla, inp, dev_inputs=dev)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])


def test_lse_may_be_omitted(mla):
    inp = mi.make_inputs(mi.WORKLOADS["tiny"])
    q, kv, bt, sl = to_device(inp)
    wl = inp.wl
    out, lse = mla.mla_decode(q, kv, bt, sl, wl.softmax_scale, want_lse=False)
    assert lse is None
    ro, _ = run_oracle(inp)
    assert orc.rel_fro(out.float().cpu().double().numpy(), ro) <= 5e-3


# ---------------------------------------------------------------------------
# the split planner on the device equals its host mirror (integer work: exact)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("lens,s_q,H,bs,maxb,split", [
    ([37, 200], 1, 16, 64, 4, 0),
    ([4096] * 128, 1, 16, 64, 64, 0),
    ([512, 16384, 777, 5000, 9000, 600] * 5 + [1, 0], 4, 128, 64, 256, 0),
    (list(range(0, 3000, 7)), 1, 16, 128, 24, 0),
    ([4096, 100, 3000, 64], 1, 16, 64, 64, 192),
])
def test_device_plan_matches_host_mirror(mla, lens, s_q, H, bs, maxb, split):
    sl = torch.tensor(lens, dtype=torch.int32, device="cuda:0")
    header, items = mla.mla_decode_plan(sl, s_q, H, bs, maxb, split_keys=split)
    host, rows, chunk = mla.mla_plan_host(lens, s_q, H, bs, maxb, split_keys=split)
    assert int(header[0]) == len(host) and int(header[1]) == chunk and int(header[3]) == 0
    np.testing.assert_array_equal(items.cpu().numpy(), host)


def test_device_plan_matches_host_mirror_random_batches(mla):
    # the device planner divides with a reciprocal estimate, the host with a
    # float division; both correct to the exact quotient, so the plans agree
    # on every batch, including very long sequences and the 1M-key range
    rng = np.random.default_rng(7)
    for case in range(24):
        B = int(rng.integers(1, 400))
        H = int(rng.choice([1, 16, 64, 128]))
        s_q = int(rng.integers(1, 4))
        bs = int(rng.choice([64, 128]))
        maxb = int(rng.choice([4, 64, 1024, 8192]))
        lens = rng.integers(0, maxb * bs + 1, size=B)
        if case % 3 == 0:
            lens[: B // 2] = rng.integers(0, 65, size=B // 2)   # a mix of tiny and long
        sl = torch.tensor(lens, dtype=torch.int32, device="cuda:0")
        header, items = mla.mla_decode_plan(sl, s_q, H, bs, maxb)
        host, _, chunk = mla.mla_plan_host(lens, s_q, H, bs, maxb)
        assert int(header[0]) == len(host) and int(header[1]) == chunk, (case, B, H, s_q, bs, maxb)
        np.testing.assert_array_equal(items.cpu().numpy(), host)


# ---------------------------------------------------------------------------
# block-table entries outside [0, num_blocks) inside a sequence's range: the
# library leaves those tokens out of the softmax and sets flag bit 2
# ---------------------------------------------------------------------------

BAD_PAGES = [
    # (tag, B, s_q, H, bs, dtype, lens, split, [(b, block index, bad id)])
    ("narrow_bf16", 3, 1, 16, 64, "bf16", (700, 300, 1500), 0, [(0, 2, -1), (2, 0, 10 ** 6)]),
    ("narrow_fp8_split", 2, 1, 16, 64, "fp8", (2000, 900), 256, [(0, 5, -1), (1, 13, -5)]),
    ("wide_h32_sq2", 2, 2, 32, 64, "bf16", (900, 300), 0, [(0, 1, -1)]),
    ("wide128_bf16", 2, 1, 128, 128, "bf16", (1500, 700), 0, [(0, 3, -1), (1, 0, 10 ** 7)]),
    ("wide128_fp8_sq4_split", 2, 4, 128, 64, "fp8", (3000, 800), 192, [(0, 7, -2), (1, 12, -1)]),
    ("whole_sequence", 2, 1, 16, 64, "bf16", (100, 200), 0, [(0, 0, -1), (0, 1, -1)]),
]


def run_gpu_ws(mla, inp, block_table, split_keys=0):
    """run_gpu with an explicit workspace, returning the header's flag word too."""
    q, kv, _, sl = to_device(inp)
    bt = torch.from_numpy(block_table).to(q.device)
    wl = inp.wl
    out = torch.full((wl.batch, wl.s_q, wl.heads, 512), float("nan"), dtype=torch.bfloat16, device=q.device)
    lse = torch.full((wl.batch, wl.s_q, wl.heads), float("nan"), dtype=torch.float32, device=q.device)
    desc = mla.make_desc(wl.batch, wl.heads, wl.block_size, kv.shape[0], bt.shape[1],
                         0 if wl.kv_dtype == "bf16" else 1, wl.causal, split_keys)
    ws = torch.empty(mla.workspace_size(wl.s_q, desc), dtype=torch.uint8, device=q.device)
    mla.mla_decode(q, kv, bt, sl, wl.softmax_scale, inp.kv_scale, causal=wl.causal, out=out, lse=lse,
                   workspace=ws, split_keys=split_keys)
    torch.cuda.synchronize()
    flags = int(ws[:16].view(torch.int32)[3].item())
    return out.float().cpu().double().numpy(), lse.cpu().double().numpy(), flags


@pytest.mark.parametrize("case", BAD_PAGES, ids=[c[0] for c in BAD_PAGES])
def test_out_of_range_block_table_entries_are_dropped_and_flagged(mla, case):
    tag, B, s_q, H, bs, dtype, lens, split, bad = case
    wl = mi.Workload(tag, B, s_q, H, bs, dtype, "fixed", lens, seed=61)
    inp = mi.make_inputs(wl)
    # the valid table sets no flag
    _, _, flags = run_gpu_ws(mla, inp, inp.block_table, split)
    assert flags & 4 == 0
    bt = inp.block_table.copy()
    for b, j, v in bad:
        assert j * bs < inp.seq_lens[b]
        bt[b, j] = v
    o, l, flags = run_gpu_ws(mla, inp, bt, split)
    assert flags & 4, f"{tag}: flag bit 2 not set ({flags})"
    r = run_oracle(inp, block_table=bt)
    assert_parity(o, l, r[0], r[1], dtype, f"bad pages {tag}", vabs=r.vabs)


# ---------------------------------------------------------------------------
# one plan, several decode calls (plan once per step, reuse for every layer)
# ---------------------------------------------------------------------------

PLAN_REUSE = [
    ("narrow_bf16", 4, 1, 16, 64, "bf16", (4096, 1000, 77, 2500)),
    ("narrow_fp8", 3, 1, 16, 128, "fp8", (3000, 129, 1800)),
    ("wide_h64", 2, 1, 64, 64, "bf16", (1200, 333)),
    ("wide128_bf16", 3, 1, 128, 128, "bf16", (1024, 2048, 1500)),
    ("wide128_fp8_sq4", 2, 4, 128, 64, "fp8", (5000, 700)),
]


@pytest.mark.parametrize("case", PLAN_REUSE, ids=[c[0] for c in PLAN_REUSE])
def test_plan_reuse_across_layers(mla, case):
    """Plan with one call, then decode two more 'layers' (new q, cache
    contents and page placement; same lengths) with mla_decode_with_plan."""
    tag, B, s_q, H, bs, dtype, lens = case
    dev = torch.device("cuda:0")
    layers = [mi.make_inputs(mi.Workload(tag, B, s_q, H, bs, dtype, "fixed", lens, seed=71), seed=s)
              for s in (71, 72, 73)]
    for inp in layers[1:]:   # same lengths and cache size, so the same description
        assert inp.kv.shape == layers[0].kv.shape and inp.block_table.shape == layers[0].block_table.shape
    wl = layers[0].wl
    q0, kv0, bt, sl = to_device(layers[0])
    desc = mla.make_desc(B, H, bs, kv0.shape[0], bt.shape[1], 0 if dtype == "bf16" else 1, True)
    ws = torch.empty(mla.workspace_size(s_q, desc), dtype=torch.uint8, device=dev)
    mla.mla_decode(q0, kv0, bt, sl, wl.softmax_scale, layers[0].kv_scale, workspace=ws)
    plan = ws[:256].clone()
    for li, inp in enumerate(layers[1:], start=1):
        q, kv, bt, _ = to_device(inp)
        out = torch.full((B, s_q, H, 512), float("nan"), dtype=torch.bfloat16, device=dev)
        lse = torch.full((B, s_q, H), float("nan"), dtype=torch.float32, device=dev)
        mla.mla_decode_with_plan(q, kv, bt, sl, wl.softmax_scale, ws, kv_scale=inp.kv_scale,
                                 out=out, lse=lse)
        torch.cuda.synchronize()
        assert torch.equal(ws[:16], plan[:16]), "the plan header changed"
        r = run_oracle(inp)
        assert_parity(out.float().cpu().double().numpy(), lse.cpu().double().numpy(), r[0], r[1],
                      dtype, f"plan reuse {tag} layer {li}", vabs=r.vabs)


# ---------------------------------------------------------------------------
# a plan that does not fit the call: items skipped and flagged, never run
# ---------------------------------------------------------------------------

STALE = [
    ("narrow_bf16", 1, 16, 64, "bf16", (900, 2500, 60, 3000, 1200, 700, 2000, 64)),
    ("wide_fp8", 1, 64, 64, "fp8", (1300, 200, 2600, 64, 900, 1800, 3000, 500)),
    ("wide128_fp8_sq2", 2, 64, 64, "fp8", (1000, 2200, 130, 1700, 600, 2900, 64, 1500)),
    ("wide128_bf16", 1, 128, 128, "bf16", (700, 1900, 2400, 256, 1300, 128, 2048, 999)),
]


@pytest.mark.parametrize("case", STALE, ids=[c[0] for c in STALE])
def test_stale_plan_items_are_skipped_and_flagged(mla, case):
    """A plan made for 8 sequences, then reused by mla_decode_with_plan for a
    call on the first 4 (views of the same buffers, the same workspace). The
    plan's items for sequences 4..7 are out of range for that call: the
    kernels skip them, set flag bit 3 and leave rows 4..7 of out and lse as
    they were. Every address such an item could form lies inside the 8-row
    buffers and the workspace, so this holds with or without the check."""
    tag, s_q, H, bs, dtype, lens = case
    inp = mi.make_inputs(mi.Workload(tag, 8, s_q, H, bs, dtype, "fixed", lens, seed=81))
    q, kv, bt, sl = to_device(inp)
    dev = q.device
    wl = inp.wl
    desc8 = mla.make_desc(8, H, bs, kv.shape[0], bt.shape[1], 0 if dtype == "bf16" else 1, True)
    ws = torch.empty(mla.workspace_size(s_q, desc8), dtype=torch.uint8, device=dev)
    out = torch.empty((8, s_q, H, 512), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((8, s_q, H), dtype=torch.float32, device=dev)
    mla.mla_decode(q, kv, bt, sl, wl.softmax_scale, inp.kv_scale, out=out, lse=lse, workspace=ws)
    torch.cuda.synchronize()
    hdr = ws[:16].view(torch.int32).cpu()
    items = ws[256:256 + 32 * int(hdr[0])].view(torch.int32).view(-1, 8).cpu()
    assert (items[:, 0] >= 4).any(), "the 8-sequence plan has items for sequences 4..7"
    assert int(hdr[3]) & 8 == 0
    out.fill_(float("nan"))
    lse.fill_(float("nan"))
    mla.mla_decode_with_plan(q[:4], kv, bt[:4], sl[:4], wl.softmax_scale, ws, kv_scale=inp.kv_scale,
                             out=out[:4], lse=lse[:4])
    torch.cuda.synchronize()
    flags = int(ws[:16].view(torch.int32)[3].item())
    assert flags & 8, f"{tag}: flag bit 3 not set ({flags})"
    assert torch.isnan(out[4:].float()).all(), "a skipped item wrote rows 4..7 of out"
    assert torch.isnan(lse[4:]).all(), "a skipped item wrote rows 4..7 of lse"
    # a fresh plan on the same views is exact again
    mla.mla_decode(q[:4], kv, bt[:4], sl[:4], wl.softmax_scale, inp.kv_scale, out=out[:4], lse=lse[:4])
    torch.cuda.synchronize()
    r = run_oracle(inp)
    assert_parity(out[:4].float().cpu().double().numpy(), lse[:4].cpu().double().numpy(), r[0][:4], r[1][:4],
                  dtype, f"after stale plan {tag}", vabs=r.vabs[:4])


# ---------------------------------------------------------------------------
# a latent cache larger than 4 GiB
# ---------------------------------------------------------------------------

# The sequences' pages are moved above the 4 GiB offset of a cache of about
# 4.3 GB, so every row address needs 64-bit arithmetic. One case per decode
# kernel (16, 32 and 128 query rows per sequence), split items included (a
# few short sequences over 256 items). The oracle reads the same pages from
# the compact cache through the original block table.
@pytest.mark.parametrize("heads,s_q,bs,kv_dtype", [(16, 1, 64, "bf16"), (32, 1, 64, "fp8"),
                                                   (128, 1, 128, "bf16"), (16, 4, 128, "fp8")])
def test_cache_beyond_4gib(mla, heads, s_q, bs, kv_dtype):
    import dataclasses
    wl = dataclasses.replace(mi.WORKLOADS["tiny"], name=f"big_cache_h{heads}_sq{s_q}_{kv_dtype}", batch=3,
                             s_q=s_q, heads=heads, block_size=bs, kv_dtype=kv_dtype,
                             lens="fixed", lens_arg=(1000, 77, 640), seed=heads + s_q)
    inp = mi.make_inputs(wl)
    print(f"[{wl.name}] cache rows past 4 GiB", flush=True)
    q, kv, bt, sl = to_device(inp)
    page_bytes = bs * 576 * (2 if kv_dtype == "bf16" else 1)
    base = (2 ** 32) // page_bytes + 1                 # first page id past 4 GiB
    n_small = kv.shape[0]
    big = torch.empty((base + n_small,) + tuple(kv.shape[1:]), dtype=kv.dtype, device=kv.device)
    assert big.numel() * big.element_size() > 2 ** 32
    big[base:] = kv
    bt_big = torch.where(bt >= 0, bt + base, bt)
    o, l = run_gpu(mla, inp, dev_inputs=(q, big, bt_big, sl))
    ro = run_oracle(inp)
    assert_parity(o, l, ro[0], ro[1], kv_dtype, tag=wl.name, vabs=ro.vabs)
