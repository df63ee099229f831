"""C-ABI library: loads, exports what the header declares, and rejects bad
arguments before touching the device (CPU only)."""
import ctypes
import os
import re

import numpy as np
import pytest

import mla_paged_decode_04_amd as mla

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mla_decode.h")

OK, INVALID, UNSUPPORTED, WS_SMALL = 0, 1, 2, 3
FAKE = 0x10000   # an aligned non-null address; only used where the call must fail first


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*[\w\s\*]+?\b(mla_\w+)\s*\(", text, flags=re.M)))


def desc(**kw):
    d = dict(batch=2, num_heads=16, block_size=64, num_blocks=8, max_blocks_per_seq=4,
             kv_dtype=0, causal=1, split_keys=0)
    d.update(kw)
    return mla.Desc(**d)


def call(d, s_q=1, ws_bytes=None, softmax_scale=0.07, kv_scale=1.0, ptrs=None, lse=FAKE):
    lib = mla.library()
    p = dict(q=FAKE, kv=FAKE, bt=FAKE, sl=FAKE, out=FAKE, ws=FAKE)
    p.update(ptrs or {})
    if ws_bytes is None:
        ws_bytes = 0        # too small for any valid description
    return lib.mla_decode(p["q"], p["kv"], p["bt"], p["sl"], s_q, softmax_scale, kv_scale,
                          p["out"], lse, ctypes.byref(d), p["ws"], ws_bytes, None)


def test_library_exports_every_declared_function():
    lib = mla.library()
    names = declared_functions()
    assert {"mla_decode", "mla_decode_workspace_size", "mla_status_string"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n
    assert lib.mla_abi_version() == 1


def test_status_strings():
    lib = mla.library()
    assert lib.mla_status_string(0) == b"MLA_OK"
    assert lib.mla_status_string(3) == b"MLA_ERR_WORKSPACE_TOO_SMALL"
    assert lib.mla_status_string(99) == b"MLA_ERR_UNKNOWN"


def test_workspace_size_is_host_only_and_monotone():
    small = mla.workspace_size(1, desc(batch=2))
    big = mla.workspace_size(1, desc(batch=200))
    assert 0 < small < big and small % 256 == 0
    assert mla.workspace_size(1, desc(num_heads=129)) == 0
    assert mla.workspace_size(513, desc()) == 0
    assert mla.workspace_size(1, desc(block_size=32)) == 0
    assert mla.workspace_size(1, desc(split_keys=100)) == 0


@pytest.mark.parametrize("kw,s_q,code", [
    (dict(num_heads=0), 1, INVALID),
    (dict(num_heads=129), 1, UNSUPPORTED),
    (dict(block_size=16), 1, UNSUPPORTED),
    (dict(block_size=256), 1, UNSUPPORTED),
    (dict(kv_dtype=7), 1, UNSUPPORTED),
    (dict(causal=2), 1, INVALID),
    (dict(batch=-1), 1, INVALID),
    (dict(num_blocks=0), 1, INVALID),
    (dict(max_blocks_per_seq=0), 1, INVALID),
    (dict(split_keys=65), 1, INVALID),
    (dict(), 0, INVALID),
    (dict(), 513, UNSUPPORTED),
])
def test_bad_descriptions_are_rejected(kw, s_q, code):
    assert call(desc(**kw), s_q=s_q) == code


@pytest.mark.parametrize("name", ["q", "kv", "bt", "sl", "out", "ws"])
def test_null_pointers_are_rejected(name):
    assert call(desc(), ptrs={name: 0}, ws_bytes=1 << 40) == INVALID


@pytest.mark.parametrize("name,addr", [("q", FAKE + 8), ("kv", FAKE + 4), ("out", FAKE + 2),
                                       ("bt", FAKE + 2), ("ws", FAKE + 128)])
def test_misaligned_pointers_are_rejected(name, addr):
    assert call(desc(), ptrs={name: addr}, ws_bytes=1 << 40) == INVALID


@pytest.mark.parametrize("sc,kvs", [(0.0, 1.0), (-1.0, 1.0), (float("nan"), 1.0),
                                    (float("inf"), 1.0), (0.1, 0.0), (0.1, float("nan"))])
def test_bad_scales_are_rejected(sc, kvs):
    assert call(desc(), softmax_scale=sc, kv_scale=kvs, ws_bytes=1 << 40) == INVALID


def test_short_workspace_is_rejected_before_launch():
    d = desc()
    need = mla.workspace_size(1, d)
    assert call(d, ws_bytes=need - 1) == WS_SMALL


def test_empty_batch_is_a_no_op():
    assert call(desc(batch=0), ws_bytes=mla.workspace_size(1, desc(batch=0))) == OK


# ---------------------------------------------------------------------------
# host mirror of the split planner
# ---------------------------------------------------------------------------

def check_plan(lens, s_q, H, bs, maxb, split_keys=0):
    items, rgs, chunk = mla.mla_plan_host(lens, s_q, H, bs, maxb, split_keys=split_keys)
    R = s_q * H
    nrg = -(-R // rgs)
    max_keys = maxb * bs
    seen = {}
    slots = []
    for b, rg, t0, t1, slot, *_ in items.tolist():
        assert 0 <= b < len(lens) and 0 <= rg < nrg
        assert t0 % 64 == 0 and t0 <= t1
        seen.setdefault((b, rg), []).append((t0, t1, slot))
        if slot >= 0:
            slots.append(slot)
    assert len(slots) == len(set(slots))
    for b, L in enumerate(lens):
        L = min(max(int(L), 0), max_keys)
        for rg in range(nrg):
            parts = sorted(seen[(b, rg)])
            # chunks tile [0, L) exactly, in order, with no empty chunk unless L == 0
            assert parts[0][0] == 0 and parts[-1][1] == L
            for (a0, a1, _), (b0, _, _) in zip(parts[:-1], parts[1:]):
                assert a1 == b0
            if len(parts) == 1:
                assert parts[0][2] == -1
            else:
                assert all(p[2] >= 0 for p in parts) and all(p[0] < p[1] for p in parts)
                if split_keys:
                    assert all(p[1] - p[0] <= split_keys for p in parts)
    return items, rgs, chunk


@pytest.mark.parametrize("lens,s_q,H,bs,maxb", [
    ([37, 200], 1, 16, 64, 4),
    ([4096] * 128, 1, 16, 64, 64),
    (list(range(1000, 2048, 17))[:64], 1, 128, 128, 16),
    ([512, 16384, 777, 5000, 9000, 600] * 5 + [1, 0], 4, 128, 64, 256),
    ([0, 0, 0], 2, 8, 64, 1),
    ([65, 129, 1], 16, 8, 128, 2),
])
def test_host_plan_covers_every_key_once(lens, s_q, H, bs, maxb):
    check_plan(lens, s_q, H, bs, maxb)


@pytest.mark.parametrize("split_keys", [64, 128, 448, 1024])
def test_forced_split_chunks(split_keys):
    items, _, chunk = check_plan([4096, 100, 3000, 64], 1, 16, 64, 64, split_keys=split_keys)
    assert chunk == split_keys


def test_plan_stays_within_workspace_bound():
    rng = np.random.default_rng(0)
    for _ in range(20):
        B = int(rng.integers(1, 300))
        H = int(rng.choice([1, 8, 16, 32, 64, 128]))
        s_q = int(rng.integers(1, 5))
        bs = int(rng.choice([64, 128]))
        maxb = int(rng.integers(1, 40))
        lens = rng.integers(0, maxb * bs + 1, size=B)
        d = desc(batch=B, num_heads=H, block_size=bs, max_blocks_per_seq=maxb)
        items, rgs, _ = check_plan(lens, s_q, H, bs, maxb)
        # items and partial slots both fit the workspace the library asked for
        slots = int((items[:, 4] >= 0).sum())
        need = len(items) * 32 + slots * (rgs * 8 + rgs * 512 * 2)   # lse, exponent, fp16 row
        assert need < mla.workspace_size(s_q, d)
        # the automatic split never needs more than 2048 partial slots
        assert slots <= 2048


@pytest.mark.parametrize("s_q,H", [(64, 16), (512, 1), (512, 128), (300, 3)])
def test_long_query_blocks_plan_and_size(s_q, H):
    # s_q up to the decode threshold: row groups tile s_q * H rows
    lens = [s_q + 5, 2 * s_q + 100, 7, 4000]
    items, rgs, _ = check_plan(lens, s_q, H, 64, 64)
    R = s_q * H
    assert rgs == (16 if R <= 16 else 64 if R <= 64 else 128)
    assert mla.workspace_size(s_q, desc(batch=4, num_heads=H, max_blocks_per_seq=64)) > 0


def test_out_of_range_lengths_are_clamped():
    items, _, _ = mla.mla_plan_host([-5, 10_000], 1, 16, 64, 2)
    ends = {(b, t1) for b, rg, t0, t1, *_ in items.tolist()}
    assert (0, 0) in ends and (1, 128) in ends


# ---------------------------------------------------------------------------
# cache append: argument checks (nothing is launched on an error)
# ---------------------------------------------------------------------------

def append_call(n=4, scale=1.0, nb=8, bs=64, dtype=0, ptrs=True):
    lib = mla.library()
    p = 4096 if ptrs else None
    return lib.mla_kv_append(p, p, n, scale, p, nb, bs, dtype, None)


@pytest.mark.parametrize("kw,code", [
    (dict(n=-1), INVALID),
    (dict(nb=0), INVALID),
    (dict(bs=32), UNSUPPORTED),
    (dict(dtype=7), UNSUPPORTED),
    (dict(scale=0.0), INVALID),
    (dict(scale=float("nan")), INVALID),
    (dict(ptrs=False), INVALID),
])
def test_kv_append_rejects_bad_arguments(kw, code):
    assert append_call(**kw) == code


def test_append_scale_product_equals_float32_division():
    """The append kernel forms x / kv_scale as float(double(x) * (1 / double(kv_scale))).
    For every bf16 x and a spread of float32 scales (powers of two, the
    workloads' amax / 448 scales, extremes that overflow or give float32
    subnormals, random magnitudes and random bit patterns) that equals the
    correctly rounded float32 division bit for bit."""
    x = (np.arange(65536, dtype=np.uint32) << 16).view(np.float32)
    rng = np.random.default_rng(5)
    scales = [1.0, 0.5, 448.0, 1 / 448, 0.0213, 0.013029, 3.0, 0.1, 1e-30, 1e30, 2.0 ** -126, 3.4e38]
    scales += list(np.exp(rng.uniform(np.log(1e-6), np.log(1e6), 40)))
    scales += list(rng.integers(0x00800000, 0x7F7FFFFF, 40, dtype=np.uint32).view(np.float32))
    with np.errstate(all="ignore"):
        for s in np.asarray(scales, dtype=np.float32):
            ref = x / s
            got = (x.astype(np.float64) * (1.0 / np.float64(s))).astype(np.float32)
            same = (ref.view(np.uint32) == got.view(np.uint32)) | (np.isnan(ref) & np.isnan(got))
            assert same.all(), (float(s), x[~same][:4])


def test_kv_append_zero_tokens_is_a_no_op():
    assert append_call(n=0, ptrs=False) == 0


@pytest.mark.parametrize("fn,args,code", [
    ("mla_absorb_q", (4096, 4096, 4096, 4096, 4, 16, 100, None), UNSUPPORTED),   # d_nope % 32
    ("mla_absorb_q", (4096, 4096, 4096, 4096, 4, 0, 128, None), INVALID),
    ("mla_absorb_q", (4096, 4096, 4096, 4096, -1, 16, 128, None), INVALID),
    ("mla_absorb_q", (None, 4096, 4096, 4096, 4, 16, 128, None), INVALID),
    ("mla_absorb_out", (4096, 4096, 4096, 4, 16, 100, None), UNSUPPORTED),      # d_v % 64
    ("mla_absorb_out", (4096, 4096, 4096, 4, 129, 128, None), INVALID),
    ("mla_absorb_out", (4096, None, 4096, 4, 16, 128, None), INVALID),
])
def test_absorb_rejects_bad_arguments(fn, args, code):
    assert getattr(mla.library(), fn)(*args) == code


def test_absorb_zero_tokens_is_a_no_op():
    lib = mla.library()
    assert lib.mla_absorb_q(None, None, None, None, 0, 16, 128, None) == 0
    assert lib.mla_absorb_out(None, None, None, 0, 16, 128, None) == 0


def list_schedule_makespan(items, overhead, workers=256):
    """Makespan, in key units, of the items run in plan order on `workers`
    single-workgroup CUs, each item costing its keys plus `overhead`."""
    import heapq
    free = [0] * workers
    for it in items:
        t = heapq.heappop(free)
        heapq.heappush(free, t + int(it[3] - it[2]) + overhead)
    return max(free)


@pytest.mark.parametrize("name", ["b64_h128_L1k2k_bs128_bf16", "b32_sq4_h128_L512_16k_fp8"])
def test_automatic_chunk_is_near_the_best_list_schedule(name):
    """For the skewed 128-head batches the planner's chunk gives a simulated
    list-schedule makespan within 3 % of the best forced chunk (64-key steps,
    same per-item overhead as the planner's model: 320 keys for 128-row items)."""
    import mla_inputs as mi
    wl = mi.WORKLOADS[name]
    lens = mi.draw_seq_lens(wl, np.random.default_rng(wl.seed))
    maxb = int(max(1, (lens.max() + wl.block_size - 1) // wl.block_size))
    items, rgs, _ = mla.mla_plan_host(lens, wl.s_q, wl.heads, wl.block_size, maxb)
    assert rgs == 128
    auto = list_schedule_makespan(items, 320)
    best = min(list_schedule_makespan(mla.mla_plan_host(lens, wl.s_q, wl.heads, wl.block_size, maxb,
                                                        split_keys=c)[0], 320)
               for c in range(256, 8192, 64))
    assert auto <= 1.03 * best, (auto, best)


def test_noalloc_entry_checks_arguments_on_the_host():
    """mla_decode_noalloc: argument errors come back before any device call
    (no GPU here), an empty batch is a no-op, and a description whose plan
    cannot fit the fixed 64 MiB array even unsplit is refused."""
    lib = mla.library()
    assert lib.mla_decode_noalloc_scratch_bytes() == 64 * 1024 * 1024

    def call_na(d, s_q=1, ptrs=None, softmax_scale=0.07):
        p = dict(q=FAKE, kv=FAKE, bt=FAKE, sl=FAKE, out=FAKE)
        p.update(ptrs or {})
        return lib.mla_decode_noalloc(p["q"], p["kv"], p["bt"], p["sl"], s_q, softmax_scale, 1.0,
                                      p["out"], None, ctypes.byref(d), None)

    assert call_na(desc(), ptrs={"q": 0}) == INVALID
    assert call_na(desc(), ptrs={"out": FAKE + 2}) == INVALID
    assert call_na(desc(), softmax_scale=float("nan")) == INVALID
    assert call_na(desc(num_heads=129)) == UNSUPPORTED
    assert call_na(desc(batch=0)) == OK
    # a forced 64-key split of 128-row items over long contexts needs far more
    # than 64 MiB of partials: refused
    assert call_na(desc(batch=64, num_heads=128, max_blocks_per_seq=256, split_keys=64), s_q=4) == WS_SMALL


# ---------------------------------------------------------------------------
# the achievable-peak probe library (include/mla_probe.h)
# ---------------------------------------------------------------------------

PROBE_HEADER = os.path.join(ROOT, "include", "mla_probe.h")


def test_probe_library_exports_every_declared_function():
    text = re.sub(r"/\*.*?\*/", "", open(PROBE_HEADER).read(), flags=re.S)
    declared = sorted(set(re.findall(r"^\s*[\w\s\*]+?\b(mla_probe_\w+)\s*\(", text, flags=re.M)))
    assert declared == ["mla_probe_mfma", "mla_probe_mfma_expected", "mla_probe_mfma_flops"]
    lib = mla.probe_library()
    for fn in declared:
        assert hasattr(lib, fn), fn


def test_probe_flop_and_result_formulas():
    lib = mla.probe_library()
    # workgroups x 8 waves x iters x 8 chains x 2 M N K
    assert lib.mla_probe_mfma_flops(0, 1024, 2048) == 1024 * 8 * 2048 * 8 * 2 * 16 * 16 * 32
    assert lib.mla_probe_mfma_flops(1, 3, 5) == 3 * 8 * 5 * 8 * 2 * 32 * 32 * 16
    assert lib.mla_probe_mfma_flops(2, 1, 1) == 8 * 8 * 2 * 16 * 16 * 128
    assert lib.mla_probe_mfma_flops(3, 1, 1) == 0 and lib.mla_probe_mfma_flops(0, 0, 1) == 0
    # per thread: 8 chains x elements per lane x iters x K x x^2 (x = 1/16)
    assert lib.mla_probe_mfma_expected(0, 16, 0.0625) == 8 * 4 * 16 * 32 / 256
    assert lib.mla_probe_mfma_expected(1, 16, 0.0625) == 8 * 16 * 16 * 16 / 256
    assert lib.mla_probe_mfma_expected(2, 16, 0.0625) == 8 * 4 * 16 * 128 / 256
    assert lib.mla_probe_mfma_expected(-1, 16, 0.0625) == 0


@pytest.mark.parametrize("args", [(3, 8, 16), (-1, 8, 16), (0, 0, 16), (0, 8, 0), (0, (1 << 20) + 1, 1),
                                  (0, 1, (1 << 24) + 1)])
def test_probe_rejects_bad_arguments_without_launching(args):
    shape, wgs, iters = args
    assert mla.probe_library().mla_probe_mfma(shape, wgs, iters, 0.0625, FAKE, None) == 1


def test_probe_rejects_null_output():
    assert mla.probe_library().mla_probe_mfma(0, 8, 16, 0.0625, None, None) == 1
