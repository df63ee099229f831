"""Float64 CPU oracle for paged MLA decode — TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this module. The product path (the C-ABI library and
its Python binding) never calls it, and this module calls nothing of theirs.

What it computes (plain reading of the pages):
  * "[WIP][Attention] FlashAttn MLA", description: MLA's decode step is
    computed as multi-query attention (MQA) — all query heads attend to a
    single shared KV head.
  * "[Attention] Blackwell FP8 MLA support with CUTLASS_MLA backend", review
    thread (the failing kernel test): h_kv = 1, d = 576 (query/key width),
    dv = 512 (value width), paged cache with page size 64, ``causal`` and
    ``varlen`` options, cache dtype bf16 or ``torch.float8_e4m3fn``.
  * Readings where the pages are silent (each listed in the design notes):
    the 512 latent columns come first and the 64 rotary columns last; V is the
    first 512 columns of the same cached row; k = decode(code) * kv_scale;
    scores = softmax_scale * (q . k); lse is the natural log of the softmax
    denominator including both scales; with s_q > 1 query tokens the causal
    mask is bottom-right aligned (query token i sees keys [0, L - s_q + 1 + i));
    a row that sees no key gets out = 0, lse = -inf; a block-table entry
    outside [0, num_blocks) inside a sequence's range holds no keys (its
    tokens are left out of the softmax).

Everything is float64 and unblocked: one numpy matmul per (sequence, query
token) for the scores and one for the weighted sum of values.
Parity status: pinned (see tests/test_oracle.py) — brute force, closed forms,
invariants and the OCP fp8 special values.
"""
from __future__ import annotations

import math
from typing import Tuple

import numpy as np

D_QK = 576
D_V = 512


# ---------------------------------------------------------------------------
# element decoding
# ---------------------------------------------------------------------------

def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 is the top half of an IEEE float32: widen exactly."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def e4m3fn_value(code: int) -> float:
    """Value of one OCP OFP8 E4M3 ("fn": finite, no infinities) code.

    OCP 8-bit Floating Point Specification v1.0, E4M3: 1 sign bit, 4 exponent
    bits with bias 7, 3 mantissa bits; exponent field 0 encodes subnormals
    (2^-6 * m/8); S.1111.111 is NaN; there is no infinity, so S.1111.110 = 448
    is the largest finite magnitude. (The pages name the dtype
    ``torch.float8_e4m3fn`` for the cache.)
    """
    s = (code >> 7) & 1
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return math.nan
    if e == 0:
        mag = math.ldexp(m / 8.0, -6)
    else:
        mag = math.ldexp(1.0 + m / 8.0, e - 7)
    return -mag if s else mag


E4M3FN_TABLE = np.array([e4m3fn_value(c) for c in range(256)], dtype=np.float64)


def e4m3fn_to_f64(codes: np.ndarray) -> np.ndarray:
    return E4M3FN_TABLE[np.asarray(codes, dtype=np.uint8)]


def decode_rows(raw: np.ndarray, kv_dtype: str) -> np.ndarray:
    if kv_dtype == "bf16":
        return bf16_bits_to_f64(raw)
    if kv_dtype == "fp8":
        return e4m3fn_to_f64(raw)
    raise ValueError(kv_dtype)


# ---------------------------------------------------------------------------
# paging
# ---------------------------------------------------------------------------

def page_is_valid(page: int, num_blocks: int) -> bool:
    """A block-table entry names a page of the cache only if it lies in
    [0, num_blocks). (Reading: the pages never show an invalid entry inside a
    sequence's range; such a page is taken to hold no keys.)"""
    return 0 <= page < num_blocks


def gather_keys(kv: np.ndarray, block_table_row: np.ndarray, seq_len: int,
                kv_dtype: str, kv_scale: float) -> np.ndarray:
    """Rows 0..seq_len-1 of one sequence, in token order, as float64.

    Token t lives at page ``block_table_row[t // bs]``, slot ``t % bs``
    (paged cache of the kernel test in the CUTLASS_MLA fp8 review thread).
    Rows of an invalid page (``page_is_valid``) are left as zeros here and
    excluded by ``valid_key_mask``.
    """
    bs = kv.shape[1]
    out = np.zeros((seq_len, D_QK), dtype=np.float64)
    for t in range(0, seq_len, bs):
        page = int(block_table_row[t // bs])
        if not page_is_valid(page, kv.shape[0]):
            continue
        n = min(bs, seq_len - t)
        out[t:t + n] = decode_rows(kv[page, :n], kv_dtype)
    return out * np.float64(kv_scale)


def valid_key_mask(block_table_row: np.ndarray, seq_len: int, block_size: int,
                   num_blocks: int) -> np.ndarray:
    """True for the tokens 0..seq_len-1 whose page is valid."""
    pages = np.asarray(block_table_row[:(seq_len + block_size - 1) // block_size], dtype=np.int64)
    ok = (pages >= 0) & (pages < num_blocks)
    return np.repeat(ok, block_size)[:seq_len]


# ---------------------------------------------------------------------------
# attention
# ---------------------------------------------------------------------------

def attend(qrows: np.ndarray, keys: np.ndarray, softmax_scale: float
           ) -> Tuple[np.ndarray, np.ndarray]:
    """Softmax attention of query rows [n, 576] over keys [T, 576]; the value
    of key t is keys[t, :512]. Returns (out [n, 512], lse [n]), natural log."""
    n = qrows.shape[0]
    T = keys.shape[0]
    if T == 0:
        return np.zeros((n, D_V)), np.full(n, -np.inf)
    s = np.float64(softmax_scale) * (qrows @ keys.T)          # [n, T]
    m = s.max(axis=1, keepdims=True)
    w = np.exp(s - m)
    den = w.sum(axis=1, keepdims=True)
    out = (w @ keys[:, :D_V]) / den
    lse = (m + np.log(den))[:, 0]
    return out, lse


def attend_abs(qrows: np.ndarray, keys: np.ndarray, softmax_scale: float) -> np.ndarray:
    """The softmax-weighted mean of |v| per output element: sum_t w_t |v_t| /
    sum_t w_t with the same weights as ``attend`` ([n, 512]; zeros when there
    is no key). It bounds |out| elementwise (convexity) and is the scale of
    the error that rounding the weights makes in out, which is what the
    elementwise parity bound of the GPU tests is stated against."""
    n = qrows.shape[0]
    if keys.shape[0] == 0:
        return np.zeros((n, D_V))
    s = np.float64(softmax_scale) * (qrows @ keys.T)
    w = np.exp(s - s.max(axis=1, keepdims=True))
    return (w @ np.abs(keys[:, :D_V])) / w.sum(axis=1, keepdims=True)


def visible_keys(seq_len: int, s_q: int, i: int, causal: bool) -> int:
    """Number of keys query token i (0-based among the s_q new tokens) sees.
    The new tokens are the last s_q of the sequence (they are already in the
    cache), so causal attention lets token i see keys [0, L - s_q + 1 + i)."""
    if not causal:
        return seq_len
    return max(0, seq_len - s_q + 1 + i)


def mla_decode(q_bits: np.ndarray, kv: np.ndarray, block_table: np.ndarray,
               seq_lens: np.ndarray, s_q: int, softmax_scale: float,
               kv_scale: float, kv_dtype: str, causal: bool = True,
               with_abs: bool = False):
    """Paged MLA decode in its weight-absorbed MQA form.

    q_bits: uint16 bf16 bits [B, s_q, H, 576]; kv: uint16 bf16 bits or uint8
    e4m3fn codes [num_blocks, bs, 576]; block_table int32 [B, max_blocks];
    seq_lens int32 [B]. Returns float64 out [B, s_q, H, 512], lse [B, s_q, H]
    (and, with ``with_abs``, ``attend_abs`` of every row as a third array).
    Keys on invalid pages are not attended (``valid_key_mask``).
    """
    B, sq, H, d = q_bits.shape
    assert sq == s_q and d == D_QK and kv.shape[2] == D_QK
    nb, bs = kv.shape[0], kv.shape[1]
    out = np.zeros((B, s_q, H, D_V), dtype=np.float64)
    lse = np.full((B, s_q, H), -np.inf, dtype=np.float64)
    vabs = np.zeros((B, s_q, H, D_V), dtype=np.float64) if with_abs else None
    for b in range(B):
        L = int(seq_lens[b])
        keys = gather_keys(kv, block_table[b], L, kv_dtype, kv_scale)
        ok = valid_key_mask(block_table[b], L, bs, nb)
        for i in range(s_q):
            n_vis = visible_keys(L, s_q, i, causal)
            qrows = bf16_bits_to_f64(q_bits[b, i])
            vis = keys[:n_vis][ok[:n_vis]]
            o, l = attend(qrows, vis, softmax_scale)
            out[b, i] = o
            lse[b, i] = l
            if with_abs:
                vabs[b, i] = attend_abs(qrows, vis, softmax_scale)
    if with_abs:
        return out, lse, vabs
    return out, lse


def combine_partials(o_parts: np.ndarray, lse_parts: np.ndarray
                     ) -> Tuple[np.ndarray, np.ndarray]:
    """Merge attention results computed over disjoint key chunks.

    o_parts [S, ..., 512] are each chunk's normalised outputs and lse_parts
    [S, ...] their log-sum-exps; a chunk that saw no key has lse = -inf and
    weight 0. The merged lse is log(sum_s exp(lse_s)) and the merged output is
    sum_s exp(lse_s - lse) * o_s (flash-decoding's split-KV reduction).
    """
    m = np.max(lse_parts, axis=0)
    m_safe = np.where(np.isfinite(m), m, 0.0)
    w = np.exp(lse_parts - m_safe)                            # [S, ...]
    den = w.sum(axis=0)
    with np.errstate(divide="ignore", invalid="ignore"):
        lse = np.where(den > 0, m_safe + np.log(den), -np.inf)
        o = np.where((den > 0)[..., None],
                     (w[..., None] * o_parts).sum(axis=0) / den[..., None], 0.0)
    return o, lse


# ---------------------------------------------------------------------------
# comparison metrics
# ---------------------------------------------------------------------------

def cos_diff(x: np.ndarray, y: np.ndarray) -> float:
    """The similarity measure the kernel test of the CUTLASS_MLA fp8 review
    thread asserts on, from its definition: the squared distance of x and y
    relative to their summed squared norms, ||x - y||^2 / (||x||^2 + ||y||^2).
    It is 0 for x = y, 1 when one of them is zero (or the two are
    orthogonal) and 2 for y = -x. Two all-zero arrays count as equal (0)."""
    x = np.asarray(x, dtype=np.float64).ravel()
    y = np.asarray(y, dtype=np.float64).ravel()
    den = float(np.dot(x, x) + np.dot(y, y))
    if den == 0.0:
        return 0.0
    d = x - y
    return float(np.dot(d, d) / den)


def rel_fro(x: np.ndarray, ref: np.ndarray) -> float:
    """Relative Frobenius error ||x - ref||_F / ||ref||_F over all elements
    (0 when both are zero, inf when only ref is)."""
    x = np.asarray(x, dtype=np.float64).ravel()
    ref = np.asarray(ref, dtype=np.float64).ravel()
    num = math.sqrt(float(np.dot(x - ref, x - ref)))
    den = math.sqrt(float(np.dot(ref, ref)))
    if den == 0.0:
        return 0.0 if num == 0.0 else math.inf
    return num / den


def rel_fro_rows(x: np.ndarray, ref: np.ndarray) -> np.ndarray:
    """``rel_fro`` of every row (last axis) on its own; rows where ref is zero
    give 0 if x is zero there too, else inf."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    num = np.sqrt(((x - ref) ** 2).sum(axis=-1))
    den = np.sqrt((ref ** 2).sum(axis=-1))
    with np.errstate(divide="ignore", invalid="ignore"):
        r = num / den
    return np.where(den > 0, r, np.where(num > 0, np.inf, 0.0))


# ---------------------------------------------------------------------------
# writing new rows into the paged cache (the step before decode)
# ---------------------------------------------------------------------------
#
# "[Attention] Blackwell FP8 MLA support with CUTLASS_MLA backend", Purpose
# and Test Plan: the latent cache is kept in torch.float8_e4m3fn. Reading
# used (the pages do not spell out the write): a new row x (bf16) is stored
# in slot `slot` (page slot // bs, row slot % bs) as the code of
# y = float32(x) / float32(kv_scale) -- for fp8 clamped to [-448, 448] and
# rounded to the nearest e4m3fn value, ties to the even mantissa; for a bf16
# cache rounded to the nearest bf16, ties to even. Decoding multiplies by
# kv_scale again. Negative slots are padding and write nothing.

_E4M3FN_POS = E4M3FN_TABLE[:0x7F]          # codes 0x00..0x7E: 0 .. 448, increasing


def quantize_e4m3fn(y: np.ndarray) -> np.ndarray:
    """float32 values -> e4m3fn codes by nearest value (ties: even mantissa)."""
    y = np.asarray(y, dtype=np.float32)
    a = np.minimum(np.abs(y.astype(np.float64)), 448.0)
    hi = np.searchsorted(_E4M3FN_POS, a, side="left")          # first value >= a
    hi = np.minimum(hi, 0x7E)
    lo = np.where(_E4M3FN_POS[hi] == a, hi, np.maximum(hi - 1, 0))
    d_lo = a - _E4M3FN_POS[lo]
    d_hi = _E4M3FN_POS[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0) & (hi != lo))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    code = np.where(np.signbit(y), code | np.uint8(0x80), code)
    code = np.where(np.isnan(y), np.uint8(0x7F) | (np.signbit(y).astype(np.uint8) << 7), code)
    return code.astype(np.uint8)


def round_bf16(y: np.ndarray) -> np.ndarray:
    """float32 values -> bf16 bit patterns, nearest with ties to even (NaN kept
    as a quiet NaN). The two candidates are the value truncated to bf16 and
    the next bf16 away from zero; the distances are compared in float64."""
    y = np.asarray(y, dtype=np.float32)
    u = y.view(np.uint32)
    t = (u >> np.uint32(16)).astype(np.uint32)                 # truncated pattern
    up = t + np.uint32(1)                                       # next magnitude up
    vt = bf16_bits_to_f64(t.astype(np.uint16))
    vu = bf16_bits_to_f64(up.astype(np.uint16))
    x = y.astype(np.float64)
    d_t = np.abs(x - vt)
    d_u = np.abs(vu - x)
    pick_up = (d_u < d_t) | ((d_u == d_t) & (t % 2 == 1))
    out = np.where(pick_up, up, t).astype(np.uint16)
    out = np.where(np.isnan(y), (t | np.uint32(0x40)).astype(np.uint16), out)
    return out


def kv_append(kv: np.ndarray, rows_bits: np.ndarray, slot_mapping: np.ndarray,
              kv_scale: float, kv_dtype: str) -> np.ndarray:
    """Copy of `kv` with row n of `rows_bits` (bf16 bits [N, 576]) written to
    slot slot_mapping[n] in the cache encoding."""
    kv = np.array(kv, copy=True)
    nb, bs = kv.shape[0], kv.shape[1]
    x = bf16_bits_to_f64(rows_bits).astype(np.float32)
    y = x / np.float32(kv_scale)
    for n, slot in enumerate(np.asarray(slot_mapping, dtype=np.int64)):
        if slot < 0 or slot >= nb * bs:
            continue
        page, off = divmod(int(slot), bs)
        kv[page, off] = quantize_e4m3fn(y[n]) if kv_dtype == "fp8" else round_bf16(y[n])
    return kv


# ---------------------------------------------------------------------------
# the absorbed projections around the MQA
# ---------------------------------------------------------------------------
#
# "[WIP][Attention] FlashAttn MLA", description: the decode step of MLA is
# computed as MQA over the latent cache, so each head's up-projection of the
# keys (W_UK) multiplies its query instead, and the value up-projection (W_UV)
# is applied to the 512-wide latent output. Reading used: q_nope [T, H, d],
# W_UK [H, d, 512], q_pe [T, H, 64] appended as the rotary part; W_UV
# [H, 512, d_v]. Plain float64 products of the bf16 inputs.

def absorb_q(q_nope_bits: np.ndarray, q_pe_bits: np.ndarray, w_uk_bits: np.ndarray) -> np.ndarray:
    qn = bf16_bits_to_f64(q_nope_bits)                     # [T, H, d]
    w = bf16_bits_to_f64(w_uk_bits)                        # [H, d, 512]
    lat = np.einsum("thd,hdn->thn", qn, w)
    return np.concatenate([lat, bf16_bits_to_f64(q_pe_bits)], axis=-1)


def absorb_out(o_bits: np.ndarray, w_uv_bits: np.ndarray) -> np.ndarray:
    return np.einsum("thn,hnv->thv", bf16_bits_to_f64(o_bits), bf16_bits_to_f64(w_uv_bits))
