"""Seeded synthetic workloads for paged MLA decode.

This module only *produces inputs*: sequence lengths, a shuffled page table,
bf16 query / latent-cache bit patterns, and (for the fp8 cache) e4m3fn codes
with their per-tensor scale. It holds none of the attention arithmetic, so
both the float64 oracle and the HIP path can consume what it makes without
sharing any computation.

Shapes follow the pages' workloads:
  * the kernel test printed in the review thread of "[Attention] Blackwell FP8
    MLA support with CUTLASS_MLA backend" (b=128, s_q=1, mean_sk=4096, h_q=16,
    h_kv=1, d=576, dv=512, page size 64, causal, fp8 e4m3fn);
  * DeepSeek-V3 serving in "[NVIDIA] Add Cutlass MLA backend" (128 heads,
    --block-size=128, 1000-token prompts with up to 2048 tokens of context);
  * 16K-token contexts of "[WIP][Attention] FlashAttn MLA" (max_model_len 16384).

Random numbers come from numpy's PCG64 (``default_rng(seed)``), drawn in a
fixed order: sequence lengths, page permutation, q, then cache rows. float32
samples are rounded to bf16 by round-to-nearest-even and to fp8 e4m3fn by
torch's cast (also round-to-nearest-even), after clamping to +-448.
Unused cache rows (tails of last pages, spare pages) are poisoned with NaN and
unused block-table entries hold -1, so any read past a sequence end shows up.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, Optional

import numpy as np

D_QK = 576      # 512 latent + 64 rotary columns per row
D_V = 512       # the latent part of each row doubles as V
BF16_NAN = 0x7FC0
FP8_NAN = 0x7F
FP8_MAX = 448.0


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    s_q: int
    heads: int
    block_size: int
    kv_dtype: str            # "bf16" or "fp8"
    lens: str                # "fixed", "uniform", "loguniform"
    lens_arg: tuple          # fixed: the lengths; uniform/loguniform: (lo, hi)
    causal: bool = True
    softmax_scale: float = 1.0 / math.sqrt(192.0)
    seed: int = 0
    spare_pages: int = 8


WORKLOADS: Dict[str, Workload] = {
    # tiny: two sequences, one shorter than a page, one with a ragged last page
    "tiny": Workload("tiny", 2, 1, 16, 64, "bf16", "fixed", (37, 200), seed=0),
    # the kernel-test shape, bf16 cache
    "b128_h16_L4096_bf16": Workload("b128_h16_L4096_bf16", 128, 1, 16, 64, "bf16",
                                     "fixed", (4096,), seed=1),
    # same shape, fp8 e4m3fn cache with per-tensor scale
    "b128_h16_L4096_fp8": Workload("b128_h16_L4096_fp8", 128, 1, 16, 64, "fp8",
                                    "fixed", (4096,), seed=2),
    # tiny shape with an fp8 cache
    "tiny_fp8": Workload("tiny_fp8", 2, 1, 16, 64, "fp8", "fixed", (37, 200), seed=5),
    # DeepSeek-V3-style 128-head decode
    "b64_h128_L1k2k_bs128_bf16": Workload("b64_h128_L1k2k_bs128_bf16", 64, 1, 128, 128,
                                           "bf16", "uniform", (1000, 2048), seed=3),
    # long skewed contexts with 4 speculative query tokens, fp8 cache
    "b32_sq4_h128_L512_16k_fp8": Workload("b32_sq4_h128_L512_16k_fp8", 32, 4, 128, 64,
                                           "fp8", "loguniform", (512, 16384), seed=4),
}


@dataclasses.dataclass
class Inputs:
    """Host-side arrays for one decode call (all numpy, C-contiguous)."""
    wl: Workload
    q_bits: np.ndarray          # uint16 [B, s_q, H, 576]  bf16 bit patterns
    kv: np.ndarray              # uint16 [nblk, bs, 576] (bf16) or uint8 (fp8 codes)
    kv_scale: float             # float32 value; 1.0 for a bf16 cache
    block_table: np.ndarray     # int32 [B, max_blocks]  (-1 = unused)
    seq_lens: np.ndarray        # int32 [B]  (counts the s_q new tokens)

    @property
    def num_blocks(self) -> int:
        return int(self.kv.shape[0])

    @property
    def max_blocks(self) -> int:
        return int(self.block_table.shape[1])


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (round-to-nearest-even) via torch; returns uint16 bits."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def f32_to_e4m3fn_codes(x: np.ndarray) -> np.ndarray:
    """Round float32 to OCP fp8 e4m3fn codes via torch's cast, saturating at +-448."""
    import torch
    t = torch.from_numpy(np.clip(np.ascontiguousarray(x, dtype=np.float32), -FP8_MAX, FP8_MAX))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def draw_seq_lens(wl: Workload, rng: np.random.Generator) -> np.ndarray:
    if wl.lens == "fixed":
        vals = list(wl.lens_arg)
        if len(vals) == 1:
            vals = vals * wl.batch
        assert len(vals) == wl.batch
        return np.asarray(vals, dtype=np.int32)
    lo, hi = wl.lens_arg
    if wl.lens == "uniform":
        return rng.integers(lo, hi + 1, size=wl.batch).astype(np.int32)
    if wl.lens == "loguniform":
        u = rng.uniform(math.log(lo), math.log(hi), size=wl.batch)
        return np.clip(np.rint(np.exp(u)), lo, hi).astype(np.int32)
    raise ValueError(wl.lens)


def make_inputs(wl: Workload, seed: Optional[int] = None,
                seq_lens: Optional[np.ndarray] = None,
                q_zero: bool = False) -> Inputs:
    """Build one seeded workload. ``seq_lens`` overrides the drawn lengths
    (the RNG stream is consumed the same way either way)."""
    rng = np.random.default_rng(wl.seed if seed is None else seed)
    drawn = draw_seq_lens(wl, rng)
    lens = drawn if seq_lens is None else np.asarray(seq_lens, dtype=np.int32)
    B, bs = wl.batch, wl.block_size
    assert lens.shape == (B,) and (lens >= 0).all()
    pages_per_seq = [(int(L) + bs - 1) // bs for L in lens]
    max_blocks = max(1, max(pages_per_seq))
    num_blocks = sum(pages_per_seq) + wl.spare_pages
    perm = rng.permutation(num_blocks).astype(np.int32)
    block_table = np.full((B, max_blocks), -1, dtype=np.int32)
    k = 0
    for b, n in enumerate(pages_per_seq):
        block_table[b, :n] = perm[k:k + n]
        k += n

    q = rng.standard_normal((B, wl.s_q, wl.heads, D_QK), dtype=np.float32)
    if q_zero:
        q[:] = 0.0
    q_bits = f32_to_bf16_bits(q)
    del q

    rows = rng.standard_normal((num_blocks, bs, D_QK), dtype=np.float32)
    # mark every cache row that no sequence owns
    used = np.zeros((num_blocks, bs), dtype=bool)
    for b, n in enumerate(pages_per_seq):
        for j in range(n):
            p = block_table[b, j]
            cnt = min(bs, int(lens[b]) - j * bs)
            used[p, :cnt] = True
    if wl.kv_dtype == "bf16":
        kv = f32_to_bf16_bits(rows)
        kv[~used] = BF16_NAN
        kv_scale = 1.0
    elif wl.kv_dtype == "fp8":
        amax = float(np.abs(rows[used]).max()) if used.any() else 1.0
        kv_scale = float(np.float32(amax / FP8_MAX))
        kv = f32_to_e4m3fn_codes(rows / np.float32(kv_scale))
        kv[~used] = FP8_NAN
    else:
        raise ValueError(wl.kv_dtype)
    del rows
    return Inputs(wl, q_bits, kv, kv_scale, block_table, lens)


def shrink(wl: Workload, batch: int, seed: Optional[int] = None, **kw) -> Workload:
    """A smaller instance of the same workload family (same distribution)."""
    lens_arg = wl.lens_arg
    if wl.lens == "fixed" and len(lens_arg) > 1:
        lens_arg = tuple((list(lens_arg) * batch)[:batch])
    return dataclasses.replace(wl, name=f"{wl.name}[B={batch}]", batch=batch,
                               lens_arg=lens_arg, seed=wl.seed if seed is None else seed, **kw)


def permute_pages(inp: Inputs, seed: int) -> Inputs:
    """Move every physical page to a new slot and rewrite the block table to match."""
    rng = np.random.default_rng(seed)
    n = inp.num_blocks
    perm = rng.permutation(n)            # new slot of old page p is perm[p]
    kv = np.empty_like(inp.kv)
    kv[perm] = inp.kv
    bt = inp.block_table.copy()
    m = bt >= 0
    bt[m] = perm[bt[m]]
    return dataclasses.replace(inp, kv=kv, block_table=bt.astype(np.int32))
