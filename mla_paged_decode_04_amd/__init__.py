"""Paged MLA decode on MI355X (gfx950): thin Python binding over the C ABI.

Every step of the computation runs in the HIP kernels of
``libmla_decode.so``; this module only checks tensors, allocates outputs and
workspace with torch, and passes raw device pointers plus the current torch
stream. If the library is missing the call raises — there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

__all__ = ["mla_decode", "mla_decode_plan", "mla_decode_with_plan", "mla_decode_noalloc",
           "mla_plan_host", "mla_kv_append", "mla_absorb_q", "mla_absorb_out", "workspace_size",
           "library", "MlaError", "D_QK", "D_V", "LIB_PATH"]

D_QK = 576
D_V = 512
LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmla_decode.so")
PROBE_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmla_probe.so")

MLA_DTYPE_BF16 = 0
MLA_DTYPE_FP8_E4M3FN = 1
ITEM_INTS = 8
HEADER_INTS = 64


class MlaError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what} failed: {_status_string(status)} ({status})")
        self.status = status


class Desc(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("num_heads", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("num_blocks", ctypes.c_int32),
        ("max_blocks_per_seq", ctypes.c_int32),
        ("kv_dtype", ctypes.c_int32),
        ("causal", ctypes.c_int32),
        ("split_keys", ctypes.c_int32),
    ]


_lib: Optional[ctypes.CDLL] = None


def library() -> ctypes.CDLL:
    """Load the in-tree HIP library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build it with `python -m mla_paged_decode_04_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, f32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
    pdesc = ctypes.POINTER(Desc)
    lib.mla_decode_workspace_size.argtypes = [i32, pdesc]
    lib.mla_decode_workspace_size.restype = sz
    lib.mla_decode.argtypes = [vp, vp, vp, vp, i32, f32, f32, vp, vp, pdesc, vp, sz, vp]
    lib.mla_decode.restype = ctypes.c_int
    lib.mla_decode_fwd_only.argtypes = [vp, vp, vp, vp, i32, f32, f32, vp, vp, pdesc, vp, sz, vp]
    lib.mla_decode_fwd_only.restype = ctypes.c_int
    lib.mla_decode_with_plan.argtypes = [vp, vp, vp, vp, i32, f32, f32, vp, vp, pdesc, vp, sz, vp]
    lib.mla_decode_with_plan.restype = ctypes.c_int
    lib.mla_decode_noalloc.argtypes = [vp, vp, vp, vp, i32, f32, f32, vp, vp, pdesc, vp]
    lib.mla_decode_noalloc.restype = ctypes.c_int
    lib.mla_decode_noalloc_scratch_bytes.argtypes = []
    lib.mla_decode_noalloc_scratch_bytes.restype = sz
    lib.mla_decode_plan.argtypes = [vp, i32, pdesc, vp, sz, vp]
    lib.mla_decode_plan.restype = ctypes.c_int
    lib.mla_plan_host.argtypes = [vp, i32, pdesc, vp, i32, vp, vp]
    lib.mla_plan_host.restype = i32
    lib.mla_kv_append.argtypes = [vp, vp, i32, f32, vp, i32, i32, i32, vp]
    lib.mla_kv_append.restype = ctypes.c_int
    lib.mla_absorb_q.argtypes = [vp, vp, vp, vp, i32, i32, i32, vp]
    lib.mla_absorb_q.restype = ctypes.c_int
    lib.mla_absorb_out.argtypes = [vp, vp, vp, i32, i32, i32, vp]
    lib.mla_absorb_out.restype = ctypes.c_int
    lib.mla_status_string.argtypes = [ctypes.c_int]
    lib.mla_status_string.restype = ctypes.c_char_p
    lib.mla_abi_version.argtypes = []
    lib.mla_abi_version.restype = i32
    _lib = lib
    return lib


_probe_lib: Optional[ctypes.CDLL] = None

PROBE_MFMA_16X16X32_BF16, PROBE_MFMA_32X32X16_BF16, PROBE_MFMA_16X16X128_FP8 = 0, 1, 2
PROBE_THREADS = 512


def probe_library() -> ctypes.CDLL:
    """Load the in-tree achievable-peak probe (include/mla_probe.h)."""
    global _probe_lib
    if _probe_lib is not None:
        return _probe_lib
    if not os.path.exists(PROBE_LIB_PATH):
        raise RuntimeError(
            f"{PROBE_LIB_PATH} is missing: build it with `python -m mla_paged_decode_04_amd.build`")
    lib = ctypes.CDLL(PROBE_LIB_PATH)
    i32, f32 = ctypes.c_int32, ctypes.c_float
    lib.mla_probe_mfma_flops.argtypes = [i32, i32, i32]
    lib.mla_probe_mfma_flops.restype = ctypes.c_double
    lib.mla_probe_mfma_expected.argtypes = [i32, i32, f32]
    lib.mla_probe_mfma_expected.restype = ctypes.c_double
    lib.mla_probe_mfma.argtypes = [i32, i32, i32, f32, ctypes.c_void_p, ctypes.c_void_p]
    lib.mla_probe_mfma.restype = i32
    _probe_lib = lib
    return lib


def mla_probe_mfma(shape: int, workgroups: int, iters: int, x: float, out: torch.Tensor) -> None:
    """Launch the MFMA probe on the current torch stream; out is float32 with
    workgroups * PROBE_THREADS elements on the GPU."""
    _check(out, "out", torch.float32, 1)
    if out.numel() < workgroups * PROBE_THREADS:
        raise ValueError(f"out needs {workgroups * PROBE_THREADS} elements")
    st = probe_library().mla_probe_mfma(shape, workgroups, iters, float(x), out.data_ptr(),
                                        torch.cuda.current_stream(out.device).cuda_stream)
    if st != 0:
        raise RuntimeError(f"mla_probe_mfma returned {st}")


def _status_string(status: int) -> str:
    try:
        return library().mla_status_string(status).decode()
    except Exception:  # pragma: no cover - only when the library itself is missing
        return "?"


def make_desc(batch: int, num_heads: int, block_size: int, num_blocks: int,
              max_blocks_per_seq: int, kv_dtype: int, causal: bool, split_keys: int = 0) -> Desc:
    return Desc(batch, num_heads, block_size, num_blocks, max_blocks_per_seq, kv_dtype,
                int(bool(causal)), split_keys)


def workspace_size(s_q: int, desc: Desc) -> int:
    return int(library().mla_decode_workspace_size(s_q, ctypes.byref(desc)))


def _kv_dtype_code(kv: torch.Tensor) -> int:
    if kv.dtype == torch.bfloat16:
        return MLA_DTYPE_BF16
    if kv.dtype in (torch.float8_e4m3fn, torch.uint8):
        return MLA_DTYPE_FP8_E4M3FN
    raise ValueError(f"kv_cache dtype {kv.dtype} is not bf16 or float8_e4m3fn")


def _check(t: torch.Tensor, name: str, dtype, ndim: int) -> None:
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU, got {t.device}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got shape {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _prepare(q, kv_cache, block_table, seq_lens, causal, out, lse, split_keys, want_lse):
    """Checks and output allocation shared by the decode entry points."""
    if kv_cache.dim() == 4 and kv_cache.shape[2] == 1:
        kv_cache = kv_cache.view(kv_cache.shape[0], kv_cache.shape[1], kv_cache.shape[3])
    _check(q, "q", torch.bfloat16, 4)
    _check(kv_cache, "kv_cache", None, 3)
    _check(block_table, "block_table", torch.int32, 2)
    _check(seq_lens, "seq_lens", torch.int32, 1)
    B, s_q, H, d = q.shape
    nb, bs, dk = kv_cache.shape
    if d != D_QK or dk != D_QK:
        raise ValueError(f"q and kv_cache rows must be {D_QK} wide")
    if block_table.shape[0] != B or seq_lens.shape[0] != B:
        raise ValueError("block_table and seq_lens must have one row per sequence")
    dev = q.device
    for name, t in (("kv_cache", kv_cache), ("block_table", block_table), ("seq_lens", seq_lens)):
        if t.device != dev:
            raise ValueError(f"{name} is on {t.device}, q on {dev}")
    desc = make_desc(B, H, bs, nb, block_table.shape[1], _kv_dtype_code(kv_cache), causal,
                     split_keys)
    if out is None:
        out = torch.empty((B, s_q, H, D_V), dtype=torch.bfloat16, device=dev)
    else:
        _check(out, "out", torch.bfloat16, 4)
        if tuple(out.shape) != (B, s_q, H, D_V):
            raise ValueError(f"out must be {(B, s_q, H, D_V)}")
    if lse is None and want_lse:
        lse = torch.empty((B, s_q, H), dtype=torch.float32, device=dev)
    elif lse is not None:
        _check(lse, "lse", torch.float32, 3)
        if tuple(lse.shape) != (B, s_q, H):
            raise ValueError(f"lse must be {(B, s_q, H)}")
    return kv_cache, desc, out, lse


def _decode_call(fn_name, q, kv_cache, block_table, seq_lens, softmax_scale, kv_scale, causal,
                 out, lse, workspace, split_keys, want_lse):
    kv_cache, desc, out, lse = _prepare(q, kv_cache, block_table, seq_lens, causal, out, lse,
                                        split_keys, want_lse)
    B, s_q, H, _ = q.shape
    lib = library()
    need = int(lib.mla_decode_workspace_size(s_q, ctypes.byref(desc)))
    if need == 0 and B > 0:
        raise MlaError(2, f"{fn_name} (B={B}, s_q={s_q}, H={H}, bs={kv_cache.shape[1]})")
    if workspace is None:
        if fn_name == "mla_decode_with_plan":
            raise ValueError("mla_decode_with_plan needs the workspace that holds the plan")
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    elif workspace.numel() < need:
        raise ValueError(f"workspace has {workspace.numel()} bytes, {need} needed")
    stream = torch.cuda.current_stream(q.device).cuda_stream
    st = getattr(lib, fn_name)(q.data_ptr(), kv_cache.data_ptr(), block_table.data_ptr(),
                               seq_lens.data_ptr(), s_q, float(softmax_scale), float(kv_scale),
                               out.data_ptr(), lse.data_ptr() if lse is not None else None,
                               ctypes.byref(desc), workspace.data_ptr(), workspace.numel(), stream)
    if st != 0:
        raise MlaError(st, fn_name)
    return out, lse


def mla_decode(q: torch.Tensor, kv_cache: torch.Tensor, block_table: torch.Tensor,
               seq_lens: torch.Tensor, softmax_scale: float, kv_scale: float = 1.0,
               causal: bool = True, out: Optional[torch.Tensor] = None,
               lse: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
               split_keys: int = 0, want_lse: bool = True
               ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Paged MLA decode (weight-absorbed MQA form).

    q [B, s_q, H, 576] bf16; kv_cache [num_blocks, bs, 576] (or [num_blocks,
    bs, 1, 576]) bf16 or float8_e4m3fn; block_table [B, max_blocks] int32;
    seq_lens [B] int32. Returns out [B, s_q, H, 512] bf16 and lse [B, s_q, H]
    fp32 (natural log), computed on the current torch stream. A workspace
    passed in (uint8, at least ``workspace_size`` bytes) keeps the plan for
    ``mla_decode_with_plan``.
    """
    return _decode_call("mla_decode", q, kv_cache, block_table, seq_lens, softmax_scale,
                        kv_scale, causal, out, lse, workspace, split_keys, want_lse)


def mla_decode_with_plan(q: torch.Tensor, kv_cache: torch.Tensor, block_table: torch.Tensor,
                         seq_lens: torch.Tensor, softmax_scale: float, workspace: torch.Tensor,
                         kv_scale: float = 1.0, causal: bool = True,
                         out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                         split_keys: int = 0, want_lse: bool = True
                         ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """``mla_decode`` on the plan an earlier ``mla_decode`` / ``mla_decode_plan``
    left in ``workspace`` for the same seq_lens values, s_q and description
    (no planner launch)."""
    return _decode_call("mla_decode_with_plan", q, kv_cache, block_table, seq_lens, softmax_scale,
                        kv_scale, causal, out, lse, workspace, split_keys, want_lse)


def mla_decode_noalloc(q: torch.Tensor, kv_cache: torch.Tensor, block_table: torch.Tensor,
                       seq_lens: torch.Tensor, softmax_scale: float, out: torch.Tensor,
                       lse: Optional[torch.Tensor], kv_scale: float = 1.0, causal: bool = True,
                       split_keys: int = 0) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """``mla_decode`` into caller-provided out / lse with the library's fixed
    device scratch array instead of a workspace: the call allocates nothing."""
    kv_cache, desc, out, lse = _prepare(q, kv_cache, block_table, seq_lens, causal, out, lse,
                                        split_keys, False)
    st = library().mla_decode_noalloc(
        q.data_ptr(), kv_cache.data_ptr(), block_table.data_ptr(), seq_lens.data_ptr(), q.shape[1],
        float(softmax_scale), float(kv_scale), out.data_ptr(),
        lse.data_ptr() if lse is not None else None, ctypes.byref(desc),
        torch.cuda.current_stream(q.device).cuda_stream)
    if st != 0:
        raise MlaError(st, "mla_decode_noalloc")
    return out, lse


def mla_decode_plan(seq_lens: torch.Tensor, s_q: int, num_heads: int, block_size: int,
                    max_blocks_per_seq: int, num_blocks: int = 1, causal: bool = True,
                    split_keys: int = 0) -> Tuple[torch.Tensor, torch.Tensor]:
    """Run only the device split planner; returns (header int32[4], items int32[n, 8])."""
    _check(seq_lens, "seq_lens", torch.int32, 1)
    desc = make_desc(seq_lens.shape[0], num_heads, block_size, num_blocks, max_blocks_per_seq,
                     MLA_DTYPE_BF16, causal, split_keys)
    lib = library()
    need = int(lib.mla_decode_workspace_size(s_q, ctypes.byref(desc)))
    if need == 0:
        raise MlaError(2, "mla_decode_plan")
    ws = torch.empty(need, dtype=torch.uint8, device=seq_lens.device)
    st = lib.mla_decode_plan(seq_lens.data_ptr(), s_q, ctypes.byref(desc), ws.data_ptr(), need,
                             torch.cuda.current_stream(seq_lens.device).cuda_stream)
    if st != 0:
        raise MlaError(st, "mla_decode_plan")
    ints = ws.view(torch.int32)
    header = ints[:4].clone()
    n = int(header[0].item())
    items = ints[HEADER_INTS:HEADER_INTS + n * ITEM_INTS].view(n, ITEM_INTS).clone()
    return header, items


def mla_plan_host(seq_lens, s_q: int, num_heads: int, block_size: int, max_blocks_per_seq: int,
                  causal: bool = True, split_keys: int = 0, max_items: int = 1 << 20):
    """Host mirror of the planner: returns (items int32[n, 8], rows_per_item, chunk_keys)."""
    import numpy as np
    lens = np.ascontiguousarray(np.asarray(seq_lens, dtype=np.int32))
    desc = make_desc(lens.shape[0], num_heads, block_size, 1, max_blocks_per_seq,
                     MLA_DTYPE_BF16, causal, split_keys)
    buf = np.zeros((max_items, ITEM_INTS), dtype=np.int32)
    rows = ctypes.c_int32(0)
    chunk = ctypes.c_int32(0)
    n = library().mla_plan_host(lens.ctypes.data, s_q, ctypes.byref(desc), buf.ctypes.data,
                                max_items, ctypes.byref(rows), ctypes.byref(chunk))
    if n < 0:
        raise MlaError(1, "mla_plan_host")
    return buf[:n].copy(), rows.value, chunk.value


def mla_kv_append(rows: torch.Tensor, slot_mapping: torch.Tensor, kv_cache: torch.Tensor,
                  kv_scale: float = 1.0) -> torch.Tensor:
    """Write rows (bf16 [n, 576]) into kv_cache ([num_blocks, bs, 576] or
    [num_blocks, bs, 1, 576], bf16 or float8_e4m3fn) at slot_mapping (int32 [n],
    slot = page * bs + offset; negative = skip), on the current torch stream.
    fp8 values are stored as e4m3fn(x / kv_scale); returns kv_cache."""
    kv = kv_cache
    if kv.dim() == 4 and kv.shape[2] == 1:
        kv = kv.view(kv.shape[0], kv.shape[1], kv.shape[3])
    _check(rows, "rows", torch.bfloat16, 2)
    _check(slot_mapping, "slot_mapping", torch.int32, 1)
    _check(kv, "kv_cache", None, 3)
    if rows.shape[1] != D_QK or kv.shape[2] != D_QK:
        raise ValueError(f"rows and kv_cache rows must be {D_QK} wide")
    if slot_mapping.shape[0] != rows.shape[0]:
        raise ValueError("slot_mapping must have one entry per row")
    for name, t in (("slot_mapping", slot_mapping), ("kv_cache", kv)):
        if t.device != rows.device:
            raise ValueError(f"{name} is on {t.device}, rows on {rows.device}")
    st = library().mla_kv_append(rows.data_ptr(), slot_mapping.data_ptr(), rows.shape[0],
                                 float(kv_scale), kv.data_ptr(), kv.shape[0], kv.shape[1],
                                 _kv_dtype_code(kv), torch.cuda.current_stream(rows.device).cuda_stream)
    if st != 0:
        raise MlaError(st, "mla_kv_append")
    return kv_cache


def mla_absorb_q(q_nope: torch.Tensor, q_pe: torch.Tensor, w_uk: torch.Tensor,
                 out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """q for mla_decode from the per-head parts: q_nope [T, H, d_nope] . w_uk
    [H, d_nope, 512] -> latent 512, with q_pe [T, H, 64] appended. All bf16."""
    _check(q_nope, "q_nope", torch.bfloat16, 3)
    _check(q_pe, "q_pe", torch.bfloat16, 3)
    _check(w_uk, "w_uk", torch.bfloat16, 3)
    T, H, dn = q_nope.shape
    if tuple(q_pe.shape) != (T, H, D_QK - D_V) or tuple(w_uk.shape) != (H, dn, D_V):
        raise ValueError("shapes must be q_nope [T,H,d], q_pe [T,H,64], w_uk [H,d,512]")
    if out is None:
        out = torch.empty((T, H, D_QK), dtype=torch.bfloat16, device=q_nope.device)
    _check(out, "out", torch.bfloat16, 3)
    st = library().mla_absorb_q(q_nope.data_ptr(), q_pe.data_ptr(), w_uk.data_ptr(), out.data_ptr(),
                                T, H, dn, torch.cuda.current_stream(q_nope.device).cuda_stream)
    if st != 0:
        raise MlaError(st, "mla_absorb_q")
    return out


def mla_absorb_out(o: torch.Tensor, w_uv: torch.Tensor, out: Optional[torch.Tensor] = None
                   ) -> torch.Tensor:
    """Per-head output projection: o [T, H, 512] . w_uv [H, 512, d_v] -> [T, H, d_v]. bf16."""
    _check(o, "o", torch.bfloat16, 3)
    _check(w_uv, "w_uv", torch.bfloat16, 3)
    T, H, dl = o.shape
    if dl != D_V or w_uv.shape[0] != H or w_uv.shape[1] != D_V:
        raise ValueError("shapes must be o [T,H,512], w_uv [H,512,d_v]")
    dv = w_uv.shape[2]
    if out is None:
        out = torch.empty((T, H, dv), dtype=torch.bfloat16, device=o.device)
    _check(out, "out", torch.bfloat16, 3)
    st = library().mla_absorb_out(o.data_ptr(), w_uv.data_ptr(), out.data_ptr(), T, H, dv,
                                  torch.cuda.current_stream(o.device).cuda_stream)
    if st != 0:
        raise MlaError(st, "mla_absorb_out")
    return out
