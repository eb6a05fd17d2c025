"""Paged-attention hot path for MI355X (gfx950): Python binding of libpaged_attn.so.

Only argument marshalling lives here: every step of the computation runs in the
HIP kernels behind the C ABI declared in ``include/paged_attn.h``.  PyTorch
supplies device memory and the current stream.  There is no fallback: if the
library is missing or a call fails, an exception is raised.

Calls (weft, "Cache layouts": write = scatter via slot_mapping, read = gather by
block_table; per-layer pool ``[N, P, H_kv, D]``):

* ``slot_mapping(block_table, cu_seqlens, context_lens, block_size)``
* ``reshape_and_cache(k, v, slot_mapping, k_cache, v_cache)``
* ``paged_decode_attention(q, k_cache, v_cache, block_table, context_lens, scale, out)``
* ``paged_prefill_attention(q, k, v, cu_seqlens, block_table, context_lens, scale, out)``
"""

from __future__ import annotations

import contextlib
import ctypes
import os
import threading

import torch

__all__ = [
    "LIB_PATH",
    "PagedAttnError",
    "load_library",
    "slot_mapping",
    "reshape_and_cache",
    "copy_blocks",
    "check_metadata",
    "hbm_read",
    "paged_decode_attention",
    "paged_decode_append",
    "paged_decode_attention_noalloc",
    "paged_prefill_attention",
    "paged_mixed_attention",
    "decode_workspace_size",
    "prefill_workspace_size",
    "mixed_workspace_size",
    "kernel_timer",
    "workspace_status",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpaged_attn.so")

_c_void_p = ctypes.c_void_p
_i32 = ctypes.c_int32
_i64 = ctypes.c_int64
_f32 = ctypes.c_float
_size = ctypes.c_size_t

# name -> (restype, argtypes); mirrors include/paged_attn.h
SIGNATURES = {
    "pa_version": (ctypes.c_int, []),
    "pa_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "pa_last_error": (ctypes.c_char_p, []),
    "pa_set_timing_events": (ctypes.c_int, [_c_void_p, _c_void_p]),
    "pa_hbm_read": (ctypes.c_int, [_c_void_p, _i64, _c_void_p, _i32, _c_void_p]),
    "pa_slot_mapping": (ctypes.c_int, [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _i32, _i64, _i32, _i32, _c_void_p]),
    "pa_reshape_and_cache": (
        ctypes.c_int,
        [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _i64, _i64, _i32, _i32, _i32, _i32, _c_void_p],
    ),
    "pa_reshape_and_cache_fp8": (
        ctypes.c_int,
        [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _i64, _i64, _i32, _i32, _i32,
         _i32, _c_void_p],
    ),
    "pa_paged_decode_attention_fp8": (
        ctypes.c_int,
        [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _f32, _c_void_p,
         _i32, _i32, _i32, _i32, _i32, _i64, _i32, _c_void_p, _size, _c_void_p],
    ),
    "pa_paged_prefill_attention_fp8": (
        ctypes.c_int,
        [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _f32, _c_void_p,
         _i32, _i64, _i32, _i32, _i32, _i32, _i64, _i32, _c_void_p, _size, _c_void_p],
    ),
    "pa_check_metadata": (
        ctypes.c_int,
        [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _i32, _i64, _i64, _i32, _i32, _c_void_p, _c_void_p],
    ),
    "pa_copy_blocks": (ctypes.c_int, [_c_void_p, _c_void_p, _c_void_p, _i64, _i64, _i32, _i32, _i32, _i32, _c_void_p]),
    "pa_decode_workspace_size": (_size, [_i32, _i32, _i32, _i32, _i32]),
    "pa_paged_decode_attention": (
        ctypes.c_int,
        [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _f32, _c_void_p,
         _i32, _i32, _i32, _i32, _i32, _i64, _i32, _i32, _c_void_p, _size, _c_void_p],
    ),
    "pa_paged_decode_attention_noalloc": (
        ctypes.c_int,
        [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _f32, _c_void_p,
         _i32, _i32, _i32, _i32, _i32, _i64, _i32, _i32, _c_void_p],
    ),
    "pa_workspace_status": (ctypes.c_int, [_c_void_p, _c_void_p, _c_void_p]),
    "pa_paged_decode_append": (
        ctypes.c_int,
        [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _f32, _c_void_p,
         _i32, _i32, _i32, _i32, _i32, _i64, _i32, _i32, _c_void_p, _size, _c_void_p],
    ),
    "pa_paged_decode_append_fp8": (
        ctypes.c_int,
        [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _f32,
         _c_void_p, _i32, _i32, _i32, _i32, _i32, _i64, _i32, _i32, _c_void_p, _size, _c_void_p],
    ),
    "pa_mixed_workspace_size": (_size, [_i32, _i32, _i32, _i32, _i32]),
    "pa_paged_mixed_attention": (
        ctypes.c_int,
        [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _f32, _c_void_p,
         _i32, _i64, _i32, _i32, _i32, _i32, _i64, _i32, _i32, _c_void_p, _size, _c_void_p],
    ),
    "pa_paged_mixed_attention_fp8": (
        ctypes.c_int,
        [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _f32, _c_void_p,
         _i32, _i64, _i32, _i32, _i32, _i32, _i64, _i32, _c_void_p, _size, _c_void_p],
    ),
    "pa_prefill_workspace_size": (_size, [_i32, _i64, _i32, _i32]),
    "pa_paged_prefill_attention": (
        ctypes.c_int,
        [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _f32, _c_void_p,
         _i32, _i64, _i32, _i32, _i32, _i32, _i64, _i32, _i32, _c_void_p, _size, _c_void_p],
    ),
}

_DTYPES = {torch.float32: 0, torch.bfloat16: 1}
_lib = None
_lock = threading.Lock()


class PagedAttnError(RuntimeError):
    """A libpaged_attn call returned an error status."""


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libpaged_attn.so (built by ``paged_kv_cache_48_amd.build``)."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(path):
                raise PagedAttnError(
                    f"{path} is missing: build it first (python -m paged_kv_cache_48_amd.build)"
                )
            lib = ctypes.CDLL(path)
            for name, (res, args) in SIGNATURES.items():
                fn = getattr(lib, name)
                fn.restype = res
                fn.argtypes = args
            _lib = lib
    return _lib


def _check(status: int) -> None:
    if status != 0:
        lib = load_library()
        msg = lib.pa_last_error().decode() or lib.pa_status_string(status).decode()
        if status in (-1, -2, -3):
            raise ValueError(msg)
        raise PagedAttnError(msg)


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _req(cond: bool, msg: str) -> None:
    if not cond:
        raise ValueError(msg)


def _dev_tensor(t: torch.Tensor, name: str, dtype=None, dim=None) -> None:
    _req(isinstance(t, torch.Tensor), f"{name} must be a tensor")
    _req(t.is_cuda, f"{name} must be a device tensor")
    _req(t.is_contiguous(), f"{name} must be contiguous")
    if dtype is not None:
        _req(t.dtype == dtype, f"{name} must be {dtype} (got {t.dtype})")
    if dim is not None:
        _req(t.dim() == dim, f"{name} must have {dim} dimensions (got {t.dim()})")


def _dtype_code(t: torch.Tensor) -> int:
    _req(t.dtype in _DTYPES, f"unsupported dtype {t.dtype} (float32 or bfloat16)")
    return _DTYPES[t.dtype]


# One cached workspace per (device, stream): calls on one stream run in order,
# so they can share it; calls on different streams must not.  A workspace may
# be baked into a captured HIP graph (torch.cuda.graph), so a cached workspace
# is never freed: when a call needs more, a larger one (rounded up to a power
# of two, so at most a few dozen ever exist) replaces it in the cache and the
# old one stays alive in ``_retired`` until the process ends.  Graphs that
# were captured on one stream share that stream's workspace and must not be
# replayed concurrently; a caller that needs otherwise passes ``workspace=``.
_workspaces: dict = {}
_retired: list = []


def _workspace(device: torch.device, stream: int, nbytes: int, given: torch.Tensor | None = None) -> torch.Tensor:
    if given is not None:
        _dev_tensor(given, "workspace", torch.uint8)
        _req(given.device == device, "workspace must be on the call's device")
        _req(given.numel() >= nbytes, f"workspace holds {given.numel()} bytes, the call needs {nbytes}")
        return given
    key = (device.index, stream)
    ws = _workspaces.get(key)
    if ws is None or ws.numel() < nbytes:
        size = 256
        while size < nbytes:
            size *= 2
        if ws is not None:
            _retired.append(ws)
        ws = torch.empty(size, dtype=torch.uint8, device=device)
        _workspaces[key] = ws
    return ws


def decode_workspace_size(num_seqs, num_q_heads, head_dim, block_size, max_blocks_per_seq) -> int:
    return int(load_library().pa_decode_workspace_size(num_seqs, num_q_heads, head_dim, block_size,
                                                       max_blocks_per_seq))


def prefill_workspace_size(num_seqs, total_q_tokens, num_q_heads, num_kv_heads) -> int:
    return int(load_library().pa_prefill_workspace_size(num_seqs, total_q_tokens, num_q_heads, num_kv_heads))


def mixed_workspace_size(num_seqs, num_q_heads, head_dim, block_size, max_blocks_per_seq) -> int:
    return int(load_library().pa_mixed_workspace_size(num_seqs, num_q_heads, head_dim, block_size,
                                                      max_blocks_per_seq))


def slot_mapping(block_table: torch.Tensor, cu_seqlens: torch.Tensor, context_lens: torch.Tensor,
                 block_size: int, num_tokens: int, out: torch.Tensor | None = None) -> torch.Tensor:
    """int32 ``[num_tokens]`` slots of the new tokens (see ``pa_slot_mapping``).
    ``num_tokens`` must equal ``cu_seqlens[-1]`` (passed explicitly so that no
    device value is read on the host)."""
    lib = load_library()
    _dev_tensor(block_table, "block_table", torch.int32, 2)
    _dev_tensor(cu_seqlens, "cu_seqlens", torch.int32, 1)
    _dev_tensor(context_lens, "context_lens", torch.int32, 1)
    B = context_lens.shape[0]
    _req(cu_seqlens.shape[0] == B + 1, "cu_seqlens must have num_seqs + 1 entries")
    _req(block_table.shape[0] == B, "block_table must have num_seqs rows")
    if out is None:
        out = torch.empty(num_tokens, dtype=torch.int32, device=block_table.device)
    _dev_tensor(out, "out", torch.int32, 1)
    _req(out.shape[0] == num_tokens, "out must have num_tokens entries")
    _check(lib.pa_slot_mapping(block_table.data_ptr(), cu_seqlens.data_ptr(), context_lens.data_ptr(),
                               out.data_ptr(), B, num_tokens, int(block_size), block_table.shape[1],
                               _stream(block_table)))
    return out


def _scales(k_scale, v_scale, H: int, device):
    _req(k_scale is not None and v_scale is not None, "fp8 (uint8) pools need k_scale and v_scale")
    for name, t in (("k_scale", k_scale), ("v_scale", v_scale)):
        _dev_tensor(t, name, torch.float32, 1)
        _req(t.shape[0] == H and t.device == device, f"{name} must be float32 [num_kv_heads] on the pools' device")


def reshape_and_cache(k: torch.Tensor, v: torch.Tensor, slot_mapping: torch.Tensor,
                      k_cache: torch.Tensor, v_cache: torch.Tensor, k_scale: torch.Tensor | None = None,
                      v_scale: torch.Tensor | None = None) -> None:
    """Scatter ``k``, ``v`` ``[T, H_kv, D]`` into the pools ``[N, P, H_kv, D]`` in place.
    uint8 pools hold fp8 (OCP E4M3) codes: the values are divided by the
    per-KV-head ``k_scale``/``v_scale`` (float32 ``[H_kv]``) and quantised
    (see ``pa_reshape_and_cache_fp8``)."""
    lib = load_library()
    for name, t in (("k", k), ("v", v)):
        _dev_tensor(t, name, dim=3)
    for name, t in (("k_cache", k_cache), ("v_cache", v_cache)):
        _dev_tensor(t, name, dim=4)
    _dev_tensor(slot_mapping, "slot_mapping", torch.int32, 1)
    T, H, D = k.shape
    N, P, H2, D2 = k_cache.shape
    _req(v.shape == k.shape, "k and v must have the same shape")
    _req(v_cache.shape == k_cache.shape, "k_cache and v_cache must have the same shape")
    _req((H, D) == (H2, D2), "k rows and cache rows differ in [H_kv, D]")
    _req(slot_mapping.shape[0] == T, "slot_mapping must have one entry per token")
    if k_cache.dtype == torch.uint8:
        _req(v_cache.dtype == torch.uint8, "k_cache and v_cache must share a dtype")
        _req(k.dtype == v.dtype, "k and v must share a dtype")
        _scales(k_scale, v_scale, H, k_cache.device)
        _check(lib.pa_reshape_and_cache_fp8(k.data_ptr(), v.data_ptr(), slot_mapping.data_ptr(), k_cache.data_ptr(),
                                            v_cache.data_ptr(), k_scale.data_ptr(), v_scale.data_ptr(), T, N, P, H, D,
                                            _dtype_code(k), _stream(k)))
        return
    _req(len({k.dtype, v.dtype, k_cache.dtype, v_cache.dtype}) == 1, "k, v and the caches must share a dtype")
    _check(lib.pa_reshape_and_cache(k.data_ptr(), v.data_ptr(), slot_mapping.data_ptr(), k_cache.data_ptr(),
                                    v_cache.data_ptr(), T, N, P, H, D, _dtype_code(k), _stream(k)))


def copy_blocks(k_cache: torch.Tensor, v_cache: torch.Tensor, block_mapping: torch.Tensor) -> None:
    """Copy-on-write block copy: for each row ``(src, dst)`` of the int32
    ``[n, 2]`` ``block_mapping``, block ``dst`` of both pools becomes a copy of
    block ``src`` (see ``pa_copy_blocks``)."""
    lib = load_library()
    for name, t in (("k_cache", k_cache), ("v_cache", v_cache)):
        _dev_tensor(t, name, dim=4)
    _dev_tensor(block_mapping, "block_mapping", torch.int32, 2)
    _req(block_mapping.shape[1] == 2, "block_mapping must be [num_pairs, 2]")
    _req(v_cache.shape == k_cache.shape and v_cache.dtype == k_cache.dtype, "k_cache and v_cache must match")
    N, P, H, D = k_cache.shape
    code = 2 if k_cache.dtype == torch.uint8 else _dtype_code(k_cache)  # uint8: fp8 codes
    _check(lib.pa_copy_blocks(k_cache.data_ptr(), v_cache.data_ptr(), block_mapping.data_ptr(),
                              block_mapping.shape[0], N, P, H, D, code, _stream(k_cache)))


def hbm_read(buf: torch.Tensor, sink: torch.Tensor, num_workgroups: int) -> None:
    """Measurement aid (see ``pa_hbm_read``): streams every byte of the
    contiguous device tensor ``buf`` (its size a multiple of 16 bytes) from
    HBM, storing nothing of consequence to the one-element int32 ``sink``."""
    lib = load_library()
    _dev_tensor(buf, "buf")
    _dev_tensor(sink, "sink", torch.int32)
    _req(sink.numel() >= 1, "sink must hold at least one element")
    _check(lib.pa_hbm_read(buf.data_ptr(), buf.numel() * buf.element_size(), sink.data_ptr(), int(num_workgroups),
                           _stream(buf)))


CHECK_RULES = {1: "context_lens out of range", 2: "block id out of range", 4: "cu_seqlens malformed",
               8: "chunk longer than its context", 16: "slot out of range"}


def check_metadata(block_table: torch.Tensor, context_lens: torch.Tensor, num_blocks: int, block_size: int,
                   cu_seqlens: torch.Tensor | None = None, slot_mapping: torch.Tensor | None = None,
                   num_tokens: int | None = None) -> tuple[int, int]:
    """Checks device metadata (see ``pa_check_metadata``); synchronises and
    returns ``(mask of violated rules, offending entries)``; ``(0, 0)`` when valid."""
    lib = load_library()
    _dev_tensor(block_table, "block_table", torch.int32, 2)
    _dev_tensor(context_lens, "context_lens", torch.int32, 1)
    B = context_lens.shape[0]
    _req(block_table.shape[0] == B, "block_table must have one row per sequence")
    if cu_seqlens is not None:
        _dev_tensor(cu_seqlens, "cu_seqlens", torch.int32, 1)
        _req(cu_seqlens.shape[0] == B + 1, "cu_seqlens must have num_seqs + 1 entries")
    if slot_mapping is not None:
        _dev_tensor(slot_mapping, "slot_mapping", torch.int32, 1)
    if num_tokens is None:
        _req(cu_seqlens is None or slot_mapping is not None, "pass num_tokens (cu_seqlens[-1]) with cu_seqlens")
        num_tokens = slot_mapping.shape[0] if slot_mapping is not None else 0
    result = torch.empty(2, dtype=torch.int32, device=block_table.device)
    _check(lib.pa_check_metadata(block_table.data_ptr(), context_lens.data_ptr(),
                                 cu_seqlens.data_ptr() if cu_seqlens is not None else None,
                                 slot_mapping.data_ptr() if slot_mapping is not None else None, B, num_tokens,
                                 int(num_blocks), int(block_size), block_table.shape[1], result.data_ptr(),
                                 _stream(block_table)))
    mask, count = result.cpu().tolist()
    return int(mask), int(count)


def _attn_common(q, k_cache, v_cache, block_table, context_lens, out):
    _dev_tensor(q, "q", dim=3)
    _dev_tensor(out, "out", dim=3)
    _dev_tensor(k_cache, "k_cache", dim=4)
    _dev_tensor(v_cache, "v_cache", dim=4)
    _dev_tensor(block_table, "block_table", torch.int32, 2)
    _dev_tensor(context_lens, "context_lens", torch.int32, 1)
    _req(out.shape == q.shape and out.dtype == q.dtype, "out must match q in shape and dtype")
    _req(out.data_ptr() != q.data_ptr(), "out must not alias q")
    _req(k_cache.shape == v_cache.shape, "k_cache and v_cache must have the same shape")
    if k_cache.dtype == torch.uint8:
        _req(v_cache.dtype == torch.uint8 and q.dtype == torch.bfloat16, "fp8 (uint8) pools take a bfloat16 q")
    else:
        _req(len({q.dtype, k_cache.dtype, v_cache.dtype}) == 1, "q and the caches must share a dtype")
    _req(q.shape[2] == k_cache.shape[3], "head_dim of q and of the caches differ")
    B = context_lens.shape[0]
    _req(block_table.shape[0] == B, "block_table must have one row per sequence")
    return B


def paged_decode_attention(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                           block_table: torch.Tensor, context_lens: torch.Tensor, scale: float,
                           out: torch.Tensor, k_scale: torch.Tensor | None = None,
                           v_scale: torch.Tensor | None = None,
                           workspace: torch.Tensor | None = None) -> torch.Tensor:
    """Decode attention: ``q``/``out`` ``[B, H_q, D]``; see ``pa_paged_decode_attention``.
    uint8 pools hold fp8 (OCP E4M3) codes with per-KV-head scales
    (``pa_paged_decode_attention_fp8``; q and out bfloat16).
    ``workspace``, if given, is a caller-owned uint8 device tensor at least the
    call's workspace size; otherwise the stream's cached workspace is used."""
    lib = load_library()
    B = _attn_common(q, k_cache, v_cache, block_table, context_lens, out)
    _req(q.shape[0] == B, "q must have one row per sequence")
    N, P, Hkv, D = k_cache.shape
    Hq = q.shape[1]
    M = block_table.shape[1]
    stream = _stream(q)
    need = decode_workspace_size(B, Hq, D, P, M)
    ws = _workspace(q.device, stream, need, workspace)
    if k_cache.dtype == torch.uint8:
        _scales(k_scale, v_scale, Hkv, k_cache.device)
        _check(lib.pa_paged_decode_attention_fp8(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
                                                 k_scale.data_ptr(), v_scale.data_ptr(), block_table.data_ptr(),
                                                 context_lens.data_ptr(), float(scale), out.data_ptr(), B, Hq, Hkv,
                                                 D, P, N, M, ws.data_ptr(), ws.numel(), stream))
        return out
    _check(lib.pa_paged_decode_attention(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
                                         block_table.data_ptr(), context_lens.data_ptr(), float(scale),
                                         out.data_ptr(), B, Hq, Hkv, D, P, N, M, _dtype_code(q),
                                         ws.data_ptr(), ws.numel(), stream))
    return out


def paged_decode_attention_noalloc(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                                   block_table: torch.Tensor, context_lens: torch.Tensor, scale: float,
                                   out: torch.Tensor) -> torch.Tensor:
    """``paged_decode_attention`` for callers that cannot allocate: the
    workspace is the library's static device array (see
    ``pa_paged_decode_attention_noalloc``), so this call allocates no device
    memory.  float32 or bfloat16 pools.  Calls that may overlap on one GPU race."""
    lib = load_library()
    B = _attn_common(q, k_cache, v_cache, block_table, context_lens, out)
    _req(q.shape[0] == B, "q must have one row per sequence")
    _req(k_cache.dtype != torch.uint8, "the allocation-free call takes float32 or bfloat16 pools")
    N, P, Hkv, D = k_cache.shape
    _check(lib.pa_paged_decode_attention_noalloc(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
                                                 block_table.data_ptr(), context_lens.data_ptr(), float(scale),
                                                 out.data_ptr(), B, q.shape[1], Hkv, D, P, N, block_table.shape[1],
                                                 _dtype_code(q), _stream(q)))
    return out


def paged_decode_append(q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor, k_cache: torch.Tensor,
                        v_cache: torch.Tensor, block_table: torch.Tensor, context_lens: torch.Tensor, scale: float,
                        out: torch.Tensor, k_scale: torch.Tensor | None = None,
                        v_scale: torch.Tensor | None = None,
                        workspace: torch.Tensor | None = None) -> torch.Tensor:
    """One decode step in one call: the new tokens ``k_new``/``v_new``
    ``[B, H_kv, D]`` are written at positions ``context_lens - 1`` and attended
    to, as ``reshape_and_cache`` + ``paged_decode_attention`` would (see
    ``pa_paged_decode_append``).  uint8 pools hold fp8 (OCP E4M3) codes: the new
    rows (float32 or bfloat16) are quantised with the per-KV-head scales.
    ``workspace``, if given, is a caller-owned uint8 device tensor at least the
    call's workspace size; otherwise the stream's cached workspace is used."""
    lib = load_library()
    B = _attn_common(q, k_cache, v_cache, block_table, context_lens, out)
    _req(q.shape[0] == B, "q must have one row per sequence")
    N, P, Hkv, D = k_cache.shape
    for name, t in (("k_new", k_new), ("v_new", v_new)):
        _dev_tensor(t, name, dim=3)
        _req(tuple(t.shape) == (B, Hkv, D), f"{name} must be [num_seqs, num_kv_heads, head_dim]")
    _req(v_new.dtype == k_new.dtype, "k_new and v_new must share a dtype")
    Hq = q.shape[1]
    M = block_table.shape[1]
    stream = _stream(q)
    ws = _workspace(q.device, stream, decode_workspace_size(B, Hq, D, P, M), workspace)
    if k_cache.dtype == torch.uint8:
        _scales(k_scale, v_scale, Hkv, k_cache.device)
        _check(lib.pa_paged_decode_append_fp8(q.data_ptr(), k_new.data_ptr(), v_new.data_ptr(), k_cache.data_ptr(),
                                              v_cache.data_ptr(), k_scale.data_ptr(), v_scale.data_ptr(),
                                              block_table.data_ptr(), context_lens.data_ptr(), float(scale),
                                              out.data_ptr(), B, Hq, Hkv, D, P, N, M, _dtype_code(k_new),
                                              ws.data_ptr(), ws.numel(), stream))
        return out
    _req(k_new.dtype == k_cache.dtype, "k_new and the caches must share a dtype")
    _check(lib.pa_paged_decode_append(q.data_ptr(), k_new.data_ptr(), v_new.data_ptr(), k_cache.data_ptr(),
                                      v_cache.data_ptr(), block_table.data_ptr(), context_lens.data_ptr(),
                                      float(scale), out.data_ptr(), B, Hq, Hkv, D, P, N, M, _dtype_code(q),
                                      ws.data_ptr(), ws.numel(), stream))
    return out


def paged_prefill_attention(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, cu_seqlens: torch.Tensor,
                            block_table: torch.Tensor, context_lens: torch.Tensor, scale: float,
                            out: torch.Tensor, k_scale: torch.Tensor | None = None,
                            v_scale: torch.Tensor | None = None,
                            workspace: torch.Tensor | None = None) -> torch.Tensor:
    """Varlen / chunked prefill: ``q``/``out`` ``[T_total, H_q, D]``; ``k``, ``v`` are the
    paged pools; see ``pa_paged_prefill_attention``.  uint8 pools hold fp8
    (OCP E4M3) codes with per-KV-head scales (``pa_paged_prefill_attention_fp8``).
    ``workspace``, if given, is a caller-owned uint8 device tensor at least the
    call's workspace size; otherwise the stream's cached workspace is used."""
    lib = load_library()
    B = _attn_common(q, k, v, block_table, context_lens, out)
    _dev_tensor(cu_seqlens, "cu_seqlens", torch.int32, 1)
    _req(cu_seqlens.shape[0] == B + 1, "cu_seqlens must have num_seqs + 1 entries")
    N, P, Hkv, D = k.shape
    T, Hq, _ = q.shape
    M = block_table.shape[1]
    stream = _stream(q)
    need = prefill_workspace_size(B, T, Hq, Hkv)
    ws = _workspace(q.device, stream, need, workspace)
    if k.dtype == torch.uint8:
        _scales(k_scale, v_scale, Hkv, k.device)
        _check(lib.pa_paged_prefill_attention_fp8(q.data_ptr(), k.data_ptr(), v.data_ptr(), k_scale.data_ptr(),
                                                  v_scale.data_ptr(), cu_seqlens.data_ptr(), block_table.data_ptr(),
                                                  context_lens.data_ptr(), float(scale), out.data_ptr(), B, T, Hq,
                                                  Hkv, D, P, N, M, ws.data_ptr(), ws.numel(), stream))
        return out
    _check(lib.pa_paged_prefill_attention(q.data_ptr(), k.data_ptr(), v.data_ptr(), cu_seqlens.data_ptr(),
                                          block_table.data_ptr(), context_lens.data_ptr(), float(scale),
                                          out.data_ptr(), B, T, Hq, Hkv, D, P, N, M, _dtype_code(q),
                                          ws.data_ptr(), ws.numel(), stream))
    return out


def paged_mixed_attention(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, cu_seqlens: torch.Tensor,
                          block_table: torch.Tensor, context_lens: torch.Tensor, scale: float,
                          out: torch.Tensor, k_scale: torch.Tensor | None = None,
                          v_scale: torch.Tensor | None = None,
                          workspace: torch.Tensor | None = None) -> torch.Tensor:
    """One step's ragged mix of decodes (one-token chunks) and prefill chunks in one
    persistent launch; same arguments and result as ``paged_prefill_attention``
    (see ``pa_paged_mixed_attention``).  uint8 pools hold fp8 (OCP E4M3) codes
    with per-KV-head scales (``pa_paged_mixed_attention_fp8``).
    ``workspace``, if given, is a caller-owned uint8 device tensor at least the
    call's workspace size; otherwise the stream's cached workspace is used."""
    lib = load_library()
    B = _attn_common(q, k, v, block_table, context_lens, out)
    _dev_tensor(cu_seqlens, "cu_seqlens", torch.int32, 1)
    _req(cu_seqlens.shape[0] == B + 1, "cu_seqlens must have num_seqs + 1 entries")
    N, P, Hkv, D = k.shape
    T, Hq, _ = q.shape
    M = block_table.shape[1]
    stream = _stream(q)
    ws = _workspace(q.device, stream, mixed_workspace_size(B, Hq, D, P, M), workspace)
    if k.dtype == torch.uint8:
        _scales(k_scale, v_scale, Hkv, k.device)
        _check(lib.pa_paged_mixed_attention_fp8(q.data_ptr(), k.data_ptr(), v.data_ptr(), k_scale.data_ptr(),
                                                v_scale.data_ptr(), cu_seqlens.data_ptr(), block_table.data_ptr(),
                                                context_lens.data_ptr(), float(scale), out.data_ptr(), B, T, Hq,
                                                Hkv, D, P, N, M, ws.data_ptr(), ws.numel(), stream))
        return out
    _check(lib.pa_paged_mixed_attention(q.data_ptr(), k.data_ptr(), v.data_ptr(), cu_seqlens.data_ptr(),
                                        block_table.data_ptr(), context_lens.data_ptr(), float(scale),
                                        out.data_ptr(), B, T, Hq, Hkv, D, P, N, M, _dtype_code(q),
                                        ws.data_ptr(), ws.numel(), stream))
    return out


GAVE_UP = {1: "a decode work queue was given up", 2: "a prefill work queue of the mixed call was given up"}


def workspace_status(workspace: torch.Tensor | None = None, device=None, noalloc: bool = False) -> int:
    """Bits of the workspace's status word (see ``pa_workspace_status``),
    gathered since the previous query; the word is cleared.  ``workspace``
    defaults to the cached workspace of ``device``'s current stream; with
    ``noalloc`` the static scratch of ``paged_decode_attention_noalloc`` is
    read.  Synchronises the stream."""
    lib = load_library()
    dev = torch.device("cuda", torch.cuda.current_device()) if device is None else torch.device(device)
    stream = torch.cuda.current_stream(dev).cuda_stream
    if noalloc:
        ptr = None
    else:
        if workspace is None:
            workspace = _workspaces.get((dev.index, stream))
            _req(workspace is not None, "no cached workspace on this stream yet")
        _dev_tensor(workspace, "workspace", torch.uint8)
        ptr = workspace.data_ptr()
    result = torch.empty(1, dtype=torch.int32, device=dev)
    _check(lib.pa_workspace_status(ptr, result.data_ptr(), stream))
    return int(result.item())


@contextlib.contextmanager
def kernel_timer(start: "torch.cuda.Event", stop: "torch.cuda.Event"):
    """While active, each attention call records ``start``/``stop`` around its
    main kernel on its stream (``pa_set_timing_events``).  The events must have
    been created (recorded once) before."""
    lib = load_library()
    _req(start.cuda_event != 0 and stop.cuda_event != 0, "record the events once before use")
    lib.pa_set_timing_events(start.cuda_event, stop.cuda_event)
    try:
        yield
    finally:
        lib.pa_set_timing_events(None, None)
