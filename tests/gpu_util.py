"""Helpers for the GPU parity tests: move a seeded case to the device, write it
into a NaN-filled pool through the HIP path, and compare with the oracle."""

from __future__ import annotations

import numpy as np
import torch

import paged_kv_cache_48_amd as pa
from oracle import ref_decode, ref_dequantize, ref_reshape_and_cache, ref_slot_mapping, widen
from workloads import nan_pool

DEV = "cuda:0"

# tolerances on |got - ref|: fp32 inputs 1e-4 absolute; bf16 inputs 1e-2 + 2e-2 * |ref|
TOL = {"f32": (1e-4, 0.0), "bf16": (1e-2, 2e-2)}


def to_dev(x: np.ndarray, dtype: str) -> torch.Tensor:
    """Host bits/values -> device tensor with identical bits."""
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to(DEV).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(DEV)


def to_host_bits(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def idx(x) -> torch.Tensor:
    return torch.as_tensor(np.asarray(x, dtype=np.int32)).to(DEV)


def dev_nan_pool(case) -> torch.Tensor:
    shape = (case.num_blocks, case.block_size, case.num_kv_heads, case.head_dim)
    if case.dtype == "bf16":
        return torch.full(shape, 0x7FC0, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    return torch.full(shape, 0x7FC00000, dtype=torch.int32, device=DEV).view(torch.float32)


class DevCase:
    """A case on the device, its pool written through the HIP path:
    the cached prefix first, then this step's new tokens."""

    def __init__(self, case, block_table=None):
        self.case = case
        self.bt_np = case.block_table if block_table is None else block_table
        self.bt = idx(self.bt_np)
        self.lens = idx(case.context_lens)
        self.cu = idx(case.cu_seqlens)
        self.q = to_dev(case.q, case.dtype)
        self.kc = dev_nan_pool(case)
        self.vc = dev_nan_pool(case)
        kp, vp, cu_pre, lens_pre = case.prefix()
        if len(kp):
            slots = pa.slot_mapping(self.bt, idx(cu_pre), idx(lens_pre), case.block_size, len(kp))
            pa.reshape_and_cache(to_dev(kp, case.dtype), to_dev(vp, case.dtype), slots, self.kc, self.vc)
        kn, vn = case.new_kv()
        self.k_new = to_dev(kn, case.dtype)
        self.v_new = to_dev(vn, case.dtype)
        self.slots = pa.slot_mapping(self.bt, self.cu, self.lens, case.block_size, case.T_total)
        pa.reshape_and_cache(self.k_new, self.v_new, self.slots, self.kc, self.vc)

    def decode(self, out=None):
        c = self.case
        out = torch.empty_like(self.q) if out is None else out
        pa.paged_decode_attention(self.q, self.kc, self.vc, self.bt, self.lens, c.scale, out)
        return out

    def prefill(self, out=None):
        c = self.case
        out = torch.empty_like(self.q) if out is None else out
        pa.paged_prefill_attention(self.q, self.kc, self.vc, self.cu, self.bt, self.lens, c.scale, out)
        return out


def oracle_pool(case, block_table=None):
    """The oracle's pool after the same two writes (its own slot math and scatter)."""
    bt = case.block_table if block_table is None else block_table
    kc = nan_pool(case.num_blocks, case.block_size, case.num_kv_heads, case.head_dim, case.dtype)
    vc = kc.copy()
    kp, vp, cu_pre, lens_pre = case.prefix()
    if len(kp):
        kc, vc = ref_reshape_and_cache(kp, vp, ref_slot_mapping(bt, cu_pre, lens_pre, case.block_size), kc, vc)
    kn, vn = case.new_kv()
    slots = ref_slot_mapping(bt, case.cu_seqlens, case.context_lens, case.block_size)
    return ref_reshape_and_cache(kn, vn, slots, kc, vc)


def assert_close(got: torch.Tensor, ref: np.ndarray, dtype: str, what: str = "", rows=None):
    """Element-wise tolerance check of device output ``got`` against fp64 ``ref``
    (only the leading-index rows in ``rows``, if given)."""
    g = widen(to_host_bits(got))
    if rows is not None:
        g, ref = g[rows], ref[rows]
    atol, rtol = TOL[dtype]
    err = np.abs(g - ref)
    bound = atol + rtol * np.abs(ref)
    bad = ~(err <= bound)
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError(
            f"{what}: {int(bad.sum())} of {bad.size} elements outside tolerance; first at {tuple(i)}: "
            f"got {g[tuple(i)]!r}, ref {ref[tuple(i)]!r}; max err {float(np.nanmax(err))}"
        )
    return float(err.max()) if err.size else 0.0


def fp8_scales(H, seed, lo=0.004, hi=0.03):
    return np.random.default_rng(seed).uniform(lo, hi, H).astype(np.float32)


class Fp8Case:
    """A case's pools written as fp8 through the HIP path (prefix, then new tokens)."""

    def __init__(self, c, ks, vs):
        self.case, self.ks, self.vs = c, ks, vs
        shape = (c.num_blocks, c.block_size, c.num_kv_heads, c.head_dim)
        # unwritten slots hold the largest code (448): a masking mistake would show
        self.kc = torch.full(shape, 0x7E, dtype=torch.uint8, device=DEV)
        self.vc = torch.full(shape, 0x7E, dtype=torch.uint8, device=DEV)
        self.dks, self.dvs = torch.from_numpy(ks).to(DEV), torch.from_numpy(vs).to(DEV)
        self.bt, self.lens, self.cu = idx(c.block_table), idx(c.context_lens), idx(c.cu_seqlens)
        kp, vp, cu_pre, lens_pre = c.prefix()
        if len(kp):
            sl = pa.slot_mapping(self.bt, idx(cu_pre), idx(lens_pre), c.block_size, len(kp))
            pa.reshape_and_cache(to_dev(kp, c.dtype), to_dev(vp, c.dtype), sl, self.kc, self.vc, self.dks, self.dvs)
        kn, vn = c.new_kv()
        sl = pa.slot_mapping(self.bt, idx(c.cu_seqlens), self.lens, c.block_size, c.T_total)
        pa.reshape_and_cache(to_dev(kn, c.dtype), to_dev(vn, c.dtype), sl, self.kc, self.vc, self.dks, self.dvs)
        self.q = to_dev(c.q, c.dtype)

    def decode(self, q=None, bt=None, lens=None):
        q = self.q if q is None else q
        out = torch.empty_like(q)
        pa.paged_decode_attention(q, self.kc, self.vc, self.bt if bt is None else bt,
                                  self.lens if lens is None else lens, self.case.scale, out, self.dks, self.dvs)
        return out

    def reference(self, select=None):
        c = self.case
        kc, vc = self.kc.cpu().numpy(), self.vc.cpu().numpy()
        return ref_decode(c.q, ref_dequantize(kc, self.ks), ref_dequantize(vc, self.vs), c.block_table,
                          c.context_lens, c.scale, select=select)
