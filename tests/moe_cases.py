"""Helpers for the GPU parity tests: device layers built from the seeded generators, the
matching oracle inputs, and the acceptance check.

Acceptance (per token, per tensor): routing indices equal exactly; every floating-point
output satisfies max|gpu - oracle| <= 2e-3 * ||oracle||_2 / sqrt(n).
"""
from __future__ import annotations

import functools
from dataclasses import dataclass, field, replace
from typing import Dict, List, Optional

import numpy as np
import torch

import bit_expert_dequant_amd as M
import oracle
import synth

REL_TOL = 2e-3
MIN_MARGIN = 1e-4      # routing margins below this are reported, never silently accepted


def max_err_ok(gpu: np.ndarray, ref: np.ndarray, rel: float = REL_TOL):
    gpu = np.asarray(gpu, dtype=np.float64).reshape(-1)
    ref = np.asarray(ref, dtype=np.float64).reshape(-1)
    bound = rel * np.linalg.norm(ref) / np.sqrt(ref.size)
    err = np.abs(gpu - ref).max() if ref.size else 0.0
    return err <= bound, err, bound


def assert_close(gpu, ref, what: str, rel: float = REL_TOL):
    ok, err, bound = max_err_ok(gpu, ref, rel)
    assert ok, f"{what}: max abs err {err:.3e} > bound {bound:.3e}"


def to_bf16_tensor(u16: np.ndarray, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(u16).view(np.int16)).to(device).view(torch.bfloat16)


def act_tensor(wl: synth.Workload, bank: np.ndarray, device="cuda") -> torch.Tensor:
    if wl.x_bf16:
        return to_bf16_tensor(bank, device)
    return torch.from_numpy(np.ascontiguousarray(bank)).to(device)


def act_f64(wl: synth.Workload, bank: np.ndarray) -> np.ndarray:
    return (synth.bf16_to_f32(bank) if wl.x_bf16 else bank).astype(np.float64)


@dataclass
class DeviceLayer:
    wl: synth.Workload
    layer_id: int
    store: torch.Tensor           # all expert blobs of the layer, `stride` bytes apart
    stride: int
    table: torch.Tensor
    router: torch.Tensor
    logit_bias: Optional[torch.Tensor]
    norm_w: Optional[torch.Tensor]
    L: M.Layer

    def expert_ptr(self, e: int) -> int:
        return self.store.data_ptr() + e * self.stride


def build_layer(wl: synth.Workload, layer_id: int = 0, host_blobs: Optional[bool] = None,
                device="cuda") -> DeviceLayer:
    """Expert blobs on the device (host-generated and copied for small stores, written by the
    device filler otherwise), descriptor table, router, bias, norm weight."""
    bits = wl.expert_bits()
    stride = wl.blob_bytes(int(bits.max()))
    store = torch.empty(wl.E * stride, dtype=torch.uint8, device=device)
    if host_blobs is None:
        host_blobs = wl.E * stride <= (64 << 20)
    if host_blobs:
        host = np.zeros((wl.E, stride), dtype=np.uint8)
        for e in range(wl.E):
            b = wl.blob(layer_id, e)
            host[e, :b.size] = b
        store.copy_(torch.from_numpy(host.reshape(-1)))
    else:
        stream = torch.cuda.current_stream().cuda_stream
        if (bits == bits[0]).all():
            synth.fill_blobs_device(store.data_ptr(), stride, wl.E, 0, layer_id, wl.seed, wl.H, wl.I,
                                    int(bits[0]), stream)
        else:
            for e in range(wl.E):
                synth.fill_blobs_device(store.data_ptr() + e * stride, stride, 1, e, layer_id, wl.seed, wl.H,
                                        wl.I, int(bits[e]), stream)
    ptrs = [store.data_ptr() + e * stride for e in range(wl.E)]
    table = M.expert_table(ptrs, bits.tolist(), device)
    r = wl.router(layer_id)
    router = to_bf16_tensor(r, device) if wl.router_bf16 else torch.from_numpy(r).to(device)
    lb = wl.logit_bias()
    logit_bias = None if lb is None else torch.from_numpy(lb).to(device)
    nw = wl.norm_w(layer_id)
    norm_w = None if nw is None else to_bf16_tensor(nw, device)
    L = M.Layer(router, table, logit_bias, norm_w, wl.norm_eps)
    return DeviceLayer(wl, layer_id, store, stride, table, router, logit_bias, norm_w, L)


@functools.lru_cache(maxsize=512)
def _cached_blob(seed, layer, e, H, I, bits) -> np.ndarray:
    return synth.expert_blob(seed, layer, e, H, I, bits)


def oracle_layer(wl: synth.Workload, layer_id: int = 0) -> oracle.LayerWeights:
    bits = wl.expert_bits()
    return oracle.LayerWeights(
        router=wl.router(layer_id), router_is_bf16=wl.router_bf16,
        blob=lambda e: _cached_blob(wl.seed, layer_id, int(e), wl.H, wl.I, int(bits[e])),
        bits=lambda e: int(bits[e]),
        logit_bias=wl.logit_bias(), norm_w=wl.norm_w(layer_id), norm_eps=wl.norm_eps)


def small_workload(name: str, seed: int, H: int, I: int, E: int, K: int, bits: int = 4, tiered: bool = False,
                   n_hot: int = 0, zipf: bool = False, router_bf16: bool = True, x_bf16: bool = True,
                   norm: bool = False, n_layers: int = 1) -> synth.Workload:
    return synth.Workload(name, 1000, H, I, E, K, n_layers=n_layers, bits_default=bits, tiered=tiered,
                          zipf=zipf, router_bf16=router_bf16, x_bf16=x_bf16, norm=norm, n_hot=n_hot,
                          seed_override=seed)
