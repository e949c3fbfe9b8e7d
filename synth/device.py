"""Device-resident copies of the seeded workloads: expert stores, descriptor tables, routers and
activation banks as torch tensors, wrapped in the library's layer struct.

Input plumbing only (no arithmetic of the method): the benchmark and the GPU tests both build their
layers here.  Expert stores of up to 64 MiB are generated on the host and copied; larger ones are
written on the device by the seeded filler, byte-identical to the host generator."""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np

from . import Workload, bf16_to_f32, fill_blobs_device


def to_bf16_tensor(u16: np.ndarray, device="cuda"):
    """bf16 bits (uint16 array) as a torch bfloat16 tensor on `device`."""
    import torch
    return torch.from_numpy(np.ascontiguousarray(u16).view(np.int16)).to(device).view(torch.bfloat16)


def act_tensor(wl: Workload, bank: np.ndarray, device="cuda"):
    """A slice of the workload's token bank (bf16 bits or fp32) as a device tensor."""
    import torch
    if wl.x_bf16:
        return to_bf16_tensor(bank, device)
    return torch.from_numpy(np.ascontiguousarray(bank)).to(device)


def act_f64(wl: Workload, bank: np.ndarray) -> np.ndarray:
    """The same tokens as float64 values (what the oracle consumes)."""
    return (bf16_to_f32(bank) if wl.x_bf16 else bank).astype(np.float64)


@dataclass
class DeviceLayer:
    wl: Workload
    layer_id: int
    store: object                 # torch uint8 tensor: all expert blobs, `stride` bytes apart
    stride: int
    table: object                 # device moe_expert_desc [E]
    router: object
    logit_bias: Optional[object]
    norm_w: Optional[object]
    L: object                     # bit_expert_dequant_amd.Layer

    def expert_ptr(self, e: int) -> int:
        return self.store.data_ptr() + e * self.stride


def build_layer(wl: Workload, layer_id: int = 0, host_blobs: Optional[bool] = None,
                device="cuda") -> DeviceLayer:
    """Expert blobs on the device (host-generated and copied for small stores, written by the
    device filler otherwise), descriptor table, router, bias, norm weight."""
    import torch

    import bit_expert_dequant_amd as M
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
            fill_blobs_device(store.data_ptr(), stride, wl.E, 0, layer_id, wl.seed, wl.H, wl.I, int(bits[0]), stream)
        else:
            for e in range(wl.E):
                fill_blobs_device(store.data_ptr() + e * stride, stride, 1, e, layer_id, wl.seed, wl.H, wl.I,
                                  int(bits[e]), stream)
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
