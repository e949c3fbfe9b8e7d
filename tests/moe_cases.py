"""Helpers for the GPU parity tests: device layers built from the seeded generators, the
matching oracle inputs, and the acceptance check.

Acceptance (per token, per tensor): routing indices equal exactly; every floating-point
output satisfies max|gpu - oracle| <= 2e-3 * ||oracle||_2 / sqrt(n).
"""
from __future__ import annotations

from typing import Optional

import numpy as np

import oracle
import synth
from synth.device import DeviceLayer, act_f64, act_tensor, build_layer, to_bf16_tensor  # noqa: F401

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


def oracle_layer(wl: synth.Workload, layer_id: int = 0) -> oracle.LayerWeights:
    return oracle.workload_layer(wl, layer_id)


def small_workload(name: str, seed: int, H: int, I: int, E: int, K: int, bits: int = 4, tiered: bool = False,
                   n_hot: int = 0, zipf: bool = False, router_bf16: bool = True, x_bf16: bool = True,
                   norm: bool = False, n_layers: int = 1) -> synth.Workload:
    return synth.Workload(name, 1000, H, I, E, K, n_layers=n_layers, bits_default=bits, tiered=tiered,
                          zipf=zipf, router_bf16=router_bf16, x_bf16=x_bf16, norm=norm, n_hot=n_hot,
                          seed_override=seed)
