"""Seeded synthetic inputs shared by the oracle-side tests and the GPU path.

Holds none of the MoE arithmetic: only random draws and the placement of those draws in
the documented packed byte format.  Two generators are used:

* Counter-based SplitMix64 (Steele, Lea & Flood, "Fast splittable pseudorandom number
  generators", OOPSLA 2014): word i of a stream with key k is mix64(k + (i+1)*gamma).
  It fills the large packed expert blobs.  The same definition is implemented on the
  device in ``synth_fill.hip`` so that a store too large for host memory can be written
  on the GPU while the host regenerates, byte for byte, any expert the oracle needs.
* numpy's PCG64 (``default_rng``) for the small dense inputs: router weights, token
  activations, RMSNorm weights, Zipf priors.  Those are generated on the host only and
  copied to the device.

Distributions (per the workload description): codes uniform over 0..2^bits-1 (uniform
random bytes), scales U(0.002, 0.02) and biases U(-0.1, 0.1) rounded to bf16, router
weights N(0, 0.02), activations N(0, 1), RMSNorm weights 1 + N(0, 0.02).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass, field
from typing import Dict, List, Optional

import numpy as np

MASK64 = (1 << 64) - 1
GAMMA = 0x9E3779B97F4A7C15
GROUP = 64

# Tensor ids inside one expert blob (also the order of the planes).
T_GATE_CODES, T_GATE_SB, T_UP_CODES, T_UP_SB, T_DOWN_CODES, T_DOWN_SB = range(6)

# Affine maps for the (scale, bias) draws: value = lo + span * u, u = k * 2^-24.
SCALE_LO, SCALE_SPAN = np.float32(0.002), np.float32(0.018)
BIAS_LO, BIAS_SPAN = np.float32(-0.1), np.float32(0.2)

# Zipf(1.1) prior strength.  Chosen so that the 128 highest-prior experts receive about
# 70% of the top-4 selections of the seeded token bank at the 4096 x 512 shape; the value
# is reproduced by oracle/calibrate_zipf.py (which calls only the oracle).
ZIPF_S = 1.1
ZIPF_BETA = 0.40
N_HOT = 128


def config_seed(c: int) -> int:
    return 0x5EED0000 + c


# ----------------------------------------------------------------------------- SplitMix64
def _mix64_int(z: int) -> int:
    z &= MASK64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & MASK64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & MASK64
    return z ^ (z >> 31)


def _mix64(z: np.ndarray) -> np.ndarray:
    z = z.astype(np.uint64, copy=True)
    with np.errstate(over="ignore"):
        z ^= z >> np.uint64(30)
        z *= np.uint64(0xBF58476D1CE4E5B9)
        z ^= z >> np.uint64(27)
        z *= np.uint64(0x94D049BB133111EB)
        z ^= z >> np.uint64(31)
    return z


def stream_key(seed: int, layer: int, expert: int, tensor: int) -> int:
    """Key of the SplitMix64 stream for one tensor of one expert of one layer."""
    assert 0 <= layer < (1 << 32) and 0 <= expert < (1 << 24) and 0 <= tensor < 256
    return _mix64_int(_mix64_int(seed) ^ ((layer << 32) | (expert << 8) | tensor))


def words(key: int, start: int, count: int) -> np.ndarray:
    """Words start..start+count-1 of the stream: mix64(key + (i+1)*gamma)."""
    i = np.arange(start + 1, start + count + 1, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = np.uint64(key) + i * np.uint64(GAMMA)
    return _mix64(z)


def random_bytes(key: int, nbytes: int) -> np.ndarray:
    """Byte j is byte (j mod 8) (little-endian) of word j // 8."""
    w = words(key, 0, (nbytes + 7) // 8)
    return w.view(np.uint8)[:nbytes].copy()


def f32_to_bf16_rne(f: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even of float32 to bf16 bits (finite inputs)."""
    u = np.ascontiguousarray(f, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return u.astype(np.uint16)


def bf16_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def sb_pairs(key: int, npairs: int) -> np.ndarray:
    """(scale, bias) bf16 pairs [npairs, 2] from one stream: the high 24 bits of a word
    give the scale draw, the low 24 bits the bias draw; all steps in float32."""
    w = words(key, 0, npairs)
    hi = (w >> np.uint64(40)).astype(np.float32) * np.float32(2.0 ** -24)
    lo = (w & np.uint64(0xFFFFFF)).astype(np.float32) * np.float32(2.0 ** -24)
    scale = (hi * SCALE_SPAN).astype(np.float32) + SCALE_LO
    bias = (lo * BIAS_SPAN).astype(np.float32) + BIAS_LO
    out = np.empty((npairs, 2), dtype=np.uint16)
    out[:, 0] = f32_to_bf16_rne(scale.astype(np.float32))
    out[:, 1] = f32_to_bf16_rne(bias.astype(np.float32))
    return out


# ----------------------------------------------------------------------------- blob format
def _r256(v: int) -> int:
    return (v + 255) & ~255


def plane_sizes(H: int, I: int, bits: int) -> List[int]:
    cin, sbin = I * H * bits // 8, I * (H // GROUP) * 4
    cout, sbout = H * I * bits // 8, H * (I // GROUP) * 4
    return [cin, sbin, cin, sbin, cout, sbout]


def blob_layout(H: int, I: int, bits: int):
    off, p = [], 0
    for s in plane_sizes(H, I, bits):
        off.append(p)
        p = _r256(p + s)
    return off, p


def expert_blob(seed: int, layer: int, expert: int, H: int, I: int, bits: int) -> np.ndarray:
    """Packed expert blob with uniform codes and seeded (scale, bias) planes."""
    off, tot = blob_layout(H, I, bits)
    sizes = plane_sizes(H, I, bits)
    blob = np.zeros(tot, dtype=np.uint8)
    for t in range(6):
        key = stream_key(seed, layer, expert, t)
        if t % 2 == 0:
            blob[off[t]:off[t] + sizes[t]] = random_bytes(key, sizes[t])
        else:
            blob[off[t]:off[t] + sizes[t]] = sb_pairs(key, sizes[t] // 4).reshape(-1).view(np.uint8)
    return blob


# ----------------------------------------------------------------------------- dense inputs
def normal_bf16(rng: np.random.Generator, shape, std: float, mean: float = 0.0) -> np.ndarray:
    return f32_to_bf16_rne((rng.standard_normal(shape) * std + mean).astype(np.float32))


def router_weights(seed: int, layer: int, E: int, H: int, bf16: bool) -> np.ndarray:
    rng = np.random.default_rng([seed, layer, 1])
    if bf16:
        return normal_bf16(rng, (E, H), 0.02)
    return (rng.standard_normal((E, H)) * 0.02).astype(np.float32)


def norm_weights(seed: int, layer: int, H: int) -> np.ndarray:
    rng = np.random.default_rng([seed, layer, 2])
    return normal_bf16(rng, (H,), 0.02, 1.0)


def token_bank(seed: int, n: int, H: int, bf16: bool) -> np.ndarray:
    """[n, H] activations: bf16 bits (uint16) or float32."""
    rng = np.random.default_rng([seed, 0xB00C])
    if bf16:
        return normal_bf16(rng, (n, H), 1.0)
    return rng.standard_normal((n, H)).astype(np.float32)


def zipf_prior(seed: int, E: int, s: float = ZIPF_S):
    """(perm, p): expert perm[r] has prior rank r+1 and probability p[perm[r]] ~ (r+1)^-s."""
    rng = np.random.default_rng([seed, 0x21FF])
    perm = rng.permutation(E)
    ranks = np.arange(1, E + 1, dtype=np.float64)
    q = ranks ** (-s)
    q /= q.sum()
    p = np.empty(E)
    p[perm] = q
    return perm, p


def zipf_logit_bias(seed: int, E: int, beta: float = ZIPF_BETA) -> np.ndarray:
    _, p = zipf_prior(seed, E)
    return (beta * np.log(p)).astype(np.float32)


def hot_set(seed: int, E: int, n_hot: int = N_HOT) -> np.ndarray:
    perm, _ = zipf_prior(seed, E)
    return np.sort(perm[:n_hot])


# ----------------------------------------------------------------------------- workloads
@dataclass
class Workload:
    """One synthetic configuration: shapes, dtypes and seeds of every input."""
    name: str
    cfg: int
    H: int
    I: int
    E: int
    K: int
    n_layers: int = 1
    tokens: int = 1                 # tokens per call (1 = decode)
    bits_default: int = 4
    tiered: bool = False            # hot experts 4-bit, the rest 2-bit
    zipf: bool = False              # add the Zipf logit bias
    router_bf16: bool = True
    x_bf16: bool = True
    norm: bool = False              # RMSNorm (eps 1e-6) before each layer; residual stream
    norm_eps: float = 1e-6
    n_hot: int = N_HOT              # tiered: experts of prior rank 1..n_hot keep 4-bit codes
    seed_override: Optional[int] = None

    @property
    def seed(self) -> int:
        return self.seed_override if self.seed_override is not None else config_seed(self.cfg)

    def expert_bits(self) -> np.ndarray:
        bits = np.full(self.E, self.bits_default, dtype=np.int32)
        if self.tiered:
            bits[:] = 2
            bits[hot_set(self.seed, self.E, min(self.n_hot, self.E))] = 4
        return bits

    def blob(self, layer: int, e: int) -> np.ndarray:
        return expert_blob(self.seed, layer, e, self.H, self.I, int(self.expert_bits()[e]))

    def blob_bytes(self, bits: int) -> int:
        return blob_layout(self.H, self.I, bits)[1]

    def router(self, layer: int) -> np.ndarray:
        return router_weights(self.seed, layer, self.E, self.H, self.router_bf16)

    def logit_bias(self) -> Optional[np.ndarray]:
        return zipf_logit_bias(self.seed, self.E) if self.zipf else None

    def norm_w(self, layer: int) -> Optional[np.ndarray]:
        return norm_weights(self.seed, layer, self.H) if self.norm else None

    def tokens_bank(self, n: int) -> np.ndarray:
        return token_bank(self.seed, n, self.H, self.x_bf16)


def shared_routing(kind: str, base: np.ndarray, E: int) -> np.ndarray:
    """Routings of a few tokens for the shared-read measurements, built from the router's choice
    `base` [T][K] on the same tokens: "router" keeps it; "draft" gives every token the first token's
    first K-1 experts and one expert of its own (draft tokens of a speculative step that agree on
    most experts); "same" gives every token the first token's K experts."""
    T, K = base.shape
    if kind == "router":
        return base.astype(np.int32).copy()
    if kind not in ("draft", "same"):
        raise ValueError(f"unknown routing {kind!r}")
    shared = [int(e) for e in base[0]]
    idx = np.empty((T, K), dtype=np.int32)
    for t in range(T):
        if kind == "same":
            idx[t] = shared
            continue
        own = (shared[-1] + 37 * t) % E
        while own in shared[:-1]:
            own = (own + 1) % E
        idx[t] = shared[:-1] + [own]
    return idx


WORKLOADS: Dict[int, Workload] = {
    0: Workload("tiny: H512 I256 E8 top2, 4-bit, fp32 router and x", 0, 512, 256, 8, 2,
                router_bf16=False, x_bf16=False),
    1: Workload("one layer 4-bit: H4096 I1024 E512 top4, 1 decode token", 1, 4096, 1024, 512, 4),
    2: Workload("one layer tiered hot-4/cold-2 with Zipf(1.1) routing prior", 2, 4096, 1024, 512, 4,
                tiered=True, zipf=True),
    3: Workload("60-layer 4-bit stack, RMSNorm + residual, 1 decode token", 3, 4096, 1024, 512, 4,
                n_layers=60, norm=True),
    4: Workload("batched 256 tokens, 4-bit, Zipf(1.1) routing prior", 4, 4096, 1024, 512, 4,
                tokens=256, zipf=True),
}


# ----------------------------------------------------------------------------- device filler
_HERE = os.path.dirname(os.path.abspath(__file__))
_FILL_SRC = os.path.join(_HERE, "synth_fill.hip")
_FILL_LIB = os.path.join(_HERE, "libsynth_fill.so")
_fill = None


def build_device_filler(force: bool = True) -> str:
    if force or not os.path.exists(_FILL_LIB):
        cmd = ["hipcc", "--offload-arch=gfx950", "-O3", "-fPIC", "-shared", "-ffp-contract=off",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               _FILL_SRC, "-o", _FILL_LIB + ".tmp"]
        subprocess.check_call(cmd, stderr=subprocess.DEVNULL)
        os.replace(_FILL_LIB + ".tmp", _FILL_LIB)
    return _FILL_LIB


def _filler():
    global _fill
    if _fill is None:
        if not os.path.exists(_FILL_LIB):
            raise RuntimeError("synth device filler not built; run __graft_entry__.build()")
        L = ctypes.CDLL(_FILL_LIB)
        L.synth_fill_blobs.restype = ctypes.c_int
        L.synth_fill_blobs.argtypes = [
            ctypes.c_void_p, ctypes.c_uint64, ctypes.c_int, ctypes.c_int,   # dst, stride, n, first_expert
            ctypes.c_int, ctypes.c_uint64,                                  # layer, seed
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,              # keys_dev? (unused), off, sizes
            ctypes.c_float, ctypes.c_float, ctypes.c_float, ctypes.c_float,
            ctypes.c_void_p]
        _fill = L
    return _fill


def fill_blobs_device(dst_ptr: int, blob_stride: int, n_experts: int, first_expert: int,
                      layer: int, seed: int, H: int, I: int, bits: int, stream_ptr: int = 0) -> None:
    """Write experts first_expert..first_expert+n_experts-1 (all with the same code
    width) into device memory at dst_ptr, blob_stride bytes apart; identical bytes to
    :func:`expert_blob`."""
    off, tot = blob_layout(H, I, bits)
    assert blob_stride >= tot and blob_stride % 256 == 0
    sizes = plane_sizes(H, I, bits)
    off_a = (ctypes.c_uint64 * 6)(*off)
    size_a = (ctypes.c_uint64 * 6)(*sizes)
    rc = _filler().synth_fill_blobs(
        ctypes.c_void_p(dst_ptr), blob_stride, n_experts, first_expert, layer, seed,
        None, off_a, size_a, float(SCALE_LO), float(SCALE_SPAN), float(BIAS_LO), float(BIAS_SPAN),
        ctypes.c_void_p(stream_ptr))
    if rc != 0:
        raise RuntimeError(f"synth_fill_blobs failed: {rc}")
