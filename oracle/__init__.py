"""CPU oracle for the MoE expert path (fp32 dequantisation, fp64 accumulation).

TEST INFRASTRUCTURE ONLY: the tests, the package smoke check and the benchmark's
CPU-baseline leg use this module; the product library never imports it.  It shares no
code with the HIP library.  The arithmetic lives in ``moe_oracle.c`` (built with gcc by
:func:`build`); this wrapper marshals numpy arrays and strings the per-token steps
together in the order the method defines them:

    [RMSNorm] -> router logits -> softmax / top-K / renormalise
             -> per selected expert: gate, up, SwiGLU, down -> weighted combine [+ x]

Where the Flash-MoE pages define a step (affine dequantisation and its FMA form, the
4-/2-bit matvec kernels, two-pass RMSNorm, the weighted-sum combine: lilting.ch,
"397Bパラメータモデルを48GB MacBookで動かすFlash-MoE", section "Metal Compute Shaders")
this follows them; where they are silent it takes the plain reading written in the
header of ``moe_oracle.c``.  Beside the per-token path: quantise-from-float (``quantize``) and the
policy side of the tiered store (``expert_usage``, ``hot_order``, ``requantize_expert``) and the
replacement policy of an expert cache (``ExpertCacheModel``).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass
from typing import Callable, Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB = os.environ.get("MOE_ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")
_lib = None

GROUP = 64


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (OpenMP, no fp contraction)."""
    if force or not os.path.exists(_LIB):
        cmd = ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
               _SRC, "-o", _LIB + ".tmp", "-lm"]
        subprocess.check_call(cmd)
        os.replace(_LIB + ".tmp", _LIB)
    return _LIB


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        L = ctypes.CDLL(_LIB)
        c_sz, c_int, c_dbl = ctypes.c_size_t, ctypes.c_int, ctypes.c_double
        P = ctypes.c_void_p
        L.orc_codes_bytes.restype = c_sz
        L.orc_codes_bytes.argtypes = [c_int, c_int, c_int]
        L.orc_sb_bytes.restype = c_sz
        L.orc_sb_bytes.argtypes = [c_int, c_int]
        L.orc_blob_layout.restype = None
        L.orc_blob_layout.argtypes = [c_int, c_int, c_int, P, P]
        L.orc_bf16_to_f32.restype = ctypes.c_float
        L.orc_bf16_to_f32.argtypes = [ctypes.c_uint16]
        L.orc_code.restype = c_int
        L.orc_code.argtypes = [P, c_int, c_int, c_int, c_int, c_int]
        L.orc_dequant.restype = None
        L.orc_dequant.argtypes = [P, P, c_int, c_int, c_int, P]
        L.orc_matvec.restype = None
        L.orc_matvec.argtypes = [P, c_int, c_int, P, P]
        L.orc_rmsnorm.restype = None
        L.orc_rmsnorm.argtypes = [P, P, c_int, c_dbl, P]
        L.orc_router_logits.restype = None
        L.orc_router_logits.argtypes = [P, c_int, c_int, c_int, P, P, P]
        L.orc_route.restype = None
        L.orc_route.argtypes = [P, c_int, c_int, P, P, P]
        L.orc_expert.restype = None
        L.orc_expert.argtypes = [P, c_int, c_int, c_int, P, P, P, P, P]
        L.orc_combine.restype = None
        L.orc_combine.argtypes = [P, P, c_int, c_int, P, P]
        L.orc_silu_export.restype = c_dbl
        L.orc_silu_export.argtypes = [c_dbl]
        L.orc_quantize.argtypes = [P, c_int, c_int, c_int, P, P, P]
        L.orc_quantize.restype = None
        _lib = L
    return _lib


def _p(a: Optional[np.ndarray]):
    return None if a is None else ctypes.c_void_p(a.ctypes.data)


# ----------------------------------------------------------------------------- format
def codes_bytes(rows: int, cols: int, bits: int) -> int:
    return int(lib().orc_codes_bytes(rows, cols, bits))


def sb_bytes(rows: int, cols: int) -> int:
    return int(lib().orc_sb_bytes(rows, cols))


def blob_layout(H: int, I: int, bits: int):
    off = np.zeros(6, dtype=np.uint64)
    tot = np.zeros(1, dtype=np.uint64)
    lib().orc_blob_layout(H, I, bits, _p(off), _p(tot))
    return [int(v) for v in off], int(tot[0])


def blob_bytes(H: int, I: int, bits: int) -> int:
    return blob_layout(H, I, bits)[1]


def bf16_to_f32(bits16: np.ndarray) -> np.ndarray:
    a = np.ascontiguousarray(bits16, dtype=np.uint16)
    return (a.astype(np.uint32) << 16).view(np.float32)


def code(codes: np.ndarray, rows: int, cols: int, bits: int, r: int, c: int) -> int:
    a = np.ascontiguousarray(codes, dtype=np.uint8)
    return int(lib().orc_code(_p(a), rows, cols, bits, r, c))


def dequant(codes: np.ndarray, sb: np.ndarray, rows: int, cols: int, bits: int) -> np.ndarray:
    """fp32 [rows, cols] matrix w = q*scale + bias from a packed code plane and sb plane."""
    c = np.ascontiguousarray(codes, dtype=np.uint8)
    s = np.ascontiguousarray(sb, dtype=np.uint16)
    assert c.size == codes_bytes(rows, cols, bits) and s.size * 2 == sb_bytes(rows, cols)
    W = np.empty((rows, cols), dtype=np.float32)
    lib().orc_dequant(_p(c), _p(s), rows, cols, bits, _p(W))
    return W


def expert_matrices(blob: np.ndarray, H: int, I: int, bits: int):
    """Dequantised (W_gate [I,H], W_up [I,H], W_down [H,I]) of one packed expert blob."""
    off, tot = blob_layout(H, I, bits)
    b = np.ascontiguousarray(blob, dtype=np.uint8)
    assert b.size >= tot
    cb_in, sb_in = codes_bytes(I, H, bits), sb_bytes(I, H)
    cb_out, sb_out = codes_bytes(H, I, bits), sb_bytes(H, I)
    Wg = dequant(b[off[0]:off[0] + cb_in], b[off[1]:off[1] + sb_in].view(np.uint16), I, H, bits)
    Wu = dequant(b[off[2]:off[2] + cb_in], b[off[3]:off[3] + sb_in].view(np.uint16), I, H, bits)
    Wd = dequant(b[off[4]:off[4] + cb_out], b[off[5]:off[5] + sb_out].view(np.uint16), H, I, bits)
    return Wg, Wu, Wd


# ----------------------------------------------------------------------------- steps
def matvec(W: np.ndarray, x: np.ndarray) -> np.ndarray:
    W = np.ascontiguousarray(W, dtype=np.float32)
    x = np.ascontiguousarray(x, dtype=np.float64)
    y = np.empty(W.shape[0], dtype=np.float64)
    lib().orc_matvec(_p(W), W.shape[0], W.shape[1], _p(x), _p(y))
    return y


def rmsnorm(x: np.ndarray, w_bf16: np.ndarray, eps: float) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float64)
    w = np.ascontiguousarray(w_bf16, dtype=np.uint16)
    out = np.empty_like(x)
    lib().orc_rmsnorm(_p(x), _p(w), x.size, eps, _p(out))
    return out


def router_logits(Wr: np.ndarray, n: np.ndarray, bias: Optional[np.ndarray] = None,
                  wr_is_bf16: bool = False) -> np.ndarray:
    """Wr: float32 [E,H] or uint16 (bf16 bits) [E,H]."""
    Wr = np.ascontiguousarray(Wr)
    if wr_is_bf16:
        assert Wr.dtype == np.uint16
    else:
        assert Wr.dtype == np.float32
    E, H = Wr.shape
    n = np.ascontiguousarray(n, dtype=np.float64)
    b = None if bias is None else np.ascontiguousarray(bias, dtype=np.float32)
    out = np.empty(E, dtype=np.float64)
    lib().orc_router_logits(_p(Wr), int(wr_is_bf16), E, H, _p(n), _p(b), _p(out))
    return out


def route(logits: np.ndarray, K: int):
    """(idx int32[K], weights float64[K], margin) -- softmax, top-K, renormalise."""
    l = np.ascontiguousarray(logits, dtype=np.float64)
    idx = np.empty(K, dtype=np.int32)
    w = np.empty(K, dtype=np.float64)
    m = np.empty(1, dtype=np.float64)
    lib().orc_route(_p(l), l.size, K, _p(idx), _p(w), _p(m))
    return idx, w, float(m[0])


def expert(blob: np.ndarray, bits: int, H: int, I: int, n: np.ndarray):
    """(g, u, h, y) of one expert on activation n."""
    b = np.ascontiguousarray(blob, dtype=np.uint8)
    assert b.size >= blob_bytes(H, I, bits)
    n = np.ascontiguousarray(n, dtype=np.float64)
    g = np.empty(I); u = np.empty(I); h = np.empty(I); y = np.empty(H)
    lib().orc_expert(_p(b), bits, H, I, _p(n), _p(g), _p(u), _p(h), _p(y))
    return g, u, h, y


def combine(y: np.ndarray, w: np.ndarray, residual: Optional[np.ndarray] = None) -> np.ndarray:
    y = np.ascontiguousarray(y, dtype=np.float64)
    K, H = y.shape
    w = np.ascontiguousarray(w, dtype=np.float64)
    r = None if residual is None else np.ascontiguousarray(residual, dtype=np.float64)
    out = np.empty(H)
    lib().orc_combine(_p(y), _p(w), K, H, _p(r), _p(out))
    return out


def quantize(W: np.ndarray, bits: int):
    """Quantise-from-float of an fp32 [rows][cols] matrix (see orc_quantize): (codes uint8
    [rows][cols], scale bf16 bits [rows][cols/64], bias bf16 bits [rows][cols/64])."""
    W = np.ascontiguousarray(W, dtype=np.float32)
    rows, cols = W.shape
    codes = np.empty((rows, cols), dtype=np.uint8)
    scale = np.empty((rows, cols // GROUP), dtype=np.uint16)
    bias = np.empty((rows, cols // GROUP), dtype=np.uint16)
    lib().orc_quantize(_p(W), rows, cols, bits, _p(codes), _p(scale), _p(bias))
    return codes, scale, bias


# ----------------------------------------------------------------------------- hot set, re-tiering
# The pages keep the frequently used experts at 4 bits and store the others at 2 bits (nzkcom.pages.dev,
# "flash-moe-romance-vs-utility", adopted-optimisation table; tomo3141592653.github.io, section
# "ハイブリッド量子化": the base is MLX 4-bit).  They do not say how "frequently used" is measured or
# how a 2-bit expert is made.  Plain reading: count the selections of each expert over a stream of
# routed tokens; the n most selected are hot (equal counts: the lower expert index first); a cold
# expert is dequantised from its base blob and quantised again at the cold width with quantize().

def expert_usage(idx: np.ndarray, E: int) -> np.ndarray:
    """counts[e] = number of entries of idx (any shape, e.g. [T][K] routing indices) equal to e;
    entries outside [0, E) are not counted.  int64 [E]."""
    idx = np.asarray(idx, dtype=np.int64).ravel()
    counts = np.zeros(E, dtype=np.int64)
    np.add.at(counts, idx[(idx >= 0) & (idx < E)], 1)
    return counts


def hot_order(counts: np.ndarray) -> np.ndarray:
    """Experts ranked by usage, most used first; equal counts rank the lower expert index first.
    int32 [E]; the first n entries are the hot set of size n."""
    counts = np.asarray(counts, dtype=np.int64)
    return np.lexsort((np.arange(counts.size), -counts)).astype(np.int32)


def requantize_matrix(codes_plane: np.ndarray, sb_plane: np.ndarray, rows: int, cols: int, bits_in: int,
                      bits_out: int):
    """A packed matrix at bits_in re-quantised at bits_out: quantize(dequant(...)).  Returns
    (codes uint8 [rows][cols], scale bf16 bits [rows][cols/64], bias bf16 bits [rows][cols/64])."""
    return quantize(dequant(codes_plane, sb_plane, rows, cols, bits_in), bits_out)


def requantize_expert(blob: np.ndarray, H: int, I: int, bits_in: int, bits_out: int):
    """The three matrices (gate I x H, up I x H, down H x I) of one packed expert, each re-quantised
    at bits_out: a list of three (codes, scale, bias) as requantize_matrix returns."""
    blob = np.asarray(blob, dtype=np.uint8)
    off, _ = blob_layout(H, I, bits_in)
    shapes = [(I, H), (I, H), (H, I)]
    out = []
    for m, (rows, cols) in enumerate(shapes):
        c0, s0 = off[2 * m], off[2 * m + 1]
        codes = blob[c0:c0 + codes_bytes(rows, cols, bits_in)]
        sb = blob[s0:s0 + sb_bytes(rows, cols)].view(np.uint16)
        out.append(requantize_matrix(codes, sb, rows, cols, bits_in, bits_out))
    return out


# ----------------------------------------------------------------------------- expert cache policy
# The pages stream each selected expert from SSD once routing is known and let the OS page cache keep
# recently read experts in memory (lilting.ch, "397Bパラメータモデルを48GB MacBookで動かすFlash-MoE",
# section "コア技術: SSDエキスパートストリーミング"); they do not define the replacement policy.  Plain
# reading for a store held in host memory with a cache of expert slots in device memory: least
# recently used replacement, one call per routing step.

class ExpertCacheModel:
    """Residency of experts in n_slots slots.  fetch(requests) processes one routing step: its
    distinct experts in [0, E) (first occurrence order; others are ignored) are each a hit when
    resident, else a miss loaded into the lowest free slot or, with no free slot, into the slot used
    least recently among those this call has not touched (equal times: the lower slot).  A call
    with more distinct experts than slots is refused (ValueError) and changes nothing."""

    def __init__(self, E: int, n_slots: int):
        self.E, self.n_slots = E, n_slots
        self.slot_of = {}                      # expert -> slot
        self.expert_of = [-1] * n_slots        # slot -> expert, -1 free
        self.last_use = [0] * n_slots
        self.tick = 0
        self.hits = self.misses = 0

    def fetch(self, requests):
        """Returns (hits, misses, loads, evicted): loads = [(expert, slot)] in load order,
        evicted = experts removed by this call."""
        distinct = []
        for e in requests:
            e = int(e)
            if 0 <= e < self.E and e not in distinct:
                distinct.append(e)
        if len(distinct) > self.n_slots:
            raise ValueError("more distinct experts than slots")
        self.tick += 1
        hits, missing = 0, []
        for e in distinct:
            if e in self.slot_of:
                hits += 1
                self.last_use[self.slot_of[e]] = self.tick
            else:
                missing.append(e)
        loads, evicted = [], []
        for e in missing:
            free = [s for s in range(self.n_slots) if self.expert_of[s] < 0]
            if free:
                s = free[0]
            else:
                s = min((s for s in range(self.n_slots) if self.last_use[s] < self.tick),
                        key=lambda s: (self.last_use[s], s))
                old = self.expert_of[s]
                del self.slot_of[old]
                evicted.append(old)
            self.slot_of[e] = s
            self.expert_of[s] = e
            self.last_use[s] = self.tick
            loads.append((e, s))
        self.hits += hits
        self.misses += len(missing)
        return hits, len(missing), loads, evicted


def silu(z: float) -> float:
    return float(lib().orc_silu_export(float(z)))


# ----------------------------------------------------------------------------- drivers
@dataclass
class LayerWeights:
    """Host copies of one MoE layer.  ``blob(e)`` returns expert e's packed bytes and
    ``bits(e)`` its code width, so that a store too large for host memory can be
    regenerated one expert at a time."""
    router: np.ndarray                  # float32 [E,H] or uint16 bf16 bits [E,H]
    router_is_bf16: bool
    blob: Callable[[int], np.ndarray]
    bits: Callable[[int], int]
    logit_bias: Optional[np.ndarray] = None   # float32 [E]
    norm_w: Optional[np.ndarray] = None       # uint16 bf16 bits [H]
    norm_eps: float = 1e-6


def workload_layer(wl, layer_id: int = 0, cache_size: Optional[int] = None) -> LayerWeights:
    """Host inputs of one layer of a seeded workload (any object with the seeded generator's
    methods: expert_bits(), blob(layer, e), router(layer), logit_bias(), norm_w(layer), and the
    fields router_bf16, norm_eps and n_layers).  Expert blobs are regenerated on demand and the most
    recent `cache_size` of them kept (default: 512 shared out over the workload's layers)."""
    import functools
    bits = wl.expert_bits()
    if cache_size is None:
        cache_size = max(8, 512 // max(1, int(getattr(wl, "n_layers", 1))))

    @functools.lru_cache(maxsize=cache_size)
    def blob(e: int) -> np.ndarray:
        return wl.blob(layer_id, int(e))

    return LayerWeights(router=wl.router(layer_id), router_is_bf16=wl.router_bf16,
                        blob=lambda e: blob(int(e)), bits=lambda e: int(bits[e]),
                        logit_bias=wl.logit_bias(), norm_w=wl.norm_w(layer_id), norm_eps=wl.norm_eps)


@dataclass
class LayerResult:
    idx: np.ndarray        # int32 [K]
    w: np.ndarray          # float64 [K]
    margin: float
    logits: np.ndarray     # float64 [E]
    n: np.ndarray          # float64 [H] activation fed to router and experts
    h: np.ndarray          # float64 [K, I]
    y: np.ndarray          # float64 [K, H]
    out: np.ndarray        # float64 [H]


def layer_token(x: np.ndarray, L: LayerWeights, H: int, I: int, K: int,
                residual: bool = False) -> LayerResult:
    """One token through one MoE layer."""
    x = np.asarray(x, dtype=np.float64)
    n = rmsnorm(x, L.norm_w, L.norm_eps) if L.norm_w is not None else x
    logits = router_logits(L.router, n, L.logit_bias, L.router_is_bf16)
    idx, w, margin = route(logits, K)
    hs = np.empty((K, I))
    ys = np.empty((K, H))
    for k in range(K):
        e = int(idx[k])
        _, _, hs[k], ys[k] = expert(L.blob(e), L.bits(e), H, I, n)
    out = combine(ys, w, x if residual else None)
    return LayerResult(idx, w, margin, logits, n, hs, ys, out)


def stack_token(x: np.ndarray, layers: Sequence[LayerWeights], H: int, I: int, K: int,
                residual: bool = True):
    """One token through a stack of layers; each layer's output feeds the next."""
    results = []
    cur = np.asarray(x, dtype=np.float64)
    for L in layers:
        r = layer_token(cur, L, H, I, K, residual=residual)
        results.append(r)
        cur = r.out
    return cur, results
