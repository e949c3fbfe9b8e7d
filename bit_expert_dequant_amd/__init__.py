"""Python binding of libmoe_dequant.so (the gfx950 MoE expert-path library).

Argument marshalling only: every function here converts torch tensors / numpy arrays to the
pointers and sizes of the C ABI declared in include/moe_dequant.h and calls it; all arithmetic
runs in the library.  The names match the C entry points.  PyTorch is used for device memory
and streams only.  Importing works without a GPU (the packer and the validation paths are
host code); compute calls need the built library and a gfx950 device, and raise if either is
missing -- there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import List, Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe_dequant.so")

MOE_OK = 0
MOE_F32, MOE_BF16 = 0, 1
MOE_OP_ROUTE, MOE_OP_EXPERT_FFN, MOE_OP_LAYER_DECODE = 1, 2, 3
MOE_FLAG_RESIDUAL = 1
MOE_FLAG_SEPARATE_KERNELS = 2
MOE_FLAG_SINGLE_LAUNCH = 4
MOE_FFN_AUTO, MOE_FFN_PER_TOKEN, MOE_FFN_SHARED, MOE_FFN_GROUPED = 0, 1, 2, 3
GROUP = 64
MAX_TOPK = 8
MAX_EXPERTS = 2048
MOE_CACHE_DRY_RUN = 1
STATUS = {0: "MOE_OK", 1: "MOE_ERR_NULL", 2: "MOE_ERR_SHAPE", 3: "MOE_ERR_DTYPE", 4: "MOE_ERR_BITS",
          5: "MOE_ERR_ALIGN", 6: "MOE_ERR_WORKSPACE", 7: "MOE_ERR_LAUNCH", 8: "MOE_ERR_UNSUPPORTED",
          9: "MOE_ERR_BUFFER", 10: "MOE_ERR_DEVICE"}


class MoeError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"{STATUS.get(status, status)}: {detail}")
        self.status = status


class moe_expert_desc(ctypes.Structure):
    _fields_ = [("blob", ctypes.c_uint64), ("bits", ctypes.c_uint32), ("reserved", ctypes.c_uint32)]


class moe_dims(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("inter", ctypes.c_int32), ("n_experts", ctypes.c_int32),
                ("top_k", ctypes.c_int32)]


class moe_layer(ctypes.Structure):
    _fields_ = [("router", ctypes.c_void_p), ("router_dtype", ctypes.c_int32), ("norm_eps", ctypes.c_float),
                ("logit_bias", ctypes.c_void_p), ("norm_w", ctypes.c_void_p), ("experts", ctypes.c_void_p)]


_lib = None


def lib():
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                               "(python -m bit_expert_dequant_amd.build)")
        L = ctypes.CDLL(LIB_PATH)
        P, I32, SZ, U = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t, ctypes.c_uint
        sig = {
            "moe_status_string": (ctypes.c_char_p, [I32]),
            "moe_last_error": (ctypes.c_char_p, []),
            "moe_version": (ctypes.c_char_p, []),
            "moe_packed_codes_bytes": (SZ, [I32, I32, I32]),
            "moe_packed_sb_bytes": (SZ, [I32, I32]),
            "moe_packed_expert_bytes": (SZ, [I32, I32, I32]),
            "moe_expert_plane_offsets": (I32, [I32, I32, I32, P]),
            "moe_pack_matrix": (I32, [P, P, P, I32, I32, I32, P, SZ, P, SZ]),
            "moe_unpack_matrix": (I32, [P, P, I32, I32, I32, P, P, P]),
            "moe_pack_expert": (I32, [P, P, P, I32, I32, I32, P, SZ]),
            "moe_check_experts": (I32, [P, I32]),
            "moe_workspace_bytes": (SZ, [I32, P, I32, I32]),
            "moe_route": (I32, [P, P, P, I32, I32, P, P, P, P, SZ, P]),
            "moe_expert_ffn": (I32, [P, P, P, I32, I32, P, P, P, SZ, P]),
            "moe_expert_ffn_path": (I32, [P, P, P, I32, I32, P, P, P, SZ, I32, P]),
            "moe_combine": (I32, [P, P, I32, I32, I32, P, P, P]),
            "moe_layer_decode": (I32, [P, P, I32, P, I32, U, P, P, P, P, SZ, P]),
            "moe_layer_decode_timed": (I32, [P, P, I32, P, I32, U, P, P, P, P, SZ, P, P]),
            "moe_layer_decode_static": (I32, [P, P, I32, P, I32, U, P, P, P, P]),
            "moe_stream_read": (I32, [P, SZ, P, P]),
            "moe_quantize_matrix": (I32, [P, I32, I32, I32, I32, P, P, P]),
            "moe_expert_usage": (I32, [P, I32, I32, P, P]),
            "moe_hot_order": (I32, [P, I32, P, P]),
            "moe_retier": (I32, [P, P, P, I32, I32, P, SZ, P, P]),
            "moe_cache_create": (I32, [P, P, P, SZ, I32, P, U, P, P]),
            "moe_cache_fetch": (I32, [P, P, I32, P, P]),
            "moe_cache_stats": (I32, [P, P, P, P]),
            "moe_cache_slot": (I32, [P, I32]),
            "moe_cache_destroy": (None, [P]),
            "moe_cache_device_state_bytes": (SZ, [P]),
            "moe_cache_attach_device": (I32, [P, P, SZ, P]),
            "moe_cache_fetch_device": (I32, [P, P, I32, P]),
            "moe_cache_device_refused": (I32, [P]),
            "moe_debug_inject_launch_failure": (I32, [I32, I32]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def exported_symbols() -> List[str]:
    return ["moe_status_string", "moe_last_error", "moe_version", "moe_packed_codes_bytes",
            "moe_packed_sb_bytes", "moe_packed_expert_bytes", "moe_expert_plane_offsets", "moe_pack_matrix",
            "moe_unpack_matrix", "moe_pack_expert", "moe_check_experts", "moe_workspace_bytes", "moe_route",
            "moe_expert_ffn", "moe_expert_ffn_path", "moe_combine", "moe_layer_decode", "moe_layer_decode_timed",
            "moe_layer_decode_static", "moe_stream_read",
            "moe_quantize_matrix", "moe_expert_usage", "moe_hot_order", "moe_retier", "moe_cache_create",
            "moe_cache_fetch", "moe_cache_stats", "moe_cache_slot", "moe_cache_destroy",
            "moe_cache_device_state_bytes", "moe_cache_attach_device", "moe_cache_fetch_device",
            "moe_cache_device_refused", "moe_debug_inject_launch_failure"]


def _check(status: int):
    if status != MOE_OK:
        raise MoeError(status, lib().moe_last_error().decode())


def _np_ptr(a: Optional[np.ndarray]):
    return None if a is None else ctypes.c_void_p(a.ctypes.data)


def _tptr(t):
    """Device pointer of a torch tensor (None -> NULL)."""
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.float32:
        return MOE_F32
    if t.dtype == torch.bfloat16:
        return MOE_BF16
    raise TypeError(f"unsupported activation dtype {t.dtype} (float32 or bfloat16)")


def _stream(stream=None):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def version() -> str:
    return lib().moe_version().decode()


# ----------------------------------------------------------------------------- format (host)
def moe_packed_codes_bytes(rows: int, cols: int, bits: int) -> int:
    return int(lib().moe_packed_codes_bytes(rows, cols, bits))


def moe_packed_sb_bytes(rows: int, cols: int) -> int:
    return int(lib().moe_packed_sb_bytes(rows, cols))


def moe_packed_expert_bytes(hidden: int, inter: int, bits: int) -> int:
    return int(lib().moe_packed_expert_bytes(hidden, inter, bits))


def moe_expert_plane_offsets(hidden: int, inter: int, bits: int) -> List[int]:
    off = (ctypes.c_size_t * 6)()
    _check(lib().moe_expert_plane_offsets(hidden, inter, bits, off))
    return list(off)


def moe_pack_matrix(codes: np.ndarray, scale: np.ndarray, bias: np.ndarray, bits: int):
    """codes uint8 [R, C]; scale, bias uint16 (bf16 bits) [R, C/64] -> (code plane, sb plane)."""
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    R, C = codes.shape
    scale = np.ascontiguousarray(scale, dtype=np.uint16)
    bias = np.ascontiguousarray(bias, dtype=np.uint16)
    if scale.size != R * (C // GROUP) or bias.size != scale.size:
        raise ValueError("scale/bias must have R*C/64 entries")
    cb, sb = max(moe_packed_codes_bytes(R, C, bits), 1), max(moe_packed_sb_bytes(R, C), 4)
    co = np.zeros(cb, dtype=np.uint8)
    so = np.zeros(sb // 2, dtype=np.uint16)
    _check(lib().moe_pack_matrix(_np_ptr(codes), _np_ptr(scale), _np_ptr(bias), R, C, bits,
                                 _np_ptr(co), co.nbytes, _np_ptr(so), so.nbytes))
    return co, so


def moe_unpack_matrix(code_plane: np.ndarray, sb_plane: np.ndarray, rows: int, cols: int, bits: int):
    cp = np.ascontiguousarray(code_plane, dtype=np.uint8)
    sp = np.ascontiguousarray(sb_plane, dtype=np.uint16)
    codes = np.zeros((rows, cols), dtype=np.uint8)
    scale = np.zeros(rows * (cols // GROUP), dtype=np.uint16)
    bias = np.zeros_like(scale)
    _check(lib().moe_unpack_matrix(_np_ptr(cp), _np_ptr(sp), rows, cols, bits, _np_ptr(codes),
                                   _np_ptr(scale), _np_ptr(bias)))
    return codes, scale, bias


def moe_pack_expert(mats: Sequence, hidden: int, inter: int, bits: int) -> np.ndarray:
    """mats = [(codes, scale, bias)] for gate [I,H], up [I,H], down [H,I] -> packed blob (uint8)."""
    arrs = []
    for codes, scale, bias in mats:
        arrs.append((np.ascontiguousarray(codes, dtype=np.uint8), np.ascontiguousarray(scale, dtype=np.uint16),
                     np.ascontiguousarray(bias, dtype=np.uint16)))
    P3 = ctypes.c_void_p * 3
    cp = P3(*[a[0].ctypes.data for a in arrs])
    sp = P3(*[a[1].ctypes.data for a in arrs])
    bp = P3(*[a[2].ctypes.data for a in arrs])
    n = moe_packed_expert_bytes(hidden, inter, bits)
    out = np.zeros(max(n, 1), dtype=np.uint8)
    _check(lib().moe_pack_expert(cp, sp, bp, hidden, inter, bits, _np_ptr(out), out.nbytes))
    return out


def moe_check_experts(table) -> None:
    """Validate a device descriptor table (torch uint8/int64 tensor of E*16 bytes)."""
    _check(lib().moe_check_experts(_tptr(table), table.numel() * table.element_size() // 16))


# ----------------------------------------------------------------------------- device helpers
def expert_table(blob_ptrs: Sequence[int], bits: Sequence[int], device="cuda"):
    """Build the device descriptor table [E] from blob device addresses and widths."""
    import torch
    E = len(blob_ptrs)
    host = np.zeros((E, 2), dtype=np.uint64)
    host[:, 0] = np.asarray(blob_ptrs, dtype=np.uint64)
    host[:, 1] = np.asarray(bits, dtype=np.uint64)       # bits in the low word, reserved = 0
    return torch.from_numpy(host.view(np.int64).reshape(-1)).to(device)


def make_dims(hidden: int, inter: int, n_experts: int, top_k: int) -> moe_dims:
    return moe_dims(hidden, inter, n_experts, top_k)


class Layer:
    """Keeps the tensors of one layer alive and exposes the C struct."""

    def __init__(self, router, experts, logit_bias=None, norm_w=None, norm_eps: float = 1e-6):
        self.router, self.experts, self.logit_bias, self.norm_w = router, experts, logit_bias, norm_w
        self.c = moe_layer(router.data_ptr(), _dtype_code(router), float(norm_eps),
                           None if logit_bias is None else logit_bias.data_ptr(),
                           None if norm_w is None else norm_w.data_ptr(), experts.data_ptr())


def moe_workspace_bytes(op: int, dims: moe_dims, T: int = 1, n_layers: int = 1) -> int:
    return int(lib().moe_workspace_bytes(op, ctypes.byref(dims), T, n_layers))


def workspace(op: int, dims: moe_dims, T: int = 1, n_layers: int = 1, device="cuda"):
    import torch
    n = moe_workspace_bytes(op, dims, T, n_layers)
    return torch.zeros(max(n, 256), dtype=torch.uint8, device=device)


# ----------------------------------------------------------------------------- compute
def moe_route(dims: moe_dims, layer: Layer, x, idx, w, logits=None, ws=None, stream=None) -> None:
    T = x.shape[0] if x.dim() == 2 else 1
    _check(lib().moe_route(ctypes.byref(dims), ctypes.byref(layer.c), _tptr(x), _dtype_code(x), T, _tptr(idx),
                           _tptr(w), _tptr(logits), _tptr(ws), 0 if ws is None else ws.numel(), _stream(stream)))


def moe_expert_ffn(dims: moe_dims, layer: Layer, x, idx, y, ws, stream=None, path: int = 0) -> None:
    """``path``: MOE_FFN_AUTO (0, what moe_expert_ffn chooses), MOE_FFN_PER_TOKEN, MOE_FFN_SHARED or
    MOE_FFN_GROUPED."""
    T = x.shape[0] if x.dim() == 2 else 1
    if path == MOE_FFN_AUTO:
        _check(lib().moe_expert_ffn(ctypes.byref(dims), ctypes.byref(layer.c), _tptr(x), _dtype_code(x), T,
                                    _tptr(idx), _tptr(y), _tptr(ws), ws.numel(), _stream(stream)))
    else:
        _check(lib().moe_expert_ffn_path(ctypes.byref(dims), ctypes.byref(layer.c), _tptr(x), _dtype_code(x), T,
                                         _tptr(idx), _tptr(y), _tptr(ws), ws.numel(), path, _stream(stream)))


def moe_combine(y, w, out, residual=None, stream=None) -> None:
    T, K, H = y.shape
    _check(lib().moe_combine(_tptr(y), _tptr(w), T, K, H, _tptr(residual), _tptr(out), _stream(stream)))


def moe_layer_decode(dims: moe_dims, layers: Sequence[Layer], x, out, idx=None, w=None, residual: bool = False,
                     ws=None, stream=None, separate_kernels: bool = False, single_launch: bool = False) -> None:
    """One decode token through the layers.  ``ws`` must come from :func:`workspace` (zero-filled)
    and be reused only by stream-ordered calls.  A layer is two launches by default (router + gate/up,
    down); ``separate_kernels`` selects three, ``single_launch`` one (a persistent grid)."""
    arr = (moe_layer * len(layers))(*[L.c for L in layers])
    flags = ((MOE_FLAG_RESIDUAL if residual else 0) | (MOE_FLAG_SEPARATE_KERNELS if separate_kernels else 0)
             | (MOE_FLAG_SINGLE_LAUNCH if single_launch else 0))
    _check(lib().moe_layer_decode(ctypes.byref(dims), arr, len(layers), _tptr(x), _dtype_code(x), flags,
                                  _tptr(out), _tptr(idx), _tptr(w), _tptr(ws), 0 if ws is None else ws.numel(),
                                  _stream(stream)))


def moe_layer_decode_static(dims: moe_dims, layers: Sequence[Layer], x, out, idx=None, w=None,
                            residual: bool = False, stream=None, separate_kernels: bool = False,
                            single_launch: bool = False) -> None:
    """moe_layer_decode with the library's per-device static workspace (allocates nothing; calls on
    one device must not overlap)."""
    arr = (moe_layer * len(layers))(*[L.c for L in layers])
    flags = ((MOE_FLAG_RESIDUAL if residual else 0) | (MOE_FLAG_SEPARATE_KERNELS if separate_kernels else 0)
             | (MOE_FLAG_SINGLE_LAUNCH if single_launch else 0))
    _check(lib().moe_layer_decode_static(ctypes.byref(dims), arr, len(layers), _tptr(x), _dtype_code(x), flags,
                                         _tptr(out), _tptr(idx), _tptr(w), _stream(stream)))


def moe_stream_read(buf, sink, stream=None) -> None:
    """Read-stream reference (see moe_stream_read in the header): XOR of every dword of `buf`
    (a contiguous device tensor, 16-byte aligned, size a multiple of 16 bytes) into sink[0]."""
    _check(lib().moe_stream_read(_tptr(buf), buf.numel() * buf.element_size(), _tptr(sink), _stream(stream)))


def moe_quantize_matrix(w, bits: int, codes, sb, stream=None) -> None:
    """Quantise a device [rows][cols] fp32 or bf16 tensor `w` into the packed code plane `codes`
    (uint8 tensor, moe_packed_codes_bytes bytes) and (scale, bias) plane `sb` (int16 tensor of
    2 * rows * cols / 64 entries); see moe_quantize_matrix in the header."""
    rows, cols = w.shape
    _check(lib().moe_quantize_matrix(_tptr(w), _dtype_code(w), rows, cols, bits, _tptr(codes), _tptr(sb),
                                     _stream(stream)))


def moe_expert_usage(idx, n_experts: int, counts, stream=None) -> None:
    """counts[e] += selections of expert e in the int32 device tensor `idx` (any shape; entries
    outside [0, n_experts) are not counted); `counts` is a uint32/int32 device tensor of n_experts."""
    _check(lib().moe_expert_usage(_tptr(idx), idx.numel(), n_experts, _tptr(counts), _stream(stream)))


def moe_hot_order(counts, order, stream=None) -> None:
    """order = experts by counts, largest first, equal counts lower index first (device tensors of
    n_experts uint32/int32 counts and int32 order)."""
    _check(lib().moe_hot_order(_tptr(counts), counts.numel(), _tptr(order), _stream(stream)))


def moe_retier(dims: moe_dims, base, order, n_hot: int, cold_bits: int, store, tiered, stream=None) -> None:
    """Hot experts (order[:n_hot]) keep their base blobs; the others are requantised at cold_bits into
    `store` (a uint8 device tensor) in rank order; `tiered` (device table, may be `base`) gets the
    new descriptors.  See moe_retier in the header."""
    _check(lib().moe_retier(ctypes.byref(dims), _tptr(base), _tptr(order), n_hot, cold_bits, _tptr(store),
                            0 if store is None else store.numel() * store.element_size(), _tptr(tiered),
                            _stream(stream)))


class ExpertCache:
    """A device-memory cache of experts whose blobs live in host memory (see moe_cache_create in the
    header).  ``host_ptrs``/``bits``: host address and width of each expert's blob (pinned memory,
    e.g. a torch tensor allocated with pin_memory=True); ``slots``: a uint8 device tensor of
    n_slots * slot_bytes bytes; ``table``: the device descriptor table the layer uses (e.g. from
    :func:`expert_table`), which the cache owns from now on.  ``dry_run`` runs the policy only."""

    def __init__(self, dims: moe_dims, host_ptrs: Sequence[int], bits: Sequence[int], slots=None,
                 slot_bytes: int = 0, n_slots: int = 0, table=None, dry_run: bool = False, stream=None):
        E = dims.n_experts
        host = np.zeros((E, 2), dtype=np.uint64)
        host[:, 0] = np.asarray(host_ptrs, dtype=np.uint64)
        host[:, 1] = np.asarray(bits, dtype=np.uint64)
        self._keep = (host, slots, table)
        self._dry = dry_run
        self._c = ctypes.c_void_p()
        _check(lib().moe_cache_create(ctypes.byref(dims), _np_ptr(host), _tptr(slots), slot_bytes, n_slots,
                                      _tptr(table), MOE_CACHE_DRY_RUN if dry_run else 0,
                                      None if dry_run else _stream(stream), ctypes.byref(self._c)))

    def fetch(self, idx, stream=None) -> int:
        """Make the experts named in ``idx`` (host int array, any shape) resident; returns the misses."""
        a = np.ascontiguousarray(idx, dtype=np.int32).reshape(-1)
        miss = ctypes.c_int(0)
        _check(lib().moe_cache_fetch(self._c, _np_ptr(a), a.size, None if self._dry else _stream(stream),
                                     ctypes.byref(miss)))
        return miss.value

    def stats(self):
        """(hits, misses, bytes copied) since creation."""
        h, m, b = ctypes.c_uint64(), ctypes.c_uint64(), ctypes.c_uint64()
        _check(lib().moe_cache_stats(self._c, ctypes.byref(h), ctypes.byref(m), ctypes.byref(b)))
        return h.value, m.value, b.value

    def slot(self, expert: int) -> int:
        return lib().moe_cache_slot(self._c, expert)

    def attach_device(self, stream=None) -> None:
        """Move the policy to the device (see moe_cache_attach_device): a device state buffer is
        allocated here and kept; from now on use :meth:`fetch_device`."""
        import torch
        nb = lib().moe_cache_device_state_bytes(self._c)
        if nb == 0:
            raise MoeError(8, "the device policy does not apply to this cache")
        self._state = torch.empty((nb + 255) // 256 * 64, dtype=torch.int32, device="cuda")
        _check(lib().moe_cache_attach_device(self._c, _tptr(self._state), self._state.numel() * 4, _stream(stream)))

    def fetch_device(self, idx, stream=None) -> None:
        """Make the experts named in ``idx`` (a device int32 tensor, any shape) resident, on the device."""
        _check(lib().moe_cache_fetch_device(self._c, _tptr(idx), idx.numel(), _stream(stream)))

    def refused(self) -> int:
        return lib().moe_cache_device_refused(self._c)

    def close(self):
        if self._c:
            lib().moe_cache_destroy(self._c)
            self._c = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def moe_layer_decode_timed(dims: moe_dims, layers: Sequence[Layer], x, out, events: Sequence, idx=None, w=None,
                           residual: bool = False, ws=None, stream=None, separate_kernels: bool = False,
                           single_launch: bool = False) -> None:
    """As moe_layer_decode, with a start/stop pair of ``events`` (torch.cuda.Event objects with
    timing enabled) per kernel: events[2j].elapsed_time(events[2j+1]) is kernel j's execution time.
    Two kernels per layer on the default schedule (router + gate/up, down), one with ``single_launch``,
    three with ``separate_kernels`` (router, gate/up, down)."""
    arr = (moe_layer * len(layers))(*[L.c for L in layers])
    need = 2 * (3 if separate_kernels else 1 if single_launch else 2) * len(layers)
    if len(events) < need:
        raise ValueError(f"{need} events needed, {len(events)} given")
    handles = [e.cuda_event for e in events]
    if not all(handles):
        raise ValueError("events must have been recorded once (torch creates HIP events lazily)")
    ev = (ctypes.c_void_p * len(events))(*handles)
    flags = ((MOE_FLAG_RESIDUAL if residual else 0) | (MOE_FLAG_SEPARATE_KERNELS if separate_kernels else 0)
             | (MOE_FLAG_SINGLE_LAUNCH if single_launch else 0))
    _check(lib().moe_layer_decode_timed(ctypes.byref(dims), arr, len(layers), _tptr(x), _dtype_code(x), flags,
                                        _tptr(out), _tptr(idx), _tptr(w), _tptr(ws), 0 if ws is None else ws.numel(),
                                        _stream(stream), ev))
