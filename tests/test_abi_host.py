"""Host-side checks of the C ABI (no GPU): exported symbols, the packer against the oracle's
independent unpack, and argument validation (each failing call returns its status before
anything is enqueued)."""
import ctypes
import os
import re

import numpy as np
import pytest

import bit_expert_dequant_amd as M

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_dequant.h")


@pytest.fixture(scope="module")
def L():
    return M.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_0-9]+)\s*\(", text)))


def test_header_declarations_are_exported(L):
    names = declared_functions()
    assert len(names) >= 15
    for n in names:
        assert hasattr(L, n), n
    assert sorted(M.exported_symbols()) == names


def test_version_and_status_strings(L):
    assert b"gfx950" in L.moe_version()
    assert L.moe_status_string(0) == b"MOE_OK"
    assert L.moe_status_string(6) == b"MOE_ERR_WORKSPACE"


def test_sizes_match_oracle(orc):
    for H, I, bits in [(4096, 1024, 4), (4096, 1024, 2), (512, 256, 4), (192, 320, 2), (3072, 768, 4)]:
        off, tot = orc.blob_layout(H, I, bits)
        assert M.moe_packed_expert_bytes(H, I, bits) == tot
        assert M.moe_expert_plane_offsets(H, I, bits) == off
        assert M.moe_packed_codes_bytes(I, H, bits) == orc.codes_bytes(I, H, bits)
        assert M.moe_packed_sb_bytes(I, H) == orc.sb_bytes(I, H)
    assert M.moe_packed_expert_bytes(4096, 1024, 4) == 7_077_888
    assert M.moe_packed_expert_bytes(100, 64, 4) == 0
    assert M.moe_packed_expert_bytes(128, 64, 3) == 0


@pytest.mark.parametrize("bits", [2, 4])
def test_pack_matrix_matches_oracle_unpack(orc, bits):
    rng = np.random.default_rng(20 + bits)
    R, C = 7, 320
    codes = rng.integers(0, 1 << bits, (R, C)).astype(np.uint8)
    scale = rng.integers(0, 1 << 16, R * (C // 64)).astype(np.uint16)
    bias = rng.integers(0, 1 << 16, R * (C // 64)).astype(np.uint16)
    cp, sp = M.moe_pack_matrix(codes, scale, bias, bits)
    for r in range(R):
        for c in range(0, C, 7):
            assert orc.code(cp, R, C, bits, r, c) == codes[r, c]
    assert np.array_equal(sp[0::2], scale) and np.array_equal(sp[1::2], bias)
    c2, s2, b2 = M.moe_unpack_matrix(cp, sp, R, C, bits)
    assert np.array_equal(c2, codes) and np.array_equal(s2, scale) and np.array_equal(b2, bias)


def test_pack_expert_matches_oracle_dequant(orc):
    rng = np.random.default_rng(30)
    H, I, bits = 192, 128, 4
    mats = []
    for R, C in [(I, H), (I, H), (H, I)]:
        codes = rng.integers(0, 16, (R, C)).astype(np.uint8)
        s = (rng.uniform(0.002, 0.02, R * C // 64).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
        b = (rng.uniform(-0.1, 0.1, R * C // 64).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
        mats.append((codes, s, b))
    blob = M.moe_pack_expert(mats, H, I, bits)
    Wg, Wu, Wd = orc.expert_matrices(blob, H, I, bits)
    for W, (codes, s, b) in zip((Wg, Wu, Wd), mats):
        sf = orc.bf16_to_f32(s).reshape(W.shape[0], -1)
        bf = orc.bf16_to_f32(b).reshape(W.shape[0], -1)
        ref = codes.astype(np.float32) * np.repeat(sf, 64, 1) + np.repeat(bf, 64, 1)
        assert np.array_equal(W, ref)


def test_pack_rejects_bad_codes_and_buffers(L):
    codes = np.full((2, 64), 4, dtype=np.uint8)
    s = np.zeros(2, dtype=np.uint16)
    with pytest.raises(M.MoeError) as e:
        M.moe_pack_matrix(codes, s, s, 2)           # code 4 does not fit in 2 bits
    assert e.value.status == 4
    out = np.zeros(8, dtype=np.uint8)
    sb = np.zeros(4, dtype=np.uint16)
    rc = L.moe_pack_matrix(codes.ctypes.data, s.ctypes.data, s.ctypes.data, 2, 64, 4, out.ctypes.data, 8,
                           sb.ctypes.data, 8)
    assert rc == 9                                   # MOE_ERR_BUFFER
    assert b"need" in L.moe_last_error()


# ----------------------------------------------------------------------------- validation
FAKE = 1 << 20        # a 1 MiB-aligned non-NULL address that is never dereferenced


def dims(H=512, I=256, E=8, K=2):
    return M.moe_dims(H, I, E, K)


def layer(router=FAKE, experts=FAKE, dtype=M.MOE_F32, bias=None, norm=None, eps=1e-6):
    return M.moe_layer(router, dtype, eps, bias, norm, experts)


def call_route(L, d, lay, x=FAKE, xdt=M.MOE_F32, T=1, idx=FAKE, w=FAKE, logits=FAKE, ws=None, wsb=0):
    return L.moe_route(ctypes.byref(d) if d is not None else None, ctypes.byref(lay) if lay is not None else None,
                       x, xdt, T, idx, w, logits, ws, wsb, None)


@pytest.mark.parametrize("d,status", [
    (dims(H=500), 2), (dims(H=0), 2), (dims(I=32), 2), (dims(H=16384), 2), (dims(E=0), 2),
    (dims(E=4096), 2), (dims(K=0), 2), (dims(K=9, E=16), 2), (dims(K=5, E=4), 2),
    (dims(I=8192, K=8), 8),
])
def test_route_rejects_bad_dims(L, d, status):
    assert call_route(L, d, layer()) == status
    assert L.moe_last_error().startswith(M.STATUS[status].encode())


def test_route_rejects_bad_arguments(L):
    d = dims()
    assert call_route(L, None, layer()) == 1
    assert call_route(L, d, None) == 1
    assert call_route(L, d, layer(router=None)) == 1
    assert call_route(L, d, layer(experts=None)) == 1
    assert call_route(L, d, layer(dtype=7)) == 3
    assert call_route(L, d, layer(), xdt=9) == 3
    assert call_route(L, d, layer(router=FAKE + 4)) == 5
    assert call_route(L, d, layer(), x=FAKE + 8) == 5
    assert call_route(L, d, layer(), x=None) == 1
    assert call_route(L, d, layer(), T=0) == 2
    assert call_route(L, d, layer(norm=FAKE, eps=float("nan"))) == 2
    # logits NULL -> the workspace must hold them
    assert call_route(L, d, layer(), logits=None) == 6
    assert call_route(L, d, layer(), logits=None, ws=FAKE, wsb=16) == 6
    assert call_route(L, d, layer(), logits=None, ws=FAKE + 16, wsb=1 << 20) == 5
    # route workspace: logits, then from 64 tokens the normalised rows and the partial logit rows of
    # the MFMA router's K splits (as many splits as bring its grid to 256 workgroups: 8 at 64 tokens
    # of 512 experts, 2 at 256 tokens, none from 512; at most 2 above 512 experts)
    r = lambda n: (n + 255) // 256 * 256  # noqa: E731
    d1 = dims(H=4096, I=1024, E=512, K=4)
    ws_route = lambda dd, T: M.moe_workspace_bytes(M.MOE_OP_ROUTE, dd, T, 1)  # noqa: E731
    assert ws_route(d1, 63) == r(63 * 512 * 4)
    assert ws_route(d1, 64) == r(64 * 512 * 4) + r(64 * 4096 * 4) + r(8 * 64 * 512 * 4)
    assert ws_route(d1, 256) == r(256 * 512 * 4) + r(256 * 4096 * 4) + r(2 * 256 * 512 * 4)
    assert ws_route(d1, 512) == r(512 * 512 * 4) + r(512 * 4096 * 4)
    dw = dims(H=2048, I=256, E=1024, K=4)
    assert ws_route(dw, 64) == r(64 * 1024 * 4) + r(64 * 2048 * 4) + r(2 * 64 * 1024 * 4)


def test_expert_ffn_and_decode_validation(L):
    d = dims()
    lay = layer()
    need = M.moe_workspace_bytes(M.MOE_OP_EXPERT_FFN, d, 1, 1)
    assert need == 2 * 256 * 4 + 256   # h [K][I] fp32, then the selected experts [K] (256-byte regions)
    assert L.moe_expert_ffn(ctypes.byref(d), ctypes.byref(lay), FAKE, M.MOE_F32, 1, FAKE, FAKE, FAKE, need - 1,
                            None) == 6
    assert L.moe_expert_ffn(ctypes.byref(d), ctypes.byref(lay), FAKE, M.MOE_F32, 1, None, FAKE, FAKE, need,
                            None) == 1
    # path selection (validated before any launch): unknown paths and T outside a path's range
    ffn = L.moe_expert_ffn_path
    big = 1 << 30

    def path_rc(T, path):
        return ffn(ctypes.byref(d), ctypes.byref(lay), FAKE, M.MOE_F32, T, FAKE, FAKE, FAKE, big, path, None)
    assert path_rc(4, 7) == 8 and path_rc(4, -1) == 8
    assert path_rc(1, M.MOE_FFN_SHARED) == 8 and path_rc(17, M.MOE_FFN_SHARED) == 8
    assert b"shared-read" in L.moe_last_error()
    assert path_rc(25, M.MOE_FFN_PER_TOKEN) == 8 and path_rc(1, M.MOE_FFN_GROUPED) == 8
    d8 = dims(K=8)
    assert ffn(ctypes.byref(d8), ctypes.byref(lay), FAKE, M.MOE_F32, 9, FAKE, FAKE, FAKE, big, M.MOE_FFN_SHARED,
               None) == 8                                          # 72 pairs: more than one wavefront
    # the workspace covers every path that can take T: at 2..16 tokens shared-read (h of every pair,
    # then the rows normalised), per-token (h of every pair, then the selected experts) and grouped
    pairs_h = 4 * 2 * 256 * 4
    assert M.moe_workspace_bytes(M.MOE_OP_EXPERT_FFN, d, 4, 1) >= max(pairs_h + 4 * 512 * 4, pairs_h + 256)
    wsn = pairs_h + 4 * 512 * 4
    assert ffn(ctypes.byref(d), ctypes.byref(lay), FAKE, M.MOE_F32, 4, FAKE, FAKE, FAKE, wsn - 1, M.MOE_FFN_SHARED,
               None) == 6
    need = M.moe_workspace_bytes(M.MOE_OP_LAYER_DECODE, d, 1, 3)
    assert need > 0 and M.moe_workspace_bytes(M.MOE_OP_LAYER_DECODE, d, 2, 3) == 0
    arr = (M.moe_layer * 3)(layer(), layer(router=None), layer())
    rc = L.moe_layer_decode(ctypes.byref(d), arr, 3, FAKE, M.MOE_F32, 0, FAKE + 4096, None, None, FAKE, need, None)
    assert rc == 1 and b"layer 1" in L.moe_last_error()
    arr = (M.moe_layer * 1)(layer())
    assert L.moe_layer_decode(ctypes.byref(d), arr, 1, FAKE, M.MOE_F32, 8, FAKE + 4096, None, None, FAKE, need,
                              None) == 8
    assert L.moe_layer_decode(ctypes.byref(d), arr, 1, FAKE, M.MOE_F32, 0, FAKE, None, None, FAKE, need, None) == 2
    assert L.moe_layer_decode(ctypes.byref(d), arr, 1, FAKE, M.MOE_F32, 0, FAKE + 4096, FAKE, None, FAKE, need,
                              None) == 1
    assert L.moe_layer_decode(ctypes.byref(d), arr, 0, FAKE, M.MOE_F32, 0, FAKE + 4096, None, None, FAKE, need,
                              None) == 2
    assert L.moe_combine(None, FAKE, 1, 2, 64, None, FAKE, None) == 1
    assert L.moe_combine(FAKE, FAKE, 1, 9, 64, None, FAKE, None) == 2
    assert L.moe_check_experts(None, 4) == 1


def test_quantize_matrix_validates_before_launch(L):
    """moe_quantize_matrix refuses bad arguments with a status and enqueues nothing (no device
    pointer is ever dereferenced: every call below fails validation)."""
    P = ctypes.c_void_p
    w, codes, sb = P(0x100000), P(0x200000), P(0x300000)
    q = L.moe_quantize_matrix
    assert q(None, M.MOE_F32, 4, 64, 4, codes, sb, None) == 1                 # MOE_ERR_NULL
    assert q(w, M.MOE_F32, 4, 64, 4, None, sb, None) == 1
    assert q(w, 7, 4, 64, 4, codes, sb, None) == 3                           # MOE_ERR_DTYPE
    assert q(w, M.MOE_F32, 0, 64, 4, codes, sb, None) == 2                   # MOE_ERR_SHAPE
    assert q(w, M.MOE_F32, 4, 96, 4, codes, sb, None) == 2
    assert q(w, M.MOE_BF16, 4, 0, 4, codes, sb, None) == 2
    assert q(w, M.MOE_F32, 4, 64, 3, codes, sb, None) == 4                   # MOE_ERR_BITS
    assert q(P(0x100004), M.MOE_F32, 4, 64, 4, codes, sb, None) == 5          # MOE_ERR_ALIGN
    assert q(w, M.MOE_F32, 4, 64, 2, P(0x200008), sb, None) == 5
    assert q(w, M.MOE_F32, 4, 64, 2, codes, P(0x300002), None) == 5
    assert b"bits" in L.moe_last_error() or b"align" in L.moe_last_error()


def test_tier_calls_validate_before_launch(L):
    """moe_expert_usage, moe_hot_order and moe_retier refuse bad arguments with a status before
    anything is enqueued (every call below fails validation, so no device pointer is touched)."""
    P = ctypes.c_void_p
    idx, counts, order = P(0x100000), P(0x200000), P(0x300000)
    u = L.moe_expert_usage
    assert u(idx, 16, 8, None, None) == 1                                    # MOE_ERR_NULL
    assert u(None, 16, 8, counts, None) == 1
    assert u(idx, -1, 8, counts, None) == 2                                  # MOE_ERR_SHAPE
    assert u(idx, 16, 0, counts, None) == 2
    assert u(idx, 16, M.MAX_EXPERTS + 1, counts, None) == 2
    assert u(P(0x100002), 16, 8, counts, None) == 5                          # MOE_ERR_ALIGN
    h = L.moe_hot_order
    assert h(None, 8, order, None) == 1
    assert h(counts, 8, None, None) == 1
    assert h(counts, 0, order, None) == 2
    assert h(counts, 8, P(0x300001), None) == 5
    dims = M.moe_dims(256, 128, 16, 2)
    base, tiered, store = P(0x400000), P(0x500000), P(0x600000)
    cold2 = L.moe_packed_expert_bytes(256, 128, 2)
    r = L.moe_retier
    assert r(ctypes.byref(dims), None, order, 4, 2, store, 12 * cold2, tiered, None) == 1
    assert r(ctypes.byref(dims), base, order, 4, 2, None, 12 * cold2, tiered, None) == 1   # cold experts, no store
    assert r(ctypes.byref(dims), base, order, 17, 2, store, 12 * cold2, tiered, None) == 2
    assert r(ctypes.byref(dims), base, order, -1, 2, store, 12 * cold2, tiered, None) == 2
    assert r(ctypes.byref(dims), base, order, 4, 3, store, 12 * cold2, tiered, None) == 4
    assert r(ctypes.byref(dims), base, order, 4, 2, P(0x600080), 12 * cold2, tiered, None) == 5
    assert r(ctypes.byref(dims), P(0x400008), order, 4, 2, store, 12 * cold2, tiered, None) == 5
    assert r(ctypes.byref(dims), base, order, 4, 2, store, 12 * cold2 - 1, tiered, None) == 9   # MOE_ERR_BUFFER
    assert b"store_bytes" in L.moe_last_error()
    bad = M.moe_dims(100, 128, 16, 2)
    assert r(ctypes.byref(bad), base, order, 4, 2, store, 12 * cold2, tiered, None) == 2


def test_cache_dry_run_follows_the_policy_model(L):
    """The expert cache's replacement decisions (dry run: policy only, no device) against the
    oracle's LRU model, step by step: hits, misses and the slot of every expert."""
    import oracle
    rng = np.random.default_rng(41)
    for E, K, n_slots, T in [(16, 2, 4, 1), (64, 4, 20, 3), (512, 4, 128, 1), (40, 8, 40, 2)]:
        dims = M.moe_dims(128, 64, E, K)
        host = [0x10000 + 0x100 * e for e in range(E)]
        c = M.ExpertCache(dims, host, [4 if e % 3 else 2 for e in range(E)], n_slots=n_slots, dry_run=True)
        model = oracle.ExpertCacheModel(E, n_slots)
        zipf = 1.0 / np.arange(1, E + 1) ** 1.1
        zipf /= zipf.sum()
        for step in range(400):
            idx = np.stack([rng.choice(E, size=K, replace=False, p=zipf) for _ in range(T)])
            if step % 50 == 7:
                idx[0, 0] = -1                       # ignored entries
            if step % 50 == 9:
                idx[-1, -1] = E + 3
            miss = c.fetch(idx)
            _, m_miss, _, _ = model.fetch(idx.reshape(-1))
            assert miss == m_miss, (E, step)
            assert [c.slot(e) for e in range(E)] == [model.slot_of.get(e, -1) for e in range(E)], (E, step)
        hits, misses, _ = c.stats()
        assert (hits, misses) == (model.hits, model.misses)
        # a dry-run cache has no device side: no state size, attach and device fetch refused
        assert L.moe_cache_device_state_bytes(c._c) == 0
        assert L.moe_cache_attach_device(c._c, FAKE, 1 << 20, None) == 8
        assert L.moe_cache_fetch_device(c._c, FAKE, 4, None) == 8
        assert L.moe_cache_device_refused(c._c) == -1
        c.close()


def test_cache_validates_and_refuses_oversized_steps(L):
    """Create refuses bad arguments before touching anything; a step naming more distinct experts
    than slots is refused and leaves the residency unchanged."""
    dims = M.moe_dims(128, 64, 8, 2)
    host = [0x10000 + 0x100 * e for e in range(8)]
    with pytest.raises(M.MoeError) as ei:
        M.ExpertCache(dims, host, [4] * 8, n_slots=1, dry_run=True)          # fewer slots than top_k
    assert ei.value.status == 2
    with pytest.raises(M.MoeError) as ei:
        M.ExpertCache(dims, host, [4] * 7 + [3], n_slots=4, dry_run=True)
    assert ei.value.status == 4
    with pytest.raises(M.MoeError) as ei:
        M.ExpertCache(dims, [0] + host[1:], [4] * 8, n_slots=4, dry_run=True)
    assert ei.value.status == 1
    P = ctypes.c_void_p
    out = P()
    hs = np.zeros((8, 2), dtype=np.uint64)
    hs[:, 0] = host
    hs[:, 1] = 4
    blob4 = L.moe_packed_expert_bytes(128, 64, 4)
    slot = (blob4 + 255) // 256 * 256
    args = (ctypes.byref(dims), P(hs.ctypes.data))
    assert L.moe_cache_create(*args, None, slot, 4, None, 0, None, ctypes.byref(out)) == 1   # no device buffers
    assert L.moe_cache_create(*args, P(0x100080), slot, 4, P(0x200000), 0, None, ctypes.byref(out)) == 5
    assert L.moe_cache_create(*args, P(0x100000), slot - 256, 4, P(0x200000), 0, None, ctypes.byref(out)) == 9
    assert L.moe_cache_create(*args, P(0x100000), slot, 4, P(0x200000), 4, None, ctypes.byref(out)) == 8
    assert not out.value
    c = M.ExpertCache(dims, host, [4] * 8, n_slots=3, dry_run=True)
    assert c.fetch([1, 2]) == 2
    with pytest.raises(M.MoeError) as ei:
        c.fetch([3, 4, 5, 6])
    assert ei.value.status == 2
    assert [c.slot(e) for e in range(8)] == [-1, 0, 1, -1, -1, -1, -1, -1]
    assert c.slot(8) == -2 and c.slot(-1) == -2
    assert c.fetch(np.array([], dtype=np.int32)) == 0
    c.close()
    assert L.moe_cache_fetch(None, None, 0, None, None) == 1
    L.moe_cache_destroy(None)


def test_injected_launch_failure_enqueues_nothing(L):
    """With the test hook armed, calls whose arguments pass validation return MOE_ERR_LAUNCH at their
    first launch step, before anything is enqueued (their fake device pointers are never touched);
    the hook counts down, and (0, 0) switches it off."""
    P = ctypes.c_void_p
    assert L.moe_debug_inject_launch_failure(-1, 1) == 2
    assert L.moe_debug_inject_launch_failure(0, 2) == 0
    try:
        assert L.moe_combine(P(0x100000), P(0x200000), 4, 2, 64, None, P(0x300000), None) == 7
        assert b"injected" in L.moe_last_error() and b"combine" in L.moe_last_error()
        assert L.moe_quantize_matrix(P(0x100000), M.MOE_F32, 4, 64, 4, P(0x200000), P(0x300000), None) == 7
        assert b"injected" in L.moe_last_error() and b"quantize" in L.moe_last_error()
        # validation still comes first: an invalid call fails as such and does not use up an injection
        assert L.moe_debug_inject_launch_failure(0, 1) == 0
        assert L.moe_combine(None, P(0x200000), 4, 2, 64, None, P(0x300000), None) == 1
        assert L.moe_combine(P(0x100000), P(0x200000), 4, 2, 64, None, P(0x300000), None) == 7
    finally:
        assert L.moe_debug_inject_launch_failure(0, 0) == 0
