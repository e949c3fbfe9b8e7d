"""GPU tests of the expert cache (store in pinned host memory, slots in device memory): a step
through the cache (route -> indices to the host -> fetch -> expert FFN -> combine) must give
exactly the outputs of the same kernels on the all-resident store, on the per-token and the
grouped path, with evictions; a few tokens are also checked against the oracle; an absent expert
(blob 0 in the table) gives zero rows on both paths."""
import sys

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import bit_expert_dequant_amd as M  # noqa: E402
import oracle  # noqa: E402
from moe_cases import (MIN_MARGIN, act_f64, act_tensor, assert_close, build_layer, oracle_layer,  # noqa: E402
                       small_workload)


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


class HostStore:
    """The layer's expert blobs copied to pinned host memory, with a cache over n_slots slots."""

    def __init__(self, dl, n_slots):
        wl = dl.wl
        self.host = torch.empty(dl.store.numel(), dtype=torch.uint8, pin_memory=True)
        self.host.copy_(dl.store)
        bits = wl.expert_bits().tolist()
        self.slots = torch.empty(n_slots * dl.stride, dtype=torch.uint8, device="cuda")
        self.table = torch.zeros_like(dl.table)
        self.dims = M.make_dims(wl.H, wl.I, wl.E, wl.K)
        self.cache = M.ExpertCache(self.dims, [self.host.data_ptr() + e * dl.stride for e in range(wl.E)], bits,
                                   self.slots, dl.stride, n_slots, self.table)
        self.L = M.Layer(dl.router, self.table, dl.logit_bias, dl.norm_w, wl.norm_eps)


def route(dl, x, T):
    wl = dl.wl
    d = M.make_dims(wl.H, wl.I, wl.E, wl.K)
    idx = torch.empty(T, wl.K, dtype=torch.int32, device="cuda")
    w = torch.empty(T, wl.K, dtype=torch.float32, device="cuda")
    M.moe_route(d, dl.L, x, idx, w, ws=M.workspace(M.MOE_OP_ROUTE, d, T, 1))
    return idx, w


def ffn(dims, L, x, idx, T, H, K):
    y = torch.full((T, K, H), float("nan"), dtype=torch.float32, device="cuda")
    M.moe_expert_ffn(dims, L, x, idx, y, M.workspace(M.MOE_OP_EXPERT_FFN, dims, T, 1))
    return y


@pytest.mark.parametrize("tiered", [False, True], ids=["4bit", "tiered"])
def test_cached_decode_matches_resident(tiered):
    """24 single-token steps over 16 experts with 3 slots (top-2): most steps evict."""
    wl = small_workload("cache_decode", 0xCAC1 + tiered, 512, 256, 16, 2, tiered=tiered, n_hot=6 if tiered else 0,
                        zipf=tiered)
    dl = build_layer(wl)
    hs = HostStore(dl, 3)
    ol = oracle_layer(wl)
    bank = wl.tokens_bank(24)
    total_miss = 0
    for t in range(24):
        x = act_tensor(wl, bank[t:t + 1])
        idx, w = route(dl, x, 1)
        idx_h = idx.cpu().numpy()
        total_miss += hs.cache.fetch(idx_h)
        y = ffn(hs.dims, hs.L, x, idx, 1, wl.H, wl.K)
        y_ref = ffn(hs.dims, dl.L, x, idx, 1, wl.H, wl.K)
        torch.cuda.synchronize()
        assert torch.equal(y, y_ref), f"token {t}: cached and resident outputs differ"
        if t % 6 == 0:
            out = torch.empty(1, wl.H, dtype=torch.float32, device="cuda")
            M.moe_combine(y, w, out)
            ref = oracle.layer_token(act_f64(wl, bank[t]), ol, wl.H, wl.I, wl.K)
            assert ref.margin > MIN_MARGIN
            assert list(idx_h[0]) == list(ref.idx)
            assert_close(out.cpu().numpy()[0], ref.out, f"token {t} out")
    hits, misses, nbytes = hs.cache.stats()
    say(f"[cache decode] hits {hits} misses {misses} bytes {nbytes}")
    assert misses == total_miss and misses > 3 and hits + misses >= 24


def test_cached_batched_matches_resident():
    """Batches of 32 tokens (grouped path) over 64 experts with 60 slots: evictions between batches."""
    wl = small_workload("cache_batched", 0xCAC3, 256, 128, 64, 2)
    dl = build_layer(wl)
    hs = HostStore(dl, 60)
    bank = wl.tokens_bank(32 * 5)
    for b in range(5):
        x = act_tensor(wl, bank[32 * b:32 * (b + 1)])
        idx, _ = route(dl, x, 32)
        idx_h = idx.cpu().numpy()
        if len(set(idx_h.reshape(-1).tolist())) > 60:
            continue
        hs.cache.fetch(idx_h)
        y = ffn(hs.dims, hs.L, x, idx, 32, wl.H, wl.K)
        y_ref = ffn(hs.dims, dl.L, x, idx, 32, wl.H, wl.K)
        torch.cuda.synchronize()
        assert torch.equal(y, y_ref), f"batch {b}: cached and resident outputs differ"
    hits, misses, _ = hs.cache.stats()
    say(f"[cache batched] hits {hits} misses {misses}")
    assert misses > 60


@pytest.mark.parametrize("T", [1, 32], ids=["per_token", "grouped"])
def test_absent_expert_gives_zero_rows(T):
    """Only some experts are fetched; indices naming absent experts give zero rows, the others
    match the resident store."""
    wl = small_workload("cache_absent", 0xCAC5, 256, 128, 16, 2)
    dl = build_layer(wl)
    hs = HostStore(dl, 8)
    hs.cache.fetch(np.arange(0, 16, 2))                  # even experts resident
    rng = np.random.default_rng(T)
    idx_h = np.stack([rng.choice(16, size=2, replace=False) for _ in range(T)]).astype(np.int32)
    idx = torch.from_numpy(idx_h).cuda()
    x = act_tensor(wl, wl.tokens_bank(T))
    y = ffn(hs.dims, hs.L, x, idx, T, wl.H, wl.K)
    y_ref = ffn(hs.dims, dl.L, x, idx, T, wl.H, wl.K)
    torch.cuda.synchronize()
    absent = torch.from_numpy(idx_h % 2 == 1).cuda()
    assert torch.all(y[absent] == 0)
    assert torch.equal(y[~absent], y_ref[~absent])


# --------------------------------------------------------------------------- device-side policy
def check_state(hs, model, dl, what):
    """The device state's residency equals the model's; table entries point at the slots; every
    resident slot holds its expert's blob byte for byte."""
    wl = dl.wl
    tab = hs.table.cpu().numpy().view(np.uint64).reshape(-1, 2)
    base = hs.slots.data_ptr()
    store = dl.store.cpu().numpy().reshape(wl.E, dl.stride)
    slots = hs.slots.cpu().numpy().reshape(-1, dl.stride)
    bits = wl.expert_bits()
    for e in range(wl.E):
        s = hs.cache.slot(e)
        assert s == model.slot_of.get(e, -1), f"{what}: expert {e} in slot {s}, model {model.slot_of.get(e, -1)}"
        if s < 0:
            assert tab[e, 0] == 0, f"{what}: absent expert {e} has a blob"
        else:
            assert tab[e, 0] == base + s * dl.stride and (tab[e, 1] & 0xFFFFFFFF) == bits[e], f"{what}: table {e}"
            nb = wl.blob_bytes(int(bits[e]))
            assert np.array_equal(slots[s, :nb], store[e, :nb]), f"{what}: slot {s} bytes of expert {e}"


def test_device_policy_matches_model():
    """The device policy against the oracle's cache model, step by step: 16 experts, 5 slots, top-2;
    three host fetches first (the state moves to the device with them), then 40 device steps of 1-2
    tokens with out-of-range indices, and two steps with more distinct experts than slots (refused)."""
    wl = small_workload("cache_device", 0xCAC7, 256, 128, 16, 2)
    dl = build_layer(wl)
    hs = HostStore(dl, 5)
    model = oracle.ExpertCacheModel(16, 5)
    rng = np.random.default_rng(7)
    for step in ([0, 3], [3, 5, 7], [9, 0]):
        hs.cache.fetch(np.array(step, dtype=np.int32))
        model.fetch(step)
    hs.cache.attach_device()
    check_state(hs, model, dl, "after attach")
    with pytest.raises(M.MoeError):
        hs.cache.fetch(np.array([1], dtype=np.int32))          # the host policy is off now
    refused = 0
    for t in range(40):
        T = int(rng.integers(1, 3))
        idx_h = rng.integers(-2, 18, size=(T, 2)).astype(np.int32)
        if t in (11, 27):
            idx_h = np.arange(12, dtype=np.int32).reshape(6, 2)  # 12 distinct > 5 slots
        try:
            model.fetch(idx_h.reshape(-1))
        except ValueError:
            refused += 1
        h0, m0, _ = hs.cache.stats()
        hs.cache.fetch_device(torch.from_numpy(idx_h).cuda())
        torch.cuda.synchronize()
        h1, m1, _ = hs.cache.stats()
        assert (h1, m1) == (model.hits, model.misses), f"step {t}: hits/misses {(h1, m1)} vs model"
        check_state(hs, model, dl, f"step {t}")
    assert hs.cache.refused() == refused and refused == 2
    say(f"[cache device] hits {model.hits} misses {model.misses}")


@pytest.mark.parametrize("T", [1, 32], ids=["decode", "grouped"])
def test_device_fetch_matches_resident(T):
    """Route on the device -> device fetch -> expert FFN through the cache table, with no host step:
    outputs equal the resident store's byte for byte (decode steps over 16 experts with 3 slots;
    batches of 32 over 64 experts with 60 slots)."""
    if T == 1:
        wl = small_workload("cache_dev_decode", 0xCAC9, 512, 256, 16, 2, tiered=True, n_hot=6, zipf=True)
        n_slots, steps = 3, 24
    else:
        wl = small_workload("cache_dev_batched", 0xCACB, 256, 128, 64, 2)
        n_slots, steps = 60, 5
    dl = build_layer(wl)
    hs = HostStore(dl, n_slots)
    hs.cache.attach_device()
    bank = wl.tokens_bank(T * steps)
    done = 0
    for t in range(steps):
        x = act_tensor(wl, bank[T * t:T * (t + 1)])
        idx, _ = route(dl, x, T)
        if T > 1 and len(set(idx.cpu().numpy().reshape(-1).tolist())) > n_slots:
            continue
        hs.cache.fetch_device(idx)
        y = ffn(hs.dims, hs.L, x, idx, T, wl.H, wl.K)
        y_ref = ffn(hs.dims, dl.L, x, idx, T, wl.H, wl.K)
        torch.cuda.synchronize()
        assert torch.equal(y, y_ref), f"step {t}: cached and resident outputs differ"
        done += 1
    hits, misses, nbytes = hs.cache.stats()
    say(f"[cache device T={T}] steps {done} hits {hits} misses {misses} bytes {nbytes}")
    assert done >= 3 and misses > n_slots
