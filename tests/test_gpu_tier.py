"""GPU parity of the tiered-store policy calls against the CPU oracle, through the C ABI:
moe_expert_usage (counts bit-exact), moe_hot_order (order bit-exact), moe_retier (every code and
(scale, bias) pair of the requantised cold experts bit-exact, the tiered table exact), and a decode
through a re-tiered table against the oracle (the decode path's tolerance)."""
import sys

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import bit_expert_dequant_amd as M  # noqa: E402
import oracle  # noqa: E402
import synth  # noqa: E402
from moe_cases import (MIN_MARGIN, act_f64, act_tensor, assert_close, build_layer, oracle_layer,  # noqa: E402
                       small_workload)


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def unpack_codes(plane: np.ndarray, rows: int, cols: int, bits: int) -> np.ndarray:
    per = 8 // bits
    b = plane.reshape(rows, cols // per)
    out = np.empty((rows, cols), dtype=np.uint8)
    for k in range(per):
        out[:, k::per] = (b >> (k * bits)) & ((1 << bits) - 1)
    return out


def pack_blob(mats, H: int, I: int, bits: int) -> np.ndarray:
    """(codes, scale, bias) of gate, up, down -> a packed blob (the tests' own packer)."""
    off, tot = synth.blob_layout(H, I, bits)
    blob = np.zeros(tot, dtype=np.uint8)
    per = 8 // bits
    for m, (codes, scale, bias) in enumerate(mats):
        rows, cols = codes.shape
        plane = np.zeros((rows, cols // per), dtype=np.uint8)
        for k in range(per):
            plane |= (codes[:, k::per] << (k * bits)).astype(np.uint8)
        sb = np.stack([scale, bias], axis=-1).astype(np.uint16).reshape(-1).view(np.uint8)
        blob[off[2 * m]:off[2 * m] + plane.size] = plane.reshape(-1)
        blob[off[2 * m + 1]:off[2 * m + 1] + sb.size] = sb
    return blob


def table_host(table) -> np.ndarray:
    """Descriptor table tensor -> uint64 [E][2] (blob, bits | reserved << 32)."""
    return table.cpu().numpy().view(np.uint64).reshape(-1, 2)


def check_cold_blob(gpu_blob: np.ndarray, base_blob: np.ndarray, H: int, I: int, bits_in: int, bits_out: int,
                    what: str):
    ref = oracle.requantize_expert(base_blob, H, I, bits_in, bits_out)
    off, _ = synth.blob_layout(H, I, bits_out)
    sizes = synth.plane_sizes(H, I, bits_out)
    for m, (rows, cols) in enumerate([(I, H), (I, H), (H, I)]):
        codes = unpack_codes(gpu_blob[off[2 * m]:off[2 * m] + sizes[2 * m]], rows, cols, bits_out)
        sb = gpu_blob[off[2 * m + 1]:off[2 * m + 1] + sizes[2 * m + 1]].view(np.uint16).reshape(rows, cols // 64, 2)
        rc, rs, rb = ref[m]
        bad = np.argwhere(codes != rc)
        assert bad.size == 0, f"{what} matrix {m}: {len(bad)} codes differ, first at {tuple(bad[0])}"
        assert np.array_equal(sb[:, :, 0], rs), f"{what} matrix {m}: scales differ"
        assert np.array_equal(sb[:, :, 1], rb), f"{what} matrix {m}: biases differ"


# --------------------------------------------------------------------------- usage
@pytest.mark.parametrize("E,shape", [(8, (300, 4)), (512, (256, 4)), (2048, (1 << 20) + 37), (1, (5, 3))])
def test_expert_usage_matches_oracle(E, shape):
    """Two calls accumulate; entries outside [0, E) are skipped; the large stream spans many
    workgroups (grid-stride loop and the global flush)."""
    say(f"[usage] E={E} shape={shape}")
    rng = np.random.default_rng(E + 1)
    a = rng.integers(-2, E + 2, size=shape).astype(np.int32)
    b = rng.integers(0, E, size=shape).astype(np.int32)
    counts = torch.zeros(E, dtype=torch.int32, device="cuda")
    M.moe_expert_usage(torch.from_numpy(a).cuda(), E, counts)
    M.moe_expert_usage(torch.from_numpy(b).cuda(), E, counts)
    torch.cuda.synchronize()
    ref = oracle.expert_usage(a, E) + oracle.expert_usage(b, E)
    assert np.array_equal(counts.cpu().numpy().astype(np.int64), ref)


def test_expert_usage_empty_stream():
    counts = torch.full((16,), 3, dtype=torch.int32, device="cuda")
    M.moe_expert_usage(torch.empty(0, dtype=torch.int32, device="cuda"), 16, counts)
    torch.cuda.synchronize()
    assert counts.cpu().tolist() == [3] * 16


# --------------------------------------------------------------------------- hot order
@pytest.mark.parametrize("E,kind", [(1, "small"), (7, "small"), (512, "ties"), (1000, "ties"), (2048, "ties"),
                                    (512, "wide"), (300, "zero")])
def test_hot_order_matches_oracle(E, kind):
    say(f"[order] E={E} {kind}")
    rng = np.random.default_rng(E + 7)
    if kind == "small":
        counts = rng.integers(0, 100, size=E)
    elif kind == "ties":
        counts = rng.integers(0, 5, size=E)
    elif kind == "wide":
        counts = rng.integers(0, 2 ** 32, size=E, dtype=np.uint64)
        counts[:4] = [2 ** 32 - 1, 0, 2 ** 32 - 1, 2 ** 31]
    else:
        counts = np.zeros(E, dtype=np.int64)
    c32 = counts.astype(np.uint32)
    dev = torch.from_numpy(c32.view(np.int32)).cuda()
    order = torch.full((E,), -1, dtype=torch.int32, device="cuda")
    M.moe_hot_order(dev, order)
    torch.cuda.synchronize()
    assert np.array_equal(order.cpu().numpy(), oracle.hot_order(c32.astype(np.int64)))


# --------------------------------------------------------------------------- re-tier
def _base_layer(H, I, E, seed, two_bit_every=0):
    """Base store on the device (host-generated blobs, one stride), its table and the host blobs."""
    bits = [2 if two_bit_every and e % two_bit_every == 0 else 4 for e in range(E)]
    stride = synth.blob_layout(H, I, 4)[1]
    host = np.zeros((E, stride), dtype=np.uint8)
    blobs = []
    for e in range(E):
        b = synth.expert_blob(seed, 0, e, H, I, bits[e])
        host[e, :b.size] = b
        blobs.append(b)
    store = torch.from_numpy(host.reshape(-1)).cuda()
    table = M.expert_table([store.data_ptr() + e * stride for e in range(E)], bits)
    return store, table, blobs, bits


@pytest.mark.parametrize("cold_bits,two_bit_every,in_place", [(2, 0, False), (2, 5, False), (4, 3, False),
                                                              (2, 4, True)],
                         ids=["4to2", "mixed_to2", "mixed_to4", "in_place"])
def test_retier_small_matches_oracle(cold_bits, two_bit_every, in_place):
    H, I, E, K, n_hot = 320, 192, 24, 2, 9
    say(f"[retier] H={H} I={I} E={E} n_hot={n_hot} cold={cold_bits} mixed={two_bit_every} in_place={in_place}")
    store, table, blobs, bits = _base_layer(H, I, E, 0x7E1, two_bit_every)
    base_host = table_host(table)
    order_np = np.random.default_rng(5).permutation(E).astype(np.int32)
    order = torch.from_numpy(order_np).cuda()
    cold_bytes = synth.blob_layout(H, I, cold_bits)[1]
    cold = torch.full(((E - n_hot) * cold_bytes,), 0xA5, dtype=torch.uint8, device="cuda")
    tiered = table if in_place else torch.zeros_like(table)
    M.moe_retier(M.make_dims(H, I, E, K), table, order, n_hot, cold_bits, cold, tiered)
    torch.cuda.synchronize()
    t = table_host(tiered)
    cold_host = cold.cpu().numpy()
    for r, e in enumerate(order_np.tolist()):
        if r < n_hot:
            assert t[e, 0] == base_host[e, 0] and t[e, 1] == base_host[e, 1], f"hot expert {e}"
        else:
            slot = r - n_hot
            assert t[e, 0] == cold.data_ptr() + slot * cold_bytes and t[e, 1] == cold_bits, f"cold expert {e}"
            check_cold_blob(cold_host[slot * cold_bytes:(slot + 1) * cold_bytes], blobs[e], H, I, bits[e], cold_bits,
                            f"expert {e} (rank {r})")
    assert M.lib().moe_check_experts(M._tptr(tiered), E) == 0


def test_retier_all_hot_writes_table_only():
    H, I, E = 128, 64, 6
    store, table, _, _ = _base_layer(H, I, E, 0x7E2)
    order = torch.arange(E, dtype=torch.int32, device="cuda").flip(0).contiguous()
    tiered = torch.zeros_like(table)
    M.moe_retier(M.make_dims(H, I, E, 2), table, order, E, 2, None, tiered)
    torch.cuda.synchronize()
    assert np.array_equal(table_host(tiered), table_host(table))


def test_retier_full_size_sampled():
    """512 experts of 4096 x 1024 at 4 bits, 128 hot (ranked from seeded Zipf-like counts), 384
    requantised to 2 bits in one call: the whole table, and the first, a middle and the last cold
    expert bit-exact against the oracle."""
    H, I, E, K, n_hot = 4096, 1024, 512, 4, 128
    say("[retier] full size: filling the base store")
    stride = synth.blob_layout(H, I, 4)[1]
    base = torch.empty(E * stride, dtype=torch.uint8, device="cuda")
    seed = synth.config_seed(2)
    synth.fill_blobs_device(base.data_ptr(), stride, E, 0, 0, seed, H, I, 4,
                            torch.cuda.current_stream().cuda_stream)
    table = M.expert_table([base.data_ptr() + e * stride for e in range(E)], [4] * E)
    rng = np.random.default_rng(9)
    counts = (1e5 * rng.permutation(np.arange(1, E + 1) ** -1.1)).astype(np.uint32)
    order_np = oracle.hot_order(counts.astype(np.int64))
    order = torch.from_numpy(order_np).cuda()
    cold_bytes = synth.blob_layout(H, I, 2)[1]
    cold = torch.empty((E - n_hot) * cold_bytes, dtype=torch.uint8, device="cuda")
    tiered = torch.zeros_like(table)
    say("[retier] full size: re-tiering")
    M.moe_retier(M.make_dims(H, I, E, K), table, order, n_hot, 2, cold, tiered)
    torch.cuda.synchronize()
    t = table_host(tiered)
    for r, e in enumerate(order_np.tolist()):
        want = (base.data_ptr() + e * stride, 4) if r < n_hot else (cold.data_ptr() + (r - n_hot) * cold_bytes, 2)
        assert (int(t[e, 0]), int(t[e, 1])) == want, f"rank {r} expert {e}"
    for r in [n_hot, n_hot + 191, E - 1]:
        e = int(order_np[r])
        slot = r - n_hot
        say(f"[retier] full size: checking rank {r} expert {e}")
        gpu = cold[slot * cold_bytes:(slot + 1) * cold_bytes].cpu().numpy()
        check_cold_blob(gpu, synth.expert_blob(seed, 0, e, H, I, 4), H, I, 4, 2, f"expert {e} (rank {r})")


def test_decode_through_retiered_table():
    """A layer re-tiered to hot 4-bit / cold 2-bit decodes like the oracle layer whose cold experts
    are the oracle's requantised blobs (routing indices exact, outputs within the tolerance)."""
    wl = small_workload("retier_decode", 0x7E3, 512, 256, 16, 2, zipf=True)
    dl = build_layer(wl)
    E, n_hot = wl.E, 6
    order_np = np.random.default_rng(3).permutation(E).astype(np.int32)
    cold_bytes = synth.blob_layout(wl.H, wl.I, 2)[1]
    cold = torch.empty((E - n_hot) * cold_bytes, dtype=torch.uint8, device="cuda")
    tiered = torch.zeros_like(dl.table)
    M.moe_retier(M.make_dims(wl.H, wl.I, E, wl.K), dl.table, torch.from_numpy(order_np).cuda(), n_hot, 2, cold,
                 tiered)
    L = M.Layer(dl.router, tiered, dl.logit_bias, dl.norm_w, wl.norm_eps)
    ol = oracle_layer(wl)
    rank = {int(e): r for r, e in enumerate(order_np)}
    cold_blobs = {}

    def blob(e):
        e = int(e)
        if rank[e] < n_hot:
            return ol.blob(e)
        if e not in cold_blobs:
            cold_blobs[e] = pack_blob(oracle.requantize_expert(ol.blob(e), wl.H, wl.I, 4, 2), wl.H, wl.I, 2)
        return cold_blobs[e]

    ot = oracle.LayerWeights(router=ol.router, router_is_bf16=ol.router_is_bf16, blob=blob,
                             bits=lambda e: 4 if rank[int(e)] < n_hot else 2, logit_bias=ol.logit_bias,
                             norm_w=ol.norm_w, norm_eps=ol.norm_eps)
    bank = wl.tokens_bank(6)
    d = M.make_dims(wl.H, wl.I, E, wl.K)
    ws = M.workspace(M.MOE_OP_LAYER_DECODE, d, 1, 1)
    for t in range(bank.shape[0]):
        x = act_tensor(wl, bank[t])
        out = torch.empty(wl.H, dtype=torch.float32, device="cuda")
        idx = torch.empty(wl.K, dtype=torch.int32, device="cuda")
        w = torch.empty(wl.K, dtype=torch.float32, device="cuda")
        M.moe_layer_decode(d, [L], x, out, idx, w, ws=ws)
        torch.cuda.synchronize()
        ref = oracle.layer_token(act_f64(wl, bank[t]), ot, wl.H, wl.I, wl.K)
        assert ref.margin > MIN_MARGIN, f"token {t}: routing margin {ref.margin:.2e} too small to compare"
        assert list(idx.cpu().numpy()) == list(ref.idx), f"token {t}"
        assert_close(out.cpu().numpy(), ref.out, f"token {t} out")
