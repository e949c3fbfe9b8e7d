"""GPU parity of the shared-read expert FFN (moe_expert_ffn_path with MOE_FFN_SHARED: 2 <= T <= 16
tokens, each distinct expert of the call streamed once for every (token, slot) pair that chose it)
against the CPU oracle, for every (token, slot) row of y.

Routings: the router's own choice on seeded tokens (mostly distinct experts), draft-style tokens
that share K-1 experts with the first token and differ in one, and tokens that all choose the same
K experts (every expert staged with T rows).  Up to four tokens without a norm weight every
workgroup stages its rows from x itself; otherwise one launch stages them for all.  Plus the edge
cases of the in-kernel expert list:
an expert chosen by more pairs than a workgroup stages, repeated experts within a token,
indices outside [0, E) and absent experts (zero rows), 2-bit and tiered experts, fp32 and
normalised activations, ragged and widest rows."""
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


def run_ffn(d, dl, x, idx, path, fill=float("nan")):
    T, K = idx.shape
    y = torch.full((T, K, d.hidden), fill, dtype=torch.float32, device="cuda")
    M.moe_expert_ffn(d, dl.L, x, idx, y, M.workspace(M.MOE_OP_EXPERT_FFN, d, T), path=path)
    torch.cuda.synchronize()
    return y.cpu().numpy()


def check_rows(wl, ol, x64, idx_h, y, what, absent=()):
    """Every (token, slot) row against the oracle's expert on that token's (normalised) row."""
    outs = {}
    for t in range(idx_h.shape[0]):
        n = oracle.rmsnorm(x64[t], ol.norm_w, ol.norm_eps) if ol.norm_w is not None else x64[t]
        for k in range(idx_h.shape[1]):
            e = int(idx_h[t, k])
            if e < 0 or e >= wl.E or e in absent:
                assert np.all(y[t, k] == 0.0), f"{what}: token {t} slot {k} (expert {e}) not a zero row"
                continue
            key = (t, e)
            if key not in outs:
                outs[key] = oracle.expert(ol.blob(e), ol.bits(e), wl.H, wl.I, n)[3]
            assert_close(y[t, k], outs[key], f"{what}: token {t} slot {k} expert {e}")


@pytest.fixture(scope="module")
def cfg1():
    wl = synth.WORKLOADS[1]
    say(f"[shared] building {wl.name}")
    dl = build_layer(wl)
    ol = oracle_layer(wl)
    yield wl, dl, ol
    del dl
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


@pytest.mark.parametrize("T", [2, 4, 8, 16])
@pytest.mark.parametrize("kind", ["router", "draft", "same"])
def test_shared_read_config1(cfg1, T, kind):
    wl, dl, ol = cfg1
    say(f"[shared] config 1 T={T} routing={kind}")
    bank = wl.tokens_bank(T)
    x = act_tensor(wl, bank)
    d = M.make_dims(wl.H, wl.I, wl.E, wl.K)
    ridx = torch.empty(T, wl.K, dtype=torch.int32, device="cuda")
    rw = torch.empty(T, wl.K, dtype=torch.float32, device="cuda")
    M.moe_route(d, dl.L, x, ridx, rw, ws=M.workspace(M.MOE_OP_ROUTE, d, T))
    torch.cuda.synchronize()
    base = ridx.cpu().numpy()
    x64 = act_f64(wl, bank)
    if kind == "router":
        for t in range(T):
            ri, _, margin = oracle.route(oracle.router_logits(ol.router, x64[t], ol.logit_bias, wl.router_bf16), wl.K)
            assert margin > MIN_MARGIN and list(base[t]) == list(ri), f"token {t}"
    idx_h = synth.shared_routing(kind, base, wl.E)
    idx = torch.from_numpy(idx_h).to("cuda")
    y = run_ffn(d, dl, x, idx, M.MOE_FFN_SHARED)
    say(f"[shared]   {len(set(idx_h.reshape(-1).tolist()))} distinct experts over {T * wl.K} pairs")
    check_rows(wl, ol, x64, idx_h, y, f"T={T} {kind}")
    # it repeats byte for byte, and from 8 tokens it is the automatic choice
    assert np.array_equal(run_ffn(d, dl, x, idx, M.MOE_FFN_SHARED), y)
    if T >= 8:
        assert np.array_equal(run_ffn(d, dl, x, idx, M.MOE_FFN_AUTO), y)


def test_shared_read_repeated_and_missing_experts(cfg1):
    """An expert chosen by all 64 pairs (four workgroup records of 16 rows), experts repeated inside
    a token, indices outside [0, E) and an absent expert (blob 0 in a copy of the table)."""
    wl, dl, ol = cfg1
    d = M.make_dims(wl.H, wl.I, wl.E, wl.K)
    for T in (16, 4):        # 16: four records of 16 pairs (staged rows); 4: two of 8 (rows staged in-kernel)
        bank = wl.tokens_bank(T)
        x, x64 = act_tensor(wl, bank), act_f64(wl, bank)
        idx_h = np.full((T, wl.K), 300, dtype=np.int32)
        y = run_ffn(d, dl, x, torch.from_numpy(idx_h).to("cuda"), M.MOE_FFN_SHARED)
        check_rows(wl, ol, x64, idx_h, y, f"one expert, {T * wl.K} pairs")

    T = 5
    idx_h = np.array([[7, 7, 8, 9], [-1, 7, 500, 511], [9, 9, 9, 9], [512, 3, 1 << 30, 7], [8, 500, 3, 2]],
                     dtype=np.int32)
    table = dl.table.clone()
    tv = table.view(torch.int64).view(-1, 2)
    tv[500, 0] = 0                                  # expert 500 absent
    L2 = M.Layer(dl.router, table, dl.logit_bias, dl.norm_w, wl.norm_eps)

    class _DL:
        pass
    dl2 = _DL()
    dl2.L = L2
    bank = wl.tokens_bank(T)
    x, x64 = act_tensor(wl, bank), act_f64(wl, bank)
    y = run_ffn(d, dl2, x, torch.from_numpy(idx_h).to("cuda"), M.MOE_FFN_SHARED, fill=7.0)
    check_rows(wl, ol, x64, idx_h, y, "repeats and missing", absent={500})
    del table


SMALL = [
    # name, T, H, I, E, K, bits, extra
    ("t3_h512_i256_e8_k2_2b", 3, 512, 256, 8, 2, 2, {}),
    ("t3_h1024_i512_e16_k4_norm_staged", 3, 1024, 512, 16, 4, 4, {"norm": True}),
    ("t4_h1024_i512_e16_k4_fp32_direct", 4, 1024, 512, 16, 4, 4, {"x_bf16": False}),
    ("t6_h1024_i512_e16_k4_tiered_fp32", 6, 1024, 512, 16, 4, 4, {"tiered": True, "n_hot": 5, "x_bf16": False}),
    ("t9_h192_i320_e5_k3_ragged", 9, 192, 320, 5, 3, 4, {}),
    ("t12_h2048_i768_e40_k4_norm", 12, 2048, 768, 40, 4, 4, {"norm": True}),
    ("t16_h3072_i2048_e24_k4_partial_slots", 16, 3072, 2048, 24, 4, 4, {}),
    ("t6_h8192_i256_e12_k4_widest", 6, 8192, 256, 12, 4, 4, {}),
    ("t2_h4096_i1024_e2048_k8_max_experts", 2, 4096, 1024, 2048, 8, 2, {"zipf": True}),
]


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_shared_read_shapes(case):
    name, T, H, I, E, K, bits, extra = case
    say(f"[shared] {name}")
    wl = small_workload(name, 0x5A4E + T + H + I + E, H, I, E, K, bits, **extra)
    dl = build_layer(wl)
    ol = oracle_layer(wl)
    bank = wl.tokens_bank(T)
    x, x64 = act_tensor(wl, bank), act_f64(wl, bank)
    d = M.make_dims(H, I, E, K)
    idx = torch.empty(T, K, dtype=torch.int32, device="cuda")
    w = torch.empty(T, K, dtype=torch.float32, device="cuda")
    M.moe_route(d, dl.L, x, idx, w, ws=M.workspace(M.MOE_OP_ROUTE, d, T))
    torch.cuda.synchronize()
    idx_h = idx.cpu().numpy()
    y = run_ffn(d, dl, x, idx, M.MOE_FFN_SHARED)
    check_rows(wl, ol, x64, idx_h, y, name)
    # the per-token kernels on the same routing agree within the same tolerance
    y_pt = run_ffn(d, dl, x, idx, M.MOE_FFN_PER_TOKEN)
    for t in range(T):
        for k in range(K):
            assert_close(y[t, k], y_pt[t, k], f"{name} shared vs per-token, token {t} slot {k}")


def test_shared_read_graph_replays(cfg1):
    """The shared-read launches captured in a HIP graph: replays with eager work in between, each
    equal byte for byte to the eager result."""
    wl, dl, ol = cfg1
    d = M.make_dims(wl.H, wl.I, wl.E, wl.K)
    T = 4
    bank = wl.tokens_bank(T)
    x = act_tensor(wl, bank)
    idx_h = np.array([[1, 2, 3, 4], [1, 2, 3, 5], [1, 2, 6, 4], [9, 2, 3, 4]], dtype=np.int32)
    idx = torch.from_numpy(idx_h).to("cuda")
    eager = run_ffn(d, dl, x, idx, M.MOE_FFN_SHARED)
    ws = M.workspace(M.MOE_OP_EXPERT_FFN, d, T)
    y = torch.full((T, wl.K, wl.H), float("nan"), dtype=torch.float32, device="cuda")
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        M.moe_expert_ffn(d, dl.L, x, idx, y, ws, stream=s, path=M.MOE_FFN_SHARED)
    for r in range(3):
        y.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(y.cpu().numpy(), eager), f"replay {r}"
        run_ffn(d, dl, x, idx, M.MOE_FFN_PER_TOKEN)          # eager work between replays
