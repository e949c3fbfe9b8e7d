"""GPU parity of the batched path (moe_expert_ffn with T >= 2: grouping by expert + MFMA grouped
dequant-GEMM, then moe_combine) against the CPU oracle, for every (token, slot)."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import bit_expert_dequant_amd as M  # noqa: E402
import oracle  # noqa: E402
from moe_cases import (MIN_MARGIN, act_f64, act_tensor, assert_close, build_layer, oracle_layer,  # noqa: E402
                       small_workload)


class ExpertCache:
    """The oracle's dequantised matrices per expert, reused across tokens."""

    def __init__(self, wl, ol):
        self.wl, self.ol, self.m = wl, ol, {}

    def y(self, e, n):
        if e not in self.m:
            self.m[e] = oracle.expert_matrices(self.ol.blob(e), self.wl.H, self.wl.I, self.ol.bits(e))
        Wg, Wu, Wd = self.m[e]
        g, u = oracle.matvec(Wg, n), oracle.matvec(Wu, n)
        h = np.array([oracle.silu(z) for z in g]) * u
        return oracle.matvec(Wd, h)


BATCH = [
    # name, T, H, I, E, K, bits, extra
    ("t2_h512_i256_e8_k2", 2, 512, 256, 8, 2, 4, {}),
    ("t7_h192_i320_e5_k2_ragged", 7, 192, 320, 5, 2, 4, {}),
    ("t33_h1024_i512_e16_k4_norm", 33, 1024, 512, 16, 4, 4, {"norm": True}),
    ("t64_h2048_i768_e8_k8_2b", 64, 2048, 768, 8, 8, 2, {}),
    ("t40_h4096_i1024_e20_k4_tiered_fp32", 40, 4096, 1024, 20, 4, 4, {"tiered": True, "n_hot": 7, "x_bf16": False}),
    ("t100_h640_i1344_e3_k3_multitile", 100, 640, 1344, 3, 3, 4, {}),
    # above 24 tokens, experts with few tokens take the integer dot-product kernels: 2-bit only, a
    # wide row (four slots per lane), a mix around the eight-token boundary with fp32 activations,
    # and partial slots
    ("t48_h1024_i512_e64_k2_2b_few", 48, 1024, 512, 64, 2, 2, {}),
    ("t30_h8192_i256_e24_k2_wide", 30, 8192, 256, 24, 2, 4, {}),
    ("t32_h2048_i576_e12_k3_fp32_boundary", 32, 2048, 576, 12, 3, 4, {"x_bf16": False}),
    ("t32_h3072_i2048_e24_k3_partial_slots", 32, 3072, 2048, 24, 3, 4, {}),
    # up to 24 tokens the decode kernels run one grid row per token
    ("t24_h4096_i1024_e40_k4_per_token", 24, 4096, 1024, 40, 4, 4, {"tiered": True, "n_hot": 12}),
    ("t5_h1024_i512_e16_k4_norm_per_token", 5, 1024, 512, 16, 4, 4, {"norm": True, "x_bf16": False}),
    # from 64 tokens the router runs as MFMA tiles; with a norm weight on normalised fp32 rows
    ("t80_h1024_i256_e32_k4_norm_mfma_router", 80, 1024, 256, 32, 4, 4, {"norm": True}),
    # the limits: K * I at the LDS bound (K = 8), and the widest intermediate
    ("t30_h512_i4608_e12_k8_lds_limit", 30, 512, 4608, 12, 8, 4, {}),
    ("t40_h256_i8192_e8_k4_2b_max_inter", 40, 256, 8192, 8, 4, 2, {}),
]


@pytest.mark.parametrize("case", BATCH, ids=[c[0] for c in BATCH])
def test_batched_expert_ffn(case):
    name, T, H, I, E, K, bits, extra = case
    print(f"[batched] {name}", flush=True)
    wl = small_workload(name, 0xBA7C + T + H + I, H, I, E, K, bits, **extra)
    dl = build_layer(wl)
    ol = oracle_layer(wl)
    bank = wl.tokens_bank(T)
    x = act_tensor(wl, bank)
    d = M.make_dims(H, I, E, K)
    idx = torch.empty(T, K, dtype=torch.int32, device="cuda")
    w = torch.empty(T, K, dtype=torch.float32, device="cuda")
    M.moe_route(d, dl.L, x, idx, w, ws=M.workspace(M.MOE_OP_ROUTE, d, T))
    y = torch.full((T, K, H), float("nan"), dtype=torch.float32, device="cuda")
    M.moe_expert_ffn(d, dl.L, x, idx, y, M.workspace(M.MOE_OP_EXPERT_FFN, d, T))
    out = torch.empty(T, H, dtype=torch.float32, device="cuda")
    M.moe_combine(y, w, out)
    torch.cuda.synchronize()
    idx_h, w_h, y_h, out_h = idx.cpu().numpy(), w.cpu().numpy(), y.cpu().numpy(), out.cpu().numpy()
    cache = ExpertCache(wl, ol)
    x64 = act_f64(wl, bank)
    for t in range(T):
        n = oracle.rmsnorm(x64[t], ol.norm_w, ol.norm_eps) if ol.norm_w is not None else x64[t]
        lg = oracle.router_logits(ol.router, n, ol.logit_bias, wl.router_bf16)
        ri, rw, margin = oracle.route(lg, K)
        assert margin > MIN_MARGIN
        assert list(idx_h[t]) == list(ri), f"token {t}"
        ys = np.stack([cache.y(int(e), n) for e in ri])
        for k in range(K):
            assert_close(y_h[t, k], ys[k], f"{name} token {t} slot {k}")
        assert_close(out_h[t], oracle.combine(ys, rw), f"{name} token {t} out")


def test_batched_deterministic_and_given_routing():
    """Same inputs twice give identical bytes; caller-chosen routing with repeated experts and an
    out-of-range index (zero rows)."""
    wl = small_workload("det_b", 5150, 512, 256, 6, 3, 4)
    dl = build_layer(wl)
    ol = oracle_layer(wl)
    T = 9
    x = act_tensor(wl, wl.tokens_bank(T))
    d = M.make_dims(wl.H, wl.I, wl.E, wl.K)
    idx = torch.tensor([[0, 1, 2]] * 4 + [[5, 0, 9]] + [[3, 4, 5]] * 4, dtype=torch.int32, device="cuda")
    ws = M.workspace(M.MOE_OP_EXPERT_FFN, d, T)
    ys = []
    for _ in range(2):
        y = torch.full((T, 3, wl.H), 7.0, dtype=torch.float32, device="cuda")
        M.moe_expert_ffn(d, dl.L, x, idx, y, ws)
        torch.cuda.synchronize()
        ys.append(y.cpu().numpy())
    assert np.array_equal(ys[0], ys[1])
    y = ys[0]
    assert np.all(y[4, 2] == 0.0)              # out-of-range index: zero row
    x64 = act_f64(wl, wl.tokens_bank(T))
    cache = ExpertCache(wl, ol)
    for t in range(T):
        for k in range(3):
            e = int(idx[t, k])
            if 0 <= e < wl.E:
                assert_close(y[t, k], cache.y(e, x64[t]), f"token {t} slot {k} expert {e}")


def test_batched_small_records_every_count():
    """Given routing where experts 0..8 receive 1..9 tokens (every record size of the small-expert
    list, and at 9 an MFMA tile) and experts 9..13 nine tokens each in the second slot; every
    (token, slot) row against the oracle."""
    wl = small_workload("recs_b", 5151, 1024, 512, 16, 2, 4)
    dl = build_layer(wl)
    ol = oracle_layer(wl)
    T = 45
    first = np.repeat(np.arange(9), np.arange(1, 10))              # expert e for e + 1 tokens
    second = 9 + np.arange(T) % 5
    idx_h = np.stack([first, second], axis=1).astype(np.int32)
    x = act_tensor(wl, wl.tokens_bank(T))
    d = M.make_dims(wl.H, wl.I, wl.E, wl.K)
    y = torch.full((T, 2, wl.H), float("nan"), dtype=torch.float32, device="cuda")
    M.moe_expert_ffn(d, dl.L, x, torch.from_numpy(idx_h).to("cuda"), y, M.workspace(M.MOE_OP_EXPERT_FFN, d, T),
                     path=M.MOE_FFN_GROUPED)
    torch.cuda.synchronize()
    y = y.cpu().numpy()
    x64 = act_f64(wl, wl.tokens_bank(T))
    cache = ExpertCache(wl, ol)
    for t in range(T):
        for k in range(2):
            e = int(idx_h[t, k])
            assert_close(y[t, k], cache.y(e, x64[t]), f"token {t} slot {k} expert {e}")


ROUTER_CASES = [
    # name, T, H, E, extra: MFMA tiles from 64 tokens (bf16 rows; normalised fp32 rows split into
    # hi + lo; ragged token and expert tiles), the matvec router below.  The MFMA router splits K
    # over workgroups (8, 4, 2 and, above 512 experts, 2 partial rows summed by the top-K kernel).
    ("t64_h4096_e512_bf16_tiles", 64, 4096, 512, {}),
    ("t96_h1024_e40_norm_split_ragged", 96, 1024, 40, {"norm": True}),
    ("t70_h512_e8_fp32_split", 70, 512, 8, {"x_bf16": False}),
    ("t64_h2048_e1024_wide", 64, 2048, 1024, {}),
    ("t8_h4096_e512_matvec", 8, 4096, 512, {"zipf": True}),
]


@pytest.mark.parametrize("ws_kind", ["full", "no_split_room"])
@pytest.mark.parametrize("case", ROUTER_CASES, ids=[c[0] for c in ROUTER_CASES])
def test_batched_router_logits(case, ws_kind):
    """moe_route's logits for T tokens against the oracle's, element by element (tolerance 1e-4 of
    the logits' rms: the fp32 sums over H and the hi + lo split of non-bf16 rows stay far below).
    With a workspace that holds the logits and normalised rows but not the partial rows, the MFMA
    router runs unsplit."""
    name, T, H, E, extra = case
    if ws_kind == "no_split_room" and T < 64:
        pytest.skip("the matvec router has no partial rows")
    print(f"[router] {name} {ws_kind}", flush=True)
    wl = small_workload(name, 0x70C0 + T + H + E, H, 256, E, 4, 4, **extra)
    dl = build_layer(wl)
    ol = oracle_layer(wl)
    bank = wl.tokens_bank(T)
    x = act_tensor(wl, bank)
    d = M.make_dims(H, 256, E, 4)
    idx = torch.empty(T, 4, dtype=torch.int32, device="cuda")
    w = torch.empty(T, 4, dtype=torch.float32, device="cuda")
    lg = torch.full((T, E), float("nan"), dtype=torch.float32, device="cuda")
    ws = M.workspace(M.MOE_OP_ROUTE, d, T)
    if ws_kind == "no_split_room":
        r256 = lambda n: (n + 255) // 256 * 256  # noqa: E731
        ws = ws[:r256(T * E * 4) + r256(T * H * 4)]
        assert ws.numel() < M.moe_workspace_bytes(M.MOE_OP_ROUTE, d, T, 1)
    M.moe_route(d, dl.L, x, idx, w, logits=lg, ws=ws)
    torch.cuda.synchronize()
    lg_h, idx_h = lg.cpu().numpy(), idx.cpu().numpy()
    x64 = act_f64(wl, bank)
    for t in range(T):
        n = oracle.rmsnorm(x64[t], ol.norm_w, ol.norm_eps) if ol.norm_w is not None else x64[t]
        ref = oracle.router_logits(ol.router, n, ol.logit_bias, wl.router_bf16)
        assert_close(lg_h[t], ref, f"{name} token {t} logits", rel=1e-4)
        ri, _, margin = oracle.route(ref, 4)
        if margin > MIN_MARGIN:
            assert list(idx_h[t]) == list(ri), f"{name} token {t}"


def test_batched_graph_replays_match_eager():
    """Route + grouped expert FFN + combine captured in one HIP graph (the busy-expert MFMA kernels
    fork onto the library's side stream and join back inside the capture), replayed on three
    different token batches with eager work in between; every replay equals the eager result of
    its batch byte for byte."""
    wl = small_workload("graph_b", 0x6A7F, 1024, 512, 16, 4, 4, norm=True)
    dl = build_layer(wl)
    T = 40
    d = M.make_dims(wl.H, wl.I, wl.E, wl.K)
    banks = [act_tensor(wl, wl.tokens_bank(4 * T)[j * T:(j + 1) * T]) for j in range(3)]
    x = torch.empty_like(banks[0])
    ws_r, ws_f = M.workspace(M.MOE_OP_ROUTE, d, T), M.workspace(M.MOE_OP_EXPERT_FFN, d, T)
    idx = torch.empty(T, wl.K, dtype=torch.int32, device="cuda")
    w = torch.empty(T, wl.K, dtype=torch.float32, device="cuda")
    y = torch.empty(T, wl.K, wl.H, dtype=torch.float32, device="cuda")
    out = torch.empty(T, wl.H, dtype=torch.float32, device="cuda")

    def step():
        M.moe_route(d, dl.L, x, idx, w, ws=ws_r)
        M.moe_expert_ffn(d, dl.L, x, idx, y, ws_f)
        M.moe_combine(y, w, out)

    eager = []
    for b in banks:
        x.copy_(b)
        step()
        torch.cuda.synchronize()
        eager.append((idx.cpu().numpy().copy(), y.cpu().numpy().copy(), out.cpu().numpy().copy()))
    counts = np.bincount(eager[0][0].reshape(-1), minlength=wl.E)
    assert counts.max() > 8 and ((counts >= 1) & (counts <= 8)).any(), counts   # both chains run
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for j in [2, 0, 1]:
        x.copy_(banks[j])
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = (idx.cpu().numpy(), y.cpu().numpy(), out.cpu().numpy())
        for a_, b_, what in zip(got, eager[j], ("idx", "y", "out")):
            assert np.array_equal(a_, b_), f"replay of batch {j}: {what} differs"


def test_batched_launch_failure_then_same_result():
    """A batched expert FFN refused after its grouping step reports MOE_ERR_LAUNCH; the same call
    made again gives exactly the bytes of a call made before the failure."""
    wl = small_workload("inject_b", 0x1F2, 1024, 512, 24, 4, 4)
    dl = build_layer(wl)
    T = 40
    x = act_tensor(wl, wl.tokens_bank(T))
    d = M.make_dims(wl.H, wl.I, wl.E, wl.K)
    idx = torch.empty(T, wl.K, dtype=torch.int32, device="cuda")
    w = torch.empty(T, wl.K, dtype=torch.float32, device="cuda")
    M.moe_route(d, dl.L, x, idx, w, ws=M.workspace(M.MOE_OP_ROUTE, d, T))
    ws = M.workspace(M.MOE_OP_EXPERT_FFN, d, T)
    y0 = torch.empty(T, wl.K, wl.H, dtype=torch.float32, device="cuda")
    M.moe_expert_ffn(d, dl.L, x, idx, y0, ws)
    y1 = torch.full_like(y0, float("nan"))
    M.lib().moe_debug_inject_launch_failure(1, 1)
    try:
        with pytest.raises(M.MoeError) as ei:
            M.moe_expert_ffn(d, dl.L, x, idx, y1, ws)
        assert ei.value.status == 7 and "injected" in str(ei.value)
    finally:
        M.lib().moe_debug_inject_launch_failure(0, 0)
    M.moe_expert_ffn(d, dl.L, x, idx, y1, ws)
    torch.cuda.synchronize()
    assert torch.equal(y0, y1)
