"""GPU parity on seeded random shapes: valid combinations of H, I, E, K, code width (2, 4 or tiered),
activation and router dtype and the norm, drawn once from a fixed seed, through moe_layer_decode (one
token per call) and through the batched route / expert FFN / combine calls, each against the oracle
(indices exact, values within the decode path's tolerance).  Tokens whose oracle routing margin is
too small to compare are skipped and counted; each case must check most of its tokens."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import bit_expert_dequant_amd as M  # noqa: E402
import oracle  # noqa: E402
from moe_cases import (MIN_MARGIN, act_f64, act_tensor, assert_close, build_layer, oracle_layer,  # noqa: E402
                       small_workload)


def draw_cases(n: int, seed: int, batched: bool):
    rng = np.random.default_rng(seed)
    cases = []
    while len(cases) < n:
        H = 64 * int(rng.integers(1, 33))
        I = 64 * int(rng.integers(1, 25))
        E = int(rng.integers(1, 65))
        K = int(rng.integers(1, min(E, 8) + 1))
        if K * I > 36864:
            continue
        kind = ["4", "2", "tiered"][int(rng.integers(0, 3))]
        if kind == "tiered" and E < 2:
            kind = "4"
        extra = {"x_bf16": bool(rng.integers(0, 2)), "router_bf16": bool(rng.integers(0, 2)),
                 "norm": bool(rng.integers(0, 2))}
        if kind == "tiered":
            extra.update(tiered=True, n_hot=int(rng.integers(1, E)))
        T = int(rng.integers(2, 81)) if batched else 2
        name = f"{'b' if batched else 'd'}{len(cases)}_t{T}_h{H}_i{I}_e{E}_k{K}_{kind}"
        cases.append((name, T, H, I, E, K, 2 if kind == "2" else 4, extra))
    return cases


DECODE = draw_cases(16, 0x5A11, batched=False)
BATCHED = draw_cases(10, 0x5A12, batched=True)


@pytest.mark.parametrize("case", DECODE, ids=[c[0] for c in DECODE])
def test_random_shape_decode(case):
    name, T, H, I, E, K, bits, extra = case
    print(f"[random decode] {name} {extra}", flush=True)
    wl = small_workload(name, 0xD0 + H + 7 * I + 13 * E, H, I, E, K, bits, **extra)
    dl = build_layer(wl)
    ol = oracle_layer(wl)
    d = M.make_dims(H, I, E, K)
    ws = M.workspace(M.MOE_OP_LAYER_DECODE, d, 1, 1)
    bank = wl.tokens_bank(T)
    checked = 0
    for t in range(T):
        out = torch.empty(H, dtype=torch.float32, device="cuda")
        idx = torch.empty(K, dtype=torch.int32, device="cuda")
        w = torch.empty(K, dtype=torch.float32, device="cuda")
        M.moe_layer_decode(d, [dl.L], act_tensor(wl, bank[t]), out, idx, w, ws=ws)
        torch.cuda.synchronize()
        ref = oracle.layer_token(act_f64(wl, bank[t]), ol, H, I, K)
        if ref.margin <= MIN_MARGIN:
            continue
        checked += 1
        assert list(idx.cpu().numpy()) == list(ref.idx), f"{name} token {t}"
        assert_close(w.cpu().numpy(), ref.w, f"{name} token {t} weights")
        assert_close(out.cpu().numpy(), ref.out, f"{name} token {t} out")
    assert checked >= 1, f"{name}: no token with a comparable routing margin"


@pytest.mark.parametrize("case", BATCHED, ids=[c[0] for c in BATCHED])
def test_random_shape_batched(case):
    name, T, H, I, E, K, bits, extra = case
    print(f"[random batched] {name} {extra}", flush=True)
    wl = small_workload(name, 0xB0 + H + 7 * I + 13 * E, H, I, E, K, bits, **extra)
    dl = build_layer(wl)
    ol = oracle_layer(wl)
    d = M.make_dims(H, I, E, K)
    bank = wl.tokens_bank(T)
    x = act_tensor(wl, bank)
    idx = torch.empty(T, K, dtype=torch.int32, device="cuda")
    w = torch.empty(T, K, dtype=torch.float32, device="cuda")
    M.moe_route(d, dl.L, x, idx, w, ws=M.workspace(M.MOE_OP_ROUTE, d, T))
    y = torch.full((T, K, H), float("nan"), dtype=torch.float32, device="cuda")
    M.moe_expert_ffn(d, dl.L, x, idx, y, M.workspace(M.MOE_OP_EXPERT_FFN, d, T))
    out = torch.empty(T, H, dtype=torch.float32, device="cuda")
    M.moe_combine(y, w, out)
    torch.cuda.synchronize()
    idx_h, w_h, out_h = idx.cpu().numpy(), w.cpu().numpy(), out.cpu().numpy()
    x64 = act_f64(wl, bank)
    checked = 0
    for t in range(T):
        ref = oracle.layer_token(x64[t], ol, H, I, K)
        if ref.margin <= MIN_MARGIN:
            continue
        checked += 1
        assert list(idx_h[t]) == list(ref.idx), f"{name} token {t}"
        assert_close(w_h[t], ref.w, f"{name} token {t} weights")
        assert_close(out_h[t], ref.out, f"{name} token {t} out")
    assert checked >= 0.8 * T, f"{name}: only {checked} of {T} tokens had a comparable routing margin"
