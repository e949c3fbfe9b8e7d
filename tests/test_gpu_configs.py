"""GPU parity at the workload sizes (all five configurations), through the C ABI.

Full-size layers are checked on sampled tokens the oracle computes one by one: every routing
index exactly, every output within 2e-3 * ||oracle||_2 / sqrt(n)."""
import sys

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import bit_expert_dequant_amd as M  # noqa: E402
import oracle  # noqa: E402
import synth  # noqa: E402
from moe_cases import (MIN_MARGIN, act_f64, act_tensor, assert_close, build_layer, oracle_layer)  # noqa: E402


def say(msg):
    print(msg, flush=True)


def free():
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def decode_tokens(wl, layers, bank, tokens, residual):
    d = M.make_dims(wl.H, wl.I, wl.E, wl.K)
    ws = M.workspace(M.MOE_OP_LAYER_DECODE, d, 1, len(layers))
    res = []
    for t in tokens:
        out = torch.empty(wl.H, dtype=torch.float32, device="cuda")
        idx = torch.empty(len(layers), wl.K, dtype=torch.int32, device="cuda")
        w = torch.empty(len(layers), wl.K, dtype=torch.float32, device="cuda")
        M.moe_layer_decode(d, [dl.L for dl in layers], act_tensor(wl, bank[t]), out, idx, w, residual=residual,
                           ws=ws)
        torch.cuda.synchronize()
        res.append((out.cpu().numpy(), idx.cpu().numpy(), w.cpu().numpy()))
    return res


@pytest.mark.parametrize("cfg,n_tok", [(0, 64), (1, 6), (2, 8)])
def test_single_layer_configs(cfg, n_tok):
    wl = synth.WORKLOADS[cfg]
    say(f"[config {cfg}] {wl.name}")
    dl = build_layer(wl)
    ol = oracle_layer(wl)
    bank = wl.tokens_bank(n_tok)
    got = decode_tokens(wl, [dl], bank, range(n_tok), residual=False)
    hot = set(synth.hot_set(wl.seed, wl.E).tolist()) if wl.tiered else None
    n_hot = 0
    for t, (out, idx, w) in enumerate(got):
        ref = oracle.layer_token(act_f64(wl, bank[t]), ol, wl.H, wl.I, wl.K)
        assert ref.margin > MIN_MARGIN, f"token {t}: margin {ref.margin:.2e}"
        assert list(idx[0]) == list(ref.idx), f"token {t}"
        assert_close(w[0], ref.w, f"cfg{cfg} token {t} w")
        assert_close(out, ref.out, f"cfg{cfg} token {t} out")
        if hot is not None:
            n_hot += sum(int(e) in hot for e in idx[0])
    if hot is not None:
        say(f"[config 2] hot share of the sampled selections: {n_hot / (n_tok * wl.K):.2f}")
    del dl
    free()


def test_config1_bank_routing_and_graph_replays():
    """Config 1 captured in a HIP graph: several replays, each checked against eager results,
    with eager work and synchronisation in between."""
    wl = synth.WORKLOADS[1]
    dl = build_layer(wl)
    d = M.make_dims(wl.H, wl.I, wl.E, wl.K)
    ws = M.workspace(M.MOE_OP_LAYER_DECODE, d, 1, 1)
    bank = wl.tokens_bank(16)
    xs = act_tensor(wl, bank)
    n = 16
    outs = torch.empty(n, wl.H, dtype=torch.float32, device="cuda")
    idx = torch.empty(n, wl.K, dtype=torch.int32, device="cuda")
    w = torch.empty(n, wl.K, dtype=torch.float32, device="cuda")
    eager = decode_tokens(wl, [dl], bank, range(n), residual=False)
    M.moe_layer_decode(d, [dl.L], xs[0], outs[0], idx[0], w[0], ws=ws)     # warm-up before capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for t in range(n):
            M.moe_layer_decode(d, [dl.L], xs[t], outs[t], idx[t], w[t], ws=ws)
    for rep in range(4):
        outs.fill_(float("nan"))
        idx.fill_(-1)
        g.replay()
        torch.cuda.synchronize()
        junk = torch.empty(wl.H, dtype=torch.float32, device="cuda")
        M.moe_layer_decode(d, [dl.L], xs[rep], junk, ws=ws)               # eager work between replays
        torch.cuda.synchronize()
        o, i_, w_ = outs.cpu().numpy(), idx.cpu().numpy(), w.cpu().numpy()
        for t in range(n):
            assert np.array_equal(o[t], eager[t][0]), f"replay {rep} token {t} out"
            assert np.array_equal(i_[t], eager[t][1][0]) and np.array_equal(w_[t], eager[t][2][0])
    del g, dl
    free()


def test_config3_sixty_layer_stack():
    wl = synth.WORKLOADS[3]
    say(f"[config 3] building {wl.n_layers} layers ({wl.n_layers * wl.E * wl.blob_bytes(4) / 2**30:.1f} GiB)")
    layers = [build_layer(wl, l) for l in range(wl.n_layers)]
    torch.cuda.synchronize()
    ols = [oracle_layer(wl, l) for l in range(wl.n_layers)]
    n_tok = 4
    bank = wl.tokens_bank(n_tok)
    got = decode_tokens(wl, layers, bank, range(n_tok), residual=True)
    for t in range(n_tok):
        out, idx, w = got[t]
        ref_out, refs = oracle.stack_token(act_f64(wl, bank[t]), ols, wl.H, wl.I, wl.K, residual=True)
        for l, r in enumerate(refs):
            assert r.margin > MIN_MARGIN, f"token {t} layer {l}: margin {r.margin:.2e}"
            assert list(idx[l]) == list(r.idx), f"token {t} layer {l}"
            assert_close(w[l], r.w, f"token {t} layer {l} w")
        assert_close(out, ref_out, f"token {t} 60-layer out")
        say(f"[config 3] token {t} checked through {wl.n_layers} layers")
    del layers
    free()


def test_config4_batched():
    wl = synth.WORKLOADS[4]
    T = wl.tokens
    dl = build_layer(wl)
    ol = oracle_layer(wl)
    d = M.make_dims(wl.H, wl.I, wl.E, wl.K)
    bank = wl.tokens_bank(T)
    x = act_tensor(wl, bank)
    idx = torch.empty(T, wl.K, dtype=torch.int32, device="cuda")
    w = torch.empty(T, wl.K, dtype=torch.float32, device="cuda")
    logits = torch.empty(T, wl.E, dtype=torch.float32, device="cuda")
    y = torch.empty(T, wl.K, wl.H, dtype=torch.float32, device="cuda")
    out = torch.empty(T, wl.H, dtype=torch.float32, device="cuda")
    M.moe_route(d, dl.L, x, idx, w, logits)
    M.moe_expert_ffn(d, dl.L, x, idx, y, M.workspace(M.MOE_OP_EXPERT_FFN, d, T))
    M.moe_combine(y, w, out)
    torch.cuda.synchronize()
    idx_h, w_h, lg_h = idx.cpu().numpy(), w.cpu().numpy(), logits.cpu().numpy()
    x64 = act_f64(wl, bank)
    # routing of every token
    for t in range(T):
        lg = oracle.router_logits(ol.router, x64[t], ol.logit_bias, True)
        ri, rw, margin = oracle.route(lg, wl.K)
        assert margin > MIN_MARGIN, f"token {t}"
        assert list(idx_h[t]) == list(ri), f"token {t}"
        assert_close(w_h[t], rw, f"token {t} w")
        assert_close(lg_h[t], lg, f"token {t} logits")
    distinct = len(np.unique(idx_h))
    say(f"[config 4] {distinct} distinct experts over {T} tokens")
    # expert outputs and combine of every token
    y_h, out_h = y.cpu().numpy(), out.cpu().numpy()
    for t in range(T):
        ref = oracle.layer_token(x64[t], ol, wl.H, wl.I, wl.K)
        for k in range(wl.K):
            assert_close(y_h[t, k], ref.y[k], f"token {t} y[{k}]")
        assert_close(out_h[t], ref.out, f"token {t} out")
    del dl
    free()
