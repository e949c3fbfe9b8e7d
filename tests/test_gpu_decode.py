"""GPU parity of the decode path (T = 1 per call) against the CPU oracle, through the C ABI.

Routing indices must match the oracle exactly; router weights, logits, per-expert outputs and
layer outputs must satisfy max|gpu - oracle| <= 2e-3 * ||oracle||_2 / sqrt(n) per token."""
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


def ws_error_word(ws) -> int:
    """The layer-decode workspace's error word (count of timed-out waits of the two-launch schedule)."""
    return int(ws[4:8].cpu().numpy().view(np.uint32)[0])


SCHEDULES = ["two_launch", "single_launch", "three_kernels"]


def sched_kw(schedule: str) -> dict:
    """moe_layer_decode keyword arguments of a layer schedule: one launch (default), two, three."""
    return {"separate_kernels": schedule == "three_kernels", "single_launch": schedule == "single_launch"}


def run_decode(dl, x, residual=False, schedule="two_launch", ws=None):
    wl = dl.wl
    d = M.make_dims(wl.H, wl.I, wl.E, wl.K)
    ws = M.workspace(M.MOE_OP_LAYER_DECODE, d, 1, 1) if ws is None else ws
    out = torch.empty(wl.H, dtype=torch.float32, device="cuda")
    idx = torch.empty(wl.K, dtype=torch.int32, device="cuda")
    w = torch.empty(wl.K, dtype=torch.float32, device="cuda")
    M.moe_layer_decode(d, [dl.L], x, out, idx, w, residual=residual, ws=ws, **sched_kw(schedule))
    torch.cuda.synchronize()
    assert ws_error_word(ws) == 0
    return out.cpu().numpy(), idx.cpu().numpy(), w.cpu().numpy()


def check_token(wl, ol, xg, x64, out, idx, w, residual=False, what=""):
    ref = oracle.layer_token(x64, ol, wl.H, wl.I, wl.K, residual=residual)
    assert ref.margin > MIN_MARGIN, f"{what}: routing margin {ref.margin:.2e} too small to compare"
    assert list(idx) == list(ref.idx), f"{what}: idx {list(idx)} != oracle {list(ref.idx)}"
    assert_close(w, ref.w, f"{what} weights")
    assert abs(float(np.sum(w)) - 1.0) < 4 * 2**-24 * wl.K
    assert_close(out, ref.out, f"{what} out")
    return ref


SMALL = [
    # name, H, I, E, K, bits, extra
    ("h64_i64_e4_k2_4b", 64, 64, 4, 2, 4, {}),
    ("h128_i192_e6_k3_2b", 128, 192, 6, 3, 2, {}),
    ("h192_i320_e5_k1_4b_ragged", 192, 320, 5, 1, 4, {}),
    ("h512_i256_e8_k2_fp32", 512, 256, 8, 2, 4, {"router_bf16": False, "x_bf16": False}),
    ("h1024_i512_e16_k4_norm", 1024, 512, 16, 4, 4, {"norm": True}),
    ("h2048_i768_e32_k8_4b", 2048, 768, 32, 8, 4, {}),
    ("h3072_i1536_e12_k4_2b_zipf", 3072, 1536, 12, 4, 2, {"zipf": True}),
    ("h4096_i1024_e20_k4_tiered", 4096, 1024, 20, 4, 4, {"tiered": True, "n_hot": 7, "zipf": True}),
    ("h8192_i256_e9_k2_fp32x", 8192, 256, 9, 2, 4, {"x_bf16": False}),
    ("h640_i1344_e7_k7_tiered_norm", 640, 1344, 7, 7, 4, {"tiered": True, "n_hot": 3, "norm": True}),
    ("h256_i64_e1_k1", 256, 64, 1, 1, 2, {}),
    ("h4096_i4096_e8_k8_4b", 4096, 4096, 8, 8, 4, {"x_bf16": False}),
    ("h256_i128_e1000_k6", 256, 128, 1000, 6, 4, {}),
    # the limits: K * I exactly at the down projection's LDS bound, and the widest intermediate
    ("h512_i4608_e10_k8_lds_limit", 512, 4608, 10, 8, 4, {}),
    ("h256_i8192_e6_k4_2b_max_inter", 256, 8192, 6, 4, 2, {}),
]


@pytest.mark.parametrize("schedule", SCHEDULES)
@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_layer_decode_small_shapes(case, schedule):
    name, H, I, E, K, bits, extra = case
    say(f"[decode small] {name} schedule={schedule}")
    wl = small_workload(name, 0xC0DE + H + I + E, H, I, E, K, bits, **extra)
    dl = build_layer(wl)
    ol = oracle_layer(wl)
    bank = wl.tokens_bank(3)
    d = M.make_dims(H, I, E, K)
    ws = M.workspace(M.MOE_OP_LAYER_DECODE, d, 1, 1)      # one workspace for the three calls
    for t in range(3):
        residual = t == 2
        x = act_tensor(wl, bank[t])
        out, idx, w = run_decode(dl, x, residual=residual, schedule=schedule, ws=ws)
        check_token(wl, ol, x, act_f64(wl, bank[t]), out, idx, w, residual, f"{name} token {t}")


@pytest.mark.parametrize("schedule", ["two_launch", "single_launch"])
def test_many_calls_one_workspace(schedule):
    """Back-to-back calls on one workspace (each launch must see only its own hand-over words):
    every call matches the three-kernel schedule on the same token, and repeats are bit-identical."""
    wl = small_workload("seq", 4711, 1024, 512, 64, 4, 4, norm=True)
    dl = build_layer(wl)
    d = M.make_dims(wl.H, wl.I, wl.E, wl.K)
    ws = M.workspace(M.MOE_OP_LAYER_DECODE, d, 1, 1)
    ws2 = M.workspace(M.MOE_OP_LAYER_DECODE, d, 1, 1)
    bank = wl.tokens_bank(8)
    first = {}
    for i in range(48):
        t = (i * 5) % 8
        x = act_tensor(wl, bank[t])
        out, idx, w = run_decode(dl, x, residual=True, schedule=schedule, ws=ws)
        ref, ridx, rw = run_decode(dl, x, residual=True, schedule="three_kernels", ws=ws2)
        assert list(idx) == list(ridx), f"call {i} token {t}"
        assert_close(out, ref, f"call {i} token {t} {schedule} vs three kernels", rel=2e-5)
        if t in first:
            assert np.array_equal(first[t], out), f"call {i} token {t} not reproducible"
        first.setdefault(t, out)


@pytest.mark.parametrize("case", SMALL[:8], ids=[c[0] for c in SMALL[:8]])
def test_route_ffn_combine_small_shapes(case):
    """The separate C-ABI calls: moe_route (idx, w, logits), moe_expert_ffn (y per expert),
    moe_combine (out)."""
    name, H, I, E, K, bits, extra = case
    say(f"[route/ffn/combine small] {name}")
    wl = small_workload(name, 0xBEEF + H + I + E, H, I, E, K, bits, **extra)
    dl = build_layer(wl)
    ol = oracle_layer(wl)
    bank = wl.tokens_bank(2)
    d = M.make_dims(H, I, E, K)
    for t in range(2):
        x = act_tensor(wl, bank[t]).reshape(1, H)
        idx = torch.empty(1, K, dtype=torch.int32, device="cuda")
        w = torch.empty(1, K, dtype=torch.float32, device="cuda")
        logits = torch.empty(1, E, dtype=torch.float32, device="cuda")
        M.moe_route(d, dl.L, x, idx, w, logits)
        y = torch.empty(1, K, H, dtype=torch.float32, device="cuda")
        ws = M.workspace(M.MOE_OP_EXPERT_FFN, d, 1)
        M.moe_expert_ffn(d, dl.L, x, idx, y, ws)
        out = torch.empty(1, H, dtype=torch.float32, device="cuda")
        M.moe_combine(y, w, out)
        torch.cuda.synchronize()
        ref = oracle.layer_token(act_f64(wl, bank[t]), ol, H, I, K)
        assert ref.margin > MIN_MARGIN
        assert list(idx.cpu().numpy()[0]) == list(ref.idx)
        assert_close(logits.cpu().numpy()[0], ref.logits, f"{name} logits")
        assert_close(w.cpu().numpy()[0], ref.w, f"{name} w")
        yk = y.cpu().numpy()[0]
        for k in range(K):
            assert_close(yk[k], ref.y[k], f"{name} y[{k}]")
        assert_close(out.cpu().numpy()[0], ref.out, f"{name} out")


def test_expert_ffn_given_routing_and_invalid_index():
    """moe_expert_ffn with caller-chosen experts (not the router's), including an out-of-range
    index, which yields a zero row."""
    wl = small_workload("given", 77, 512, 256, 8, 3, 4)
    dl = build_layer(wl)
    ol = oracle_layer(wl)
    x64 = act_f64(wl, wl.tokens_bank(1)[0])
    x = act_tensor(wl, wl.tokens_bank(1)).reshape(1, wl.H)
    d = M.make_dims(wl.H, wl.I, wl.E, wl.K)
    idx = torch.tensor([[5, 8, 0]], dtype=torch.int32, device="cuda")
    y = torch.full((1, 3, wl.H), 7.0, dtype=torch.float32, device="cuda")
    M.moe_expert_ffn(d, dl.L, x, idx, y, M.workspace(M.MOE_OP_EXPERT_FFN, d, 1))
    torch.cuda.synchronize()
    yk = y.cpu().numpy()[0]
    for k, e in [(0, 5), (2, 0)]:
        _, _, _, ref = oracle.expert(ol.blob(e), 4, wl.H, wl.I, x64)
        assert_close(yk[k], ref, f"y[{k}] expert {e}")
    assert np.all(yk[1] == 0.0)


def test_decode_is_deterministic():
    wl = small_workload("det", 99, 4096, 1024, 16, 4, 4, norm=True)
    dl = build_layer(wl)
    x = act_tensor(wl, wl.tokens_bank(1)[0])
    a = run_decode(dl, x, residual=True)
    b = run_decode(dl, x, residual=True)
    for u, v in zip(a, b):
        assert np.array_equal(u, v)


@pytest.mark.parametrize("H,I,n", [(512, 256, 3), (4096, 1024, 2)])
def test_device_filler_matches_host_generator(H, I, n):
    """Every byte the device filler writes (codes and the fp32-derived scale/bias draws) equals the
    host generator's, at the full expert shape too."""
    for bits in (4, 2):
        stride = synth.blob_layout(H, I, bits)[1]
        buf = torch.full((n * stride,), 0xAB, dtype=torch.uint8, device="cuda")
        synth.fill_blobs_device(buf.data_ptr(), stride, n, 5, 2, 1234, H, I, bits,
                                torch.cuda.current_stream().cuda_stream)
        host = buf.cpu().numpy().reshape(n, stride)
        for i in range(n):
            ref = synth.expert_blob(1234, 2, 5 + i, H, I, bits)
            bad = np.flatnonzero(host[i] != ref)
            assert bad.size == 0, f"bits {bits} expert {i}: {bad.size} bytes differ, first at {bad[:4]}"


def test_two_layer_stack_small():
    wl = small_workload("stack2", 4242, 1024, 512, 16, 4, 4, norm=True, n_layers=3, x_bf16=True)
    dls = [build_layer(wl, l) for l in range(3)]
    ols = [oracle_layer(wl, l) for l in range(3)]
    d = M.make_dims(wl.H, wl.I, wl.E, wl.K)
    ws = M.workspace(M.MOE_OP_LAYER_DECODE, d, 1, 3)
    bank = wl.tokens_bank(2)
    for t in range(2):
        x = act_tensor(wl, bank[t])
        out = torch.empty(wl.H, dtype=torch.float32, device="cuda")
        idx = torch.empty(3, wl.K, dtype=torch.int32, device="cuda")
        w = torch.empty(3, wl.K, dtype=torch.float32, device="cuda")
        M.moe_layer_decode(d, [dl.L for dl in dls], x, out, idx, w, residual=True, ws=ws)
        torch.cuda.synchronize()
        ref_out, refs = oracle.stack_token(act_f64(wl, bank[t]), ols, wl.H, wl.I, wl.K, residual=True)
        for l, r in enumerate(refs):
            assert r.margin > MIN_MARGIN
            assert list(idx.cpu().numpy()[l]) == list(r.idx), f"layer {l}"
            assert_close(w.cpu().numpy()[l], r.w, f"layer {l} w")
        assert_close(out.cpu().numpy(), ref_out, "stack out")


@pytest.mark.parametrize("schedule", SCHEDULES)
def test_timed_decode_matches_untimed(schedule):
    """moe_layer_decode_timed runs the same schedule as moe_layer_decode (bit-identical outputs and
    routing on a 2-layer stack) and stamps a start/stop event pair per kernel, in stream order."""
    wl = small_workload("timed", 777, 1024, 512, 16, 4, 4, norm=True, n_layers=2)
    dls = [build_layer(wl, l) for l in range(2)]
    L = [dl.L for dl in dls]
    d = M.make_dims(wl.H, wl.I, wl.E, wl.K)
    ws = M.workspace(M.MOE_OP_LAYER_DECODE, d, 1, 2)
    x = act_tensor(wl, wl.tokens_bank(1)[0])
    res = []
    for timed in (False, True):
        out = torch.empty(wl.H, dtype=torch.float32, device="cuda")
        idx = torch.empty(2, wl.K, dtype=torch.int32, device="cuda")
        w = torch.empty(2, wl.K, dtype=torch.float32, device="cuda")
        if timed:
            evs = [torch.cuda.Event(enable_timing=True) for _ in range({'two_launch': 4, 'single_launch': 2, 'three_kernels': 6}[schedule]) for _ in range(2)]
            for e in evs:
                e.record()
            torch.cuda.synchronize()
            with pytest.raises(ValueError):
                M.moe_layer_decode_timed(d, L, x, out, evs[:-1], idx, w, residual=True, ws=ws, **sched_kw(schedule))
            M.moe_layer_decode_timed(d, L, x, out, evs, idx, w, residual=True, ws=ws, **sched_kw(schedule))
        else:
            M.moe_layer_decode(d, L, x, out, idx, w, residual=True, ws=ws, **sched_kw(schedule))
        torch.cuda.synchronize()
        res.append((out.cpu().numpy(), idx.cpu().numpy(), w.cpu().numpy()))
        if timed:
            kernels = [evs[2 * j].elapsed_time(evs[2 * j + 1]) for j in range(len(evs) // 2)]
            assert all(0 < k < 1e3 for k in kernels), kernels
            starts = [evs[0].elapsed_time(evs[2 * j]) for j in range(len(evs) // 2)]
            assert all(b >= a for a, b in zip(starts, starts[1:])), starts
    for u, v in zip(*res):
        assert np.array_equal(u, v)
    assert ws_error_word(ws) == 0


@pytest.mark.parametrize("schedule", SCHEDULES)
@pytest.mark.parametrize("E,K", [(40, 8), (512, 4), (700, 8), (2048, 3)])
def test_layer_decode_routing_ties(E, K, schedule):
    """Routing inside moe_layer_decode on logits with exact ties, +0/-0, -inf and NaN: an fp32
    router and a one-hot fp32 token make each logit equal to one router entry, so the selection
    (equal logits -> lower index; NaN ranks as -inf) and the weights are fixed exactly."""
    H, I = 64, 64
    rng = np.random.default_rng(E + K)
    col = rng.choice([-1.5, -0.0, 0.0, 0.25, 2.0, 3.0], size=E).astype(np.float32)
    col[E // 3] = -np.inf
    col[1] = np.nan
    wl = small_workload("ties", 31 + E, H, I, E, K, 4, router_bf16=False, x_bf16=False)
    dl = build_layer(wl)
    router = np.zeros((E, H), dtype=np.float32)
    router[:, 0] = col
    L = M.Layer(torch.from_numpy(router).cuda(), dl.table)
    x = torch.zeros(H, dtype=torch.float32, device="cuda")
    x[0] = 1.0
    d = M.make_dims(H, I, E, K)
    ws = M.workspace(M.MOE_OP_LAYER_DECODE, d, 1, 1)
    out = torch.empty(H, dtype=torch.float32, device="cuda")
    idx = torch.empty(K, dtype=torch.int32, device="cuda")
    w = torch.empty(K, dtype=torch.float32, device="cuda")
    for _ in range(2):                     # the second call reuses the workspace
        M.moe_layer_decode(d, [L], x, out, idx, w, ws=ws, **sched_kw(schedule))
        torch.cuda.synchronize()
        ri, rw, _ = oracle.route(col.astype(np.float64), K)
        assert list(idx.cpu().numpy()) == list(ri)
        assert_close(w.cpu().numpy(), rw, "tie weights")
    assert ws_error_word(ws) == 0


@pytest.mark.parametrize("schedule", SCHEDULES)
@pytest.mark.parametrize("case", ["nan_in_topk", "all_nan"])
def test_layer_decode_nan_logits_against_oracle(case, schedule):
    """NaN logits inside the top K, and a row with no finite logit, routed by moe_layer_decode and
    moe_route on the very logits the oracle gets (NaN ranks as -inf with weight 0; no finite logit
    gives weights 1/K).  The output is checked too, for the experts with nonzero weight."""
    H, I, E, K = 64, 64, 16, 4
    col = np.full(E, np.nan, dtype=np.float32)
    if case == "nan_in_topk":
        col[1], col[4], col[2] = 2.0, 1.0, -np.inf
    wl = small_workload("nan_" + case, 77, H, I, E, K, 4, router_bf16=False, x_bf16=False)
    dl = build_layer(wl)
    router = np.zeros((E, H), dtype=np.float32)
    router[:, 0] = col
    L = M.Layer(torch.from_numpy(router).cuda(), dl.table)
    x_np = np.zeros(H, dtype=np.float32)
    x_np[0] = 1.0
    x = torch.from_numpy(x_np).cuda()
    d = M.make_dims(H, I, E, K)
    ws = M.workspace(M.MOE_OP_LAYER_DECODE, d, 1, 1)
    out = torch.empty(H, dtype=torch.float32, device="cuda")
    idx = torch.empty(K, dtype=torch.int32, device="cuda")
    w = torch.empty(K, dtype=torch.float32, device="cuda")
    M.moe_layer_decode(d, [L], x, out, idx, w, ws=ws, **sched_kw(schedule))
    torch.cuda.synchronize()
    ri, rw, _ = oracle.route(col.astype(np.float64), K)
    assert list(idx.cpu().numpy()) == list(ri)
    assert_close(w.cpu().numpy(), rw, "NaN weights")
    ol = oracle_layer(wl)
    ol.router = router
    ref = oracle.layer_token(x_np.astype(np.float64), ol, H, I, K)
    assert list(ref.idx) == list(ri)
    assert_close(out.cpu().numpy(), ref.out, "out with NaN logits")
    assert ws_error_word(ws) == 0
    idx2 = torch.empty(1, K, dtype=torch.int32, device="cuda")
    w2 = torch.empty(1, K, dtype=torch.float32, device="cuda")
    lg2 = torch.empty(1, E, dtype=torch.float32, device="cuda")
    M.moe_route(d, L, x.view(1, H), idx2, w2, lg2)
    torch.cuda.synchronize()
    assert list(idx2.cpu().numpy()[0]) == list(ri)
    assert_close(w2.cpu().numpy()[0], rw, "NaN weights (moe_route)")


@pytest.mark.parametrize("E", [40, 700])
def test_route_ties_zeros_and_infinities(E):
    """Top-K on logits with exact ties, +0/-0 and -inf: an fp32 router and a one-hot fp32 token
    make each logit equal to one router entry, so the expected order is exact."""
    K = 8
    H = 64
    rng = np.random.default_rng(E)
    col = rng.choice([-1.5, -0.0, 0.0, 0.25, 2.0, 3.0], size=E).astype(np.float32)
    col[E // 3] = -np.inf
    col[E // 2] = 3.0
    router = np.zeros((E, H), dtype=np.float32)
    router[:, 0] = col
    x = np.zeros((1, H), dtype=np.float32)
    x[0, 0] = 1.0
    d = M.make_dims(H, 64, E, K)
    table = M.expert_table([1 << 20] * E, [4] * E)          # never dereferenced by moe_route
    L = M.Layer(torch.from_numpy(router).cuda(), table)
    idx = torch.empty(1, K, dtype=torch.int32, device="cuda")
    w = torch.empty(1, K, dtype=torch.float32, device="cuda")
    logits = torch.empty(1, E, dtype=torch.float32, device="cuda")
    M.moe_route(d, L, torch.from_numpy(x).cuda(), idx, w, logits)
    torch.cuda.synchronize()
    lg = col.astype(np.float64)
    ri, rw, _ = oracle.route(lg, K)
    assert list(idx.cpu().numpy()[0]) == list(ri)
    assert_close(w.cpu().numpy()[0], rw, "tie weights")
    # NaN counts as -inf: never chosen while finite logits remain
    col2 = col.copy()
    col2[:3] = np.nan
    router[:, 0] = col2
    L2 = M.Layer(torch.from_numpy(router).cuda(), table)
    M.moe_route(d, L2, torch.from_numpy(x).cuda(), idx, w, logits)
    torch.cuda.synchronize()
    ri2, rw2, _ = oracle.route(col2.astype(np.float64), K)
    assert list(idx.cpu().numpy()[0]) == list(ri2)
    assert_close(w.cpu().numpy()[0], rw2, "NaN weights")


def test_stream_read_xor():
    """The read-stream reference reads every byte: its XOR of all dwords matches numpy's."""
    rng = np.random.default_rng(5)
    for n in (16, 4096, 1 << 20, (1 << 22) + 48):
        host = rng.integers(0, 2**32, size=n // 4, dtype=np.uint32)
        buf = torch.from_numpy(host.view(np.int32)).cuda()
        sink = torch.zeros(1, dtype=torch.int32, device="cuda")
        M.moe_stream_read(buf, sink)
        torch.cuda.synchronize()
        assert int(sink.cpu().numpy().view(np.uint32)[0]) == int(np.bitwise_xor.reduce(host)), n
    with pytest.raises(M.MoeError):        # 12 bytes: not a multiple of 16
        M.moe_stream_read(torch.zeros(3, dtype=torch.int32, device="cuda"), sink)


@pytest.mark.parametrize("schedule", ["two_launch", "single_launch"])
def test_launch_failure_between_kernels_then_recovery(schedule):
    """A decode call refused at its second launch step (two launches: router + gate/up ran, down did
    not; one launch: the first of two stacked layers ran, the second did not) reports MOE_ERR_LAUNCH;
    after the workspace is zero-filled again, as the header asks, the next calls are correct."""
    n_layers = 2 if schedule == "single_launch" else 1
    wl = small_workload("inject_dec", 0x1F1, 1024, 512, 16, 4, 4, n_layers=n_layers, norm=n_layers > 1)
    dls = [build_layer(wl, l) for l in range(n_layers)]
    ols = [oracle_layer(wl, l) for l in range(n_layers)]
    bank = wl.tokens_bank(3)
    d = M.make_dims(wl.H, wl.I, wl.E, wl.K)
    ws = M.workspace(M.MOE_OP_LAYER_DECODE, d, 1, n_layers)
    kw = sched_kw(schedule)
    res = n_layers > 1

    def run_check(t, what):
        out = torch.empty(wl.H, dtype=torch.float32, device="cuda")
        idx = torch.empty(n_layers, wl.K, dtype=torch.int32, device="cuda")
        w = torch.empty(n_layers, wl.K, dtype=torch.float32, device="cuda")
        M.moe_layer_decode(d, [dl.L for dl in dls], act_tensor(wl, bank[t]), out, idx, w, residual=res, ws=ws, **kw)
        torch.cuda.synchronize()
        ref_out, refs = oracle.stack_token(act_f64(wl, bank[t]), ols, wl.H, wl.I, wl.K, residual=res)
        for l, r in enumerate(refs):
            assert list(idx.cpu().numpy()[l]) == list(r.idx), f"{what} layer {l}"
        assert_close(out.cpu().numpy(), ref_out, f"{what} out")

    run_check(0, "before")
    o = torch.empty(wl.H, dtype=torch.float32, device="cuda")
    M.lib().moe_debug_inject_launch_failure(1, 1)
    try:
        with pytest.raises(M.MoeError) as ei:
            M.moe_layer_decode(d, [dl.L for dl in dls], act_tensor(wl, bank[1]), o, residual=res, ws=ws, **kw)
        assert ei.value.status == 7 and "injected" in str(ei.value)
    finally:
        M.lib().moe_debug_inject_launch_failure(0, 0)
    torch.cuda.synchronize()
    ws.zero_()
    for t in (1, 2):
        run_check(t, f"after, token {t}")


def test_error_word_forces_nan_until_zero_fill():
    """The header's contract for a timed-out logit wait, forced from the host (no wait has to time
    out): with a nonzero error word every call writes NaN outputs and leaves the word set; after the
    workspace is zero-filled the calls match the oracle again."""
    wl = small_workload("errword", 0x2E2, 1024, 512, 16, 4, 4)
    dl = build_layer(wl)
    ol = oracle_layer(wl)
    bank = wl.tokens_bank(2)
    d = M.make_dims(wl.H, wl.I, wl.E, wl.K)
    ws = M.workspace(M.MOE_OP_LAYER_DECODE, d, 1, 1)
    out, idx, w = run_decode(dl, act_tensor(wl, bank[0]), ws=ws)
    check_token(wl, ol, None, act_f64(wl, bank[0]), out, idx, w, what="before")
    ws[4:8] = torch.tensor(np.array([3], dtype=np.uint32).view(np.uint8), device="cuda")
    o = torch.empty(wl.H, dtype=torch.float32, device="cuda")
    for _ in range(2):
        o.fill_(0.0)
        M.moe_layer_decode(d, [dl.L], act_tensor(wl, bank[1]), o, ws=ws)
        torch.cuda.synchronize()
        assert torch.isnan(o).all(), "outputs must be NaN while the error word is set"
        assert ws_error_word(ws) != 0
    ws.zero_()
    out, idx, w = run_decode(dl, act_tensor(wl, bank[1]), ws=ws)
    check_token(wl, ol, None, act_f64(wl, bank[1]), out, idx, w, what="after zero-fill")


@pytest.mark.parametrize("H", [66, 4096])
@pytest.mark.parametrize("offset", [0, 1])
@pytest.mark.parametrize("resid", ["none", "separate", "aliased"])
def test_combine_shapes_offsets_and_residual(H, offset, resid):
    """moe_combine on rows that are not a multiple of 4 and on views one float off 16-byte
    alignment (the one-element-per-thread kernel), and on aligned rows (the 16-byte kernel); the
    residual as its own buffer and with out aliasing it, as the header allows."""
    T, K = 3, 4
    rng = np.random.default_rng(H * 10 + offset)
    y_np = rng.standard_normal((T, K, H)).astype(np.float32)
    w_np = rng.random((T, K)).astype(np.float32)
    r_np = rng.standard_normal((T, H)).astype(np.float32)
    ybuf = torch.zeros(T * K * H + offset, dtype=torch.float32, device="cuda")
    y = ybuf[offset:].view(T, K, H)
    y.copy_(torch.from_numpy(y_np))
    w = torch.from_numpy(w_np).cuda()
    obuf = torch.zeros(T * H + offset, dtype=torch.float32, device="cuda")
    out = obuf[offset:].view(T, H)
    residual = None
    if resid == "separate":
        rbuf = torch.zeros(T * H + offset, dtype=torch.float32, device="cuda")
        residual = rbuf[offset:].view(T, H)
        residual.copy_(torch.from_numpy(r_np))
    elif resid == "aliased":
        out.copy_(torch.from_numpy(r_np))
        residual = out
    M.moe_combine(y, w, out, residual=residual)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    for t in range(T):
        ref = oracle.combine(y_np[t].astype(np.float64), w_np[t].astype(np.float64),
                             None if resid == "none" else r_np[t].astype(np.float64))
        assert_close(got[t], ref, f"combine t={t}")
    if resid == "separate":
        assert np.array_equal(residual.cpu().numpy(), r_np)


@pytest.mark.parametrize("bits_mix", ["4bit", "mixed"])
def test_decode_through_packer_blobs(bits_mix):
    """Experts packed by moe_pack_expert from code, scale and bias arrays (not by the seeded
    generator's own byte placement), decoded on the GPU: routing against the oracle on the same
    blobs, and each expert's output against a float64 product of the raw arrays themselves."""
    H, I, E, K = 1024, 512, 8, 4
    rng = np.random.default_rng(0x9AC + len(bits_mix))
    bits = [4] * E if bits_mix == "4bit" else [4, 2, 2, 4, 2, 4, 4, 2]
    stride = M.moe_packed_expert_bytes(H, I, 4)
    host = np.zeros((E, stride), dtype=np.uint8)
    dense = []
    for e in range(E):
        mats, Ws = [], []
        for R, C in [(I, H), (I, H), (H, I)]:
            codes = rng.integers(0, 1 << bits[e], (R, C)).astype(np.uint8)
            s = synth.f32_to_bf16_rne(rng.uniform(0.002, 0.02, R * C // 64).astype(np.float32))
            b = synth.f32_to_bf16_rne(rng.uniform(-0.1, 0.1, R * C // 64).astype(np.float32))
            mats.append((codes, s, b))
            sf = np.repeat(synth.bf16_to_f32(s).reshape(R, -1), 64, 1).astype(np.float64)
            bf = np.repeat(synth.bf16_to_f32(b).reshape(R, -1), 64, 1).astype(np.float64)
            Ws.append(codes.astype(np.float64) * sf + bf)
        blob = M.moe_pack_expert(mats, H, I, bits[e])
        host[e, :blob.size] = blob
        dense.append(Ws)
    store = torch.from_numpy(host.reshape(-1)).cuda()
    table = M.expert_table([store.data_ptr() + e * stride for e in range(E)], bits)
    router_np = synth.f32_to_bf16_rne((rng.standard_normal((E, H)) * 0.02).astype(np.float32))
    router = torch.from_numpy(router_np.view(np.int16)).cuda().view(torch.bfloat16)
    L = M.Layer(router, table)
    ol = oracle.LayerWeights(router_np, True, lambda e: host[e], lambda e: bits[e])
    d = M.make_dims(H, I, E, K)
    ws = M.workspace(M.MOE_OP_LAYER_DECODE, d, 1, 1)
    for t in range(3):
        x_u16 = synth.f32_to_bf16_rne(rng.standard_normal(H).astype(np.float32))
        x = torch.from_numpy(x_u16.view(np.int16)).cuda().view(torch.bfloat16)
        x64 = synth.bf16_to_f32(x_u16).astype(np.float64)
        out = torch.empty(H, dtype=torch.float32, device="cuda")
        idx = torch.empty(K, dtype=torch.int32, device="cuda")
        w = torch.empty(K, dtype=torch.float32, device="cuda")
        M.moe_layer_decode(d, [L], x, out, idx, w, ws=ws)
        y = torch.empty(1, K, H, dtype=torch.float32, device="cuda")
        M.moe_expert_ffn(d, L, x.view(1, H), idx.view(1, K), y, M.workspace(M.MOE_OP_EXPERT_FFN, d, 1))
        torch.cuda.synchronize()
        ref = oracle.layer_token(x64, ol, H, I, K)
        assert ref.margin > MIN_MARGIN
        assert list(idx.cpu().numpy()) == list(ref.idx)
        assert_close(out.cpu().numpy(), ref.out, f"token {t} out")
        yk = y.cpu().numpy()[0]
        for k, e in enumerate(ref.idx):
            Wg, Wu, Wd = dense[int(e)]
            g, u = Wg @ x64, Wu @ x64
            y_ref = Wd @ (g / (1.0 + np.exp(-g)) * u)
            assert_close(yk[k], y_ref, f"token {t} expert {int(e)} ({bits[int(e)]}-bit) y from the raw arrays")
