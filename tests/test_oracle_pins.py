"""Pins of the CPU oracle against facts the pages and the mathematics fix.

Each test names what pins which part of the oracle, chosen so that a plausible
mistake (wrong group size or scale dtype, wrong nibble order, swapped scale/bias,
transposed operand, dropped bias term, wrong SiLU, wrong renormalisation, wrong
tie-break) fails at least one of them.  None of these tests re-calls the oracle's
own formula: they compare it with page figures, hand-derived values, closed forms,
brute force, exact integer arithmetic or numpy's float64 matmul.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
MiB = 1 << 20


def bf16(v: float) -> int:
    """bf16 bits of a float that is exactly representable in bf16."""
    u = np.array([v], dtype=np.float32).view(np.uint32)[0]
    assert u & 0xFFFF == 0, v
    return int(u >> 16)


def pack_codes_by_hand(codes: np.ndarray, bits: int) -> np.ndarray:
    """Independent packer for the tests: per row, codes packed LSB-first with
    np.packbits on the reversed bit order of each code."""
    rows, cols = codes.shape
    per = 8 // bits
    out = np.zeros((rows, cols // per), dtype=np.uint8)
    for k in range(per):
        out |= (codes[:, k::per].astype(np.uint8) << (k * bits)).astype(np.uint8)
    return out.reshape(-1)


def sb_plane(scale: np.ndarray, bias: np.ndarray) -> np.ndarray:
    """[rows, G] float scales and biases (exact in bf16) -> uint16 [rows*G*2]."""
    s = (scale.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    b = (bias.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    return np.stack([s, b], axis=-1).reshape(-1)


# --------------------------------------------------------------------------- sizes
def test_expert_size_is_the_pages_6_75_MB(orc):
    # "each expert ~6.75 MB at 4-bit" (lilting.ch page, SSD expert streaming section).
    # With group 64 and one bf16 (scale, bias) pair per group, gate+up+down of a
    # 4096 x 1024 expert is exactly 6.75 MiB; group 32 or fp32 pairs would not be.
    assert orc.blob_bytes(4096, 1024, 4) == int(6.75 * MiB) == 7_077_888


def test_token_read_is_the_pages_27_MB(orc):
    # "4 x 6.75 MB ~= 27 MB per token" (same page, same section).
    assert 4 * orc.blob_bytes(4096, 1024, 4) == 27 * MiB


def test_sixty_layers_read_is_the_pages_1_62_GB(orc):
    # M5 Max table on the yamamurasyouten.com page: 1.62 GB of experts per token.
    per_token = 60 * 4 * orc.blob_bytes(4096, 1024, 4)
    assert per_token == 1_698_693_120
    assert per_token / MiB == pytest.approx(1620.0)


def test_two_bit_store_and_tiered_saving(orc):
    # 2-bit model ~120 GB (lilting.ch results table; tomo3141592653 page storage line);
    # tiered hot-4/cold-2 "disk -34%" (nzkcom page, adopted-optimisations table).
    b2, b4 = orc.blob_bytes(4096, 1024, 2), orc.blob_bytes(4096, 1024, 4)
    assert b2 == 3_932_160
    store2 = 60 * 512 * b2
    assert 110e9 < store2 < 125e9
    tier = (128 * b4 + 384 * b2) / (512 * b4)
    assert abs((1 - tier) - 0.34) < 0.01
    # the 4-bit store of 60 x 512 experts plus ~5.5 GB resident weights ~ "209GB" in GiB
    store4 = 60 * 512 * b4
    assert abs((store4 + 5.5e9) / 2**30 - 209) < 3


def test_layout_offsets_are_256_aligned_and_disjoint(orc):
    for H, I, bits in [(4096, 1024, 4), (4096, 1024, 2), (512, 256, 4), (192, 320, 2), (64, 64, 4)]:
        off, tot = orc.blob_layout(H, I, bits)
        sizes = [orc.codes_bytes(I, H, bits), orc.sb_bytes(I, H)] * 2 + [orc.codes_bytes(H, I, bits), orc.sb_bytes(H, I)]
        for i in range(6):
            assert off[i] % 256 == 0
            end = off[i] + sizes[i]
            assert end <= (off[i + 1] if i < 5 else tot)
        assert tot % 256 == 0


# --------------------------------------------------------------------------- code order
@pytest.mark.parametrize("bits", [2, 4])
def test_code_order_lsb_first_one_hot_bytes(orc, bits):
    # A single set byte at a known position decodes to the expected (row, col) codes:
    # low bits hold the lowest column.
    rows, cols = 2, 128
    row_bytes = cols * bits // 8
    plane = np.zeros(rows * row_bytes, dtype=np.uint8)
    plane[row_bytes + 3] = 0x2D if bits == 4 else 0b11_10_01_00  # row 1, byte 3
    per = 8 // bits
    got = [orc.code(plane, rows, cols, bits, 1, c) for c in range(3 * per, 4 * per)]
    expect = [0xD, 0x2] if bits == 4 else [0, 1, 2, 3]
    assert got == expect
    # every other code is zero
    nz = [(r, c) for r in range(rows) for c in range(cols) if orc.code(plane, rows, cols, bits, r, c)]
    assert nz == [(1, 3 * per + i) for i in range(per) if expect[i]]


@pytest.mark.parametrize("bits", [2, 4])
def test_one_hot_probe_returns_column_codes(orc, bits):
    # With scale 1 and bias 0, W e_j is column j's codes: pins every bit position.
    rng = np.random.default_rng(1)
    rows, cols = 5, 192
    codes = rng.integers(0, 1 << bits, size=(rows, cols))
    plane = pack_codes_by_hand(codes, bits)
    G = cols // 64
    sb = sb_plane(np.ones((rows, G)), np.zeros((rows, G)))
    W = orc.dequant(plane, sb, rows, cols, bits)
    for j in range(cols):
        x = np.zeros(cols)
        x[j] = 1.0
        assert np.array_equal(orc.matvec(W, x), codes[:, j].astype(np.float64))


def test_dequant_hand_values(orc):
    # q * s + b with bf16 s and b, per group of 64 along the input dimension.
    rows, cols, bits = 1, 128, 4
    codes = np.zeros((rows, cols), dtype=np.int64)
    codes[0, 0], codes[0, 64], codes[0, 127] = 3, 15, 7
    plane = pack_codes_by_hand(codes, bits)
    sb = sb_plane(np.array([[0.25, 2.0]]), np.array([[-0.125, 0.5]]))
    W = orc.dequant(plane, sb, rows, cols, bits)
    assert W[0, 0] == 3 * 0.25 - 0.125        # 0.625 (group 0)
    assert W[0, 1] == -0.125                    # code 0 -> bias only
    assert W[0, 64] == 15 * 2.0 + 0.5           # 30.5  (group 1: scale/bias of group 1)
    assert W[0, 127] == 7 * 2.0 + 0.5


# --------------------------------------------------------------------------- matvec
def unpack_numpy(plane: np.ndarray, rows: int, cols: int, bits: int) -> np.ndarray:
    """Independent unpack for the tests (vectorised shifts)."""
    per = 8 // bits
    b = plane.reshape(rows, cols // per).astype(np.int64)
    out = np.empty((rows, cols), dtype=np.int64)
    for k in range(per):
        out[:, k::per] = (b >> (k * bits)) & ((1 << bits) - 1)
    return out


@pytest.mark.parametrize("bits", [2, 4])
def test_integer_matvec_exact(orc, bits):
    rng = np.random.default_rng(2)
    rows, cols = 37, 320
    plane = rng.integers(0, 256, size=rows * cols * bits // 8, dtype=np.uint8)
    sb = sb_plane(np.ones((rows, cols // 64)), np.zeros((rows, cols // 64)))
    x = rng.integers(-50, 50, size=cols)
    W = orc.dequant(plane, sb, rows, cols, bits)
    y = orc.matvec(W, x.astype(np.float64))
    q = unpack_numpy(plane, rows, cols, bits)
    assert np.array_equal(y.astype(np.int64), q @ x)


@pytest.mark.parametrize("bits", [2, 4])
def test_fma_group_fold_identity(orc, bits):
    # The pages rewrite (q*s + b)*x as fma(q, s*x, b*x); summed over a group this is
    # s * sum(q x) + b * sum(x).  Evaluate that folded form in float64 from an
    # independent unpack and compare with the oracle's dequantise-then-dot.
    rng = np.random.default_rng(3)
    rows, cols = 23, 256
    G = cols // 64
    plane = rng.integers(0, 256, size=rows * cols * bits // 8, dtype=np.uint8)
    scale = (rng.uniform(0.002, 0.02, (rows, G)).astype(np.float32).view(np.uint32) & 0xFFFF0000).view(np.float32)
    bias = (rng.uniform(-0.1, 0.1, (rows, G)).astype(np.float32).view(np.uint32) & 0xFFFF0000).view(np.float32)
    x = rng.standard_normal(cols)
    y = orc.matvec(orc.dequant(plane, sb_plane(scale, bias), rows, cols, bits), x)
    q = unpack_numpy(plane, rows, cols, bits).astype(np.float64)
    xg = x.reshape(G, 64)
    qx = np.einsum("rgc,gc->rg", q.reshape(rows, G, 64), xg)
    folded = (scale.astype(np.float64) * qx + bias.astype(np.float64) * xg.sum(1)[None, :]).sum(1)
    assert np.allclose(y, folded, rtol=1e-12, atol=1e-12)


def test_matvec_matches_numpy_float64(orc):
    rng = np.random.default_rng(4)
    W = rng.standard_normal((64, 512)).astype(np.float32)
    x = rng.standard_normal(512)
    assert np.allclose(orc.matvec(W, x), W.astype(np.float64) @ x, rtol=1e-12, atol=1e-12)


# --------------------------------------------------------------------------- expert
def make_expert_blob(orc, H, I, bits, gate, up, down):
    """gate/up/down: (codes [R,C], scale [R,G], bias [R,G]) -> packed blob via the
    tests' own packer at the oracle's documented plane offsets."""
    off, tot = orc.blob_layout(H, I, bits)
    blob = np.zeros(tot, dtype=np.uint8)
    for t, (codes, s, b) in enumerate([gate, up, down]):
        cp = pack_codes_by_hand(codes, bits)
        sp = sb_plane(s, b).view(np.uint8)
        blob[off[2 * t]:off[2 * t] + cp.size] = cp
        blob[off[2 * t + 1]:off[2 * t + 1] + sp.size] = sp
    return blob


def silu_ref(z):
    return z / (1 + math.exp(-z))


@pytest.mark.parametrize("bits", [2, 4])
def test_all_equal_codes_closed_form(orc, bits):
    # With q == c, s == s_m, b == b_m in matrix m every weight is a_m = c s_m + b_m, so
    # g_r = a_g S, u_r = a_u S (S = sum x), h_j = silu(a_g S) a_u S, y_r = a_d I h.
    H, I = 256, 128
    c = 3 if bits == 2 else 11
    mats = []
    for (R, C, s, b) in [(I, H, 0.0078125, -0.0625), (I, H, 0.015625, 0.03125), (H, I, 0.00390625, -0.015625)]:
        mats.append((np.full((R, C), c), np.full((R, C // 64), s), np.full((R, C // 64), b)))
    blob = make_expert_blob(orc, H, I, bits, *mats)
    rng = np.random.default_rng(5)
    x = rng.standard_normal(H)
    S = x.sum()
    ag, au, ad = (c * 0.0078125 - 0.0625), (c * 0.015625 + 0.03125), (c * 0.00390625 - 0.015625)
    h = silu_ref(ag * S) * au * S
    g, u, hh, y = orc.expert(blob, bits, H, I, x)
    assert np.allclose(g, ag * S, rtol=1e-12) and np.allclose(u, au * S, rtol=1e-12)
    assert np.allclose(hh, h, rtol=1e-12)
    assert np.allclose(y, ad * I * h, rtol=1e-12)


def test_hand_computed_tiny_expert(orc):
    # Worked example with dyadic values; expected numbers derived by hand in the golden
    # file (every quantity before the SiLU is exact in binary).
    spec = json.load(open(os.path.join(GOLDEN, "tiny_expert.json")))
    H = I = 64
    bits = 4
    x = np.array(spec["x"], dtype=np.float64)
    r = np.arange(I)
    gate = (np.full((I, H), 1), np.full((I, 1), 0.25), np.full((I, 1), -0.125))
    up = (np.repeat((r % 4)[:, None], H, 1), np.full((I, 1), 0.5), np.full((I, 1), 0.0))
    down = (np.full((H, I), 3), np.full((H, 1), 0.25), np.full((H, 1), 0.0))
    blob = make_expert_blob(orc, H, I, bits, gate, up, down)
    g, u, h, y = orc.expert(blob, bits, H, I, x)
    assert np.all(g == spec["g"])
    assert np.array_equal(u, np.array(spec["u_by_row_mod_4"])[r % 4])
    assert np.allclose(h, np.array(spec["h_by_row_mod_4"])[r % 4], rtol=1e-15)
    assert np.allclose(y, spec["y"], rtol=1e-14)


# --------------------------------------------------------------------------- routing
def brute_force_topk(logits, K):
    """argmax over all K-subsets of the summed logits, ties -> lexicographically
    smallest index set; then ordered by descending logit, ascending index."""
    E = len(logits)
    best = max(itertools.combinations(range(E), K), key=lambda s: (sum(logits[i] for i in s), [-i for i in s]))
    return sorted(best, key=lambda i: (-logits[i], i))


@pytest.mark.parametrize("E,K", [(8, 2), (12, 4), (9, 1), (6, 6)])
def test_topk_brute_force_and_weights(orc, E, K):
    rng = np.random.default_rng(E * 10 + K)
    for _ in range(20):
        logits = rng.standard_normal(E) * 2
        idx, w, margin = orc.route(logits, K)
        assert list(idx) == brute_force_topk(list(logits), K)
        sel = logits[idx]
        ref = np.exp(sel - sel.max()) / np.exp(sel - sel.max()).sum()   # softmax over the selected
        assert np.allclose(w, ref, rtol=1e-13)
        assert abs(w.sum() - 1) < 1e-14
        assert np.all(np.diff(w) <= 0)
        if K < E:
            rest = np.delete(logits, idx)
            assert margin == pytest.approx(sel[-1] - rest.max())


def test_route_zero_logits_and_ties(orc):
    idx, w, margin = orc.route(np.zeros(8), 3)
    assert list(idx) == [0, 1, 2] and np.allclose(w, 1 / 3) and margin == 0.0
    logits = np.array([0.5, 2.0, 2.0, -1.0, 2.0])
    idx, w, _ = orc.route(logits, 2)
    assert list(idx) == [1, 2] and np.allclose(w, 0.5)


def test_route_nan_counts_as_minus_inf(orc):
    """Reading for non-finite logits (the pages are silent): NaN ranks as -inf in the selection and
    weighs exp(-inf) = 0; with no finite logit at all the weights are 1/K.  Hand cases."""
    nan, inf = np.nan, np.inf
    # NaN at index 0, two finite logits: the finite ones win, softmax over them
    idx, w, margin = orc.route(np.array([nan, 2.0, 1.0, nan, 0.5]), 2)
    assert list(idx) == [1, 2]
    e = np.exp(-1.0)
    assert np.allclose(w, [1 / (1 + e), e / (1 + e)], rtol=1e-15) and np.all(np.isfinite(w))
    assert margin == pytest.approx(0.5)
    # K beyond the finite logits: NaN and -inf follow in index order, with weight exactly 0
    idx, w, _ = orc.route(np.array([nan, 2.0, -inf, nan, 1.0]), 4)
    assert list(idx) == [1, 4, 0, 2]
    assert np.allclose(w[:2], [1 / (1 + e), e / (1 + e)], rtol=1e-15) and w[2] == 0.0 and w[3] == 0.0
    # no finite logit: lower indices first, equal weights
    idx, w, _ = orc.route(np.array([nan, -inf, nan, -inf]), 3)
    assert list(idx) == [0, 1, 2] and np.array_equal(w, np.full(3, 1 / 3))
    # the NaN reading equals routing the same logits with NaN replaced by -inf
    rng = np.random.default_rng(11)
    for _ in range(20):
        lg = rng.standard_normal(12)
        lg[rng.random(12) < 0.4] = nan
        a_i, a_w, _ = orc.route(lg, 4)
        b_i, b_w, _ = orc.route(np.where(np.isnan(lg), -inf, lg), 4)
        assert list(a_i) == list(b_i) and np.array_equal(a_w, b_w)


def test_route_permutation_equivariance(orc):
    rng = np.random.default_rng(7)
    logits = rng.standard_normal(32)
    perm = rng.permutation(32)
    idx, w, _ = orc.route(logits, 4)
    idx_p, w_p, _ = orc.route(logits[perm], 4)
    assert list(perm[idx_p]) == list(idx) and np.allclose(w, w_p, rtol=1e-15)


def test_router_logits_bf16_and_bias(orc):
    rng = np.random.default_rng(8)
    Wf = rng.integers(-8, 8, size=(6, 128)).astype(np.float32) * 0.25   # exact in bf16
    Wb = (Wf.view(np.uint32) >> 16).astype(np.uint16)
    x = rng.integers(-4, 5, size=128).astype(np.float64)
    bias = np.arange(6, dtype=np.float32) * 0.5
    exact = Wf.astype(np.int64 if False else np.float64) @ x + bias
    assert np.array_equal(orc.router_logits(Wf, x, bias), exact)
    assert np.array_equal(orc.router_logits(Wb, x, bias, wr_is_bf16=True), exact)


# --------------------------------------------------------------------------- norm, silu, combine
def test_rmsnorm_constant_vector_closed_form(orc):
    H, c, eps = 128, -1.5, 1e-6
    w = np.full(H, bf16(1.25), dtype=np.uint16)
    out = orc.rmsnorm(np.full(H, c), w, eps)
    assert np.allclose(out, c / math.sqrt(c * c + eps) * 1.25, rtol=1e-15)


def test_rmsnorm_unit_rms_and_weight(orc):
    rng = np.random.default_rng(9)
    x = rng.standard_normal(256) * 7
    w = np.full(256, bf16(1.0), dtype=np.uint16)
    n = orc.rmsnorm(x, w, 0.0)
    assert math.sqrt(np.mean(n * n)) == pytest.approx(1.0, rel=1e-14)
    assert np.allclose(n / x, n[0] / x[0], rtol=1e-13)          # a common positive scalar


def test_silu_special_values(orc):
    assert orc.silu(0.0) == 0.0
    assert orc.silu(50.0) == pytest.approx(50.0, rel=1e-15)
    assert abs(orc.silu(-50.0)) < 1e-19
    for z in [0.3, 1.7, 4.0, 9.5]:
        assert orc.silu(z) - orc.silu(-z) == pytest.approx(z, rel=1e-14)   # z*sig(z) + z*sig(-z) = z
    assert orc.silu(1.0) == pytest.approx(0.7310585786300049, rel=1e-15)   # 1 / (1 + 1/e)


def test_combine_k1_and_residual(orc):
    rng = np.random.default_rng(10)
    y = rng.standard_normal((1, 64))
    assert np.array_equal(orc.combine(y, np.array([1.0])), y[0])
    y = rng.standard_normal((3, 64))
    w = np.array([0.5, 0.25, 0.25])
    x = rng.standard_normal(64)
    assert np.allclose(orc.combine(y, w, x), 0.5 * y[0] + 0.25 * y[1] + 0.25 * y[2] + x, rtol=1e-15)


def test_layer_identical_experts_output_equals_expert(orc):
    # Weights sum to 1, so with every expert identical the layer output equals y.
    import oracle as O
    H, I, E, K = 128, 64, 6, 3
    rng = np.random.default_rng(11)
    mats = [(rng.integers(0, 16, (I, H)), np.full((I, H // 64), 0.0078125), np.full((I, H // 64), -0.0625)),
            (rng.integers(0, 16, (I, H)), np.full((I, H // 64), 0.0078125), np.full((I, H // 64), 0.015625)),
            (rng.integers(0, 16, (H, I)), np.full((H, I // 64), 0.00390625), np.full((H, I // 64), -0.03125))]
    blob = make_expert_blob(orc, H, I, 4, *mats)
    router = rng.standard_normal((E, H)).astype(np.float32)
    L = O.LayerWeights(router, False, lambda e: blob, lambda e: 4)
    x = rng.standard_normal(H)
    res = O.layer_token(x, L, H, I, K)
    _, _, _, y = orc.expert(blob, 4, H, I, x)
    assert np.allclose(res.out, y, rtol=1e-13)
    assert abs(res.w.sum() - 1) < 1e-14


@pytest.mark.parametrize("bits", [2, 4])
def test_random_expert_matches_independent_numpy(orc, bits):
    # Non-square expert (H != I) with random codes, scales and biases: the oracle's
    # g, u, h, y equal a float64 numpy evaluation built from the tests' own packer and
    # unpacker (catches transposed operands, swapped planes and per-group mix-ups).
    H, I = 192, 128
    rng = np.random.default_rng(12 + bits)

    def mat(R, C):
        codes = rng.integers(0, 1 << bits, (R, C))
        s = (rng.uniform(0.002, 0.02, (R, C // 64)).astype(np.float32).view(np.uint32) & 0xFFFF0000).view(np.float32)
        b = (rng.uniform(-0.1, 0.1, (R, C // 64)).astype(np.float32).view(np.uint32) & 0xFFFF0000).view(np.float32)
        W = (codes.astype(np.float32) * np.repeat(s, 64, 1) + np.repeat(b, 64, 1)).astype(np.float64)
        return (codes, s, b), W

    (gm, Wg), (um, Wu), (dm, Wd) = mat(I, H), mat(I, H), mat(H, I)
    blob = make_expert_blob(orc, H, I, bits, gm, um, dm)
    x = rng.standard_normal(H)
    g, u, h, y = orc.expert(blob, bits, H, I, x)
    gr, ur = Wg @ x, Wu @ x
    hr = gr / (1 + np.exp(-gr)) * ur
    assert np.allclose(g, gr, rtol=1e-12, atol=1e-12) and np.allclose(u, ur, rtol=1e-12, atol=1e-12)
    assert np.allclose(h, hr, rtol=1e-12, atol=1e-12)
    assert np.allclose(y, Wd @ hr, rtol=1e-11, atol=1e-11)


# ----------------------------------------------------------------------------- quantise-from-float
def _bf16_value(bits16: np.ndarray) -> np.ndarray:
    return (bits16.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _rne_bf16(x: float) -> float:
    """bf16 round-to-nearest-even of an fp32 value, by exhaustive neighbour search in float64
    (independent of bit tricks): the nearest of the two bf16 neighbours, ties to even mantissa."""
    f = float(np.float32(x))
    u = int(np.array([f], dtype=np.float32).view(np.uint32)[0])
    lo_u = u & 0xFFFF0000
    cand = [lo_u, lo_u + 0x10000]
    vals = [float(np.array([c], dtype=np.uint32).view(np.float32)[0]) for c in cand]
    d = [abs(v - f) for v in vals]
    if d[0] != d[1]:
        return vals[0] if d[0] < d[1] else vals[1]
    return vals[0] if ((cand[0] >> 16) & 1) == 0 else vals[1]


@pytest.mark.parametrize("bits", [4, 2])
def test_quantize_exact_grid(bits):
    """Pins orc_quantize on groups that lie exactly on a bf16 grid: w = lo + k * s with lo, s and
    the extremes exactly representable, both k = 0 and k = 2^b - 1 present.  Then the scale, the
    bias and every code are known exactly (a wrong qmax, swapped scale/bias, an offset code or a
    floor instead of round fails)."""
    import oracle
    qmax = (1 << bits) - 1
    rng = np.random.default_rng(7 + bits)
    rows, G = 3, 4
    W = np.empty((rows, 64 * G), dtype=np.float32)
    ks = rng.integers(0, qmax + 1, size=(rows, 64 * G))
    ks[:, ::64] = 0
    ks[:, 1::64] = qmax
    los = np.array([-0.75, 0.125, -3.0, 2.5], dtype=np.float64)
    ss = np.array([2.0 ** -5, 2.0 ** -3, 0.375, 2.0 ** -9], dtype=np.float64)
    for g in range(G):
        W[:, 64 * g:64 * (g + 1)] = (los[g] + ks[:, 64 * g:64 * (g + 1)] * ss[g]).astype(np.float32)
    codes, scale, bias = oracle.quantize(W, bits)
    assert np.array_equal(codes, ks)
    for g in range(G):
        assert np.all(_bf16_value(scale[:, g]) == ss[g]) and np.all(_bf16_value(bias[:, g]) == los[g])


def test_quantize_constant_group():
    """A constant group has scale 0, codes 0, and the bf16-rounded value as its bias (so it
    dequantises to bf16(v)); neighbouring groups are unaffected."""
    import oracle
    W = np.zeros((2, 128), dtype=np.float32)
    W[0, :64] = 0.1
    W[1, :64] = -7.3
    W[:, 64:] = np.linspace(-1, 1, 64, dtype=np.float32)
    codes, scale, bias = oracle.quantize(W, 4)
    assert np.all(codes[:, :64] == 0) and np.all(scale[:, 0] == 0)
    assert _bf16_value(bias[0, 0]) == _rne_bf16(0.1) and _bf16_value(bias[1, 0]) == _rne_bf16(-7.3)
    assert codes[0, 64] == 0 and codes[0, 127] == 15


@pytest.mark.parametrize("bits", [4, 2])
def test_quantize_nearest_code_brute_force(bits):
    """Pins the codes of random groups (normal, uniform, negative-only, wide and narrow ranges,
    values far from zero) against brute force in float64: with the stored bf16 scale s and bias b,
    every code is the nearest of all 2^b codes to w (up to fp32 rounding of the ratio), and s and
    b are the round-to-nearest-even bf16 of (max - min) / (2^b - 1) and of min (checked against an
    independent neighbour search)."""
    import oracle
    qmax = (1 << bits) - 1
    rng = np.random.default_rng(11 + bits)
    groups = [rng.normal(0, 1, 64), rng.uniform(-0.02, 0.02, 64), -rng.uniform(1, 2, 64),
              rng.normal(0, 30, 64), 100.3 + rng.uniform(0, 1e-3, 64), rng.normal(0, 1e-4, 64),
              np.concatenate([rng.normal(0, 1, 63), [40.0]])]
    W = np.concatenate(groups).astype(np.float32).reshape(1, -1)
    codes, scale, bias = oracle.quantize(W, bits)
    for g in range(len(groups)):
        w = W[0, 64 * g:64 * (g + 1)].astype(np.float64)
        s, b = _bf16_value(scale[0, g]), _bf16_value(bias[0, g])
        lo, hi = float(np.float32(w.min())), float(np.float32(w.max()))
        assert s == _rne_bf16(float(np.float32(np.float32(hi - lo) / np.float32(qmax))))
        assert b == _rne_bf16(lo)
        grid = b + s * np.arange(qmax + 1)
        for i in range(64):
            err = np.abs(w[i] - grid)
            best = err.min()
            c = int(codes[0, 64 * g + i])
            assert err[c] <= best + 1e-5 * max(s, 1e-30) * 2, (g, i, c, int(err.argmin()))


# --------------------------------------------------------------------------- hot set and re-tiering
def test_expert_usage_brute_force():
    """Pins oracle.expert_usage against a plain dictionary count on routing indices with
    out-of-range entries (which are not counted), and the total against the valid entry count."""
    import oracle
    rng = np.random.default_rng(21)
    E = 37
    idx = rng.integers(-3, E + 3, size=(200, 4)).astype(np.int32)
    counts = oracle.expert_usage(idx, E)
    ref = {}
    for v in idx.ravel().tolist():
        if 0 <= v < E:
            ref[v] = ref.get(v, 0) + 1
    assert [int(c) for c in counts] == [ref.get(e, 0) for e in range(E)]
    assert int(counts.sum()) == int(((idx >= 0) & (idx < E)).sum())


def test_hot_order_hand_case_and_invariants():
    """Pins oracle.hot_order on a hand case with ties, and on random counts with many ties by the
    properties that fix the order uniquely: a permutation, counts non-increasing along it, and the
    expert index increasing inside each run of equal counts."""
    import oracle
    assert oracle.hot_order(np.array([3, 5, 5, 0, 3, 7])).tolist() == [5, 1, 2, 0, 4, 3]
    rng = np.random.default_rng(22)
    counts = rng.integers(0, 6, size=300)
    order = oracle.hot_order(counts)
    assert sorted(order.tolist()) == list(range(300))
    c = counts[order]
    assert np.all(c[:-1] >= c[1:])
    same = c[:-1] == c[1:]
    assert np.all(order[:-1][same] < order[1:][same])


def _exact_matrix(rng, rows, cols, bits, k_set, s_vals, b_vals):
    """Codes drawn from k_set with every member present in every group, dyadic scales and
    biases: (codes, scale, bias) as make_expert_blob takes them."""
    G = cols // 64
    k_set = np.asarray(k_set)
    codes = k_set[rng.integers(0, k_set.size, size=(rows, cols))]
    for g in range(G):
        codes[:, 64 * g:64 * g + k_set.size] = k_set
    scale = np.array([[s_vals[(r + g) % len(s_vals)] for g in range(G)] for r in range(rows)])
    bias = np.array([[b_vals[(2 * r + g) % len(b_vals)] for g in range(G)] for r in range(rows)])
    return codes.astype(np.uint8), scale, bias


def _check_requant(result, expected):
    for (codes, scale, bias), (ec, es, eb) in zip(result, expected):
        assert np.array_equal(codes, ec)
        assert np.array_equal(_bf16_value(scale), es) and np.array_equal(_bf16_value(bias), eb)


def test_requantize_expert_exact_cases(orc):
    """Pins oracle.requantize_expert where the answer is exact, with different patterns in gate,
    up and down (a swapped or mis-offset matrix fails):
      4 -> 4 with codes 0 and 15 in every group returns the same codes and pairs;
      4 -> 2 with codes {0, 5, 10, 15} gives code / 5, scale 5s and the same bias;
      2 -> 4 with codes {0..3} and s = 5 * 2^-7 gives 5 * code, scale s / 5 and the same bias."""
    import oracle
    H, I = 192, 128
    rng = np.random.default_rng(23)
    s4 = [2.0 ** -6, 2.0 ** -4, 0.375 * 2.0 ** -5]
    b4 = [-0.5, 0.25, -2.0 ** -3, 1.5]
    for bits_in, bits_out, k_set, s_vals, mult in [
            (4, 4, list(range(16)), s4, None),
            (4, 2, [0, 5, 10, 15], s4, 5),
            (2, 4, [0, 1, 2, 3], [5 * 2.0 ** -7, 5 * 2.0 ** -9], 0.2)]:
        mats = [_exact_matrix(rng, I, H, bits_in, k_set, s_vals, b4),
                _exact_matrix(rng, I, H, bits_in, k_set[::-1], s_vals[::-1], b4[1:]),
                _exact_matrix(rng, H, I, bits_in, k_set, s_vals[1:] + s_vals[:1], b4[::-1])]
        blob = make_expert_blob(orc, H, I, bits_in, *mats)
        got = oracle.requantize_expert(blob, H, I, bits_in, bits_out)
        if mult is None:
            exp = [(c, s, b) for c, s, b in mats]
        elif mult == 5:
            exp = [(c // 5, s * 5, b) for c, s, b in mats]
        else:
            exp = [(c * 5, s / 5, b) for c, s, b in mats]
        _check_requant(got, exp)


@pytest.mark.parametrize("bits_in,bits_out", [(4, 2), (2, 4), (4, 4)])
def test_requantize_error_bound(orc, bits_in, bits_out):
    """Pins oracle.requantize_matrix by the quantiser's error bound on random packed matrices: with
    the new pair (s', b') of a group whose dequantised weights span [lo, hi], every weight w is
    within s'/2 + |lo - b'| + qmax |s' - (hi - lo)/qmax| (+ fp32 rounding) of q' s' + b'."""
    import oracle
    rng = np.random.default_rng(24 + bits_in + 3 * bits_out)
    rows, cols = 16, 512
    G = cols // 64
    codes = rng.integers(0, 1 << bits_in, size=(rows, cols)).astype(np.uint8)
    scale = np.array([[_rne_bf16(float(v)) for v in row] for row in rng.uniform(1e-3, 0.05, (rows, G))])
    bias = np.array([[_rne_bf16(float(v)) for v in row] for row in rng.uniform(-0.5, 0.5, (rows, G))])
    plane = pack_codes_by_hand(codes, bits_in)
    sb = sb_plane(scale, bias)
    W = np.repeat(scale, 64, axis=1) * codes + np.repeat(bias, 64, axis=1)      # float64, as stored
    c2, s2, b2 = oracle.requantize_matrix(plane, sb, rows, cols, bits_in, bits_out)
    qmax = (1 << bits_out) - 1
    for r in range(rows):
        for g in range(G):
            w = W[r, 64 * g:64 * (g + 1)]
            s, b = float(_bf16_value(s2[r, g])), float(_bf16_value(b2[r, g]))
            lo, hi = w.min(), w.max()
            bound = s / 2 + abs(lo - b) + qmax * abs(s - (hi - lo) / qmax) + 1e-6 * max(abs(lo), abs(hi), 1e-3)
            err = np.abs(w - (c2[r, 64 * g:64 * (g + 1)] * s + b))
            assert err.max() <= bound, (r, g, err.max(), bound)


# --------------------------------------------------------------------------- expert cache policy
def test_expert_cache_model_hand_trace():
    """Pins oracle.ExpertCacheModel on a trace worked out by hand with 3 slots:
    {1,2} -> misses into slots 0,1; {2,3} -> 2 hit, 3 into free slot 2; {4,1} -> 1 hit (slot 0, now
    newest), 4 evicts the least recently used untouched slot: slot 1 (expert 2, last used in call 2)
    ties with slot 2 (expert 3, call 2) -> the lower slot 1; {3,5,5,-1,9} with E = 8 -> 3 hit,
    5 evicts slot 0 (expert 1, call 3) vs slot 1 (expert 4, call 3) -> slot 0."""
    import oracle
    m = oracle.ExpertCacheModel(8, 3)
    assert m.fetch([1, 2]) == (0, 2, [(1, 0), (2, 1)], [])
    assert m.fetch([2, 3]) == (1, 1, [(3, 2)], [])
    assert m.fetch([4, 1]) == (1, 1, [(4, 1)], [2])
    assert m.fetch([3, 5, 5, -1, 9]) == (1, 1, [(5, 0)], [1])
    assert m.slot_of == {3: 2, 4: 1, 5: 0} and m.hits == 3 and m.misses == 5
    with pytest.raises(ValueError):
        m.fetch([0, 1, 2, 6])
    assert m.slot_of == {3: 2, 4: 1, 5: 0} and m.tick == 4


def test_expert_cache_model_properties():
    """On random routing traces: every expert of a call is resident after it; a call never evicts
    one of its own experts; no eviction while a slot is free; an expert requested in two
    consecutive calls is a hit the second time; with at least as many slots as experts, the misses
    are exactly the first requests of each expert."""
    import oracle
    rng = np.random.default_rng(31)
    for E, n_slots, K in [(16, 4, 2), (40, 9, 4), (12, 12, 3)]:
        m = oracle.ExpertCacheModel(E, n_slots)
        seen, prev = set(), set()
        for _ in range(300):
            req = rng.choice(E, size=K, replace=False)
            occupied = sum(1 for x in m.expert_of if x >= 0)
            hits, misses, loads, evicted = m.fetch(req)
            cur = set(int(e) for e in req)
            assert all(e in m.slot_of for e in cur)
            assert not (set(evicted) & cur)
            if occupied + misses <= n_slots:
                assert not evicted
            assert all(e in m.slot_of for e in prev & cur) and hits >= len(prev & cur)
            if n_slots >= E:
                assert misses == len(cur - seen)
            seen |= cur
            prev = cur
