"""GPU parity of quantise-from-float (moe_quantize_matrix) against the CPU oracle: every code and
every (scale, bias) pair bit-exact, over shapes from one group to a full expert matrix, both code
widths, fp32 and bf16 weights, and groups that are constant, negative-only, of huge or tiny range,
or far from zero."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import bit_expert_dequant_amd as M  # noqa: E402
import oracle  # noqa: E402


def unpack_codes(plane: np.ndarray, rows: int, cols: int, bits: int) -> np.ndarray:
    """Codes of a packed plane, LSB-first within each byte (the header's layout)."""
    per = 8 // bits
    b = plane.reshape(rows, cols // per)
    out = np.empty((rows, cols), dtype=np.uint8)
    for k in range(per):
        out[:, k::per] = (b >> (k * bits)) & ((1 << bits) - 1)
    return out


def weights(rows: int, cols: int, seed: int) -> np.ndarray:
    rng = np.random.default_rng(seed)
    W = rng.normal(0, 0.05, size=(rows, cols)).astype(np.float32)
    G = cols // 64
    special = [
        lambda: np.full(64, 0.1),                                    # constant
        lambda: -rng.uniform(1, 2, 64),                              # negative-only
        lambda: rng.normal(0, 300, 64),                              # huge range
        lambda: rng.normal(0, 1e-6, 64),                             # tiny range
        lambda: 100.3 + rng.uniform(0, 1e-3, 64),                    # far from zero, narrow
        lambda: np.concatenate([rng.normal(0, 1, 63), [40.0]]),      # one outlier
        lambda: np.zeros(64),                                        # all zero
        # exact half-integer quotients (w - bias) / scale = k + 1/2 under a scale whose reciprocal is
        # inexact (3 * 2^-6): the codes follow ties-to-even only if the IEEE quotient decides them
        lambda: np.concatenate([[-1.0, -1.0 + 15 * 3 * 2.0 ** -6],
                                -1.0 + (np.arange(62) % 15 + 0.5) * 3 * 2.0 ** -6]),
    ]
    for i, f in enumerate(special):
        g = (7 * i + 3) % G
        r = (5 * i + 1) % rows
        W[r, 64 * g:64 * (g + 1)] = f()
    return W


CASES = [
    # rows, cols, bits, dtype
    (1, 64, 4, "f32"),
    (37, 192, 2, "f32"),
    (64, 640, 4, "bf16"),
    (3, 4096, 2, "bf16"),
    (1024, 4096, 4, "f32"),      # a full gate/up matrix of the 4-bit experts
    (4096, 1024, 2, "f32"),      # a full down matrix, 2-bit
]


@pytest.mark.parametrize("case", CASES, ids=[f"{r}x{c}_{b}bit_{d}" for r, c, b, d in CASES])
def test_quantize_matches_oracle(case):
    rows, cols, bits, dt = case
    print(f"[quant] {rows}x{cols} {bits}-bit {dt}", flush=True)
    W = weights(rows, cols, 0x9A47 + rows + cols + bits)
    if dt == "bf16":
        wb = (W.view(np.uint32) + 0x7FFF + ((W.view(np.uint32) >> 16) & 1)) >> 16
        W = (wb.astype(np.uint32) << 16).view(np.float32)       # exactly bf16 values
        wt = torch.from_numpy(wb.astype(np.uint16).view(np.int16)).cuda().view(torch.bfloat16)
    else:
        wt = torch.from_numpy(W).cuda()
    codes = torch.zeros(M.lib().moe_packed_codes_bytes(rows, cols, bits), dtype=torch.uint8, device="cuda")
    sb = torch.zeros(2 * rows * (cols // 64), dtype=torch.int16, device="cuda")
    M.moe_quantize_matrix(wt, bits, codes, sb)
    torch.cuda.synchronize()
    oc, os_, ob = oracle.quantize(W, bits)
    gc = unpack_codes(codes.cpu().numpy(), rows, cols, bits)
    bad = np.argwhere(gc != oc)
    assert len(bad) == 0, f"{len(bad)} codes differ, first at {bad[0]}: gpu {gc[tuple(bad[0])]} oracle {oc[tuple(bad[0])]}"
    gsb = sb.cpu().numpy().view(np.uint16).reshape(rows, cols // 64, 2)
    assert np.array_equal(gsb[:, :, 0], os_), "scales differ"
    assert np.array_equal(gsb[:, :, 1], ob), "biases differ"
