"""The allocation-free decode entry point (moe_layer_decode_static) against moe_layer_decode on the
same inputs: two calls in a row, the second with a smaller layer, and a rejected oversize request."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import bit_expert_dequant_amd as M  # noqa: E402
from moe_cases import act_tensor, assert_close, build_layer, small_workload  # noqa: E402


def _decode(fn, dl, x, residual, **kw):
    wl = dl.wl
    d = M.make_dims(wl.H, wl.I, wl.E, wl.K)
    out = torch.empty(wl.H, dtype=torch.float32, device="cuda")
    idx = torch.empty(wl.K, dtype=torch.int32, device="cuda")
    w = torch.empty(wl.K, dtype=torch.float32, device="cuda")
    fn(d, [dl.L], x, out, idx, w, residual=residual, **kw)
    torch.cuda.synchronize()
    return out.cpu().numpy(), idx.cpu().numpy(), w.cpu().numpy()


@pytest.mark.parametrize("schedule", ["two_launch", "single_launch", "three_kernels"])
def test_static_decode_matches_workspace_decode(schedule):
    kw = {"separate_kernels": schedule == "three_kernels", "single_launch": schedule == "single_launch"}
    big = small_workload("static_big", 0x5A7, 4096, 1024, 512, 4, 4, norm=True)    # 117.5 KiB of workspace
    small = small_workload("static_small", 0x5A8, 1024, 512, 16, 2, 2)
    for wl, residual in ((big, True), (small, False)):
        dl = build_layer(wl)
        bank = wl.tokens_bank(2)
        d = M.make_dims(wl.H, wl.I, wl.E, wl.K)
        ws = M.workspace(M.MOE_OP_LAYER_DECODE, d, 1, 1)
        for t in range(2):
            x = act_tensor(wl, bank[t])
            ref = _decode(M.moe_layer_decode, dl, x, residual, ws=ws, **kw)
            got = _decode(M.moe_layer_decode_static, dl, x, residual, **kw)
            assert list(got[1]) == list(ref[1]), f"{wl.name} token {t} idx"
            assert np.array_equal(got[0], ref[0]), f"{wl.name} token {t}: same kernels, same result"
            assert_close(got[2], ref[2], f"{wl.name} token {t} w")


def test_static_decode_rejects_oversize_dims():
    d = M.make_dims(8192, 4608, 2048, 8)     # decode workspace larger than the static scratch
    assert M.moe_workspace_bytes(M.MOE_OP_LAYER_DECODE, d) > (1 << 18)
    wl = small_workload("static_tiny", 0x5A9, 256, 128, 4, 2, 4)
    dl = build_layer(wl)
    x = act_tensor(wl, wl.tokens_bank(1)[0])
    out = torch.empty(8192, dtype=torch.float32, device="cuda")
    with pytest.raises(M.MoeError) as ei:
        M.moe_layer_decode_static(d, [dl.L], x, out)
    assert ei.value.status == 6 and "static scratch" in str(ei.value)     # MOE_ERR_WORKSPACE
