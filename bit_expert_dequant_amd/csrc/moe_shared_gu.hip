// moe_shared_gu.hip -- shared-read expert FFN for a few tokens, first half: the activation rows
// staged once per call, then the gate/up rows of every distinct expert of the call with SwiGLU
// (the work split and the staging are described in moe_small.h).  moe_shared_gux.hip holds the
// same gate/up launch with every workgroup staging its rows from x itself.
#include "moe_small.h"

namespace moe {
namespace {

// The call's T activation rows (normalised first when the layer has a norm weight) as digit planes
// in both code widths, once for all workgroups: row t at out + t * (H + H / 16), the 4-bit order,
// the 2-bit order, then xs.  One workgroup per row, two 16-column chunks per thread (H <= 8192).
__global__ void __launch_bounds__(kBlock) k_stage_rows(const void *x, int x_dtype, int H, const uint16_t *norm_w,
                                                       float eps, uint32_t *out) {
    __shared__ float red[kWaves];
    const int t = blockIdx.x, nch = H / 16;
    const size_t rowb = (size_t)H * (x_dtype == MOE_BF16 ? 2 : 4);
    const void *xr = (const char *)x + (size_t)t * rowb;
    Chunk16 xc[2], nc[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int m = min((int)threadIdx.x + kBlock * j, nch - 1);
        issue_chunk16(xr, x_dtype, m, xc[j]);
        if (norm_w) issue_chunk16(norm_w, MOE_BF16, m, nc[j]);
    }
    float v[2][16];
#pragma unroll
    for (int j = 0; j < 2; ++j) chunk16_f32(xc[j], x_dtype, v[j]);
    if (norm_w) {
        float ss = 0.f;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            float w[16];
            chunk16_f32(nc[j], MOE_BF16, w);
            if ((int)threadIdx.x + kBlock * j < nch) {
#pragma unroll
                for (int i = 0; i < 16; ++i) ss += v[j][i] * v[j][i];
            }
#pragma unroll
            for (int i = 0; i < 16; ++i) v[j][i] *= w[i];
        }
        ss = block_sum(ss, red);
        const float inv = 1.0f / sqrtf(ss / (float)H + eps);
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int i = 0; i < 16; ++i) v[j][i] *= inv;
    }
    uint32_t *row = out + (size_t)t * (H + H / 16);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int m = threadIdx.x + kBlock * j;
        stage_chunk(m, m < nch, v[j], row, row + H / 2, (float2 *)(row + H));
    }
}

}  // namespace

hipError_t launch_shared_gateup(const GroupedLaunch &a, hipStream_t s, const KernelEvents &ev) {
    hipLaunchKernelGGL(k_stage_rows, dim3(a.T), dim3(kBlock), 0, s, a.x, a.x_dtype, a.H, a.norm_w, a.norm_eps,
                       a.planes);
    if (hipError_t e = hipGetLastError()) return e;
    return launch_gu_sh<true>(a, s, ev);
}

}  // namespace moe
