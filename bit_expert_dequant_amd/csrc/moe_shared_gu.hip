// moe_shared_gu.hip -- shared-read expert FFN for a few tokens, first half: the activation rows
// staged once per call, then the gate/up rows of every distinct expert of the call with SwiGLU
// (the work split and the staging are described in moe_small.h).
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

// An entry's rows in at most two batches of `cap`, written out rather than looped: a loop around the
// body keeps its hoisted addresses live throughout and spills.
// UPW: the unrolled pipeline's length, kSharedUPW when upw <= kSharedUPW (many rows per expert:
// many short slices) else kGuUPW / kDnUPW.
template <int NJ, int GS, int UPW>
__device__ __forceinline__ void gu_batch(const GroupedLaunch &a, const SharedWork &w, int tb, uint32_t *lds) {
    TokRec<kSmallTokens> r;
    row_batch(w, tb, a.cap, r);
    if (r.bits == 2) gu8_body<2, NJ, GS, UPW, kSmallTokens, true>(a, r, w.sl, w.upw, lds);
    else gu8_body<4, NJ, GS, UPW, kSmallTokens, true>(a, r, w.sl, w.upw, lds);
}
template <int NJ, int GS, int UPW>
__device__ __forceinline__ void gu_entry(const GroupedLaunch &a, const SharedWork &w, uint32_t *lds) {
    gu_batch<NJ, GS, UPW>(a, w, 0, lds);
    if (w.n > a.cap) {
        __syncthreads();                          // the first batch's rows are no longer read
        gu_batch<NJ, GS, UPW>(a, w, a.cap, lds);
    }
}
template <int NJ, int GS>
__global__ void __launch_bounds__(kBlock) k_gu_sh(GroupedLaunch a) {
    extern __shared__ __align__(16) uint32_t lds[];
    SharedWork w;
    shared_work(a, a.geo.nblk, shared_rec_off(a.H, a.cap, a.E), lds, w);
    if (w.upw == 0) return;
    if (w.upw <= kSharedUPW) gu_entry<NJ, GS, kSharedUPW>(a, w, lds);
    else gu_entry<NJ, GS, kGuUPW>(a, w, lds);
}

}  // namespace

hipError_t launch_shared_gateup(const GroupedLaunch &a, hipStream_t s, const KernelEvents &ev) {
    hipLaunchKernelGGL(k_stage_rows, dim3(a.T), dim3(kBlock), 0, s, a.x, a.x_dtype, a.H, a.norm_w, a.norm_eps,
                       a.planes);
    if (hipError_t e = hipGetLastError()) return e;
    const dim3 grid(shared_grid(a.geo.nblk, a.T * a.K));
    const size_t lds = shared_lds_bytes(a.H, a.cap, a.E);
    const int nj = nj_for(a.H), gs = small_gs(a.H, nj);
    switch (nj) {
        case 1:
            return gs == 64   ? launch_lds<k_gu_sh<1, 64>>(grid, lds, s, ev, a)
                   : gs == 32 ? launch_lds<k_gu_sh<1, 32>>(grid, lds, s, ev, a)
                              : launch_lds<k_gu_sh<1, 0>>(grid, lds, s, ev, a);
        case 2: return gs ? launch_lds<k_gu_sh<2, 64>>(grid, lds, s, ev, a) : launch_lds<k_gu_sh<2, 0>>(grid, lds, s, ev, a);
        default: return gs ? launch_lds<k_gu_sh<4, 64>>(grid, lds, s, ev, a) : launch_lds<k_gu_sh<4, 0>>(grid, lds, s, ev, a);
    }
}

}  // namespace moe
