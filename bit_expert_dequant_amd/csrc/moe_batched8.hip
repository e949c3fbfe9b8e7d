// moe_batched8.hip -- batched (T > 1) expert FFN for the experts of a batch that received few
// tokens (the small-expert list the grouping pass writes), on the integer dot-product building
// blocks of moe_small.h:
//
//   k_gu8 : gate/up rows of one small expert, h = silu(g) * u for each of its tokens (rows of
//           the expert-ordered h buffer, as the MFMA kernels write them)
//   k_dn8 : down rows of one small expert, each token's output row written to y[token][slot]
#include "moe_small.h"

namespace moe {
namespace {

template <int NJ, int GS>
__global__ void __launch_bounds__(kBlock) k_gu8(GroupedLaunch a) {
    extern __shared__ __align__(16) uint32_t lds[];
    SmallRec se;
    if (!small_entry(a, se)) return;
    if (se.bits == 2) gu8_body<2, NJ, GS, kGuUPW>(a, se, blockIdx.x, kGuUPW, lds);
    else gu8_body<4, NJ, GS, kGuUPW>(a, se, blockIdx.x, kGuUPW, lds);
}

template <int NJ, int GS>
__global__ void __launch_bounds__(kBlock) k_dn8(GroupedLaunch a) {
    extern __shared__ __align__(16) uint32_t lds[];
    SmallRec se;
    if (!small_entry(a, se)) return;
    if (se.bits == 2) dn8_body<2, NJ, GS, kDnUPW>(a, se, blockIdx.x, kDnUPW, lds);
    else dn8_body<4, NJ, GS, kDnUPW>(a, se, blockIdx.x, kDnUPW, lds);
}

}  // namespace

bool small_path_fits(int H, int I) {
    return small_lds_bytes(H) <= kMaxLds && small_lds_bytes(I) <= kMaxLds && H % 64 == 0 && I % 64 == 0;
}

hipError_t launch_small_gateup(const GroupedLaunch &a_in, int max_small, hipStream_t s) {
    GroupedLaunch a = a_in;
    a.geo = gateup_geo(a.H, a.I);
    a.pt = plane_table(a.H, a.I);
    a.upw = kGuUPW;
    const dim3 grid((a.geo.nblk + kWaves * kGuUPW - 1) / (kWaves * kGuUPW), max_small);
    const size_t lds = small_lds_bytes(a.H);
    const KernelEvents ev{};
    const int nj = nj_for(a.H), gs = small_gs(a.H, nj);
    switch (nj) {
        case 1:
            return gs == 64   ? launch_lds<k_gu8<1, 64>>(grid, lds, s, ev, a)
                   : gs == 32 ? launch_lds<k_gu8<1, 32>>(grid, lds, s, ev, a)
                              : launch_lds<k_gu8<1, 0>>(grid, lds, s, ev, a);
        case 2: return gs ? launch_lds<k_gu8<2, 64>>(grid, lds, s, ev, a) : launch_lds<k_gu8<2, 0>>(grid, lds, s, ev, a);
        default: return gs ? launch_lds<k_gu8<4, 64>>(grid, lds, s, ev, a) : launch_lds<k_gu8<4, 0>>(grid, lds, s, ev, a);
    }
}

hipError_t launch_small_down(const GroupedLaunch &a_in, int max_small, hipStream_t s) {
    GroupedLaunch a = a_in;
    const int nj = nj_for(a.I), gs = small_gs(a.I, nj);
    a.geo = row_geo(a.I, a.H, nj == 1 ? dn8_rg<1>() : nj == 2 ? dn8_rg<2>() : dn8_rg<4>());
    a.pt = plane_table(a.H, a.I);
    a.upw = kDnUPW;
    const dim3 grid((a.geo.nblk + kWaves * kDnUPW - 1) / (kWaves * kDnUPW), max_small);
    const size_t lds = small_lds_bytes(a.I);
    const KernelEvents ev{};
    switch (nj) {
        case 1:
            return gs == 64   ? launch_lds<k_dn8<1, 64>>(grid, lds, s, ev, a)
                   : gs == 32 ? launch_lds<k_dn8<1, 32>>(grid, lds, s, ev, a)
                              : launch_lds<k_dn8<1, 0>>(grid, lds, s, ev, a);
        case 2: return gs ? launch_lds<k_dn8<2, 64>>(grid, lds, s, ev, a) : launch_lds<k_dn8<2, 0>>(grid, lds, s, ev, a);
        default: return gs ? launch_lds<k_dn8<4, 64>>(grid, lds, s, ev, a) : launch_lds<k_dn8<4, 0>>(grid, lds, s, ev, a);
    }
}

}  // namespace moe
