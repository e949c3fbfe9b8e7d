// moe_shared_dn.hip -- shared-read expert FFN for a few tokens, second half: the down rows of every
// distinct expert of the call for the pairs that chose it, and the launcher of the whole path.
#include "moe_small.h"

namespace moe {
namespace {

// The down kernel stages up to a.cap_dn rows at once (16 when they fit in LDS: the rows of I inputs
// are short), so an entry is usually one batch.
template <int NJ, int GS, int UPW>
__device__ __forceinline__ void dn_batch(const GroupedLaunch &a, const SharedWork &w, int tb, uint32_t *lds) {
    TokRec<kSharedCap> r;
    row_batch(w, tb, a.cap_dn, r);
    if (r.bits == 2) dn8_body<2, NJ, GS, UPW>(a, r, w.sl, w.upw, lds);
    else dn8_body<4, NJ, GS, UPW>(a, r, w.sl, w.upw, lds);
}
template <int NJ, int GS, int UPW>
__device__ __forceinline__ void dn_entry(const GroupedLaunch &a, const SharedWork &w, uint32_t *lds) {
    dn_batch<NJ, GS, UPW>(a, w, 0, lds);
    if (w.n > a.cap_dn) {
        __syncthreads();
        dn_batch<NJ, GS, UPW>(a, w, a.cap_dn, lds);
    }
}
template <int NJ, int GS>
__global__ void __launch_bounds__(kBlock) k_dn_sh(GroupedLaunch a) {
    extern __shared__ __align__(16) uint32_t lds[];
    SharedWork w;
    shared_work(a, a.geo.nblk, shared_rec_off(a.I, a.cap_dn, a.E), lds, w);
    // zero rows for the pairs without an expert, spread over the whole grid
    for (uint64_t m = w.inval; m; m &= m - 1) {
        float *yr = a.y + (size_t)(__ffsll((unsigned long long)m) - 1) * a.H;
        for (int c = blockIdx.x * kBlock + threadIdx.x; c < a.H; c += gridDim.x * kBlock) yr[c] = 0.f;
    }
    if (w.upw == 0) return;
    if (w.upw <= kSharedUPW) dn_entry<NJ, GS, kSharedUPW>(a, w, lds);
    else dn_entry<NJ, GS, kDnUPW>(a, w, lds);
}

}  // namespace

bool shared_path_fits(int H, int I, int E, int T) {
    const int cap = shared_cap(T);
    return H % 64 == 0 && I % 64 == 0 && shared_lds_bytes(H, cap, E) <= kMaxLds &&
           shared_lds_bytes(I, cap, E) <= kMaxLds;
}

hipError_t launch_shared_ffn(const GroupedLaunch &a_in, hipStream_t s, const KernelEvents &gu_ev,
                             const KernelEvents &dn_ev) {
    GroupedLaunch a = a_in;
    a.cap = shared_cap(a.T);
    a.cap_dn = shared_cap_dn(a.I, a.T, a.E);
    a.pt = plane_table(a.H, a.I);
    a.upw = 0;
    a.geo = gateup_geo(a.H, a.I);
    // up to four tokens without a norm weight: no staging launch (measured faster there)
    const bool direct = a.T <= kSharedDirectMaxT && a.norm_w == nullptr;
    if (hipError_t e = direct ? launch_shared_gateup_direct(a, s, gu_ev) : launch_shared_gateup(a, s, gu_ev)) return e;
    const int nj = nj_for(a.I), gs = small_gs(a.I, nj);
    a.geo = row_geo(a.I, a.H, nj == 1 ? dn8_rg<1>() : nj == 2 ? dn8_rg<2>() : dn8_rg<4>());
    const dim3 grid(shared_grid(a.geo.nblk, a.T * a.K));
    const size_t lds = shared_lds_bytes(a.I, a.cap_dn, a.E);
    switch (nj) {
        case 1:
            return gs == 64   ? launch_lds<k_dn_sh<1, 64>>(grid, lds, s, dn_ev, a)
                   : gs == 32 ? launch_lds<k_dn_sh<1, 32>>(grid, lds, s, dn_ev, a)
                              : launch_lds<k_dn_sh<1, 0>>(grid, lds, s, dn_ev, a);
        case 2: return gs ? launch_lds<k_dn_sh<2, 64>>(grid, lds, s, dn_ev, a) : launch_lds<k_dn_sh<2, 0>>(grid, lds, s, dn_ev, a);
        default: return gs ? launch_lds<k_dn_sh<4, 64>>(grid, lds, s, dn_ev, a) : launch_lds<k_dn_sh<4, 0>>(grid, lds, s, dn_ev, a);
    }
}
}  // namespace moe
