// moe_layer.hip -- router and gate/up of one decode token in ONE launch.
//
// The router and gate/up phases of a layer run as two groups of workgroups of a single grid, in
// that blockIdx order, and the logits pass between them through words in the workspace instead
// of a kernel boundary (a boundary costs about 1.5 us on this part plus the memory latency of the
// next kernel's first loads):
//
//   router workgroups   publish each logit as one 64-bit word, launch tag << 32 | fp32 bits,
//                       into kLogitCopies copies of the logit row;
//   gate/up workgroups  issue their descriptor-table and activation loads, then wave 0 polls one
//                       copy until all E words carry this launch's tag; routing (top-K in
//                       registers, every wave), the gate/up stream and h follow as in the
//                       separate gate/up kernel.
//
// The down projection stays a kernel of its own: every down workgroup needs all of h, and the
// kernel boundary publishes h to all L2 slices at once, where in-kernel hand-over would need a
// release fence per producer and uncached reads per consumer (both measured far slower here).
//
// Copies.  Hundreds of workgroups polling one 4 KB row with cache-bypassing loads all land on
// the few memory channels that hold it; each workgroup polls copy (index % kLogitCopies), which
// spreads the polls over the channels.
//
// Progress.  A gate/up workgroup only waits for router workgroups, which have lower indices and
// are started first, so the wait cannot deadlock whether or not the whole grid is resident.  The
// wait is also bounded: if it runs out, the workspace error word counts it, and the down kernel
// writes NaN outputs while that word is nonzero, so a failure shows in the output instead of
// hanging the device.
//
// Launch tags.  The tag is seq + 1 (never 0), where seq is a workspace word every workgroup reads
// when it starts; the down kernel that follows on the stream stores the tag into seq, so the
// next launch uses a new tag and no word left by an earlier launch can pass for a fresh one.  The
// workspace must therefore be zero-filled before its first use.
#include "moe_handoff.h"

namespace moe {
namespace {

// ----------------------------------------------------------------------------------- kernel
template <int NP, int NJ>
__global__ void __launch_bounds__(kBlock) k_route_gateup(LayerLaunch a) {
    extern __shared__ __align__(16) uint32_t lds[];
    __shared__ uint64_t s_tab[kTabMax];
    __shared__ float red[kWaves];
    __shared__ __align__(8) uint32_t s_cand[2 * kWaves * MOE_MAX_TOPK];
    // The launch counter is loaded through an offset the compiler cannot prove uniform, so it stays
    // in a vector register and is waited for where the tag is first used, not here.
    int zero;
    asm volatile("v_mov_b32 %0, 0" : "=v"(zero));
    const uint32_t seq = ld_word(a.seq + zero);
    const int b = blockIdx.x;
    if (a.clear_err && b == 0 && threadIdx.x == 0) st_word(a.err, 0u);
    if (b < a.nr) {
        // (a raised wave priority for the router waves helped while the router was staged through LDS;
        // with its rows computed in registers the gate/up staging it delayed is the later of the two:
        // 15.83 -> 15.65 us per H4096/E512 step without it, three alternating runs)
        router_phase(a, b, lds, red, seq);
    } else {
        gateup_phase<NJ, NP>(a, b - a.nr, lds, s_tab, s_cand, red, seq);
    }
}

template <int NP, int NJ>
hipError_t layer_impl(const LayerLaunch &a, size_t lds, hipStream_t s, const KernelEvents &ev) {
    auto fn = k_route_gateup<NP, NJ>;
    if (hipError_t e = lds_for<k_route_gateup<NP, NJ>>(lds)) return e;
    return dispatch(fn, dim3(a.nr + a.ng), dim3(kBlock), lds, s, ev, a);
}

template <int NP>
hipError_t layer_nj(const LayerLaunch &a, size_t lds, hipStream_t s, const KernelEvents &ev) {
    switch (nj_for(a.H)) {
        case 1: return layer_impl<NP, 1>(a, lds, s, ev);
        case 2: return layer_impl<NP, 2>(a, lds, s, ev);
        default: return layer_impl<NP, 4>(a, lds, s, ev);
    }
}

}  // namespace

void layer_grid(int H, int I, int E, int K, int *nr, int *ng) {
    const RowGeo gg = gateup_geo(H, I);
    *nr = (E * kRouterWPR + kWaves - 1) / kWaves;
    *ng = (K * gg.nblk + kWaves - 1) / kWaves;
}

int layer_logit_copies() { return kLogitCopies; }

size_t layer_lds_bytes(int H, int E) {
    const size_t e4 = (size_t)((E + 3) & ~3) * 4;
    const size_t r = (size_t)H * 4;                             // router: x layouts
    const size_t g = e4 + gateup_lds_bytes(H);                  // gate/up: logits + x layouts
    return r > g ? r : g;
}

hipError_t launch_layer(const LayerLaunch &a_in, hipStream_t s, const KernelEvents &ev) {
    LayerLaunch a = a_in;
    layer_grid(a.H, a.I, a.E, a.K, &a.nr, &a.ng);
    a.geo = gateup_geo(a.H, a.I);
    a.pt = plane_table(a.H, a.I);
    const size_t lds = layer_lds_bytes(a.H, a.E);
    return a.E <= 512 ? layer_nj<8>(a, lds, s, ev) : layer_nj<32>(a, lds, s, ev);
}

}  // namespace moe
