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
#include "moe_device.h"

namespace moe {
namespace {

constexpr int kSpinLimit = 1 << 18;       // polls per wait (each at least one memory round trip)
constexpr int kLogitCopies = 16;          // copies of the tagged logit row (<= 64)
constexpr int kRouterWPR = 1;             // waves per router row (2 measured equal, 4 slower)

__device__ __forceinline__ uint32_t ld_word(const uint32_t *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ld_word64(const uint64_t *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}
__device__ __forceinline__ void st_word(uint32_t *p, uint32_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Published with an agent-scope atomic exchange rather than a store: the atomic is performed
// where every L2 slice sees it, while a plain store can sit in the writer's L2 slice for
// microseconds before the polling workgroups of other slices observe it.
__device__ __forceinline__ void publish_word64(uint64_t *p, uint64_t v) {
    (void)__hip_atomic_exchange(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}
__device__ __forceinline__ uint32_t launch_tag(uint32_t seq) {
    const uint32_t t = seq + 1u;
    return t ? t : 1u;
}

// One wave waits until the E logit words carry `tag` and copies the logits to LDS.  It polls a
// single word (the last expert's: the router workgroups finish within a fraction of a
// microsecond of each other) and only then reads the whole row, which it re-reads until every
// tag matches: polling the full row from hundreds of workgroups would swamp the memory system.
// Returns false if the wait ran out (the logits are then NaN, which ranks last, and the error
// word counts it).
template <int NP>
__device__ bool wait_logits(const uint64_t *slots, int E, uint32_t tag, float *s_lg, uint32_t *err) {
    const int lane = threadIdx.x & 63;
    int it = 0;
    for (; it < kSpinLimit; ++it) {
        if ((uint32_t)(ld_word64(slots + E - 1) >> 32) == tag) break;
        __builtin_amdgcn_s_sleep(16);   // back-off 1, 4, 8, 16, 32, 64, 127: 17.47, 17.44, 17.39, 17.28, 17.26, 17.53, 19.15 us per step
    }
    for (; it < kSpinLimit; ++it) {
        uint64_t v[NP];
#pragma unroll
        for (int t = 0; t < NP; ++t) v[t] = ld_word64(slots + min(NP * lane + t, E - 1));
        bool ok = true;
#pragma unroll
        for (int t = 0; t < NP; ++t) ok = ok && (NP * lane + t >= E || (uint32_t)(v[t] >> 32) == tag);
        if (__all(ok)) {
#pragma unroll
            for (int t = 0; t < NP; ++t)
                if (NP * lane + t < E) s_lg[NP * lane + t] = __uint_as_float((uint32_t)v[t]);
            return true;
        }
        __builtin_amdgcn_s_sleep(2);
    }
#pragma unroll
    for (int t = 0; t < NP; ++t)
        if (NP * lane + t < E) s_lg[NP * lane + t] = __uint_as_float(0x7FC00000u);
    if (lane == 0) atomicAdd(err, 1u);
    return false;
}

// ----------------------------------------------------------------------------------- router
__device__ __forceinline__ void router_phase(const LayerLaunch a, int b, uint32_t *lds, float *red, uint32_t seq) {
    float lg = 0.f;
    bool ok;
    if (a.r.router_dtype == MOE_BF16)
        ok = a.split ? router_row<MOE_BF16, true, kRouterWPR>(a.r, b, 0, lds, red, lg)
                     : router_row<MOE_BF16, false, kRouterWPR>(a.r, b, 0, lds, red, lg);
    else
        ok = router_row<MOE_F32, false, kRouterWPR>(a.r, b, 0, lds, red, lg);
    const int lane = threadIdx.x & 63;
    const int e = b * (kWaves / kRouterWPR) + (threadIdx.x >> 6) / kRouterWPR;
    if (ok && lane < kLogitCopies)
        publish_word64(a.slots + (size_t)lane * a.E + e, ((uint64_t)launch_tag(seq) << 32) | __float_as_uint(lg));
}

// ----------------------------------------------------------------------------------- gate/up
template <int NJ, int NP>
__device__ __forceinline__ void gateup_phase(const LayerLaunch a, int gb, uint32_t *lds, uint64_t *s_tab,
                                             uint32_t *s_cand, float *red, uint32_t seq) {
    constexpr int RG = gu_rg<NJ>();
    const int H = a.H, I = a.I, E = a.E, K = a.K;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const bool use_tab = E <= kTabMax;
    float *s_lg = (float *)lds;
    uint32_t *act = lds + ((E + 3) & ~3);

    // 1. independent loads: descriptor table, activation, norm weight
    u32x4 dsc[kTabMax / kBlock];
    if (use_tab) {
#pragma unroll
        for (int j = 0; j < kTabMax / kBlock; ++j)
            dsc[j] = *(const GLOBAL_AS u32x4 *)(a.experts + min((int)threadIdx.x + kBlock * j, E - 1));
    }
    const void *x = a.r.x;
    const int xdt = a.r.x_dtype;
    const int nch = H / 16;
    Chunk16 xc[2], nc[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int m = min((int)threadIdx.x + kBlock * j, nch - 1);
        issue_chunk16(x, xdt, m, xc[j]);
        if (a.r.norm_w) issue_chunk16(a.r.norm_w, MOE_BF16, m, nc[j]);
    }

    // 2. while the router workgroups run: descriptor table and activation layouts (both code
    //    widths; with a norm, x * w_norm scaled by 1/rms once the block sum is known)
    if (use_tab) {
#pragma unroll
        for (int j = 0; j < kTabMax / kBlock; ++j) {
            const int e = threadIdx.x + kBlock * j;
            if (e < E) s_tab[e] = pack_sel(((uint64_t)dsc[j].y << 32) | dsc[j].x, dsc[j].z);
        }
    }
    float v[2][16];
#pragma unroll
    for (int j = 0; j < 2; ++j) chunk16_f32(xc[j], xdt, v[j]);
    if (a.r.norm_w) {
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
        const float inv = 1.0f / sqrtf(ss / (float)H + a.r.eps);
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int i = 0; i < 16; ++i) v[j][i] *= inv;
    }
    uint32_t *d4 = act, *d2 = act + H / 2;
    float2 *xs = (float2 *)(act + H);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int m = threadIdx.x + kBlock * j;
        stage_chunk(m, m < nch, v[j], d4, d2, xs);
    }
    const ActView v4{d4, xs}, v2{d2, xs};

    // 3. wave 0 waits for this launch's logits and copies them to LDS; the barrier publishes the
    //    logits, the table and the layouts
    if (wave == 0) wait_logits<NP>(a.slots + (size_t)(gb % kLogitCopies) * E, E, launch_tag(seq), s_lg, a.err);
    __syncthreads();

    // 4. routing: each wave takes a quarter of the logits, then the candidates meet in LDS (every
    //    wave ends with the same selection in lanes 0..K-1)
    int my_idx = 0;
    float my_w = 0.f;
    block_topk<NP>(s_lg, E, K, s_cand, my_idx, my_w);
    if (gb == 0 && wave == 0 && lane < K) {
        if (a.idx_out) a.idx_out[lane] = my_idx;
        if (a.w_out) a.w_out[lane] = my_w;
        a.w_ws[lane] = my_w;
        a.sel_ws[lane] = lookup_sel(my_idx, E, use_tab, s_tab, a.experts);
    }

    // 5. geometry of the work units
    const Geo g = make_geo(a.geo);
    const int RB = a.geo.rb;
    const int nblk = a.geo.nblk;
    const int units = K * nblk;
    const int stride = a.ng * kWaves;
    int u = gb * kWaves + wave;
    GULoads<NJ, RG> L;
    uint64_t sel = 0;
    Planes pl[3];

    // 6. work units -> h
    for (; u < units; u += stride) {
        const int k = blk_of(u, a.geo);
        const int r0 = (u - k * nblk) * RB;
        float *hout = a.h + (size_t)k * I;
        sel = lookup_sel(__builtin_amdgcn_readlane(my_idx, k), E, use_tab, s_tab, a.experts);
        if (!sel) {
            for (int r = r0 + lane; r < r0 + RB && r < I; r += 64) hout[r] = 0.f;
            continue;
        }
        // Loads and arithmetic of one code width sit in one branch, so the arithmetic on the first
        // slots waits only for their own loads while the later ones are still arriving.
        expert_planes(sel_blob(sel), sel_bits(sel), a.pt, pl);
        if (sel_bits(sel) == 2) {
            gu_issue<2, NJ, RG>(pl, g, H, I, r0, RB, L);
            gu_finish<2, NJ, RG>(g, I, r0, RB, v2, L, hout);
        } else {
            gu_issue<4, NJ, RG>(pl, g, H, I, r0, RB, L);
            gu_finish<4, NJ, RG>(g, I, r0, RB, v4, L, hout);
        }
    }
}

// ----------------------------------------------------------------------------------- kernel
template <int NP, int NJ>
__global__ void __launch_bounds__(kBlock) k_route_gateup(LayerLaunch a) {
    extern __shared__ __align__(16) uint32_t lds[];
    __shared__ uint64_t s_tab[kTabMax];
    __shared__ float red[kWaves];
    __shared__ uint32_t s_cand[2 * kWaves * MOE_MAX_TOPK];
    // The launch counter is loaded through an offset the compiler cannot prove uniform, so it stays
    // in a vector register and is waited for where the tag is first used, not here.
    int zero;
    asm volatile("v_mov_b32 %0, 0" : "=v"(zero));
    const uint32_t seq = ld_word(a.seq + zero);
    const int b = blockIdx.x;
    if (b < a.nr) {
        // the router waves issue ahead of the gate/up waves that share their CUs while staging and
        // polling: every gate/up workgroup waits for the logits (17.62 -> 17.47 us per step)
        __builtin_amdgcn_s_setprio(3);
        router_phase(a, b, lds, red, seq);
    } else {
        gateup_phase<NJ, NP>(a, b - a.nr, lds, s_tab, s_cand, red, seq);
    }
}

template <int NP, int NJ>
hipError_t layer_impl(const LayerLaunch &a, size_t lds, hipStream_t s, const KernelEvents &ev) {
    auto fn = k_route_gateup<NP, NJ>;
    if (lds > 64 * 1024)
        if (hipError_t e = hipFuncSetAttribute((const void *)fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds))
            return e;
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
