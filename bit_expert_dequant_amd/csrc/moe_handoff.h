// moe_handoff.h -- the router and gate/up phases of a decode layer and the hand-over of their
// results between workgroups of one grid: the two-launch layer kernel (moe_layer.hip) uses the
// phases, the single-launch layer kernel (moe_fused.hip) the hand-over words and the router.
//
// Hand-over words carry a launch tag: tag << 32 | payload.  The tag is seq + 1 (never 0), where seq
// is a workspace word every workgroup reads when it starts and that a later step advances, so no
// word left by an earlier launch can pass for a fresh one.  Words are written with system-scope
// stores or atomics (written through to memory, seen by every XCD's polls after about 0.6 us on
// this part) and polled with system-scope loads; every wait is bounded and counts a timeout in the
// workspace error word.
#pragma once

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
        // back-off between polls: 16 x 64 cycles measured 17.54 us per config-1 step against 17.64 with 1
        // and 17.82 with 64 (medians of five alternating runs, each within +-0.01 us)
        __builtin_amdgcn_s_sleep(16);
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

// wait_logits for a wave that ranks the logits itself: lane l ends with the order-preserving keys
// of experts NP*l .. NP*l+NP-1 in registers (absent experts 0; after a timed-out wait the keys of
// NaN, which rank as -inf) and nothing goes through LDS.
template <int NP>
__device__ bool wait_logit_keys(const uint64_t *slots, int E, uint32_t tag, uint32_t (&key)[NP], uint32_t *err) {
    const int lane = threadIdx.x & 63;
    int it = 0;
    for (; it < kSpinLimit; ++it) {
        if ((uint32_t)(ld_word64(slots + E - 1) >> 32) == tag) break;
        __builtin_amdgcn_s_sleep(16);     // back-off as in wait_logits
    }
    float lg[NP];
    for (; it < kSpinLimit; ++it) {
        uint64_t v[NP];
#pragma unroll
        for (int t = 0; t < NP; ++t) v[t] = ld_word64(slots + min(NP * lane + t, E - 1));
        bool ok = true;
#pragma unroll
        for (int t = 0; t < NP; ++t) ok = ok && (NP * lane + t >= E || (uint32_t)(v[t] >> 32) == tag);
        if (__all(ok)) {
#pragma unroll
            for (int t = 0; t < NP; ++t) lg[t] = __uint_as_float((uint32_t)v[t]);
            logit_keys<NP>(lg, E, key);
            return true;
        }
        __builtin_amdgcn_s_sleep(2);
    }
#pragma unroll
    for (int t = 0; t < NP; ++t) lg[t] = __uint_as_float(0x7FC00000u);
    logit_keys<NP>(lg, E, key);
    if (lane == 0) atomicAdd(err, 1u);
    return false;
}

// ----------------------------------------------------------------------------------- router
// The bf16 router row for a bf16 activation without a norm, in registers only: lane l's columns of
// the row, eight at a time ((l + 64 j) * 8 ..), meet the same columns of x loaded straight from
// memory, already in the dot2 operand format, so there is no LDS staging and no barrier between the
// loads and the dot products.  The same products in the same order as router_row.  H a multiple of
// 512, at most 4096 (one batch of row loads); wave w of workgroup bx takes expert bx * kWaves + w.
__device__ __forceinline__ bool router_row_bf16x(const RouterLaunch &a, int bx, float &logit) {
    const int H = a.H, lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int e = bx * kWaves + wave;
    const int nld = H / 512;
    const GLOBAL_AS u32x4 *row =
        (const GLOBAL_AS u32x4 *)((const GLOBAL_AS uint8_t *)a.router + (size_t)(e < a.E ? e : 0) * H * 2);
    const GLOBAL_AS u32x4 *xv = (const GLOBAL_AS u32x4 *)a.x;
    const float bias = e < a.E && a.logit_bias ? a.logit_bias[e] : 0.f;
    // pairs in issue order, so the first products wait for the first pair only (loads complete in
    // issue order); clamped, so every load is in bounds and the extra ones are not used
    u32x4 xq[kRouterBatch], wq[kRouterBatch];
#pragma unroll
    for (int j = 0; j < kRouterBatch; ++j) {
        const int i = lane + 64 * min(j, nld - 1);
        xq[j] = xv[i];
        wq[j] = row[i];
    }
    float acc = 0.f;
#pragma unroll
    for (int j = 0; j < kRouterBatch; ++j)
        if (j < nld) {
#pragma unroll
            for (int q = 0; q < 4; ++q) acc = dot2(wq[j][q], xq[j][q], acc);
        }
    logit = group_sum(acc, 64) + bias;
    return e < a.E;
}

__device__ __forceinline__ void router_phase(const LayerLaunch a, int b, uint32_t *lds, float *red, uint32_t seq) {
    float lg = 0.f;
    bool ok;
    if (kRouterWPR == 1 && a.r.router_dtype == MOE_BF16 && !a.split && a.H % 512 == 0 && a.H <= 512 * kRouterBatch)
        ok = router_row_bf16x(a.r, b, lg);
    else if (a.r.router_dtype == MOE_BF16)
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

    // 3. the first work unit's load offsets for 4-bit experts (they do not depend on the routing), then
    //    wave 0 waits for this launch's logits and copies them to LDS; the barrier publishes the
    //    logits, the table and the layouts
    const Geo g = make_geo(a.geo);
    const int RB = a.geo.rb;
    const int nblk = a.geo.nblk;
    const int units = K * nblk;
    int u = gb * kWaves + wave;
    GUOffs<NJ, RG> o4;
    {
        const int k = blk_of(min(u, units - 1), a.geo);
        gu_offsets<4, NJ, RG>(a.pt, g, H, I, (min(u, units - 1) - k * nblk) * RB, o4);
    }
    const uint32_t tag = launch_tag(seq);
    const uint64_t *row = a.slots + (size_t)(gb % kLogitCopies) * E;
    // s_cand holds the K selected experts' (blob | bits) words in this path
    uint64_t *s_sel = (uint64_t *)s_cand;
    int my_idx = 0;
    if constexpr (NP <= 8) {
        // 4. routing by wave 0 alone, straight from the polled words (at most 8 keys per lane: the K
        //    rounds take no list upkeep), while the other waves wait at the barrier that also publishes
        //    the selection.  The barrier before it publishes the table and the layouts while the router
        //    workgroups still run.
        __syncthreads();
        if (wave == 0) {
            uint32_t key[NP];
            wait_logit_keys<NP>(row, E, tag, key, a.err);
            uint32_t mk;
            int pos;
            wave_topk_core<NP>(key, K, mk, pos);
            const float w = topk_weight(mk, K);
            if (lane < K) {
                const uint64_t sl = lookup_sel(pos, E, use_tab, s_tab, a.experts);
                s_sel[lane] = sl;
                if (gb == 0) {
                    if (a.idx_out) a.idx_out[lane] = pos;
                    if (a.w_out) a.w_out[lane] = w;
                    a.w_ws[lane] = w;
                    a.sel_ws[lane] = sl;
                }
            }
        }
        __syncthreads();
    } else {
        // 4. routing: wave 0 copies the logits to LDS; each wave takes a quarter of them, then the
        //    candidates meet in LDS (every wave ends with the same selection in lanes 0..K-1)
        if (wave == 0) wait_logits<NP>(row, E, tag, s_lg, a.err);
        __syncthreads();
        float my_w = 0.f;
        block_topk<NP>(s_lg, E, K, s_cand, my_idx, my_w);
        if (gb == 0 && wave == 0 && lane < K) {
            if (a.idx_out) a.idx_out[lane] = my_idx;
            if (a.w_out) a.w_out[lane] = my_w;
            a.w_ws[lane] = my_w;
            a.sel_ws[lane] = lookup_sel(my_idx, E, use_tab, s_tab, a.experts);
        }
    }
    auto sel_of = [&](int k) {
        if constexpr (NP <= 8) return s_sel[k];
        else return lookup_sel(__builtin_amdgcn_readlane(my_idx, k), E, use_tab, s_tab, a.experts);
    };

    // 5. work units -> h; the first one (the only one when the grid covers every unit) is peeled so
    //    that its loads follow the selection directly
    const int stride = a.ng * kWaves;
    GULoads<NJ, RG> L;
    Planes pl[3];
    auto unit = [&](int uu, bool at) {
        const int k = blk_of(uu, a.geo);
        const int r0 = (uu - k * nblk) * RB;
        float *hout = a.h + (size_t)k * I;
        const uint64_t sel = sel_of(k);
        if (!sel) {
            for (int r = r0 + lane; r < r0 + RB && r < I; r += 64) hout[r] = 0.f;
            return;
        }
        // Loads and arithmetic of one code width sit in one branch, so the arithmetic on the first
        // slots waits only for their own loads while the later ones are still arriving.
        if (sel_bits(sel) == 2) {
            expert_planes(sel_blob(sel), 2, a.pt, pl);
            gu_issue<2, NJ, RG>(pl, g, H, I, r0, RB, L);
            gu_finish<2, NJ, RG>(g, I, r0, RB, v2, L, hout);
        } else {
            if (at) {
                gu_issue_at<4, NJ, RG>(sel_blob(sel), o4, L);
            } else {
                expert_planes(sel_blob(sel), 4, a.pt, pl);
                gu_issue<4, NJ, RG>(pl, g, H, I, r0, RB, L);
            }
            gu_finish<4, NJ, RG>(g, I, r0, RB, v4, L, hout);
        }
    };
    if (u < units) unit(u, true);
    for (u += stride; u < units; u += stride) unit(u, false);
}

}  // namespace
}  // namespace moe
