// moe_fused.hip -- one decode layer (router, routing, gate/up + SwiGLU, down + combine) in ONE launch
// of a persistent grid: nw workgroups, all resident at once, each taking every role in turn.
//
//   1. router    rows b, b + nw, ... of the router (all four waves on a row), each logit published as
//                a tagged word into kLogitCopies copies of the logit row (moe_handoff.h);
//   2. staging   the descriptor table and the activation's digit planes, while the logits arrive;
//   3. routing   wave 0 collects the whole logit row of one copy, every wave takes the top K;
//   4. loads     the wave's first gate/up unit and, right behind it, its first down unit: the down
//                rows depend on the routing only, so they stream during gate/up instead of after it;
//   5. gate/up   SwiGLU rows stored as tagged words (below), then the workgroup raises its flag;
//   6. hand-over every workgroup waits for all nw flags, reads h and stages it as digit planes;
//   7. down      the projection of all K experts for the wave's output rows, weighted combine and
//                residual in registers.
//
// Compared with two launches (router + gate/up, then down + combine) this removes the kernel boundary
// and the down kernel's prologue, and the down weights are in registers when h arrives.  The price is
// that the grid must be resident at once (every workgroup waits for every other's flag): the launcher
// sizes nw to the occupancy the runtime reports, and every wait is bounded, so a grid that is not
// resident after all (other kernels running concurrently) ends with NaN outputs and the error word
// set, not a hang.
//
// Tagged h.  A SwiGLU value is stored with its lowest 4 mantissa bits replaced by a 4-bit launch tag
// (1..15, never the tag of the previous launch, never 0 as a zero-filled workspace holds), written
// through to memory.  A reader checks every value's tag and reads again what is stale, so the flag
// can be raised without waiting for the h stores to be acknowledged; it then clears the tag bits, so
// h enters the down projection truncated to 19 mantissa bits whatever the tag (results do not depend
// on the launch).  That changes h by less than 2^-19 of its value, below the 2^-16 of the slot
// maximum that the digit-plane staging keeps.
//
// Launch counter.  Every workgroup reads seq first; workgroup 0 advances it once it has seen every
// workgroup's flag (each carries this launch's tag, so every workgroup has read seq by then).
#include "moe_handoff.h"

namespace moe {
namespace {

constexpr int kFlagCopies = 8;            // copies of the flag row (workgroup b polls copy b % 8)
constexpr int kMaxFlagsPerLane = 16;      // nw <= 64 * 16

__device__ __forceinline__ uint32_t ld_sys(const uint32_t *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}
__device__ __forceinline__ void st_sys(uint32_t *p, uint32_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}
__device__ __forceinline__ uint32_t h_tag(uint32_t tag) { return tag % 15u + 1u; }

// One wave collects the E tagged logit words of a copy into LDS.  A lane reads its NP words until all
// carry the tag, then stops reading (lanes that are done leave the loads), so later polls touch only
// what is still missing.  False when the wait ran out (missing logits are then NaN, which ranks last).
template <int NP>
__device__ bool collect_logits(const uint64_t *row, int E, uint32_t tag, float *s_lg) {
    const int lane = threadIdx.x & 63;
    uint32_t have = 0;                                     // bit t: word NP*lane + t seen
    uint32_t want = 0;
#pragma unroll
    for (int t = 0; t < NP; ++t) want |= (NP * lane + t < E ? 1u : 0u) << t;
    for (int it = 0; it < kSpinLimit; ++it) {
        if (have != want) {
            uint64_t v[NP];
#pragma unroll
            for (int t = 0; t < NP; ++t) v[t] = ld_word64(row + min(NP * lane + t, E - 1));
#pragma unroll
            for (int t = 0; t < NP; ++t) {
                if (((want >> t) & 1u) && !((have >> t) & 1u) && (uint32_t)(v[t] >> 32) == tag) {
                    s_lg[NP * lane + t] = __uint_as_float((uint32_t)v[t]);
                    have |= 1u << t;
                }
            }
        }
        if (__all(have == want)) return true;
    }
#pragma unroll
    for (int t = 0; t < NP; ++t)
        if (((want >> t) & 1u) && !((have >> t) & 1u)) s_lg[NP * lane + t] = __uint_as_float(0x7FC00000u);
    return false;
}

// One wave waits until the n (<= 64 * kMaxFlagsPerLane) flag words at w all equal tag; lanes stop
// reading the words they have seen.  False when the wait ran out.
__device__ bool collect_flags(const uint32_t *w, int n, uint32_t tag) {
    const int lane = threadIdx.x & 63;
    uint32_t have = 0, want = 0;
#pragma unroll
    for (int j = 0; j < kMaxFlagsPerLane; ++j) want |= (lane + 64 * j < n ? 1u : 0u) << j;
    for (int it = 0; it < kSpinLimit; ++it) {
        if (have != want) {
            uint32_t v[kMaxFlagsPerLane];
#pragma unroll
            for (int j = 0; j < kMaxFlagsPerLane; ++j)
                v[j] = ((want >> j) & 1u) ? ld_sys(w + min(lane + 64 * j, n - 1)) : tag;
#pragma unroll
            for (int j = 0; j < kMaxFlagsPerLane; ++j) have |= (v[j] == tag ? 1u : 0u) << j;
            have &= want;
        }
        if (__all(have == want)) return true;
    }
    return false;
}

// Router rows of this workgroup (rows b, b + nw, ...): all four waves on one row, kLogitCopies
// copies published.
template <int RDT, bool SPLIT>
__device__ __forceinline__ void router_rows(const LayerLaunch &L, int b, int nw, uint32_t *work, float *red,
                                            uint32_t tag) {
    const int lane = threadIdx.x & 63;
    for (int e = b; e < L.E; e += nw) {
        float lg = 0.f;
        const bool ok = router_row<RDT, SPLIT, kWaves>(L.r, e, 0, work, red, lg);
        if (ok && lane < kLogitCopies)
            publish_word64(L.slots + (size_t)lane * L.E + e, ((uint64_t)tag << 32) | __float_as_uint(lg));
        __syncthreads();                                   // the staging region is reused
    }
}

template <int NP, int NJ, int DNJ, int KM>
__global__ void __launch_bounds__(kBlock) k_layer(FusedLaunch a) {
    extern __shared__ __align__(16) uint32_t lds[];
    __shared__ uint64_t s_tab[kTabMax];
    __shared__ float red[kWaves];
    __shared__ uint32_t s_cand[2 * kWaves * MOE_MAX_TOPK];
    __shared__ uint32_t s_bad;
    constexpr int RG = gu_rg<NJ>();
    const LayerLaunch &L = a.L;
    const int H = L.H, I = L.I, E = L.E, K = L.K;
    const int b = blockIdx.x, nw = a.nw;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const bool use_tab = E <= kTabMax;
    // The launch counter is loaded through an offset the compiler cannot prove uniform, so it stays
    // in a vector register and is waited for where the tag is first used.
    int zero;
    asm volatile("v_mov_b32 %0, 0" : "=v"(zero));
    const uint32_t seq = ld_word(L.seq + zero);
    const uint32_t tag = launch_tag(seq);
    if (L.clear_err && b == 0 && threadIdx.x == 0) st_word(L.err, 0u);
    if (threadIdx.x == 0) s_bad = 0u;
    float *s_lg = (float *)lds;
    uint32_t *work = lds + ((E + 3) & ~3);

    // 1. router rows
    if (L.r.router_dtype == MOE_BF16) {
        if (L.split) router_rows<MOE_BF16, true>(L, b, nw, work, red, tag);
        else router_rows<MOE_BF16, false>(L, b, nw, work, red, tag);
    } else {
        router_rows<MOE_F32, false>(L, b, nw, work, red, tag);
    }

    // 2. descriptor table and the activation's digit planes (both code widths)
    u32x4 dsc[kTabMax / kBlock];
    if (use_tab) {
#pragma unroll
        for (int j = 0; j < kTabMax / kBlock; ++j)
            dsc[j] = *(const GLOBAL_AS u32x4 *)(L.experts + min((int)threadIdx.x + kBlock * j, E - 1));
    }
    const void *x = L.r.x;
    const int xdt = L.r.x_dtype;
    const int nch = H / 16;
    Chunk16 xc[2], nc[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int m = min((int)threadIdx.x + kBlock * j, nch - 1);
        issue_chunk16(x, xdt, m, xc[j]);
        if (L.r.norm_w) issue_chunk16(L.r.norm_w, MOE_BF16, m, nc[j]);
    }
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
    if (L.r.norm_w) {
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
        const float inv = 1.0f / sqrtf(ss / (float)H + L.r.eps);
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int i = 0; i < 16; ++i) v[j][i] *= inv;
    }
    uint32_t *d4 = work, *d2 = work + H / 2;
    float2 *xs = (float2 *)(work + H);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int m = threadIdx.x + kBlock * j;
        stage_chunk(m, m < nch, v[j], d4, d2, xs);
    }
    const ActView v4{d4, xs}, v2{d2, xs};

    // 3. routing
    if (wave == 0) {
        const bool ok = collect_logits<NP>(L.slots + (size_t)(b % kLogitCopies) * E, E, tag, s_lg);
        if (!ok && lane == 0) {
            atomicAdd(L.err, 1u);
            s_bad = 1u;
        }
    }
    __syncthreads();
    int my_idx = 0;
    float my_w = 0.f;
    block_topk<NP>(s_lg, E, K, s_cand, my_idx, my_w);
    if (b == 0 && wave == 0 && lane < K) {
        if (L.idx_out) L.idx_out[lane] = my_idx;
        if (L.w_out) L.w_out[lane] = my_w;
    }
    uint64_t sel[KM];
    float wk[KM];
    uint32_t two_mask = 0;                                 // bit k: expert k has 2-bit codes
#pragma unroll
    for (int k = 0; k < KM; ++k) {
        const int kc = min(k, K - 1);
        sel[k] = k < K ? lookup_sel(__builtin_amdgcn_readlane(my_idx, kc), E, use_tab, s_tab, L.experts) : 0;
        wk[k] = k < K ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_w), kc)) : 0.f;
        if (sel_bits(sel[k]) == 2) two_mask |= 1u << k;
    }

    // 4. the first gate/up unit's loads, then the first down unit's
    const Geo g = make_geo(L.geo);
    const int RB = L.geo.rb, nblk = L.geo.nblk, units = K * nblk;
    const Geo dg = make_geo(a.dgeo);
    const int DRB = a.dgeo.rb, dnblk = a.dgeo.nblk;
    const int stride = nw * kWaves;
    int u = b * kWaves + wave;
    GULoads<NJ, RG> GL;
    Planes pl[3];
    uint64_t gsel = 0;
    if (u < units) {
        const int k = blk_of(u, L.geo);
        gsel = lookup_sel(__builtin_amdgcn_readlane(my_idx, k), E, use_tab, s_tab, L.experts);
        if (gsel) {
            expert_planes(sel_blob(gsel), sel_bits(gsel), L.pt, pl);
            if (sel_bits(gsel) == 2) gu_issue<2, NJ, RG>(pl, g, H, I, (u - k * nblk) * RB, RB, GL);
            else gu_issue<4, NJ, RG>(pl, g, H, I, (u - k * nblk) * RB, RB, GL);
        }
    }
    int ud = b * kWaves + wave;
    DLoads<DNJ, 1, KM> DL;
    if (ud < dnblk) dn_issue_all<DNJ, 1, KM>(sel, K, dg, H, I, ud * DRB, L.pt, DL);

    // 5. gate/up units -> tagged h
    const uint32_t htag = h_tag(tag);
    bool first = true;
    for (; u < units; u += stride) {
        const int k = blk_of(u, L.geo);
        const int r0 = (u - k * nblk) * RB;
        uint32_t *hout = (uint32_t *)L.h + (size_t)k * I;
        if (!first) {
            gsel = lookup_sel(__builtin_amdgcn_readlane(my_idx, k), E, use_tab, s_tab, L.experts);
            if (gsel) {
                expert_planes(sel_blob(gsel), sel_bits(gsel), L.pt, pl);
                if (sel_bits(gsel) == 2) gu_issue<2, NJ, RG>(pl, g, H, I, r0, RB, GL);
                else gu_issue<4, NJ, RG>(pl, g, H, I, r0, RB, GL);
            }
        }
        first = false;
        float hv[RG];
#pragma unroll
        for (int gi = 0; gi < RG; ++gi) hv[gi] = 0.f;
        if (gsel) {
            if (sel_bits(gsel) == 2) gu_values<2, NJ, RG>(g, v2, GL, hv);
            else gu_values<4, NJ, RG>(g, v4, GL, hv);
        }
#pragma unroll
        for (int gi = 0; gi < RG; ++gi) {
            const int rr = gi * g.rpi + g.lrow;
            if (g.lsl == 0 && rr < RB && r0 + rr < I) st_sys(hout + r0 + rr, (__float_as_uint(hv[gi]) & ~0xFu) | htag);
        }
    }
    __syncthreads();
    if ((int)threadIdx.x < kFlagCopies) st_sys(a.flags + (size_t)threadIdx.x * nw + b, tag);

    // 6. every workgroup's h, then h staged as digit planes (in the region of the activation's)
    if (wave == 0) {
        const bool ok = collect_flags(a.flags + (size_t)(b % kFlagCopies) * nw, nw, tag);
        if (!ok && lane == 0) {
            atomicAdd(L.err, 1u);
            s_bad = 1u;
        }
    }
    __syncthreads();
    if (b == 0 && threadIdx.x == 0) st_word(a.seq, tag);   // every workgroup has read seq
    const int per = down_lds_per_expert(I);
    const int cpe = I / 16;
    const int hch = K * cpe;
    const __amdgpu_buffer_rsrc_t hr = __builtin_amdgcn_make_buffer_rsrc((void *)L.h, 0, K * I * 4, 0x00020000);
    const uint32_t err_word = ld_sys(L.err);
    bool stale = false;
    for (int base = 0; base < hch; base += kBlock) {
        const int m = base + (int)threadIdx.x;
        u32x4 q[4];
        bool fresh = m >= hch;
#pragma unroll
        for (int i = 0; i < 4; ++i) q[i] = u32x4{0u, 0u, 0u, 0u};
        for (int it = 0; it < kSpinLimit && !fresh; ++it) {
#pragma unroll
            for (int i = 0; i < 4; ++i) q[i] = __builtin_amdgcn_raw_buffer_load_b128(hr, m * 64 + 16 * i, 0, 17);
            bool ok = true;
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int c = 0; c < 4; ++c) ok = ok && (q[i][c] & 0xFu) == htag;
            fresh = ok;
        }
        stale |= !fresh;
        float hvv[16];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int c = 0; c < 4; ++c) hvv[4 * i + c] = __uint_as_float(q[i][c] & ~0xFu);   // tag bits cleared
        const bool valid = m < hch;
        const int kk = valid ? m / cpe : 0;
        const int mm = m - kk * cpe;
        uint32_t *dst = work + kk * per;
        const bool two = (two_mask >> kk) & 1u;
        stage_chunk(mm, valid, hvv, two ? nullptr : dst, two ? dst : nullptr, (float2 *)(dst + I / 2));
    }
    if (stale) {
        atomicAdd(L.err, 1u);
        s_bad = 1u;
    }
    __syncthreads();

    // 7. down units: all experts of a block of output rows, combined in registers
    const char *res = a.residual ? (const char *)a.residual : nullptr;
    const bool bad = s_bad != 0 || err_word != 0;
    first = true;
    for (; ud < dnblk; ud += stride) {
        const int r0 = ud * DRB;
        if (!first) dn_issue_all<DNJ, 1, KM>(sel, K, dg, H, I, r0, L.pt, DL);
        first = false;
        float acc = 0.f;
#pragma unroll
        for (int k = 0; k < KM; ++k) {
            if (k >= K) break;
            float part = 0.f;
            if (sel[k]) {
                const uint32_t *dk = work + k * per;
                const ActView av{dk, (const float2 *)(dk + I / 2)};
#pragma unroll
                for (int j = 0; j < DNJ; ++j) {
                    const int slot = dg.lsl + 64 * j;
                    uint32_t D[kSlotDw];
                    float2 xsv;
                    load_act_slot(av, slot, slot < dg.spr, D, xsv);
                    if ((two_mask >> k) & 1u) part += slot_dot<2>(DL.q[k][0][j], D, DL.sb[k][0][j], xsv);
                    else part += slot_dot<4>(DL.q[k][0][j], D, DL.sb[k][0][j], xsv);
                }
            }
            acc += wk[k] * part;
        }
        const float sum = group_sum(acc, dg.gsz);
        const int r = r0 + dg.lrow;
        if (dg.lsl == 0 && dg.lrow < DRB && r < H)
            a.out[r] = bad ? __uint_as_float(0x7FC00000u) : sum + (res ? load_act(res, a.residual_dtype, r) : 0.f);
    }
}

template <int NP, int NJ, int DNJ, int KM>
struct RunLaunch {
    static hipError_t run(const FusedLaunch &a, size_t lds, hipStream_t s, const KernelEvents &ev) {
        auto fn = k_layer<NP, NJ, DNJ, KM>;
        if (hipError_t e = lds_for<k_layer<NP, NJ, DNJ, KM>>(lds)) return e;
        return dispatch(fn, dim3(a.nw), dim3(kBlock), lds, s, ev, a);
    }
};
template <int NP, int NJ, int DNJ, int KM>
struct RunOcc {
    static hipError_t run(int *blocks, size_t lds) {
        auto fn = k_layer<NP, NJ, DNJ, KM>;
        if (hipError_t e = lds_for<k_layer<NP, NJ, DNJ, KM>>(lds)) return e;
        return hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks, fn, kBlock, lds);
    }
};

// F<NP, NJ, DNJ, KM>::run(args...) for the layer's shape.
template <template <int, int, int, int> class F, typename... Args>
hipError_t fused_dispatch(int H, int I, int E, int K, Args &&...args) {
    auto km = [&](auto np, auto nj, auto dnj) -> hipError_t {
        constexpr int NP = decltype(np)::value, NJ = decltype(nj)::value, DNJ = decltype(dnj)::value;
        if (K <= 2) return F<NP, NJ, DNJ, 2>::run(args...);
        if (K <= 4) return F<NP, NJ, DNJ, 4>::run(args...);
        return F<NP, NJ, DNJ, 8>::run(args...);
    };
    auto dnj = [&](auto np, auto nj) -> hipError_t {
        switch (nj_for(I)) {
            case 1: return km(np, nj, std::integral_constant<int, 1>{});
            case 2: return km(np, nj, std::integral_constant<int, 2>{});
            default: return km(np, nj, std::integral_constant<int, 4>{});
        }
    };
    auto nj = [&](auto np) -> hipError_t {
        switch (nj_for(H)) {
            case 1: return dnj(np, std::integral_constant<int, 1>{});
            case 2: return dnj(np, std::integral_constant<int, 2>{});
            default: return dnj(np, std::integral_constant<int, 4>{});
        }
    };
    return E <= 512 ? nj(std::integral_constant<int, 8>{}) : nj(std::integral_constant<int, 32>{});
}

size_t fused_lds_bytes(int H, int I, int E, int K) {
    size_t work = (size_t)H * 4;                                   // router staging
    const size_t act = gateup_lds_bytes(H);                        // digit planes, both widths
    const size_t hs = down_lds_bytes(I, K);                        // h digit planes
    if (act > work) work = act;
    if (hs > work) work = hs;
    return (size_t)((E + 3) & ~3) * 4 + work;
}

}  // namespace

RowGeo fused_down_geo(int H, int I) { return row_geo(I, H, 1); }

int fused_flag_copies() { return kFlagCopies; }

int fused_max_workgroups() { return 64 * kMaxFlagsPerLane; }

hipError_t fused_workgroups(int H, int I, int E, int K, int *nw) {
    *nw = 0;
    int dev = 0, cus = 0, per_cu = 0;
    if (hipError_t e = hipGetDevice(&dev)) return e;
    if (hipError_t e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev)) return e;
    const size_t lds = fused_lds_bytes(H, I, E, K);
    if (hipError_t e = fused_dispatch<RunOcc>(H, I, E, K, &per_cu, lds)) return e;
    const int resident = cus * per_cu;
    const RowGeo gg = gateup_geo(H, I), dg = fused_down_geo(H, I);
    int want = E;                                                  // one router row per workgroup
    const int gu = (K * gg.nblk + kWaves - 1) / kWaves, dn = (dg.nblk + kWaves - 1) / kWaves;
    if (gu > want) want = gu;
    if (dn > want) want = dn;
    int n = want < resident ? want : resident;
    if (n > fused_max_workgroups()) n = fused_max_workgroups();
    *nw = n;
    return hipSuccess;
}

hipError_t launch_layer_fused(const FusedLaunch &a_in, hipStream_t s, const KernelEvents &ev) {
    FusedLaunch a = a_in;
    if (a.nw < 1 || a.nw > fused_max_workgroups()) return hipErrorInvalidValue;
    a.L.geo = gateup_geo(a.L.H, a.L.I);
    a.L.pt = plane_table(a.L.H, a.L.I);
    a.dgeo = fused_down_geo(a.L.H, a.L.I);
    const size_t lds = fused_lds_bytes(a.L.H, a.L.I, a.L.E, a.L.K);
    return fused_dispatch<RunLaunch>(a.L.H, a.L.I, a.L.E, a.L.K, a, lds, s, ev);
}

}  // namespace moe
