// moe_batched8.hip -- batched (T > 1) expert FFN for experts that received few tokens.
//
// With top-K routing over many experts most experts of a batch see one to a handful of tokens
// (a Zipf-skewed router still leaves a long tail of them), and a 32-token MFMA tile would then be
// almost empty: the matrix cores would do up to 32x the useful work and, worse, a tile's chain of
// MFMA steps per weight chunk sets its pace.  For such experts the work is a handful of matvecs
// that share one stream of weights, so these kernels reuse the decode path's building blocks:
// the expert's n <= kSmallTokens activation rows are staged once per workgroup as 16-bit digit
// planes in the expert's code order, each wave streams units of weight rows with the next unit's
// loads in flight, and every loaded code dword meets all n staged rows through v_dot8_i32_i4.
// Cost therefore grows with the tokens an expert really has.
//
//   k_gu8 : gate/up rows of one small expert, h = silu(g) * u for each of its tokens (rows of
//           the expert-ordered h buffer, as the MFMA kernels write them)
//   k_dn8 : down rows of one small expert, each token's output row written to y[token][slot]
//
// The dequantisation is the decode path's: w = q*s + b summed per slot as s * sum(q x) +
// b * sum(x) (the FMA rewrite on the lilting.ch page "397Bパラメータモデルを48GB MacBookで動かす
// Flash-MoE", section "Metal Compute Shaders"), with sum(q x) an exact integer dot product.
#include "moe_device.h"

namespace moe {
namespace {

// Per wave: UPW work units, NB register buffers (NB - 1 units in flight while one is computed).
// A gate/up unit is gu_rg rows of gate and of up (8 KiB of 4-bit codes at H = 4096); a down unit
// is dn8_rg wave instructions of rows (8 KiB at I = 1024).
constexpr int kGuUPW = 8, kGuNB = 3;
constexpr int kDnUPW = 8, kDnNB = 3;
template <int NJ>
__host__ __device__ constexpr int dn8_rg() { return NJ >= 4 ? 2 : NJ == 2 ? 4 : 8; }

// Digit-plane staging of one chunk of token row t (see stage_finish): row t occupies row_dw(cols)
// dwords at lds + t * row_dw(cols), digit planes in the order of code width BITS, then its slots'
// {sx, sum of x}.
template <int BITS>
struct DigitStage {
    uint32_t *lds;
    int cols;
    __device__ __forceinline__ void operator()(int t, int mc, bool valid, const float (&v)[16]) const {
        uint32_t *d = lds + t * row_dw(cols);
        stage_chunk(mc, valid, v, BITS == 4 ? d : nullptr, BITS == 2 ? d : nullptr, (float2 *)(d + cols / 2));
    }
};

// --------------------------------------------------------------------------- gate/up
// GS: lanes per row group when it is a compile-time 32 or 64 and every lane's slots exist, else 0
// (run-time group size, idle slots masked).
template <int BITS, int NJ, int GS>
__device__ __forceinline__ void gu8_body(const GroupedLaunch &a, const SmallRec &se, uint32_t *lds) {
    constexpr int RG = gu_rg<NJ>();
    const int H = a.H, I = a.I, lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const Geo g = make_geo(a.geo);
    const int RB = a.geo.rb, nblk = a.geo.nblk;
    Planes pl[3];
    expert_planes(se.blob, BITS, a.pt, pl);
    // unit i of this wave: ub + i * kWaves; nu of them (0 for a wave past the matrix)
    const int ub = blockIdx.x * kWaves * kGuUPW + wave;
    const int nu = max(0, min(kGuUPW, (nblk - ub + kWaves - 1) / kWaves));
    const int last = max(nu - 1, 0);
    auto r0_of = [&](int i) { return min(ub + min(i, last) * kWaves, nblk - 1) * RB; };

    // 1. activation chunks of the expert's tokens, then the first units' weights
    const size_t rowb = (size_t)H * (a.x_dtype == MOE_BF16 ? 2 : 4);
    auto row_addr = [&](int t) { return (const void *)((const char *)a.x + (size_t)(se.pair[t] / a.K) * rowb); };
    StageBatch sb;
    stage_issue(row_addr, H, a.x_dtype, sb);
    GULoads<NJ, RG> L[kGuNB];
    auto issue = [&](int i, GULoads<NJ, RG> &B) { gu_issue<BITS, NJ, RG>(pl, g, H, I, r0_of(i), RB, B); };
    static_for<0, kGuNB - 1>([&](auto ic) { issue(decltype(ic)::value, L[decltype(ic)::value]); });

    // 2. staging (registers first, so the weight loads stay in flight)
    stage_finish(row_addr, se.n, H, a.x_dtype, sb, DigitStage<BITS>{lds, H});
    __syncthreads();

    // 3. units: each loaded unit meets every token
    const int rd = row_dw(H);
    unit_pipeline<kGuUPW>(nu, L, issue, [&](int i, const GULoads<NJ, RG> &B) {
        const int r0 = r0_of(i);
        for (int t = 0; t < se.n; ++t) {
            const uint32_t *d = lds + t * rd;
            uint32_t D[NJ][kSlotDw];
            float2 XS[NJ];
            row_slots<NJ, GS>(ActView{d, (const float2 *)(d + H / 2)}, g, D, XS);
            float pg[RG], pu[RG];
#pragma unroll
            for (int gi = 0; gi < RG; ++gi) {
                pg[gi] = pu[gi] = 0.f;
#pragma unroll
                for (int j = 0; j < NJ; ++j) {
                    pg[gi] += slot_dot<BITS>(B.qg[gi][j], D[j], B.sg[gi][j], XS[j]);
                    pu[gi] += slot_dot<BITS>(B.qu[gi][j], D[j], B.su[gi][j], XS[j]);
                }
            }
            float *hout = a.hbuf + (size_t)(se.base + t) * I;
            if constexpr (GS != 0 && RG == 1) {
                // one row per wave instruction (GS = 64): gate in the lower half, up in the upper
                const float s = pair_sum<GS>(pg[0], pu[0]);
                const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(s), __float_as_uint(s), false, false);
                const int r = r0 + g.lrow;
                if (lane == 0 && r < I) hout[r] = silu(__uint_as_float(p[0])) * __uint_as_float(p[1]);
            } else if constexpr (GS != 0) {
                // rows 2q and 2q+1 of the unit: the lower half-group holds row 2q, the upper row 2q+1
#pragma unroll
                for (int q = 0; q < RG / 2; ++q) {
                    const float sg = pair_sum<GS>(pg[2 * q], pg[2 * q + 1]);
                    const float su = pair_sum<GS>(pu[2 * q], pu[2 * q + 1]);
                    const int hi = (lane % GS) >= GS / 2;
                    const int rr = (2 * q + hi) * g.rpi + g.lrow;
                    if (lane % (GS / 2) == 0 && rr < RB && r0 + rr < I) hout[r0 + rr] = silu(sg) * su;
                }
            } else {
#pragma unroll
                for (int gi = 0; gi < RG; ++gi) {
                    const float sg = group_sum(pg[gi], g.gsz), su = group_sum(pu[gi], g.gsz);
                    const int rr = gi * g.rpi + g.lrow;
                    if (g.lsl == 0 && rr < RB && r0 + rr < I) hout[r0 + rr] = silu(sg) * su;
                }
            }
        }
    });
}

template <int NJ, int GS>
__global__ void __launch_bounds__(kBlock) k_gu8(GroupedLaunch a) {
    extern __shared__ __align__(16) uint32_t lds[];
    SmallRec se;
    if (!small_entry(a, se)) return;
    if (se.bits == 2) gu8_body<2, NJ, GS>(a, se, lds);
    else gu8_body<4, NJ, GS>(a, se, lds);
}

// --------------------------------------------------------------------------- down
template <int NJ, int RG>
struct D8Loads {
    u32x4 q[RG][NJ];
    uint32_t sb[RG][NJ];
};
template <int BITS, int NJ, int RG>
__device__ __forceinline__ void dn8_issue(const Planes &pl, const Geo &g, int H, int I, int r0, D8Loads<NJ, RG> &L) {
    const int G = I / 64;
    const size_t rowb = (size_t)I * BITS / 8;
#pragma unroll
    for (int gi = 0; gi < RG; ++gi) {
        const int r = min(r0 + gi * g.rpi + g.lrow, H - 1);     // clamped; rows past H are not written
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            const int slot = min(g.lsl + 64 * j, g.spr - 1);
            L.q[gi][j] = load_slot<BITS>(pl.q + (size_t)r * rowb, slot);
            L.sb[gi][j] = __builtin_nontemporal_load(pl.sb + ((size_t)r * G + (slot >> 1)));
        }
    }
}

template <int BITS, int NJ, int GS>
__device__ __forceinline__ void dn8_body(const GroupedLaunch &a, const SmallRec &se, uint32_t *lds) {
    constexpr int RG = dn8_rg<NJ>();
    const int H = a.H, I = a.I, lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const Geo g = make_geo(a.geo);
    const int RB = a.geo.rb, nblk = a.geo.nblk;
    Planes pl[3];
    expert_planes(se.blob, BITS, a.pt, pl);
    const int ub = blockIdx.x * kWaves * kDnUPW + wave;
    const int nu = max(0, min(kDnUPW, (nblk - ub + kWaves - 1) / kWaves));
    const int last = max(nu - 1, 0);
    auto r0_of = [&](int i) { return min(ub + min(i, last) * kWaves, nblk - 1) * RB; };

    // 1. h rows (consecutive in the expert-ordered buffer), then the first units' weights
    auto row_addr = [&](int t) { return (const void *)(a.hbuf + (size_t)(se.base + min(t, se.n - 1)) * I); };
    StageBatch sb;
    stage_issue(row_addr, I, MOE_F32, sb);
    D8Loads<NJ, RG> L[kDnNB];
    auto issue = [&](int i, D8Loads<NJ, RG> &B) { dn8_issue<BITS, NJ, RG>(pl[2], g, H, I, r0_of(i), B); };
    static_for<0, kDnNB - 1>([&](auto ic) { issue(decltype(ic)::value, L[decltype(ic)::value]); });

    // 2. staging
    stage_finish(row_addr, se.n, I, MOE_F32, sb, DigitStage<BITS>{lds, I});
    __syncthreads();

    // 3. units
    const int rd = row_dw(I);
    unit_pipeline<kDnUPW>(nu, L, issue, [&](int i, const D8Loads<NJ, RG> &B) {
        const int r0 = r0_of(i);
        for (int t = 0; t < se.n; ++t) {
            const uint32_t *d = lds + t * rd;
            uint32_t D[NJ][kSlotDw];
            float2 XS[NJ];
            row_slots<NJ, GS>(ActView{d, (const float2 *)(d + I / 2)}, g, D, XS);
            float part[RG];
#pragma unroll
            for (int gi = 0; gi < RG; ++gi) {
                part[gi] = 0.f;
#pragma unroll
                for (int j = 0; j < NJ; ++j) part[gi] += slot_dot<BITS>(B.q[gi][j], D[j], B.sb[gi][j], XS[j]);
            }
            float *yrow = a.y + (size_t)se.pair[0] * H;
#pragma unroll
            for (int q = 1; q < kSmallTokens; ++q) yrow = t == q ? a.y + (size_t)se.pair[q] * H : yrow;
            if constexpr (GS != 0) {
#pragma unroll
                for (int q = 0; q < RG / 2; ++q) {
                    const float s = pair_sum<GS>(part[2 * q], part[2 * q + 1]);
                    const int hi = (lane % GS) >= GS / 2;
                    const int rr = (2 * q + hi) * g.rpi + g.lrow;
                    if (lane % (GS / 2) == 0 && rr < RB && r0 + rr < H) yrow[r0 + rr] = s;
                }
            } else {
#pragma unroll
                for (int gi = 0; gi < RG; ++gi) {
                    const float s = group_sum(part[gi], g.gsz);
                    const int rr = gi * g.rpi + g.lrow;
                    if (g.lsl == 0 && rr < RB && r0 + rr < H) yrow[r0 + rr] = s;
                }
            }
        }
    });
}

template <int NJ, int GS>
__global__ void __launch_bounds__(kBlock) k_dn8(GroupedLaunch a) {
    extern __shared__ __align__(16) uint32_t lds[];
    SmallRec se;
    if (!small_entry(a, se)) return;
    if (se.bits == 2) dn8_body<2, NJ, GS>(a, se, lds);
    else dn8_body<4, NJ, GS>(a, se, lds);
}

// Compile-time group size for rows of `cols` inputs taken NJ slots per lane: 32 or 64 when every
// lane's slots exist (cols = 64 * 32 * NJ for NJ >= 1, or 32 slots exactly), else 0.
int small_gs(int cols, int nj) {
    const int spr = cols / 32;
    if (spr == 64 * nj) return 64;
    if (nj == 1 && spr == 32) return 32;
    return 0;
}

size_t small_lds_bytes(int cols) { return (size_t)kSmallTokens * row_dw(cols) * 4; }

hipError_t set_small_lds(const void *fn, size_t lds) {
    if (lds <= 64 * 1024) return hipSuccess;
    return hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
}

}  // namespace

bool small_path_fits(int H, int I) {
    return small_lds_bytes(H) <= 160 * 1024 && small_lds_bytes(I) <= 160 * 1024 && H % 64 == 0 && I % 64 == 0;
}

hipError_t launch_small_gateup(const GroupedLaunch &a_in, int max_small, hipStream_t s) {
    GroupedLaunch a = a_in;
    a.geo = gateup_geo(a.H, a.I);
    a.pt = plane_table(a.H, a.I);
    const dim3 grid((a.geo.nblk + kWaves * kGuUPW - 1) / (kWaves * kGuUPW), max_small);
    const size_t lds = small_lds_bytes(a.H);
    auto launch = [&](auto fn) -> hipError_t {
        if (hipError_t e = set_small_lds((const void *)fn, lds)) return e;
        hipLaunchKernelGGL(fn, grid, dim3(kBlock), lds, s, a);
        return hipGetLastError();
    };
    const int nj = nj_for(a.H), gs = small_gs(a.H, nj);
    switch (nj) {
        case 1: return gs == 64 ? launch(k_gu8<1, 64>) : gs == 32 ? launch(k_gu8<1, 32>) : launch(k_gu8<1, 0>);
        case 2: return gs ? launch(k_gu8<2, 64>) : launch(k_gu8<2, 0>);
        default: return gs ? launch(k_gu8<4, 64>) : launch(k_gu8<4, 0>);
    }
}

hipError_t launch_small_down(const GroupedLaunch &a_in, int max_small, hipStream_t s) {
    GroupedLaunch a = a_in;
    const int nj = nj_for(a.I), gs = small_gs(a.I, nj);
    a.geo = row_geo(a.I, a.H, nj == 1 ? dn8_rg<1>() : nj == 2 ? dn8_rg<2>() : dn8_rg<4>());
    a.pt = plane_table(a.H, a.I);
    const dim3 grid((a.geo.nblk + kWaves * kDnUPW - 1) / (kWaves * kDnUPW), max_small);
    const size_t lds = small_lds_bytes(a.I);
    auto launch = [&](auto fn) -> hipError_t {
        if (hipError_t e = set_small_lds((const void *)fn, lds)) return e;
        hipLaunchKernelGGL(fn, grid, dim3(kBlock), lds, s, a);
        return hipGetLastError();
    };
    switch (nj) {
        case 1: return gs == 64 ? launch(k_dn8<1, 64>) : gs == 32 ? launch(k_dn8<1, 32>) : launch(k_dn8<1, 0>);
        case 2: return gs ? launch(k_dn8<2, 64>) : launch(k_dn8<2, 0>);
        default: return gs ? launch(k_dn8<4, 64>) : launch(k_dn8<4, 0>);
    }
}

}  // namespace moe
