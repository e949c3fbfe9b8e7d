// moe_small.h -- building blocks of the integer dot-product expert kernels for a few tokens per
// expert: the small-expert kernels of the batched path (moe_batched8.hip) and the shared-read
// kernels of calls with a few tokens (moe_shared_gu.hip, moe_shared_dn.hip).
//
// With top-K routing over many experts most experts of a batch see one to a handful of tokens
// (a Zipf-skewed router still leaves a long tail of them), and a 32-token MFMA tile would then be
// almost empty: the matrix cores would do up to 32x the useful work and, worse, a tile's chain of
// MFMA steps per weight chunk sets its pace.  For such experts the work is a handful of matvecs
// that share one stream of weights, so these kernels reuse the decode path's building blocks:
// the expert's activation rows are staged once per workgroup as 16-bit digit planes in the
// expert's code order, each wave streams units of weight rows with the next units' loads in
// flight, and every loaded code dword meets all staged rows through v_dot8_i32_i4.  Cost
// therefore grows with the tokens an expert really has.
//
// The dequantisation is the decode path's: w = q*s + b summed per slot as s * sum(q x) +
// b * sum(x) (the FMA rewrite on the lilting.ch page "397Bパラメータモデルを48GB MacBookで動かす
// Flash-MoE", section "Metal Compute Shaders"), with sum(q x) an exact integer dot product.
#pragma once

#include "moe_device.h"

#include <algorithm>
#include <atomic>

namespace moe {
namespace {

// Per wave: UPW work units, NB register buffers (NB - 1 units in flight while one is computed).
// A gate/up unit is gu_rg rows of gate and of up (8 KiB of 4-bit codes at H = 4096); a down unit
// is dn8_rg wave instructions of rows (8 KiB at I = 1024).
constexpr int kGuUPW = 8, kGuNB = 3;
constexpr int kDnUPW = 8, kDnNB = 3;
constexpr int kSharedUPW = 2;             // shared-read path: every unit's loads issued up front
// Dependency chains of a slot's dot products (slot_dot): the token loop interleaves the slots of a
// unit, so fewer chains than planes save the zeroed accumulators and the combination (250 instead of
// 282 vector instructions per unit and token).  Config-4 batch: two chains 525-526 us, one chain
// 530-531, four 531-532 (two runs each).
constexpr int kSmallDotCh = 2;
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
// Units of one workgroup: slice `sl` of an expert's matrix takes units [sl, sl + 1) * kWaves * upw;
// unit i of a wave is ub + i * kWaves, nu of them (0 for a wave past the matrix), upw <= UPW (the
// unrolled pipeline's length).  The small-expert list runs with sl = blockIdx.x and upw = UPW =
// kGuUPW / kDnUPW; the shared-read path sizes both per expert, with UPW = kSharedUPW.
// Copy of pre-staged rows (k_stage_rows' layout: 4-bit planes, 2-bit planes, xs) into LDS rows of
// code width BITS: row t of the record from token se.pair[t] / K.
template <int BITS, int CAP>
__device__ __forceinline__ void copy_staged(const GroupedLaunch &a, const TokRec<CAP> &se, uint32_t *lds) {
    const int H = a.H, rd = row_dw(H), nq = rd / 4, pq = H / 8;       // 16-byte pieces per row, of planes
    const size_t srow = (size_t)H + H / 16;
    static_for<0, CAP>([&](auto tc) {
        constexpr int t = decltype(tc)::value;
        if (t < se.n) {                                                     // uniform
            const uint32_t *src = a.planes + (size_t)(se.pair[t] / a.K) * srow;
            for (int i = threadIdx.x; i < nq; i += kBlock) {
                const int o = i < pq ? (BITS == 2 ? H / 2 : 0) + 4 * i : H + 4 * (i - pq);
                *(u32x4 *)(lds + t * rd + 4 * i) = *(const GLOBAL_AS u32x4 *)(src + o);
            }
        }
    });
}

// PRE: the rows come pre-staged from k_stage_rows (a.planes) instead of being converted here.
template <int BITS, int NJ, int GS, int UPW, int CAP, bool PRE = false>
__device__ __forceinline__ void gu8_body(const GroupedLaunch &a, const TokRec<CAP> &se, int sl, int upw,
                                         uint32_t *lds) {
    constexpr int RG = gu_rg<NJ>();
    const int H = a.H, I = a.I, lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const Geo g = make_geo(a.geo);
    const int RB = a.geo.rb, nblk = a.geo.nblk;
    Planes pl[3];
    expert_planes(se.blob, BITS, a.pt, pl);
    const int ub = sl * kWaves * upw + wave;
    const int nu = max(0, min(upw, (nblk - ub + kWaves - 1) / kWaves));
    const int last = max(nu - 1, 0);
    auto r0_of = [&](int i) { return min(ub + min(i, last) * kWaves, nblk - 1) * RB; };

    // 1. activation chunks of the expert's tokens, then the first units' weights
    const size_t rowb = (size_t)H * (a.x_dtype == MOE_BF16 ? 2 : 4);
    auto row_addr = [&](int t) { return (const void *)((const char *)a.x + (size_t)(se.pair[t] / a.K) * rowb); };
    StageBatch sb;
    if constexpr (!PRE) stage_issue(row_addr, H, a.x_dtype, sb);
    GULoads<NJ, RG> L[kGuNB];
    auto issue = [&](int i, GULoads<NJ, RG> &B) { gu_issue<BITS, NJ, RG>(pl, g, H, I, r0_of(i), RB, B); };
    static_for<0, kGuNB - 1>([&](auto ic) { issue(decltype(ic)::value, L[decltype(ic)::value]); });

    // 2. staging (registers first, so the weight loads stay in flight)
    if constexpr (PRE) copy_staged<BITS>(a, se, lds);
    else stage_finish<CAP / 4>(row_addr, se.n, H, a.x_dtype, sb, DigitStage<BITS>{lds, H});
    __syncthreads();

    // 3. units: each loaded unit meets every token
    const int rd = row_dw(H);
    unit_pipeline<UPW>(nu, L, issue, [&](int i, const GULoads<NJ, RG> &B) {
        const int r0 = r0_of(i);
        // the slots' dot-product operands, once per unit for all of its tokens
        SlotOps og[RG][NJ], ou[RG][NJ];
#pragma unroll
        for (int gi = 0; gi < RG; ++gi)
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                og[gi][j] = slot_ops<BITS>(B.qg[gi][j], B.sg[gi][j]);
                ou[gi][j] = slot_ops<BITS>(B.qu[gi][j], B.su[gi][j]);
            }
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
                    pg[gi] += slot_dot_ops<kSmallDotCh>(og[gi][j], D[j], XS[j]);
                    pu[gi] += slot_dot_ops<kSmallDotCh>(ou[gi][j], D[j], XS[j]);
                }
            }
            float *hout = a.hbuf + (size_t)(se.base + t) * I;
            if constexpr (GS != 0 && RG == 1) {
                // one row per wave instruction (GS = 64): gate in the lower half, up in the upper
                const float s = pair_sum<GS>(pg[0], pu[0]);
                const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(s), __float_as_uint(s), false, false);
                const int r = r0 + g.lrow;
                if (lane == 0 && r < I) hout[r] = silu_fast(__uint_as_float(p[0])) * __uint_as_float(p[1]);
            } else if constexpr (GS != 0) {
                // rows 2q and 2q+1 of the unit: the lower half-group holds row 2q, the upper row 2q+1
#pragma unroll
                for (int q = 0; q < RG / 2; ++q) {
                    const float sg = pair_sum<GS>(pg[2 * q], pg[2 * q + 1]);
                    const float su = pair_sum<GS>(pu[2 * q], pu[2 * q + 1]);
                    const int hi = (lane % GS) >= GS / 2;
                    const int rr = (2 * q + hi) * g.rpi + g.lrow;
                    if (lane % (GS / 2) == 0 && rr < RB && r0 + rr < I) hout[r0 + rr] = silu_fast(sg) * su;
                }
            } else {
#pragma unroll
                for (int gi = 0; gi < RG; ++gi) {
                    const float sg = group_sum(pg[gi], g.gsz), su = group_sum(pu[gi], g.gsz);
                    const int rr = gi * g.rpi + g.lrow;
                    if (g.lsl == 0 && rr < RB && r0 + rr < I) hout[r0 + rr] = silu_fast(sg) * su;
                }
            }
        }
    });
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

template <int BITS, int NJ, int GS, int UPW, int CAP>
__device__ __forceinline__ void dn8_body(const GroupedLaunch &a, const TokRec<CAP> &se, int sl, int upw,
                                         uint32_t *lds) {
    constexpr int RG = dn8_rg<NJ>();
    const int H = a.H, I = a.I, lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const Geo g = make_geo(a.geo);
    const int RB = a.geo.rb, nblk = a.geo.nblk;
    Planes pl[3];
    expert_planes(se.blob, BITS, a.pt, pl);
    const int ub = sl * kWaves * upw + wave;
    const int nu = max(0, min(upw, (nblk - ub + kWaves - 1) / kWaves));
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
    stage_finish<CAP / 4>(row_addr, se.n, I, MOE_F32, sb, DigitStage<BITS>{lds, I});
    __syncthreads();

    // 3. units
    const int rd = row_dw(I);
    unit_pipeline<UPW>(nu, L, issue, [&](int i, const D8Loads<NJ, RG> &B) {
        const int r0 = r0_of(i);
        SlotOps op[RG][NJ];
#pragma unroll
        for (int gi = 0; gi < RG; ++gi)
#pragma unroll
            for (int j = 0; j < NJ; ++j) op[gi][j] = slot_ops<BITS>(B.q[gi][j], B.sb[gi][j]);
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
                for (int j = 0; j < NJ; ++j)
                    part[gi] += slot_dot_ops<kSmallDotCh>(op[gi][j], D[j], XS[j]);
            }
            float *yrow = a.y + (size_t)se.pair[0] * H;
#pragma unroll
            for (int q = 1; q < CAP; ++q) yrow = t == q ? a.y + (size_t)se.pair[q] * H : yrow;
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

// --------------------------------------------------------------------------- shared-read path
// A call with a few tokens (T*K <= kSharedMaxPairs pairs) takes no grouping pass: wavefront 0 of
// every workgroup derives the call's distinct experts from idx by itself.  Each valid pair marks a
// two-word LDS entry of its expert (first pair, pair count) with LDS atomics, so the pairs that
// their entry names first stand for the distinct experts, in order of first appearance.  Expert d
// with its pairs in pair order is one entry of the work list (an expert with more than 2 * cap pairs
// becomes several entries of at most that many, each streaming the expert once); its rows
// of the expert-ordered h buffer start after the pairs of the experts that appear before it.  The
// grid's workgroups are dealt to the entries in proportion to their rows + 1, and an entry's workgroups split its
// matrix into as many slices as there are of them (one or two units per wave: with many rows per
// expert the dot products, not the weight stream, set the pace).  Gate/up and down derive the same
// entries, so the h rows match between them.  A workgroup stages at most `cap` (4 or 8) of its
// entry's rows at a time and makes one pass over its units per batch of rows: the second pass reads
// the slice's weights again from L2.
struct SharedWork {
    uint64_t blob;
    int n, base, bits;      // the entry's pairs (1..kSharedCap), first h row, code width
    int sl, upw;            // slice of the expert's matrix and units per wave (upw 0: no work)
    uint64_t inval;         // pairs whose index is outside [0, E) or whose expert is absent
    const uint32_t *pairs;  // LDS: the entry's pairs in pair order
};
constexpr int kSharedRecDw = 32;
__host__ __device__ __forceinline__ int shared_rec_off(int cols, int cap, int E) {
    const int st = cap * row_dw(cols), tb = 2 * E;
    return ((st > tb ? st : tb) + 3) & ~3;
}
constexpr int kSharedDirectMaxT = 4;      // up to this many tokens (no norm): rows staged by each workgroup
// Rows a workgroup stages at a time: 4 for up to four tokens, else 8.
__host__ __device__ __forceinline__ int shared_cap(int T) { return T <= 4 ? 4 : kSmallTokens; }

__device__ __forceinline__ int mbcnt64(uint64_t m) {
    return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// The work of this workgroup; every thread calls it (it ends with a barrier).  lds: the staging area
// (its first 2E dwords serve as the expert table), then the record at rec_off.
__device__ __forceinline__ void shared_work(const GroupedLaunch &a, int nblk, int rec_off, uint32_t *lds,
                                            SharedWork &w) {
    uint32_t *rec = lds + rec_off;
    if (threadIdx.x < 64) {
        const int lane = threadIdx.x, P = a.T * a.K;
        int e = -1, bits = 4;
        uint64_t blob = 0;
        if (lane < P) {
            e = a.idx[lane];
            if (e >= 0 && e < a.E) {
                const moe_expert_desc d = a.experts[e];
                blob = d.blob;
                bits = d.bits == 2 ? 2 : 4;
            }
        }
        const bool valid = blob != 0;
        uint32_t *tab = lds;            // [2e] first pair of expert e, [2e + 1] its pair count
        if (valid) {
            tab[2 * e] = 64u;
            tab[2 * e + 1] = 0u;
        }
        if (valid) {                    // after the stores above: one wavefront's LDS operations run in order
            atomicMin(&tab[2 * e], (uint32_t)lane);
            atomicAdd(&tab[2 * e + 1], 1u);
        }
        int first = 64, cnt = 0;
        if (valid) {
            first = (int)tab[2 * e];
            cnt = (int)tab[2 * e + 1];
        }
        const bool is_first = valid && first == lane;
        const uint64_t fm = __ballot(is_first);
        const int C = 2 * a.cap;        // pairs per entry: two batches of staged rows
        const uint64_t big = __ballot(is_first && cnt > C);
        // entries: one per distinct expert, or ceil(cnt / C) when some expert has more pairs
        int nent = __popcll(fm);
        if (big) {
            nent = 0;
            for (uint64_t m = fm; m; m &= m - 1) {
                const int l = __ffsll((unsigned long long)m) - 1;
                nent += (__builtin_amdgcn_readlane(cnt, l) + C - 1) / C;
            }
        }
        int f = 0, c = 0, n = 0, base = 0, sl = 0, upw = 0, pe = 0, pbits = 4;
        uint64_t pblob = 0;
        uint32_t pairs[kSharedCap] = {};
        if (nent > 0) {
            const int G = gridDim.x, L = blockIdx.x;
            int s = 0, avail = 0;
            if (!big) {
                // workgroups dealt to the experts in proportion to their rows + 1 (the dot products
                // grow with the rows, the weight stream does not): expert of first lane l takes the
                // workgroups [G * pre_l / W, G * (pre_l + w_l) / W)
                const int wgt = is_first ? cnt + 1 : 0;
                int inc = wgt;
#pragma unroll
                for (int d = 1; d < 64; d <<= 1) {
                    const int y = __shfl_up(inc, d);
                    if (lane >= d) inc += y;
                }
                const int W = __builtin_amdgcn_readlane(inc, 63);
                const int lo = (G * (inc - wgt)) / W, hi = (G * inc) / W;
                f = __ffsll((unsigned long long)__ballot(is_first && lo <= L && L < hi)) - 1;
                s = L - __builtin_amdgcn_readlane(lo, f);
                avail = __builtin_amdgcn_readlane(hi, f) - __builtin_amdgcn_readlane(lo, f);
            } else {
                const int j = L % nent;
                s = L / nent;
                avail = G / nent + (j < G % nent ? 1 : 0);
                int acc = 0;
                for (uint64_t m = fm; m; m &= m - 1) {
                    const int l = __ffsll((unsigned long long)m) - 1;
                    const int nch = (__builtin_amdgcn_readlane(cnt, l) + C - 1) / C;
                    if (j < acc + nch) {
                        f = l;
                        c = j - acc;
                        break;
                    }
                    acc += nch;
                }
            }
            pe = __builtin_amdgcn_readlane(e, f);
            pblob = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(blob >> 32), f) << 32) |
                    (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)blob, f);
            pbits = __builtin_amdgcn_readlane(bits, f);
            uint64_t m = __ballot(valid && e == pe);
            n = min(C, __popcll(m) - c * C);
            base = __popcll(__ballot(valid && first < f)) + c * C;
            for (int q = 0; q < c * C; ++q) m &= m - 1;
#pragma unroll
            for (int t = 0; t < kSharedCap; ++t) {
                pairs[t] = t < n ? (uint32_t)(__ffsll((unsigned long long)m) - 1) : pairs[t > 0 ? t - 1 : 0];
                if (t < n) m &= m - 1;
            }
            // slices: as many as the entry has workgroups, down to one unit per wave (the grid gives
            // every entry at least ceil(nblk / 32) workgroups, so upw <= 8)
            const int nsl = min(avail, (nblk + kWaves - 1) / kWaves);
            if (s < nsl) {
                sl = s;
                upw = (nblk + kWaves * nsl - 1) / (kWaves * nsl);
            }
        }
        const uint64_t inval = __ballot(lane < P && !valid);
        if (lane == 0) {
            rec[0] = (uint32_t)pblob;
            rec[1] = (uint32_t)(pblob >> 32);
            rec[2] = (uint32_t)pe;
            rec[3] = (uint32_t)n;
            rec[4] = (uint32_t)base;
            rec[5] = (uint32_t)pbits;
            rec[6] = (uint32_t)sl;
            rec[7] = (uint32_t)upw;
            rec[8] = (uint32_t)inval;
            rec[9] = (uint32_t)(inval >> 32);
#pragma unroll
            for (int t = 0; t < kSharedCap; ++t) rec[10 + t] = pairs[t];
        }
    }
    __syncthreads();
    // readfirstlane returns int: take the word back as unsigned before widening it into a 64-bit
    // address or mask (a sign-extended low word would corrupt the upper half)
    auto rd = [&](int i) { return (uint32_t)__builtin_amdgcn_readfirstlane((int)rec[i]); };
    w.blob = ((uint64_t)rd(1) << 32) | rd(0);
    w.n = (int)rd(3);
    w.base = (int)rd(4);
    w.bits = (int)rd(5);
    w.sl = (int)rd(6);
    w.upw = (int)rd(7);
    w.inval = ((uint64_t)rd(9) << 32) | rd(8);
    w.pairs = rec + 10;
}

// Rows tb .. tb + cap - 1 of an entry as a record of its own (tb a multiple of cap, uniform); the
// pairs come from the entry's LDS record.
template <int CAP>
__device__ __forceinline__ void row_batch(const SharedWork &w, int tb, int cap, TokRec<CAP> &o) {
    o.blob = w.blob;
    o.e = 0;
    o.bits = w.bits;
    o.n = min(cap, w.n - tb);
    o.base = w.base + tb;
#pragma unroll
    for (int t = 0; t < CAP; ++t)
        o.pair[t] = __builtin_amdgcn_readfirstlane((int)w.pairs[min(tb + min(t, o.n - 1), kSharedCap - 1)]);
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

constexpr size_t kMaxLds = kCuLds;
template <auto FN>
hipError_t launch_lds(dim3 grid, size_t lds, hipStream_t s, const KernelEvents &ev, const GroupedLaunch &a) {
    if (hipError_t e = lds_for<FN>(lds)) return e;
    return dispatch(FN, grid, dim3(kBlock), lds, s, ev, a);
}

size_t shared_lds_bytes(int cols, int cap, int E) { return ((size_t)shared_rec_off(cols, cap, E) + kSharedRecDw) * 4; }
// Rows the down kernel stages at once: an entry's 2 * cap pairs when they fit, else cap.
int shared_cap_dn(int I, int T, int E) {
    const int cap = shared_cap(T);
    return shared_lds_bytes(I, 2 * cap, E) <= kMaxLds ? 2 * cap : cap;
}
// Workgroups of a shared-read launch: at least ceil(nblk / 32) per entry whatever the split (at most
// P entries, and an entry's share of the grid is at least 1/P), so no wave has more than eight
// units; and the grid fills the chip at least twice.
int shared_grid(int nblk, int P) {
    const int per = (nblk + kWaves * kGuUPW - 1) / (kWaves * kGuUPW);
    return std::max(P * per, 512);
}
// An entry's rows in at most two batches of `cap`, written out rather than looped: a loop around the
// body keeps its hoisted addresses live throughout and spills.
// UPW: the unrolled pipeline's length, kSharedUPW when upw <= kSharedUPW (many rows per expert:
// many short slices) else kGuUPW / kDnUPW.
// PRE: the rows come pre-staged by k_stage_rows (a.planes); otherwise every workgroup converts its
// rows from x itself (few tokens and no norm weight: no staging launch).
template <int NJ, int GS, int UPW, bool PRE>
__device__ __forceinline__ void gu_batch(const GroupedLaunch &a, const SharedWork &w, int tb, uint32_t *lds) {
    TokRec<kSmallTokens> r;
    row_batch(w, tb, a.cap, r);
    if (r.bits == 2) gu8_body<2, NJ, GS, UPW, kSmallTokens, PRE>(a, r, w.sl, w.upw, lds);
    else gu8_body<4, NJ, GS, UPW, kSmallTokens, PRE>(a, r, w.sl, w.upw, lds);
}
template <int NJ, int GS, int UPW, bool PRE>
__device__ __forceinline__ void gu_entry(const GroupedLaunch &a, const SharedWork &w, uint32_t *lds) {
    gu_batch<NJ, GS, UPW, PRE>(a, w, 0, lds);
    if (w.n > a.cap) {
        __syncthreads();                          // the first batch's rows are no longer read
        gu_batch<NJ, GS, UPW, PRE>(a, w, a.cap, lds);
    }
}
template <int NJ, int GS, bool PRE>
__global__ void __launch_bounds__(kBlock) k_gu_sh(GroupedLaunch a) {
    extern __shared__ __align__(16) uint32_t lds[];
    SharedWork w;
    shared_work(a, a.geo.nblk, shared_rec_off(a.H, a.cap, a.E), lds, w);
    if (w.upw == 0) return;
    if (w.upw <= kSharedUPW) gu_entry<NJ, GS, kSharedUPW, PRE>(a, w, lds);
    else gu_entry<NJ, GS, kGuUPW, PRE>(a, w, lds);
}

// The gate/up launch of the shared-read path with PRE staging or without.
template <bool PRE>
hipError_t launch_gu_sh(const GroupedLaunch &a, hipStream_t s, const KernelEvents &ev) {
    const dim3 grid(shared_grid(a.geo.nblk, a.T * a.K));
    const size_t lds = shared_lds_bytes(a.H, a.cap, a.E);
    const int nj = nj_for(a.H), gs = small_gs(a.H, nj);
    switch (nj) {
        case 1:
            return gs == 64   ? launch_lds<k_gu_sh<1, 64, PRE>>(grid, lds, s, ev, a)
                   : gs == 32 ? launch_lds<k_gu_sh<1, 32, PRE>>(grid, lds, s, ev, a)
                              : launch_lds<k_gu_sh<1, 0, PRE>>(grid, lds, s, ev, a);
        case 2:
            return gs ? launch_lds<k_gu_sh<2, 64, PRE>>(grid, lds, s, ev, a)
                      : launch_lds<k_gu_sh<2, 0, PRE>>(grid, lds, s, ev, a);
        default:
            return gs ? launch_lds<k_gu_sh<4, 64, PRE>>(grid, lds, s, ev, a)
                      : launch_lds<k_gu_sh<4, 0, PRE>>(grid, lds, s, ev, a);
    }
}

}  // namespace
}  // namespace moe
