// moe_tier.hip -- the policy side of the tiered store: expert usage, hot order, re-tiering.
//
// The pages keep the experts a model uses often at 4 bits and store the others at 2 bits
// (nzkcom.pages.dev, "flash-moe-romance-vs-utility", adopted-optimisation table; the base is an
// MLX 4-bit model: tomo3141592653.github.io, "iPhone 17 Proで400Bパラメータ LLM を動かす
// 「flash-moe」", section "ハイブリッド量子化").  They say neither how use is measured nor how a
// 2-bit expert is made; the plain reading built here:
//   usage    counts[e] += number of routing selections of expert e over a stream of tokens;
//   order    experts by count, most used first, equal counts lower index first; the first n_hot
//            are hot;
//   re-tier  a hot expert keeps its base blob; a cold one is dequantised from its base blob
//            (w = q * scale + bias in fp32) and quantised again at the cold width with the
//            quantiser's rounding, into a store of cold blobs; a new descriptor table points at
//            each expert's blob.
//
// k_usage: LDS histogram per workgroup, flushed with one global atomic add per touched expert.
// k_hot_order: one workgroup sorts the E keys (~count << 32 | expert) in LDS (bitonic).
// k_requant: HBM-bound stream over the cold experts' blobs: a quad of lanes per group of 64 (16
//   codes per lane: 8 bytes at 4-bit, 4 at 2-bit, so a wave instruction reads 512 or 256 bytes
//   contiguous), 4 groups per quad.  Per group: the range from the smallest and largest code, the
//   new pair, and a table of the new code of each possible input code (the quad shares the
//   evaluations through DPP), which every weight then looks up.  Bytes = base blob read + cold
//   blob written per expert.
// k_retier_table: the tiered descriptor table, after the requantisation (so it may overwrite the
//   base table in place).
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "moe_device.h"

namespace moe {
namespace {

constexpr int kUsageBlock = 256;
constexpr int kOrderBlock = 1024;
constexpr int kRqBlock = 256;                 // 4 waves, each over 64 groups

__global__ void __launch_bounds__(kUsageBlock) k_usage(const int32_t *idx, size_t n, int E, uint32_t *counts) {
    extern __shared__ uint32_t hist[];
    for (int e = threadIdx.x; e < E; e += kUsageBlock) hist[e] = 0;
    __syncthreads();
    const size_t stride = (size_t)gridDim.x * kUsageBlock;
    for (size_t i = (size_t)blockIdx.x * kUsageBlock + threadIdx.x; i < n; i += stride) {
        const int v = idx[i];
        if ((unsigned)v < (unsigned)E) atomicAdd(&hist[v], 1u);
    }
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += kUsageBlock)
        if (hist[e]) atomicAdd(&counts[e], hist[e]);
}

// P: the power of two at or above E.  Ascending keys = descending count, then ascending expert.
__global__ void __launch_bounds__(kOrderBlock) k_hot_order(const uint32_t *counts, int E, int P, int32_t *order) {
    extern __shared__ uint64_t key[];
    for (int i = threadIdx.x; i < P; i += kOrderBlock)
        key[i] = i < E ? ((uint64_t)(~counts[i]) << 32) | (uint32_t)i : ~(uint64_t)0;
    __syncthreads();
    for (int k = 2; k <= P; k <<= 1) {
        for (int j = k >> 1; j > 0; j >>= 1) {
            for (int i = threadIdx.x; i < P; i += kOrderBlock) {
                const int l = i ^ j;
                if (l > i) {
                    const uint64_t a = key[i], b = key[l];
                    if ((a > b) == ((i & k) == 0)) {
                        key[i] = b;
                        key[l] = a;
                    }
                }
            }
            __syncthreads();
        }
    }
    for (int i = threadIdx.x; i < E; i += kOrderBlock) order[i] = (int32_t)(uint32_t)key[i];
}

struct RequantArgs {
    const moe_expert_desc *base;
    const int32_t *order;
    int E, n_hot;
    uint64_t store, cold_bytes;
    uint32_t gm;                  // groups of one matrix (I * H / 64, the same for gate, up and down)
    PlaneTable pt;
};

constexpr int kRqGroups = 4;      // groups per quad of lanes (16 per wave instruction, 64 per wave)

template <int CTRL>
__device__ __forceinline__ uint32_t dppu(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, true);
}

// One wave re-quantises kRqGroups * 16 consecutive groups of one matrix; pass k covers groups
// g0 + 16k .. + 15, quad lane j holding codes 16j .. 16j + 15 of group g0 + 16k + lane / 4, so every
// load instruction reads 16 groups' codes contiguous.
//
// Inside a group every weight with input code c dequantises to the same fp32 value
// w(c) = c * scale + bias (c * scale is exact: one rounding), so its new code is a function of c
// alone: the quad evaluates that function once per possible input code (4 per lane at 4 bits in,
// 1 at 2 bits) into a table of 2^BIN new codes, and each weight takes its entry.  The group's
// dequantised minimum and maximum are w(cmin) and w(cmax) (in either order with the sign of the
// scale): rounding is monotone, so they equal the minimum and maximum over the 64 weights.
template <int BIN, int BOUT>
__device__ __forceinline__ void requant_wave(const GLOBAL_AS uint8_t *src, GLOBAL_AS uint8_t *dst, const uint64_t (&oin)[6],
                                             const uint64_t (&oout)[6], int m, uint32_t g0, uint32_t gm, int lane) {
    constexpr int kIn = 1 << BIN;                       // input codes
    constexpr int kPer = kIn / 4;                       // table entries per quad lane
    const int j = lane & 3;
    uint32_t w[kRqGroups][2], sb[kRqGroups];
#pragma unroll
    for (int k = 0; k < kRqGroups; ++k) {
        const uint32_t g = min(g0 + 16 * k + (lane >> 2), gm - 1);     // clamped; results past gm unused
        const GLOBAL_AS uint8_t *q = src + oin[2 * m] + (uint64_t)g * (8 * BIN) + j * (2 * BIN);
        if (BIN == 4) {
            const u32x2 t = __builtin_nontemporal_load((const GLOBAL_AS u32x2 *)q);
            w[k][0] = t.x;
            w[k][1] = t.y;
        } else {
            w[k][0] = __builtin_nontemporal_load((const GLOBAL_AS uint32_t *)q);
            w[k][1] = 0;
        }
        sb[k] = *(const GLOBAL_AS uint32_t *)(src + oin[2 * m + 1] + (uint64_t)g * 4);
    }
#pragma unroll
    for (int k = 0; k < kRqGroups; ++k) {
        const uint32_t g = g0 + 16 * k + (lane >> 2);
        if (g0 + 16 * k >= gm) break;                    // uniform: gm is a multiple of 16
        // t[i] = BOUT * (input code of weight i): the bit offset of its table entry
        uint32_t t[16];
#pragma unroll
        for (int i = 0; i < 16; ++i)
            t[i] = (BIN == 4 ? (w[k][i >> 3] >> (4 * (i & 7))) & 15u : (w[k][0] >> (2 * i)) & 3u) * BOUT;
        uint32_t tmin = t[0], tmax = t[0];
#pragma unroll
        for (int i = 1; i < 16; ++i) {
            tmin = min(tmin, t[i]);
            tmax = max(tmax, t[i]);
        }
        tmin = min(tmin, dppu<0xB1>(tmin));             // quad_perm [1,0,3,2]
        tmax = max(tmax, dppu<0xB1>(tmax));
        tmin = min(tmin, dppu<0x4E>(tmin));             // quad_perm [2,3,0,1]
        tmax = max(tmax, dppu<0x4E>(tmax));
        const float s = bf16_f32(sb[k] & 0xFFFFu), b = bf16_f32(sb[k] >> 16);
        const float wa = (float)(tmin / BOUT) * s + b, wb = (float)(tmax / BOUT) * s + b;
        const QPair p = quant_pair<BOUT>(fminf(wa, wb), fmaxf(wa, wb));
        // this lane's table entries: input codes kPer * j .. kPer * j + kPer - 1
        uint32_t tab[2] = {0, 0};
        bool redo = p.slow;
        float wc[kPer];
#pragma unroll
        for (int e = 0; e < kPer; ++e) {
            wc[e] = (float)(kPer * j + e) * s + b;
            const uint32_t o = quant_code_fast<BOUT>(wc[e], p, redo);
            const int bit = BOUT * (kPer * j + e);
            tab[bit >> 5] |= o << (bit & 31);
        }
        if (redo) {
            tab[0] = tab[1] = 0;
#pragma unroll
            for (int e = 0; e < kPer; ++e) {
                const int bit = BOUT * (kPer * j + e);
                tab[bit >> 5] |= quant_code<BOUT>(wc[e], p) << (bit & 31);
            }
        }
        // the whole table in every lane of the quad (2^BIN entries of BOUT bits: at most 64 bits)
#pragma unroll
        for (int h = 0; h < (kIn * BOUT + 31) / 32; ++h) {
            tab[h] |= dppu<0xB1>(tab[h]);
            tab[h] |= dppu<0x4E>(tab[h]);
        }
        uint32_t out[2] = {0, 0};
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            uint32_t o;
            if (kIn * BOUT <= 32) o = __builtin_amdgcn_ubfe(tab[0], t[i], BOUT);
            else o = __builtin_amdgcn_ubfe(t[i] < 32 ? tab[0] : tab[1], t[i] & 31, BOUT);   // 16 entries of 4 bits
            const int bit = BOUT * i;
            out[bit >> 5] |= o << (bit & 31);
        }
        GLOBAL_AS uint8_t *qo = dst + oout[2 * m] + (uint64_t)g * (8 * BOUT) + j * (2 * BOUT);
        if (BOUT == 4) *(GLOBAL_AS u32x2 *)qo = u32x2{out[0], out[1]};
        else *(GLOBAL_AS uint32_t *)qo = out[0];
        if (j == 0) *(GLOBAL_AS uint32_t *)(dst + oout[2 * m + 1] + (uint64_t)g * 4) = p.word;
    }
}

// blockIdx.z: matrix (gate, up, down); blockIdx.y: cold slot c (expert order[n_hot + c]);
// blockIdx.x: 4 waves of kRqGroups * 16 groups each.
template <int BOUT>
__global__ void __launch_bounds__(kRqBlock) k_requant(RequantArgs a) {
    const uint32_t c = blockIdx.y;
    const int e = a.order[a.n_hot + c];
    if ((unsigned)e >= (unsigned)a.E) return;
    const moe_expert_desc d = a.base[e];
    const int m = blockIdx.z;
    const uint32_t g0 = (blockIdx.x * (kRqBlock / 64) + (threadIdx.x >> 6)) * (16 * kRqGroups);
    if (g0 >= a.gm) return;                                // whole wave past the matrix
    const GLOBAL_AS uint8_t *src = (const GLOBAL_AS uint8_t *)d.blob;
    GLOBAL_AS uint8_t *dst = (GLOBAL_AS uint8_t *)(a.store + (uint64_t)c * a.cold_bytes);
    uint64_t oout[6];
#pragma unroll
    for (int i = 0; i < 6; ++i) oout[i] = a.pt.off[BOUT == 2 ? 0 : 1][i];
    const int lane = threadIdx.x & 63;
    if (d.bits == 2) {
        uint64_t oin[6];
#pragma unroll
        for (int i = 0; i < 6; ++i) oin[i] = a.pt.off[0][i];
        requant_wave<2, BOUT>(src, dst, oin, oout, m, g0, a.gm, lane);
    } else {
        uint64_t oin[6];
#pragma unroll
        for (int i = 0; i < 6; ++i) oin[i] = a.pt.off[1][i];
        requant_wave<4, BOUT>(src, dst, oin, oout, m, g0, a.gm, lane);
    }
}

__global__ void __launch_bounds__(256) k_retier_table(const moe_expert_desc *base, const int32_t *order, int E,
                                                     int n_hot, int cold_bits, uint64_t store, uint64_t cold_bytes,
                                                     moe_expert_desc *tiered) {
    const int r = blockIdx.x * 256 + threadIdx.x;
    if (r >= E) return;
    const int e = order[r];
    if ((unsigned)e >= (unsigned)E) return;
    moe_expert_desc d;
    if (r < n_hot) {
        d = base[e];
    } else {
        d.blob = store + (uint64_t)(r - n_hot) * cold_bytes;
        d.bits = (uint32_t)cold_bits;
        d.reserved = 0;
    }
    tiered[e] = d;
}

}  // namespace

hipError_t launch_usage(const int32_t *idx, size_t n, int E, uint32_t *counts, hipStream_t s) {
    if (n == 0) return hipSuccess;
    const size_t want = (n + (size_t)kUsageBlock * 16 - 1) / ((size_t)kUsageBlock * 16);
    const unsigned grid = (unsigned)(want < 1024 ? want : 1024);
    hipLaunchKernelGGL(k_usage, dim3(grid), dim3(kUsageBlock), (size_t)E * 4, s, idx, n, E, counts);
    return hipGetLastError();
}

hipError_t launch_hot_order(const uint32_t *counts, int E, int32_t *order, hipStream_t s) {
    int P = 1;
    while (P < E) P <<= 1;
    hipLaunchKernelGGL(k_hot_order, dim3(1), dim3(kOrderBlock), (size_t)P * 8, s, counts, E, P, order);
    return hipGetLastError();
}

hipError_t launch_retier(const RetierLaunch &r, hipStream_t s) {
    const int n_cold = r.E - r.n_hot;
    if (n_cold > 0) {
        RequantArgs a;
        a.base = r.base;
        a.order = r.order;
        a.E = r.E;
        a.n_hot = r.n_hot;
        a.store = (uint64_t)(uintptr_t)r.store;
        a.cold_bytes = r.cold_bytes;
        a.gm = (uint32_t)((uint64_t)r.I * (uint64_t)(r.H / 64));
        a.pt = plane_table(r.H, r.I);
        const uint32_t per_block = (kRqBlock / 64) * 16 * kRqGroups;
        const dim3 grid((a.gm + per_block - 1) / per_block, (unsigned)n_cold, 3);
        if (r.cold_bits == 2) hipLaunchKernelGGL(k_requant<2>, grid, dim3(kRqBlock), 0, s, a);
        else hipLaunchKernelGGL(k_requant<4>, grid, dim3(kRqBlock), 0, s, a);
        if (hipError_t e = hipGetLastError()) return e;
    }
    hipLaunchKernelGGL(k_retier_table, dim3((unsigned)((r.E + 255) / 256)), dim3(256), 0, s, r.base, r.order, r.E,
                       r.n_hot, r.cold_bits, (uint64_t)(uintptr_t)r.store, (uint64_t)r.cold_bytes, r.tiered);
    return hipGetLastError();
}

}  // namespace moe
