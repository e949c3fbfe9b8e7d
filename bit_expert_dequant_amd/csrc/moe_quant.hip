// moe_quant.hip -- quantise-from-float: real weights -> packed affine codes (group of 64).
//
// The step before packing: the pages name an MLX 4-bit affine base (tomo3141592653.github.io,
// "iPhone 17 Proで400Bパラメータ LLM を動かす「flash-moe」", section "ハイブリッド量子化") and
// the affine form w = q * scale + bias (lilting.ch, "397Bパラメータモデルを48GB MacBookで動かす
// Flash-MoE", section "Metal Compute Shaders"), not the rounding.  Per group of 64 along a row:
//   lo, hi = min and max;  scale = bf16((hi - lo) / (2^b - 1));  bias = bf16(lo);
//   code = nearest integer (ties to even) to (w - bias) / scale, clamped to [0, 2^b - 1],
//          0 when the bf16 scale is 0,
// every step in fp32 with the stored bf16 pair, so the pair dequantises the codes.
//
// k_quantize: 16 lanes per group, each with 4 consecutive weights of it; every load instruction
// of a wave reads 1 KiB (fp32) contiguous, the 16 lanes share the group's minimum and maximum
// through DPP, each writes its 4 codes (2 bytes at 4-bit, 1 at 2-bit) and the first the (scale,
// bias) pair.  HBM-bound: bytes = weights read + codes and pairs written.  (A quad of lanes per
// group with 16 weights each, 64-byte strided loads, measured 3.9 TB/s.)
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "moe_device.h"

namespace moe {
namespace {

// The matrix is a flat run of rows * cols / 64 groups of 64 consecutive weights, and both planes
// follow the same flat group order (a row's codes and pairs are contiguous, rows follow each
// other).  A wave takes 16 consecutive groups: load k (k < 4) of lane l holds the 4 weights at
// offset 256k + 4l of the wave's 1024, so every load instruction reads 1 KiB (fp32) or 512 B
// (bf16) contiguous, and the 16 lanes of a DPP row hold group 4k + l/16 between them.
template <int BITS, int DT>
__global__ void __launch_bounds__(256) k_quantize(QuantLaunch a) {
    const size_t ng = (size_t)a.rows * (a.cols / 64);
    const int lane = threadIdx.x & 63, r16 = lane >> 4, c16 = lane & 15;
    const size_t g0 = ((size_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * 16;
    float v[4][4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const size_t gk = min(g0 + 4 * k + r16, ng - 1);        // clamped; results past ng unused
        const size_t e = gk * 64 + 4 * c16;
        if (DT == MOE_BF16) {
            const u32x2 x = __builtin_nontemporal_load((const GLOBAL_AS u32x2 *)((const uint16_t *)a.w + e));
            v[k][0] = __uint_as_float(x.x << 16);
            v[k][1] = __uint_as_float(x.x & 0xFFFF0000u);
            v[k][2] = __uint_as_float(x.y << 16);
            v[k][3] = __uint_as_float(x.y & 0xFFFF0000u);
        } else {
            const u32x4 x = __builtin_nontemporal_load((const GLOBAL_AS u32x4 *)((const float *)a.w + e));
#pragma unroll
            for (int j = 0; j < 4; ++j) v[k][j] = __uint_as_float(x[j]);
        }
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const size_t gk = g0 + 4 * k + r16;
        float lo = fminf(fminf(v[k][0], v[k][1]), fminf(v[k][2], v[k][3]));
        float hi = fmaxf(fmaxf(v[k][0], v[k][1]), fmaxf(v[k][2], v[k][3]));
        // minimum and maximum over the 16 lanes of the DPP row (the group's 64 weights)
        lo = fminf(lo, dppf<0xB1>(lo));     // quad_perm [1,0,3,2]
        hi = fmaxf(hi, dppf<0xB1>(hi));
        lo = fminf(lo, dppf<0x4E>(lo));     // quad_perm [2,3,0,1]
        hi = fmaxf(hi, dppf<0x4E>(hi));
        lo = fminf(lo, dppf<0x141>(lo));    // row_half_mirror
        hi = fmaxf(hi, dppf<0x141>(hi));
        lo = fminf(lo, dppf<0x140>(lo));    // row_mirror
        hi = fmaxf(hi, dppf<0x140>(hi));
        if (gk >= ng) continue;
        const QPair p = quant_pair<BITS>(lo, hi);
        uint32_t packed = 0;
        bool redo = p.slow;
#pragma unroll
        for (int j = 0; j < 4; ++j) packed |= quant_code_fast<BITS>(v[k][j], p, redo) << (j * BITS);
        if (redo) {
            packed = 0;
#pragma unroll
            for (int j = 0; j < 4; ++j) packed |= quant_code<BITS>(v[k][j], p) << (j * BITS);
        }
        if (BITS == 4) *(GLOBAL_AS uint16_t *)(a.codes + gk * 32 + 2 * c16) = (uint16_t)packed;
        else *(GLOBAL_AS uint8_t *)(a.codes + gk * 16 + c16) = (uint8_t)packed;
        if (c16 == 0) *(GLOBAL_AS uint32_t *)(a.sb + 2 * gk) = p.word;   // scale, then bias
    }
}

}  // namespace

hipError_t launch_quantize(const QuantLaunch &a, hipStream_t s) {
    const size_t groups = (size_t)a.rows * (a.cols / 64);
    const dim3 grid((unsigned)((groups + 63) / 64));           // 16 groups per wave, 4 waves
    if (a.bits == 2) {
        if (a.w_dtype == MOE_BF16) hipLaunchKernelGGL((k_quantize<2, MOE_BF16>), grid, dim3(256), 0, s, a);
        else hipLaunchKernelGGL((k_quantize<2, MOE_F32>), grid, dim3(256), 0, s, a);
    } else {
        if (a.w_dtype == MOE_BF16) hipLaunchKernelGGL((k_quantize<4, MOE_BF16>), grid, dim3(256), 0, s, a);
        else hipLaunchKernelGGL((k_quantize<4, MOE_F32>), grid, dim3(256), 0, s, a);
    }
    return hipGetLastError();
}

}  // namespace moe
