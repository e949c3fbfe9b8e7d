// moe_device.h -- device-side building blocks shared by the decode kernels (moe_decode.hip) and the
// router + gate/up layer kernel (moe_layer.hip): activation staging, in-register dequant dot
// products, the wave top-K, and the per-unit load/compute steps of the gate/up and down phases.
// Everything lives in an unnamed namespace, so each translation unit gets its own copy.
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <type_traits>

#include "moe_internal.h"

namespace moe {
namespace {

#define GLOBAL_AS __attribute__((address_space(1)))
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kBlock = 256;               // threads per workgroup (4 wavefronts)
constexpr int kWaves = kBlock / 64;
constexpr int kTabMax = 512;              // experts whose descriptors are prefetched into LDS

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c,
                                           false);
}
__device__ __forceinline__ uint32_t bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}
__device__ __forceinline__ float bf16_f32(uint32_t b) { return __uint_as_float(b << 16); }

// Quantise-from-float of one group of 64 (moe_quantize_matrix, and the requantisation of a cold
// expert): the (scale, bias) pair from the group's minimum and maximum, scale = bf16((hi - lo) /
// (2^BITS - 1)) and bias = bf16(lo), then a weight's code under the stored pair: the nearest
// integer (ties to even) to the fp32 quotient (w - bias) / scale under IEEE division, clamped to
// [0, 2^BITS - 1], 0 when the scale is 0.
//
// quant_code is that definition.  quant_code_fast takes the quotient as (w - bias) * rcp(scale)
// instead (v_rcp_f32, within 1 ulp): for |quotient| < 32 it is within 2^-17 of the IEEE quotient,
// so both round to the same integer unless the fast one lies within 2^-15 of a half-integer; at
// |quotient| >= 32 every code clamps to 0 or 2^BITS - 1 either way.  A lane that meets such a near
// tie, or a scale outside [2^-64, 2^64] (where the reciprocal may leave the normal range), sets
// `redo` and recomputes its codes with quant_code, so the codes equal the definition's.
struct QPair {
    uint32_t word;      // scale bits | bias bits << 16, as the sb plane stores it
    float s, b;
    float r;            // rcp(s), or 0 when s is 0 or outside [2^-64, 2^64]
    bool slow;          // s is nonzero and outside [2^-64, 2^64]
};
template <int BITS>
__device__ __forceinline__ QPair quant_pair(float lo, float hi) {
    constexpr float kQMax = (float)((1 << BITS) - 1);
    const uint32_t sbits = bf16_rne((hi - lo) / kQMax), bbits = bf16_rne(lo);
    const float s = bf16_f32(sbits);
    const bool fast = s >= 0x1p-64f && s <= 0x1p64f;
    return {sbits | (bbits << 16), s, bf16_f32(bbits), fast ? __builtin_amdgcn_rcpf(s) : 0.f, !fast && s != 0.f};
}
template <int BITS>
__device__ __forceinline__ uint32_t quant_code(float w, const QPair &p) {
    constexpr float kQMax = (float)((1 << BITS) - 1);
    return p.s > 0.f ? (uint32_t)fminf(fmaxf(rintf((w - p.b) / p.s), 0.f), kQMax) : 0u;
}
template <int BITS>
__device__ __forceinline__ uint32_t quant_code_fast(float w, const QPair &p, bool &redo) {
    constexpr float kQMax = (float)((1 << BITS) - 1);
    const float q = (w - p.b) * p.r;
    const float n = rintf(q);
    redo |= fabsf(q - n) > 0.5f - 0x1p-15f;           // |q - n| <= 1/2: within 2^-15 of a half-integer
    return (uint32_t)fminf(fmaxf(n, 0.f), kQMax);
}
__device__ __forceinline__ float load_act(const void *x, int dtype, size_t i) {
    return dtype == MOE_BF16 ? bf16_f32(((const uint16_t *)x)[i]) : ((const float *)x)[i];
}
__device__ __forceinline__ float silu(float z) { return z / (1.0f + expf(-z)); }
// silu with the hardware exponential (2^x) and reciprocal, about 2^-21 relative error: for kernels
// that evaluate it once per row and token, where the IEEE division's dozen instructions show.
__device__ __forceinline__ float silu_fast(float z) {
    return z * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-z * 1.4426950408889634f));
}

// Sum over aligned groups of GS lanes (GS a power of two <= 64); every lane gets its group's sum.
// Butterfly in registers: quad permutes and row mirrors (DPP) inside 16-lane rows, then the gfx950
// row swaps (v_permlane16/32_swap) across rows.  After the steps below GS, every lane holds the sum
// of its aligned group of GS lanes, and both partners of a step add the same two values, so all
// lanes of a group hold identical bits.  The group size is a compile-time constant so that each
// step is one DPP-fused add; group_sum dispatches a uniform run-time size to it.
template <int CTRL>
__device__ __forceinline__ float dppf(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true));
}
template <int GS>
__device__ __forceinline__ float group_sum_c(float v) {
    if constexpr (GS > 1) v += dppf<0xB1>(v);      // quad_perm [1,0,3,2]
    if constexpr (GS > 2) v += dppf<0x4E>(v);      // quad_perm [2,3,0,1]
    if constexpr (GS > 4) v += dppf<0x141>(v);     // row_half_mirror
    if constexpr (GS > 8) v += dppf<0x140>(v);     // row_mirror
    if constexpr (GS > 16) {
        const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
        v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    }
    if constexpr (GS > 32) {
        const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
        v = __uint_as_float(b[0]) + __uint_as_float(b[1]);
    }
    return v;
}
__device__ __forceinline__ float group_sum(float v, int gs) {
    switch (gs) {
        case 1: return v;
        case 2: return group_sum_c<2>(v);
        case 4: return group_sum_c<4>(v);
        case 8: return group_sum_c<8>(v);
        case 16: return group_sum_c<16>(v);
        case 32: return group_sum_c<32>(v);
        default: return group_sum_c<64>(v);
    }
}
// Group sums of two values at once (GS = 32 or 64): the first butterfly step exchanges a's upper
// half-group for b's lower one, so afterwards the lower half of every group carries a and the
// upper half b, and the remaining steps reduce both together.  Lane l receives the sum of a over
// its group when l % GS < GS / 2, else that of b.
template <int GS>
__device__ __forceinline__ float pair_sum(float a, float b) {
    static_assert(GS == 32 || GS == 64, "pair_sum: groups of 32 or 64 lanes");
    if constexpr (GS == 64) {
        const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
        return group_sum_c<32>(__uint_as_float(p[0]) + __uint_as_float(p[1]));
    } else {
        const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
        return group_sum_c<16>(__uint_as_float(p[0]) + __uint_as_float(p[1]));
    }
}

__device__ __forceinline__ float block_sum(float v, float *red) {
    v = group_sum(v, 64);
    const int w = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) red[w] = v;
    __syncthreads();
    float t = 0.f;
    for (int i = 0; i < (int)(blockDim.x >> 6); ++i) t += red[i];
    __syncthreads();
    return t;
}

__host__ __device__ __forceinline__ int next_pow2(int v) {
    int p = 1;
    while (p < v) p <<= 1;
    return p;
}
__host__ __device__ __forceinline__ size_t round256(size_t v) { return (v + 255) & ~(size_t)255; }

// Selected expert, packed for the down kernel: blob address (256-byte aligned) | code width.
__device__ __forceinline__ uint64_t pack_sel(uint64_t blob, uint32_t bits) { return blob ? (blob | (bits == 2 ? 2u : 4u)) : 0; }
__device__ __forceinline__ uint64_t sel_blob(uint64_t s) { return s & ~(uint64_t)255; }
__device__ __forceinline__ int sel_bits(uint64_t s) { return (int)(s & 255u) == 2 ? 2 : 4; }

// Packed selection of expert e (0 for an index outside [0, E)).
__device__ __forceinline__ uint64_t lookup_sel(int e, int E, bool use_tab, const uint64_t *tab,
                                               const moe_expert_desc *experts) {
    if (e < 0 || e >= E) return 0;
    if (use_tab) return tab[e];
    const moe_expert_desc d = experts[e];
    return pack_sel(d.blob, d.bits);
}

// --------------------------------------------------------------------------- activation staging
// An activation vector is held in LDS as 16-bit fixed point per 32-column slot: column c of slot s
// is X_c * sx_s, with X_c an integer in [-kXMax, kXMax] and sx_s = (largest |x| of the slot) / kXMax,
// plus the slot's exact fp32 sum of x for the bias term.  X is kept as four balanced base-16 digits,
// X = d0 + 16 d1 + 256 d2 + 4096 d3 with every d_p in [-8, 7] (kXMax is the largest X four such
// digits reach), and digit p of eight columns is one dword of 4-bit two's-complement nibbles.  A
// dword of eight weight codes then meets one such "plane" dword per v_dot8_i32_i4, which does eight
// multiply-adds in the time a bf16 dot2 does two.
//
// Slot layout (kSlotDw dwords): plane p occupies dwords 4q .. 4q+3, q = p ^ plane_swz(slot) (below).
// 4-bit order: dword 4p + j (p the plane, unswizzled) holds
// columns 8j .. 8j+7 (nibble n = column 8j+n), matching code dword j of the slot.  2-bit order: dword
// 4p + 2j + e holds columns 16j + 2n + e (n < 8), matching the even (e = 0) and odd (e = 1) codes of
// code dword j once they are spread to nibbles.  A thread stages one 16-column chunk m = 2s + h;
// in both orders it owns dwords 4p + 2h and 4p + 2h + 1 of every plane.
//
// Precision: a column's rounding error is at most sx/2, 2^-16 of the slot's largest |x|.
//
// LDS banks.  A lane reads its slot's four planes as 16-byte loads, and neighbouring lanes own
// neighbouring slots, 64 bytes apart; stored in plane order every lane of a load would hit the same
// four banks.  Plane p of slot s therefore sits at plane position p ^ plane_swz(s), which spreads the
// 16-byte loads of any 8 (32 banks) or 16 (64 banks) consecutive slots over distinct banks.
constexpr int kSlotDw = 16;
constexpr float kXMax = 30583.f;
__device__ __forceinline__ int plane_swz(int s) { return ((s >> 1) ^ (s >> 2)) & 3; }

// A chunk of 16 consecutive activations (32 bytes of bf16 or 64 of fp32) is loaded in two steps:
// issue_chunk16 starts four 16-byte loads with no data-dependent branch (bf16 repeats its second
// load), chunk16_f32 converts once the data is needed.  Keeping the conversion out of the issue
// step lets every chunk a thread needs be in flight at once instead of one memory latency each.
struct Chunk16 {
    u32x4 q[4];
};
__device__ __forceinline__ void issue_chunk16(const void *x, int dtype, int m, Chunk16 &c) {
    const int cb = dtype == MOE_BF16 ? 32 : 64;
    const GLOBAL_AS uint8_t *p = (const GLOBAL_AS uint8_t *)x + (size_t)m * cb;
#pragma unroll
    for (int i = 0; i < 4; ++i) c.q[i] = *(const GLOBAL_AS u32x4 *)(p + min(16 * i, cb - 16));
}
__device__ __forceinline__ void chunk16_f32(const Chunk16 &c, int dtype, float v[16]) {
    if (dtype == MOE_BF16) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            v[2 * j] = bf16_f32(c.q[0][j] & 0xFFFFu); v[2 * j + 1] = bf16_f32(c.q[0][j] >> 16);
            v[8 + 2 * j] = bf16_f32(c.q[1][j] & 0xFFFFu); v[8 + 2 * j + 1] = bf16_f32(c.q[1][j] >> 16);
        }
    } else {
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int j = 0; j < 4; ++j) v[4 * q + j] = __uint_as_float(c.q[q][j]);
    }
}

// Plane dwords of eight columns.  y[n] = X_n + 0x8888, whose hex digits are the balanced digits
// plus 8; out[p] nibble n = digit p of column n in two's complement (hex digit XOR 8).
__device__ __forceinline__ void planes8(const uint32_t (&y)[8], uint32_t (&out)[4]) {
    uint32_t P[4];
#pragma unroll
    for (int a = 0; a < 4; ++a) P[a] = y[a] | (y[a + 4] << 16);   // columns a and a+4
    // digits 0/1 (low byte of each column) and 2/3 (high byte) of the even and odd columns:
    // byte i of e01 = low byte of column 2i, etc.
    const uint32_t e01 = __builtin_amdgcn_perm(P[2], P[0], 0x06020400u);
    const uint32_t o01 = __builtin_amdgcn_perm(P[3], P[1], 0x06020400u);
    const uint32_t e23 = __builtin_amdgcn_perm(P[2], P[0], 0x07030501u);
    const uint32_t o23 = __builtin_amdgcn_perm(P[3], P[1], 0x07030501u);
    constexpr uint32_t lo = 0x0F0F0F0Fu;
    out[0] = ((e01 & lo) | ((o01 << 4) & ~lo)) ^ 0x88888888u;
    out[1] = (((e01 >> 4) & lo) | (o01 & ~lo)) ^ 0x88888888u;
    out[2] = ((e23 & lo) | ((o23 << 4) & ~lo)) ^ 0x88888888u;
    out[3] = (((e23 >> 4) & lo) | (o23 & ~lo)) ^ 0x88888888u;
}

// Stages chunk m (columns v[0..15]) into the 4-bit order at d4 and/or the 2-bit order at d2 (a
// null pointer skips that order) and, from the slot's even chunk, writes xs[s] = {sx, sum of x}.
// Every lane of the wave calls it together: the slot's two chunks sit in lanes l and l^1 and meet
// through DPP.  A lane with !valid takes part in the exchange only.
__device__ __forceinline__ void stage_chunk(int m, bool valid, const float (&v)[16], uint32_t *d4, uint32_t *d2,
                                            float2 *xs) {
    float mx = 0.f, sum = 0.f;
    if (valid) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            mx = fmaxf(mx, fabsf(v[i]));
            sum += v[i];
        }
    }
    mx = fmaxf(mx, dppf<0xB1>(mx));
    sum += dppf<0xB1>(sum);
    if (!valid) return;
    int ex = 0;
    const float mant = frexpf(mx, &ex);                    // mx = mant * 2^ex, mant in [0.5, 1)
    const float f = mx > 0.f ? kXMax / mant : 0.f;         // X = round(x * 2^-ex * f)
    uint32_t y[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        // 1.5 * 2^23 + X rounds to the nearest integer in one fma; its bits are 0x4B400000 + X
        const float t = fmaf(ldexpf(v[i], -ex), f, 12582912.f);
        y[i] = __float_as_uint(t) - (0x4B400000u - 0x8888u);
    }
    const int h = m & 1;
    const int swz = plane_swz(m >> 1);
    uint32_t *base4 = d4 ? d4 + (m >> 1) * kSlotDw + 2 * h : nullptr;
    uint32_t *base2 = d2 ? d2 + (m >> 1) * kSlotDw + 2 * h : nullptr;
    if (base4) {
        uint32_t a[8], b[8], pa[4], pb[4];
#pragma unroll
        for (int n = 0; n < 8; ++n) { a[n] = y[n]; b[n] = y[8 + n]; }
        planes8(a, pa);
        planes8(b, pb);
#pragma unroll
        for (int p = 0; p < 4; ++p) *(u32x2 *)(base4 + 4 * (p ^ swz)) = u32x2{pa[p], pb[p]};
    }
    if (base2) {
        uint32_t a[8], b[8], pa[4], pb[4];
#pragma unroll
        for (int n = 0; n < 8; ++n) { a[n] = y[2 * n]; b[n] = y[2 * n + 1]; }
        planes8(a, pa);
        planes8(b, pb);
#pragma unroll
        for (int p = 0; p < 4; ++p) *(u32x2 *)(base2 + 4 * (p ^ swz)) = u32x2{pa[p], pb[p]};
    }
    if (!h) xs[m >> 1] = float2{mant > 0.f ? ldexpf(mant / kXMax, ex) : 0.f, sum};
}

// One code width's view of a staged activation vector.
struct ActView {
    const uint32_t *d;   // [cols/32][kSlotDw] digit planes in that width's order
    const float2 *xs;    // [cols/32] {sx, sum of x}
};

// Loads slot s of a view into registers, for a lane whose slot exists.
__device__ __forceinline__ void load_act_slot_full(const ActView &av, int s, uint32_t (&D)[kSlotDw], float2 &xs) {
    const int swz = plane_swz(s);
#pragma unroll
    for (int i = 0; i < kSlotDw; i += 4) {
        const u32x4 d = *(const u32x4 *)(av.d + s * kSlotDw + 4 * ((i >> 2) ^ swz));
        D[i] = d.x; D[i + 1] = d.y; D[i + 2] = d.z; D[i + 3] = d.w;
    }
    xs = av.xs[s];
}
// Loads slot ss of a view into registers (zeros when !ok: an idle lane's slot adds nothing).
__device__ __forceinline__ void load_act_slot(const ActView &av, int ss, bool ok, uint32_t (&D)[kSlotDw], float2 &xs) {
    const int s = ok ? ss : 0;
    const int swz = plane_swz(s);
#pragma unroll
    for (int i = 0; i < kSlotDw; i += 4) {
        const u32x4 d = *(const u32x4 *)(av.d + s * kSlotDw + 4 * ((i >> 2) ^ swz));
        D[i] = ok ? d.x : 0u; D[i + 1] = ok ? d.y : 0u; D[i + 2] = ok ? d.z : 0u; D[i + 3] = ok ? d.w : 0u;
    }
    const float2 t = av.xs[s];
    xs = ok ? t : float2{0.f, 0.f};
}

// --------------------------------------------------------------------------- slot dot products
// s * sum(q x) + b * sum(x) over one slot, given its codes, (scale, bias) dword and staged
// activation.  4-bit codes enter v_dot8_i32_i4 as q - 8 (the code XOR 8 read as a signed nibble),
// so the bias becomes b + 8 s; 2-bit codes spread to nibbles are already in [0, 3].  Per plane
// the integer sums are at most 32 * 8 * 8, so the combined sum is exact in int32 and in fp32.
// The digit planes combine in Horner form, acc = ((A3 * 16 + A2) * 16 + A1) * 16 + A0, over CH
// dependency chains: CH = 4 gives each plane its own register (four independent chains of four dot
// products: with one or two waves per SIMD the chain latency, not the issue rate, bounds a decode
// unit); CH = 1 runs one chain from the top plane down, scaling by 16 between planes, and CH = 2 two
// chains (A3, A2 and A1, A0) -- fewer instructions (no zeroed accumulator and no combination per
// plane) where many tokens' slots interleave.  The integer sum is the same in every form.
// The token-independent part of a slot: its code dwords as v_dot8_i32_i4 operands and its scale and
// folded bias.  Kernels that meet one loaded slot with several staged rows compute it once per slot.
struct SlotOps {
    int c[4];
    float s, bb;
};
template <int BITS>
__device__ __forceinline__ SlotOps slot_ops(const u32x4 q, uint32_t sb) {
    SlotOps o;
    if (BITS == 4) {
#pragma unroll
        for (int j = 0; j < 4; ++j) o.c[j] = (int)(q[j] ^ 0x88888888u);
    } else {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            o.c[2 * j] = (int)(q[j] & 0x33333333u);
            o.c[2 * j + 1] = (int)((q[j] >> 2) & 0x33333333u);
        }
    }
    o.s = bf16_f32(sb & 0xFFFFu);
    const float b = bf16_f32(sb >> 16);
    o.bb = BITS == 4 ? fmaf(8.f, o.s, b) : b;
    return o;
}
template <int CH = 4>
__device__ __forceinline__ float slot_dot_ops(const SlotOps &o, const uint32_t (&D)[kSlotDw], float2 xs) {
    static_assert(CH == 1 || CH == 2 || CH == 4, "one, two or four chains");
    // the four dot products of plane p added to acc (2-bit: the two nibble spreads of each code dword
    // meet consecutive plane dwords)
    auto plane = [&](int p, int acc) {
#pragma unroll
        for (int j = 0; j < 4; ++j) acc = __builtin_amdgcn_sdot8(o.c[j], (int)D[4 * p + j], acc, false);
        return acc;
    };
    int acc;
    if constexpr (CH == 4) {
        const int a0 = plane(0, 0), a1 = plane(1, 0), a2 = plane(2, 0), a3 = plane(3, 0);
        acc = ((a3 * 16 + a2) * 16 + a1) * 16 + a0;
    } else if constexpr (CH == 2) {
        const int hi = plane(2, plane(3, 0) * 16), lo = plane(0, plane(1, 0) * 16);
        acc = hi * 256 + lo;
    } else {
        acc = plane(0, plane(1, plane(2, plane(3, 0) * 16) * 16) * 16);
    }
    return fmaf(o.s * xs.x, (float)acc, o.bb * xs.y);
}
// The same sum from the loaded dwords (one staged row per loaded slot: the decode kernels).
template <int BITS, int CH = 4>
__device__ __forceinline__ float slot_dot(const u32x4 q, const uint32_t (&D)[kSlotDw], uint32_t sb, float2 xs) {
    return slot_dot_ops<CH>(slot_ops<BITS>(q, sb), D, xs);
}
// slot_dot written out, with the scale and bias decoded after the dot products: the same value.  The
// per-token gate/up kernel uses it -- through slot_ops its register count grows from 128 to 130 and its
// occupancy from four waves per SIMD to three (multi-token calls 30.6 vs 33.2 us at 4 tokens), while
// the two-launch decode kernels are faster through slot_ops (15.64 vs 15.79 us per step).
template <int BITS, int CH = 4>
__device__ __forceinline__ float slot_dot_late(const u32x4 q, const uint32_t (&D)[kSlotDw], uint32_t sb, float2 xs) {
    static_assert(CH == 1 || CH == 2 || CH == 4, "one, two or four chains");
    int c[4];
    if (BITS == 4) {
#pragma unroll
        for (int j = 0; j < 4; ++j) c[j] = (int)(q[j] ^ 0x88888888u);
    } else {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            c[2 * j] = (int)(q[j] & 0x33333333u);
            c[2 * j + 1] = (int)((q[j] >> 2) & 0x33333333u);
        }
    }
    auto plane = [&](int p, int acc) {
#pragma unroll
        for (int j = 0; j < 4; ++j) acc = __builtin_amdgcn_sdot8(c[j], (int)D[4 * p + j], acc, false);
        return acc;
    };
    int acc;
    if constexpr (CH == 4) {
        const int a0 = plane(0, 0), a1 = plane(1, 0), a2 = plane(2, 0), a3 = plane(3, 0);
        acc = ((a3 * 16 + a2) * 16 + a1) * 16 + a0;
    } else if constexpr (CH == 2) {
        const int hi = plane(2, plane(3, 0) * 16), lo = plane(0, plane(1, 0) * 16);
        acc = hi * 256 + lo;
    } else {
        acc = plane(0, plane(1, plane(2, plane(3, 0) * 16) * 16) * 16);
    }
    const float s = bf16_f32(sb & 0xFFFFu), b = bf16_f32(sb >> 16);
    const float bb = BITS == 4 ? fmaf(8.f, s, b) : b;
    return fmaf(s * xs.x, (float)acc, bb * xs.y);
}

typedef const GLOBAL_AS uint8_t *gbytes;
typedef const GLOBAL_AS uint32_t *gwords;

// Weight bytes are read once per step, so they are loaded non-temporally: streaming them must not
// push the kernels' code, the activations and the descriptor tables out of the L2.
template <int BITS>
__device__ __forceinline__ u32x4 load_slot(gbytes row, int slot) {
    if (BITS == 4) return __builtin_nontemporal_load((const GLOBAL_AS u32x4 *)(row + (size_t)slot * 16));
    const u32x2 v = __builtin_nontemporal_load((const GLOBAL_AS u32x2 *)(row + (size_t)slot * 8));
    return u32x4{v.x, v.y, 0u, 0u};
}

// Lane geometry for rows of `cols` inputs.
struct Geo {
    int spr;    // slots per row
    int gsz;    // lanes per row group
    int rpi;    // rows per wave instruction
    int lrow;   // this lane's row within the instruction
    int lsl;    // this lane's first slot
};
__device__ __forceinline__ Geo make_geo(const RowGeo &r) {
    Geo g;
    const int lane = threadIdx.x & 63;
    g.spr = r.spr;
    g.gsz = 1 << r.gsh;
    g.rpi = r.rpi;
    g.lrow = lane >> r.gsh;
    g.lsl = lane & (g.gsz - 1);
    return g;
}
// u / nblk for a unit index u < 2^16 (see RowGeo).
__device__ __forceinline__ int blk_of(int u, const RowGeo &r) {
    return (int)(((uint64_t)(uint32_t)u * r.blk_mul) >> 32);
}

// Weight planes are read through global (address space 1) pointers: the blob addresses come from
// the descriptor table as integers, and generic pointers would turn every load into a flat load.
struct Planes {
    gbytes q; gwords sb;
};
__device__ __forceinline__ void expert_planes(uint64_t blob_addr, int bits, const PlaneTable &t, Planes p[3]) {
    gbytes blob = (gbytes)blob_addr;
    const uint64_t *o = t.off[bits == 2 ? 0 : 1];
#pragma unroll
    for (int m = 0; m < 3; ++m) {
        p[m].q = blob + o[2 * m];
        p[m].sb = (gwords)(blob + o[2 * m + 1]);
    }
}

// --------------------------------------------------------------------------- top-K (one wave)
// Largest K logits, descending, equal values -> lower index; NaN counts as -inf.  The weights are
// the softmax over the selected logits, which equals the softmax over all E renormalised.
//
// A logit is compared through an order-preserving 32-bit key (its fp32 bits with the sign folded;
// -0 is first canonicalised to +0 so that equal floats give equal keys); key 0 marks an absent
// expert and is below every real key.  The experts are laid out lane-major: lane l holds experts
// NP*l .. NP*l+NP-1 in registers, so among lanes whose best keys tie the lowest lane holds the lowest
// index, and inside a lane the lowest slot does.  Each lane keeps its best two untaken keys.  A
// round takes the wave maximum of the lane heads with DPP inside 16-lane rows and the gfx950 row
// swaps across rows (every lane gets it, no scalar round trip), finds the lowest lane holding it
// with one ballot, and promotes that lane's second key.  A lane that wins twice recomputes its
// two best untaken keys.  The winner records its slot in a per-round bit field; lane k reads the
// field of round k's winner once, after the last round.  Everything stays in registers: a round
// is a short dependent chain, which is what bounds a single wave here.
__device__ __forceinline__ uint32_t logit_key(float v) {
    v = (v != v) ? -INFINITY : v + 0.0f;
    const uint32_t u = __float_as_uint(v);
    return u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);
}
__device__ __forceinline__ float key_logit(uint32_t o) {
    return __uint_as_float((o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o);
}
template <int CTRL>
__device__ __forceinline__ uint32_t dpp0(uint32_t v) {   // DPP move; lanes without a source read 0
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, true);
}
// Wave-wide maximum, returned in every lane.
__device__ __forceinline__ uint32_t wave_max_all(uint32_t v) {
    v = max(v, dpp0<0xB1>(v));      // quad_perm [1,0,3,2]
    v = max(v, dpp0<0x4E>(v));      // quad_perm [2,3,0,1]
    v = max(v, dpp0<0x141>(v));     // row_half_mirror
    v = max(v, dpp0<0x140>(v));     // row_mirror: the 16-lane row maximum
    const auto a = __builtin_amdgcn_permlane16_swap(v, v, false, false);    // rows 0<->1, 2<->3
    v = max(a[0], a[1]);
    const auto b = __builtin_amdgcn_permlane32_swap(v, v, false, false);    // halves
    return max(b[0], b[1]);
}
// The two best keys of this lane that are not in `taken` (ties: lower slot first).  Pairwise
// tree: list A always comes from lower slots than list B.
struct Top2 {
    uint32_t h1, h2;
    int s1, s2;
};
__device__ __forceinline__ Top2 top2_merge(const Top2 &A, const Top2 &B) {
    const bool bw = B.h1 > A.h1;
    Top2 r;
    r.h1 = bw ? B.h1 : A.h1;
    r.s1 = bw ? B.s1 : A.s1;
    const bool a2 = bw ? (A.h1 >= B.h2) : (A.h2 >= B.h1);   // second: A's candidate wins ties
    r.h2 = bw ? (a2 ? A.h1 : B.h2) : (a2 ? A.h2 : B.h1);
    r.s2 = bw ? (a2 ? A.s1 : B.s2) : (a2 ? A.s2 : B.s1);
    return r;
}
template <int N>
__device__ __forceinline__ Top2 top2_range(const uint32_t *key, uint32_t taken, int t0) {
    if constexpr (N == 1) {
        return Top2{((taken >> t0) & 1u) ? 0u : key[t0], 0u, t0, t0};
    } else {
        return top2_merge(top2_range<N / 2>(key, taken, t0), top2_range<N / 2>(key, taken, t0 + N / 2));
    }
}

// The K rounds for few keys per lane (NP <= 8): each lane keeps its best untaken key; a round takes
// the wave maximum, the lowest lane holding it (one ballot), and that lane drops the key and takes
// its next best -- with eight keys or fewer a lane recomputes that from scratch in a handful of
// compares, branch-free, which costs less per round than keeping a second-best list.  Winners are
// read back as scalars (readlane), so no cross-lane shuffle is needed at the end.
template <int NP>
__device__ __forceinline__ void wave_topk_lean(const uint32_t (&key_in)[NP], int K, uint32_t &my_key, int &my_pos) {
    const int lane = threadIdx.x & 63;
    uint32_t key[NP];
#pragma unroll
    for (int t = 0; t < NP; ++t) key[t] = key_in[t];
    uint32_t bk = key[0];
    int bs = 0;
#pragma unroll
    for (int t = 1; t < NP; ++t) {
        const bool gt = key[t] > bk;
        bk = gt ? key[t] : bk;
        bs = gt ? t : bs;
    }
    my_key = 0;
    my_pos = 0;
    for (int k = 0; k < K; ++k) {
        const uint32_t m = wave_max_all(bk);
        const int wl = __ffsll((unsigned long long)__ballot(bk == m)) - 1;
        const int ws = __builtin_amdgcn_readlane(bs, wl);
        my_key = lane == k ? m : my_key;
        my_pos = lane == k ? wl * NP + ws : my_pos;
        if (NP > 1) {
            const bool win = lane == wl;
#pragma unroll
            for (int t = 0; t < NP; ++t) key[t] = (win && t == ws) ? 0u : key[t];
            uint32_t nk = key[0];
            int ns = 0;
#pragma unroll
            for (int t = 1; t < NP; ++t) {
                const bool gt = key[t] > nk;
                nk = gt ? key[t] : nk;
                ns = gt ? t : ns;
            }
            bk = win ? nk : bk;
            bs = win ? ns : bs;
        } else {
            bk = lane == wl ? 0u : bk;
        }
    }
}

// The K rounds.  `key`: this lane's NP keys (positions NP*lane + t of the wave).  Lane k < K
// returns the k-th largest key and its position (equal keys: lower position first).
template <int NP>
__device__ __forceinline__ void wave_topk_core(const uint32_t (&key)[NP], int K, uint32_t &my_key, int &my_pos) {
    if constexpr (NP <= 8) {
        wave_topk_lean<NP>(key, K, my_key, my_pos);
        return;
    }
    constexpr int FW = NP <= 8 ? 3 : 5;                            // bits per recorded slot
    typedef typename std::conditional<NP <= 8, uint32_t, uint64_t>::type rec_t;
    const int lane = threadIdx.x & 63;
    Top2 c = top2_range<NP>(key, 0u, 0);
    uint32_t taken = 0;
    my_key = 0;
    rec_t rec = 0;
    int my_wl = 0;
    uint64_t second_stale = 0;     // lanes whose second key was promoted and not yet recomputed
    for (int k = 0; k < K; ++k) {
        const uint32_t m = wave_max_all(c.h1);
        const int wl = __ffsll((unsigned long long)__ballot(c.h1 == m)) - 1;
        const bool me = lane == wl;
        rec |= me ? (rec_t)c.s1 << (FW * k) : (rec_t)0;
        taken |= me ? 1u << c.s1 : 0u;
        my_key = lane == k ? m : my_key;
        my_wl = lane == k ? wl : my_wl;
        if (NP > 2 && ((second_stale >> wl) & 1ull)) {
            const Top2 r = top2_range<NP>(key, taken, 0);
            c.h1 = me ? r.h1 : c.h1; c.s1 = me ? r.s1 : c.s1;
            c.h2 = me ? r.h2 : c.h2; c.s2 = me ? r.s2 : c.s2;
            second_stale &= ~(1ull << wl);
        } else {
            // with two keys a lane holds no third: after its second win it offers key 0
            c.h1 = me ? c.h2 : c.h1;
            c.s1 = me ? c.s2 : c.s1;
            if (NP <= 2) c.h2 = me ? 0u : c.h2;
            second_stale |= 1ull << wl;
        }
    }
    rec_t r;
    if constexpr (NP == 1) {
        r = 0;
    } else if constexpr (NP <= 8) {
        r = (rec_t)__shfl((int)rec, my_wl);
    } else {
        r = (rec_t)(uint32_t)__shfl((int)(uint32_t)rec, my_wl) | ((rec_t)(uint32_t)__shfl((int)(uint32_t)(rec >> 32), my_wl) << 32);
    }
    const int slot = lane < K ? (int)((r >> (FW * lane)) & ((1u << FW) - 1)) : 0;
    my_pos = my_wl * NP + slot;
}

// Routing weight of lane k < K (0 elsewhere): the softmax over the K selected logits,
// max-subtracted (the largest is lane 0's), summed over lanes 0..7.
__device__ __forceinline__ float topk_weight(uint32_t my_key, int K) {
    const int lane = threadIdx.x & 63;
    const float val = key_logit(my_key), top0 = key_logit(__builtin_amdgcn_readfirstlane(my_key));
    const float ex = lane < K ? (top0 > -INFINITY ? expf(val - top0) : 1.f) : 0.f;
    float z = ex;
    z += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(z), 0xB1, 0xF, 0xF, true));
    z += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(z), 0x4E, 0xF, 0xF, true));
    z += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(z), 0x141, 0xF, 0xF, true));
    return ex / z;
}

// One wave: lane k < K returns selection k (expert NP*lane + t layout) and its weight.
template <int NP>
__device__ __forceinline__ void wave_topk(const uint32_t (&key)[NP], int K, int &my_idx, float &my_w) {
    uint32_t mk;
    wave_topk_core<NP>(key, K, mk, my_idx);
    my_w = topk_weight(mk, K);
}

// A whole workgroup (kWaves waves, every wave gets the result): wave w takes experts
// [w * 64 * NP/kWaves, (w+1) * 64 * NP/kWaves) from the logits in LDS and finds its own top K;
// the kWaves * K candidates meet in LDS (wave-major, each wave's in rank order, so among equal
// keys a lower candidate is a lower expert) and K rounds over one candidate per lane finish the
// selection.  A quarter of the keys per wave and no recomputation make this several times
// cheaper than one wave walking all E keys.  s_cand: 2 * kWaves * K dwords of LDS.  Contains a
// barrier: the whole workgroup calls it.
template <int NP>
__device__ __forceinline__ void block_topk(const float *s_lg, int E, int K, uint32_t *s_cand, int &my_idx,
                                           float &my_w) {
    constexpr int NPW = NP / kWaves;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int base = wave * 64 * NPW;
    uint32_t key[NPW];
#pragma unroll
    for (int t = 0; t < NPW; ++t) {
        const int e = base + NPW * lane + t;
        key[t] = e < E ? logit_key(s_lg[min(e, E - 1)]) : 0u;
    }
    uint32_t ck;
    int cp;
    wave_topk_core<NPW>(key, K, ck, cp);
    const int nc = kWaves * K;
    if (lane < K) {
        s_cand[wave * K + lane] = ck;
        s_cand[nc + wave * K + lane] = (uint32_t)(base + cp);
    }
    __syncthreads();
    const uint32_t fk[1] = {lane < nc ? s_cand[lane] : 0u};
    const int fi = lane < nc ? (int)s_cand[nc + lane] : 0;
    uint32_t mk;
    int pos;
    wave_topk_core<1>(fk, K, mk, pos);
    my_idx = __shfl(fi, pos);
    my_w = topk_weight(mk, K);
}

// Keys of this lane's experts NP*lane .. NP*lane+NP-1 from a logit row (absent experts: 0).  The
// loads are branch-free (clamped address) so they are all in flight together.
template <int NP>
__device__ __forceinline__ void issue_logits(const float *row, int E, float (&lg)[NP]) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int t = 0; t < NP; ++t) lg[t] = ((const GLOBAL_AS float *)row)[min(NP * lane + t, E - 1)];
}
template <int NP>
__device__ __forceinline__ void logit_keys(const float (&lg)[NP], int E, uint32_t (&key)[NP]) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int t = 0; t < NP; ++t) key[t] = NP * lane + t < E ? logit_key(lg[t]) : 0u;
}

// --------------------------------------------------------------------------- router
// Row loads per batch and lane (16 bytes each).
constexpr int kRouterBatch = 8;

// bf16 router: the activation is staged as bf16 pairs (columns 2i, 2i+1) plus the bf16 remainder
// when it is not exactly bf16, so a 16-byte chunk of 8 weights meets one 16-byte LDS read per part
// and four v_dot2_f32_bf16.  fp32 router: fp32 activation, float4 LDS reads, fp32 FMAs.
// WPR waves share a row (each takes H/WPR consecutive columns; their sums meet in LDS in a fixed
// order), so a workgroup covers kWaves/WPR experts: bx*(kWaves/WPR) + wave/WPR.  `logit` is that
// expert's logit in every lane of every wave of the row; the return value is true for the row's
// first wave when the expert exists.  s_r: H*4 bytes of LDS (bf16: hi [H/2] + lo [H/2]; fp32:
// x [H]); red: kWaves floats.  Contains barriers: the whole workgroup calls it.
template <int RDT, bool SPLIT, int WPR = 1>
__device__ __forceinline__ bool router_row(const RouterLaunch &a, int bx, int t, uint32_t *s_r, float *red,
                                           float &logit) {
    const int H = a.H;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int e = bx * (kWaves / WPR) + wave / WPR;
    const int part = wave % WPR;
    constexpr int EB = RDT == MOE_BF16 ? 2 : 4;           // bytes per weight
    constexpr int EPL = 16 / EB;                          // weights per 16-byte load
    const int cols = H / WPR, c0 = part * cols;           // this wave's columns
    const int nld = (cols / EPL + 63) / 64;
    const GLOBAL_AS uint8_t *row = (const GLOBAL_AS uint8_t *)a.router + (size_t)(e < a.E ? e : 0) * H * EB;
    // 1. activation (+ norm weight) first: its wait then does not include the row loads issued after
    const void *x = (const char *)a.x + (size_t)t * a.x_stride * (a.x_dtype == MOE_BF16 ? 2 : 4);
    const int nch = H / 16;
    Chunk16 xc[2], nc[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int m = min((int)threadIdx.x + kBlock * j, nch - 1);   // clamped; extra chunks unused
        issue_chunk16(x, a.x_dtype, m, xc[j]);
        if (a.norm_w) issue_chunk16(a.norm_w, MOE_BF16, m, nc[j]);
    }
    // 2. first batch of this wave's part of the row.  Router rows go through the caches (unlike the
    //    expert weights): every step reads the same rows, and a workgroup index always lands on the
    //    same XCD, so each XCD's share of the router stays in its L2 between steps (17.58 -> 17.31 us
    //    per H4096/E512 decode step, three alternating runs each)
    u32x4 wv[kRouterBatch];
#pragma unroll
    for (int j = 0; j < kRouterBatch; ++j) {
        const int c = c0 + min((lane + 64 * j) * EPL, cols - EPL);   // clamped; unused lanes ignore it
        wv[j] = *(const GLOBAL_AS u32x4 *)(row + (size_t)c * EB);
    }
    // 3. activation (+ RMSNorm) into LDS
    float v[2][16];
    float ss = 0.f;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        chunk16_f32(xc[j], a.x_dtype, v[j]);
        if ((int)threadIdx.x + kBlock * j < nch) {
#pragma unroll
            for (int i = 0; i < 16; ++i) ss += v[j][i] * v[j][i];
        }
    }
    float inv = 1.f;
    if (a.norm_w) {
        ss = block_sum(ss, red);
        inv = 1.0f / sqrtf(ss / (float)H + a.eps);
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int m = threadIdx.x + kBlock * j;
        if (m < nch) {
            if (a.norm_w) {
                float w[16];
                chunk16_f32(nc[j], MOE_BF16, w);
#pragma unroll
                for (int i = 0; i < 16; ++i) v[j][i] = v[j][i] * inv * w[i];
            }
            if (RDT == MOE_BF16) {
                uint32_t hv[16], lv[16];
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    hv[i] = bf16_rne(v[j][i]);
                    lv[i] = SPLIT ? bf16_rne(v[j][i] - bf16_f32(hv[i])) : 0u;
                }
                uint32_t *hi = s_r + 8 * m, *lo = s_r + H / 2 + 8 * m;
#pragma unroll
                for (int q = 0; q < 8; q += 4) {
                    *(u32x4 *)(hi + q) = u32x4{hv[2 * q] | (hv[2 * q + 1] << 16), hv[2 * q + 2] | (hv[2 * q + 3] << 16),
                                               hv[2 * q + 4] | (hv[2 * q + 5] << 16), hv[2 * q + 6] | (hv[2 * q + 7] << 16)};
                    if (SPLIT)
                        *(u32x4 *)(lo + q) = u32x4{lv[2 * q] | (lv[2 * q + 1] << 16), lv[2 * q + 2] | (lv[2 * q + 3] << 16),
                                                   lv[2 * q + 4] | (lv[2 * q + 5] << 16), lv[2 * q + 6] | (lv[2 * q + 7] << 16)};
                }
            } else {
                float *xs = (float *)s_r + 16 * m;
#pragma unroll
                for (int q = 0; q < 16; q += 4)
                    *(u32x4 *)(xs + q) = u32x4{__float_as_uint(v[j][q]), __float_as_uint(v[j][q + 1]),
                                               __float_as_uint(v[j][q + 2]), __float_as_uint(v[j][q + 3])};
            }
        }
    }
    __syncthreads();
    // 4. dot product over this wave's columns, further batches for long rows
    float acc = 0.f, acc2 = 0.f;
    if (e < a.E) {
        for (int base = 0; base < nld; base += kRouterBatch) {
            if (base > 0) {
#pragma unroll
                for (int j = 0; j < kRouterBatch; ++j) {
                    const int c = c0 + min((lane + 64 * (base + j)) * EPL, cols - EPL);
                    wv[j] = *(const GLOBAL_AS u32x4 *)(row + (size_t)c * EB);
                }
            }
#pragma unroll
            for (int j = 0; j < kRouterBatch; ++j) {
                const int cl = (lane + 64 * (base + j)) * EPL;
                const int c = c0 + cl;
                if (base + j < nld && cl < cols) {
                    if (RDT == MOE_BF16) {
                        const u32x4 xh = *(const u32x4 *)(s_r + c / 2);
#pragma unroll
                        for (int q = 0; q < 4; ++q) acc = dot2(wv[j][q], xh[q], acc);
                        if (SPLIT) {
                            const u32x4 xl = *(const u32x4 *)(s_r + H / 2 + c / 2);
#pragma unroll
                            for (int q = 0; q < 4; ++q) acc2 = dot2(wv[j][q], xl[q], acc2);
                        }
                    } else {
                        const u32x4 xf = *(const u32x4 *)((const float *)s_r + c);
#pragma unroll
                        for (int q = 0; q < 4; ++q) acc = fmaf(__uint_as_float(wv[j][q]), __uint_as_float(xf[q]), acc);
                    }
                }
            }
        }
    }
    acc = group_sum(acc + acc2, 64);
    if (WPR > 1) {
        if (lane == 0) red[wave] = acc;
        __syncthreads();
        const int w0 = wave - part;
        acc = red[w0];
#pragma unroll
        for (int q = 1; q < WPR; ++q) acc += red[w0 + q];
    }
    logit = acc + (e < a.E && a.logit_bias ? a.logit_bias[e] : 0.f);
    return e < a.E && part == 0;
}

// --------------------------------------------------------------------------- gate/up + SwiGLU
// Instruction groups per work unit: enough loads in flight per lane (about 16 slots of gate+up).
template <int NJ>
__host__ __device__ constexpr int gu_rg() { return NJ >= 4 ? 1 : 4 / NJ; }

template <int NJ, int RG>
struct GULoads {
    u32x4 qg[RG][NJ], qu[RG][NJ];
    uint32_t sg[RG][NJ], su[RG][NJ];
};

// Issue the loads of one work unit: RB consecutive rows of gate and up of one expert.
template <int BITS, int NJ, int RG>
__device__ __forceinline__ void gu_issue(const Planes *pl, const Geo &g, int H, int I, int r0, int RB,
                                         GULoads<NJ, RG> &L) {
    // Branch-free: rows past the matrix and idle slots read a clamped, in-bounds address.  Their
    // contribution vanishes (idle slots have zero activation operands and sum; rows past the
    // block are never written), so nothing needs masking here.
    const int G = H / 64;
    const size_t rowb = (size_t)H * BITS / 8;
#pragma unroll
    for (int gi = 0; gi < RG; ++gi) {
        const int r = min(r0 + gi * g.rpi + g.lrow, I - 1);
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            const int slot = min(g.lsl + 64 * j, g.spr - 1);
            L.qg[gi][j] = load_slot<BITS>(pl[0].q + (size_t)r * rowb, slot);
            L.qu[gi][j] = load_slot<BITS>(pl[1].q + (size_t)r * rowb, slot);
            const size_t sbi = (size_t)r * G + (slot >> 1);
            L.sg[gi][j] = __builtin_nontemporal_load(pl[0].sb + sbi);
            L.su[gi][j] = __builtin_nontemporal_load(pl[1].sb + sbi);
        }
    }
}

// Byte offsets of one gate/up unit's loads inside an expert blob of code width BITS (32 bits: a blob
// of the largest supported shape is far below 4 GiB).  They depend on the unit and the lane only, so
// a kernel computes them before the routing is known; once it is, every load is the expert's blob
// address (wave-uniform, in scalar registers) plus one of these, and no address arithmetic is left
// between the selection and the loads.
template <int NJ, int RG>
struct GUOffs {
    uint32_t qg[RG][NJ], qu[RG][NJ], sg[RG][NJ], su[RG][NJ];
};
template <int BITS, int NJ, int RG>
__device__ __forceinline__ void gu_offsets(const PlaneTable &t, const Geo &g, int H, int I, int r0,
                                           GUOffs<NJ, RG> &o) {
    const uint64_t *po = t.off[BITS == 2 ? 0 : 1];
    const uint32_t G = (uint32_t)H / 64, rowb = (uint32_t)H * BITS / 8;
#pragma unroll
    for (int gi = 0; gi < RG; ++gi) {
        const uint32_t r = (uint32_t)min(r0 + gi * g.rpi + g.lrow, I - 1);     // clamped as in gu_issue
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            const uint32_t slot = (uint32_t)min(g.lsl + 64 * j, g.spr - 1);
            const uint32_t qo = r * rowb + slot * (BITS == 4 ? 16u : 8u);
            const uint32_t so = (r * G + (slot >> 1)) * 4u;
            o.qg[gi][j] = (uint32_t)po[0] + qo;
            o.qu[gi][j] = (uint32_t)po[2] + qo;
            o.sg[gi][j] = (uint32_t)po[1] + so;
            o.su[gi][j] = (uint32_t)po[3] + so;
            // materialised here, ahead of the wait they are meant to precede
            asm volatile("" : "+v"(o.qg[gi][j]), "+v"(o.qu[gi][j]), "+v"(o.sg[gi][j]), "+v"(o.su[gi][j]));
        }
    }
}
__device__ __forceinline__ uint64_t uniform64(uint64_t v) {
    return ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(v >> 32)) << 32) |
           (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)v);
}
// The loads of gu_issue from precomputed offsets; `blob` is wave-uniform.
template <int BITS, int NJ, int RG>
__device__ __forceinline__ void gu_issue_at(uint64_t blob, const GUOffs<NJ, RG> &o, GULoads<NJ, RG> &L) {
    const gbytes b = (gbytes)uniform64(blob);
#pragma unroll
    for (int gi = 0; gi < RG; ++gi) {
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            if (BITS == 4) {
                L.qg[gi][j] = __builtin_nontemporal_load((const GLOBAL_AS u32x4 *)(b + o.qg[gi][j]));
                L.qu[gi][j] = __builtin_nontemporal_load((const GLOBAL_AS u32x4 *)(b + o.qu[gi][j]));
            } else {
                const u32x2 vg = __builtin_nontemporal_load((const GLOBAL_AS u32x2 *)(b + o.qg[gi][j]));
                const u32x2 vu = __builtin_nontemporal_load((const GLOBAL_AS u32x2 *)(b + o.qu[gi][j]));
                L.qg[gi][j] = u32x4{vg.x, vg.y, 0u, 0u};
                L.qu[gi][j] = u32x4{vu.x, vu.y, 0u, 0u};
            }
            L.sg[gi][j] = __builtin_nontemporal_load((gwords)(b + o.sg[gi][j]));
            L.su[gi][j] = __builtin_nontemporal_load((gwords)(b + o.su[gi][j]));
        }
    }
}

template <int BITS, int NJ, int RG, bool LATE = false>
__device__ __forceinline__ void gu_finish(const Geo &g, int I, int r0, int RB, const ActView &av,
                                          const GULoads<NJ, RG> &L, float *hout) {
    uint32_t D[NJ][kSlotDw];
    float2 XS[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        const int slot = g.lsl + 64 * j;
        load_act_slot(av, slot, slot < g.spr, D[j], XS[j]);
    }
#pragma unroll
    for (int gi = 0; gi < RG; ++gi) {
        float pg = 0.f, pu = 0.f;
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            if constexpr (LATE) {
                pg += slot_dot_late<BITS>(L.qg[gi][j], D[j], L.sg[gi][j], XS[j]);
                pu += slot_dot_late<BITS>(L.qu[gi][j], D[j], L.su[gi][j], XS[j]);
            } else {
                pg += slot_dot<BITS>(L.qg[gi][j], D[j], L.sg[gi][j], XS[j]);
                pu += slot_dot<BITS>(L.qu[gi][j], D[j], L.su[gi][j], XS[j]);
            }
        }
        pg = group_sum(pg, g.gsz);
        pu = group_sum(pu, g.gsz);
        const int rr = gi * g.rpi + g.lrow;
        if (g.lsl == 0 && rr < RB && r0 + rr < I) hout[r0 + rr] = silu(pg) * pu;
    }
}

// The RG SwiGLU values of one unit, in every lane of each row group (no store).
template <int BITS, int NJ, int RG>
__device__ __forceinline__ void gu_values(const Geo &g, const ActView &av, const GULoads<NJ, RG> &L, float (&hv)[RG]) {
    uint32_t D[NJ][kSlotDw];
    float2 XS[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        const int slot = g.lsl + 64 * j;
        load_act_slot(av, slot, slot < g.spr, D[j], XS[j]);
    }
#pragma unroll
    for (int gi = 0; gi < RG; ++gi) {
        float pg = 0.f, pu = 0.f;
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            pg += slot_dot<BITS>(L.qg[gi][j], D[j], L.sg[gi][j], XS[j]);
            pu += slot_dot<BITS>(L.qu[gi][j], D[j], L.su[gi][j], XS[j]);
        }
        pg = group_sum(pg, g.gsz);
        pu = group_sum(pu, g.gsz);
        hv[gi] = silu(pg) * pu;
    }
}

// --------------------------------------------------------------------------- down + combine
template <int NJ>
__host__ __device__ constexpr int dn_rg() { return NJ >= 2 ? 1 : 2; }

template <int NJ, int RG, int KM>
struct DLoads {
    u32x4 q[KM][RG][NJ];
    uint32_t sb[KM][RG][NJ];
};

// Loads of one expert's down rows for one unit.  The code width is a run-time value and every slot
// is read as 16 bytes (a 2-bit slot uses the first 8; the extra 8 stay inside the blob, since a
// scale/bias plane follows every code plane), so the loads of all experts issue without a branch
// and the arithmetic on the first expert waits for its own loads only.
template <int NJ, int RG, int KM>
__device__ __forceinline__ void dn_issue(const Planes &pl, int bits, const Geo &g, int H, int I, int r0, int k,
                                         DLoads<NJ, RG, KM> &L) {
    const int G = I / 64;
    const size_t rowb = (size_t)I * bits / 8;
    const int ssh = bits == 4 ? 4 : 3;
#pragma unroll
    for (int gi = 0; gi < RG; ++gi) {
        const int r = min(r0 + gi * g.rpi + g.lrow, H - 1);     // clamped; see gu_issue
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            const int slot = min(g.lsl + 64 * j, g.spr - 1);
            L.q[k][gi][j] = __builtin_nontemporal_load((const GLOBAL_AS u32x4 *)(pl.q + (size_t)r * rowb + ((size_t)slot << ssh)));
            L.sb[k][gi][j] = __builtin_nontemporal_load(pl.sb + ((size_t)r * G + (slot >> 1)));
        }
    }
}

// Issue every selected expert's loads for one unit (output rows r0..r0+RB-1) as straight-line
// code.  Slots past K and absent experts (sel 0) read a present expert's rows instead (their
// results are never used), so no branch separates the loads from the arithmetic; with no expert
// present at all nothing is loaded.
template <int NJ, int RG, int KM>
__device__ __forceinline__ void dn_issue_all(const uint64_t (&sel)[KM], int K, const Geo &g, int H, int I, int r0,
                                             const PlaneTable &pt, DLoads<NJ, RG, KM> &L) {
    uint64_t any = 0;
#pragma unroll
    for (int k = KM - 1; k >= 0; --k)
        if (k < K && sel[k]) any = sel[k];
    if (!any) return;
#pragma unroll
    for (int k = 0; k < KM; ++k) {
        const uint64_t sk = (k < K && sel[k]) ? sel[k] : any;
        Planes pl[3];
        expert_planes(sel_blob(sk), sel_bits(sk), pt, pl);
        dn_issue<NJ, RG, KM>(pl[2], sel_bits(sk), g, H, I, r0, k, L);
    }
}

// Byte offsets of one down unit's loads inside an expert blob, for both code widths ([0] 2-bit, [1]
// 4-bit), computed before the selection is known (see GUOffs).
template <int NJ, int RG>
struct DNOffs {
    uint32_t q[2][RG][NJ], sb[2][RG][NJ];
};
template <int NJ, int RG>
__device__ __forceinline__ void dn_offsets(const PlaneTable &t, const Geo &g, int H, int I, int r0, DNOffs<NJ, RG> &o) {
    const uint32_t G = (uint32_t)I / 64;
#pragma unroll
    for (int w = 0; w < 2; ++w) {
        const uint32_t rowb = (uint32_t)I * (w ? 4u : 2u) / 8;
#pragma unroll
        for (int gi = 0; gi < RG; ++gi) {
            const uint32_t r = (uint32_t)min(r0 + gi * g.rpi + g.lrow, H - 1);     // clamped; see gu_issue
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                const uint32_t slot = (uint32_t)min(g.lsl + 64 * j, g.spr - 1);
                o.q[w][gi][j] = (uint32_t)t.off[w][4] + r * rowb + (slot << (w ? 4 : 3));
                o.sb[w][gi][j] = (uint32_t)t.off[w][5] + (r * G + (slot >> 1)) * 4u;
                asm volatile("" : "+v"(o.q[w][gi][j]), "+v"(o.sb[w][gi][j]));
            }
        }
    }
}
// dn_issue_all from precomputed offsets: the same loads (every slot read as 16 bytes; slots past K
// and absent experts read a present expert's rows), each the expert's blob address plus an offset.
// Branch-free, so that the waits for loads issued before these (h) can count them: with no expert
// present at all every load reads the first 16 bytes of `spare` (any buffer of at least 16 bytes)
// and its results go unused.
template <int NJ, int RG, int KM>
__device__ __forceinline__ void dn_issue_all_at(const uint64_t (&sel)[KM], int K, const DNOffs<NJ, RG> &o,
                                                const void *spare, DLoads<NJ, RG, KM> &L) {
    uint64_t any = 0;
#pragma unroll
    for (int k = KM - 1; k >= 0; --k)
        if (k < K && sel[k]) any = sel[k];
    const bool none = any == 0;
#pragma unroll
    for (int k = 0; k < KM; ++k) {
        const uint64_t sk = (k < K && sel[k]) ? sel[k] : any;
        const gbytes b = (gbytes)uniform64(none ? (uint64_t)spare : sel_blob(sk));
        const bool two = sel_bits(sk) == 2;
#pragma unroll
        for (int gi = 0; gi < RG; ++gi) {
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                const uint32_t qo = none ? 0u : two ? o.q[0][gi][j] : o.q[1][gi][j];
                const uint32_t so = none ? 0u : two ? o.sb[0][gi][j] : o.sb[1][gi][j];
                L.q[k][gi][j] = __builtin_nontemporal_load((const GLOBAL_AS u32x4 *)(b + qo));
                L.sb[k][gi][j] = __builtin_nontemporal_load((gwords)(b + so));
            }
        }
    }
}

// LDS dwords per expert: digit planes [I/32][kSlotDw] in the expert's code width's order, then
// xs [I/32] float2 (I is a multiple of 64, so every part stays 16-byte aligned).
__host__ __device__ __forceinline__ int down_lds_per_expert(int I) { return I / 2 + I / 16; }

// --------------------------------------------------------------------------- small-expert helpers
// Compile-time loop: f(std::integral_constant<int, i>) for i = I .. N-1.
template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F &&f) {
    if constexpr (I < N) {
        f(std::integral_constant<int, I>{});
        static_for<I + 1, N>(f);
    }
}

// The unit pipeline of one wave: UPW units, NB register buffers, the loads of unit i + NB - 1 issued
// before unit i is finished, so NB - 1 units are in flight while one is computed.  Fully unrolled
// (buffer indices are compile-time) and branch-free around the loads: a wave with fewer than UPW
// units (the ragged end of a matrix) re-reads its last unit's rows instead, and only the finishing
// step is skipped.  (Skipping those loads behind a branch instead keeps every buffer live across
// the branch and spills.)  issue(i, buf) must clamp i itself.
template <int UPW, int NB, typename Buf, typename Issue, typename Finish>
__device__ __forceinline__ void unit_pipeline(int nu, Buf (&B)[NB], Issue &&issue, Finish &&finish) {
    static_for<0, UPW>([&](auto ic) {
        constexpr int i = decltype(ic)::value;
        if constexpr (i + NB - 1 < UPW) issue(i + NB - 1, B[(i + NB - 1) % NB]);
        if (i < nu) finish(i, B[i % NB]);
    });
}

// Slot operands of this lane for one staged row: FULL (GS != 0) when every lane's slots exist.
template <int NJ, int GS>
__device__ __forceinline__ void row_slots(const ActView &av, const Geo &g, uint32_t (&D)[NJ][kSlotDw], float2 (&XS)[NJ]) {
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        const int slot = g.lsl + 64 * j;
        if constexpr (GS != 0) load_act_slot_full(av, slot, D[j], XS[j]);
        else load_act_slot(av, slot, slot < g.spr, D[j], XS[j]);
    }
}

// The workgroup's list entry (one scalar load; entries past the list end exit at once).
__device__ __forceinline__ bool small_entry(const GroupedLaunch &a, SmallRec &r) {
    const int j = blockIdx.y;
    const int ns = *a.nsmall;
    r = a.small[j];
    return j < ns;
}

// Staging of an expert's token rows into LDS.  Thread `tid` takes chunk tid (+ kBlock, ... for rows
// of more than kBlock chunks) of 16 activations of every row, so a token's index is a compile-time
// constant everywhere and its row address a uniform value: row_addr(t) for t < 4 * NBATCH (t >= n
// gives a duplicate of a present row).  Tokens go in NBATCH batches of four; the loads of the first
// pass's first batch are issued by stage_issue, before the caller's first weight loads, and
// everything else happens in stage_finish, which hands every chunk to conv(t, chunk, valid, v).
// Every thread of the workgroup calls both (conv may exchange data between the lanes of a wave);
// the caller puts a barrier after stage_finish.
struct StageBatch {
    Chunk16 c[4];
};
template <int B, typename RowAddr>
__device__ __forceinline__ void stage_batch_issue(RowAddr &&row_addr, int dtype, int mc, StageBatch &sb) {
    static_for<0, 4>([&](auto jc) {
        constexpr int j = decltype(jc)::value;
        issue_chunk16(row_addr(4 * B + j), dtype, mc, sb.c[j]);
    });
}
template <int B, typename Conv>
__device__ __forceinline__ void stage_batch_convert(int n, int nch, int dtype, int m, const StageBatch &sb, Conv &&conv) {
    const bool valid = m < nch;
    const int mc = min(m, nch - 1);
    static_for<0, 4>([&](auto jc) {
        constexpr int t = 4 * B + decltype(jc)::value;
        if (t < n) {                                                         // uniform
            float v[16];
            chunk16_f32(sb.c[t - 4 * B], dtype, v);
            conv(t, mc, valid, v);
        }
    });
}
template <typename RowAddr>
__device__ __forceinline__ void stage_issue(RowAddr &&row_addr, int cols, int dtype, StageBatch &sb) {
    stage_batch_issue<0>(row_addr, dtype, min((int)threadIdx.x, cols / 16 - 1), sb);
}
template <int NBATCH, typename RowAddr, typename Conv>
__device__ __forceinline__ void stage_finish(RowAddr &&row_addr, int n, int cols, int dtype, StageBatch &sb,
                                             Conv &&conv) {
    const int nch = cols / 16;
    for (int m0 = 0; m0 < nch; m0 += kBlock) {                               // uniform; usually one pass
        const int m = m0 + (int)threadIdx.x, mc = min(m, nch - 1);
        if (m0 > 0) stage_batch_issue<0>(row_addr, dtype, mc, sb);
        stage_batch_convert<0>(n, nch, dtype, m, sb, conv);
        static_for<1, NBATCH>([&](auto bc) {
            constexpr int B = decltype(bc)::value;
            if (n > 4 * B) {                                                 // uniform
                stage_batch_issue<B>(row_addr, dtype, mc, sb);
                stage_batch_convert<B>(n, nch, dtype, m, sb, conv);
            }
        });
    }
}

__host__ __device__ __forceinline__ int row_dw(int cols) { return cols / 2 + cols / 16; }   // planes + xs

int nj_for(int cols) {
    const int spr = cols / 32;
    const int nj = spr >= 64 ? (spr + 63) / 64 : 1;
    return nj <= 1 ? 1 : nj <= 2 ? 2 : 4;
}
int rpi_for(int cols) {
    const int spr = cols / 32;
    return spr >= 64 ? 1 : 64 / next_pow2(spr);
}

}  // namespace
}  // namespace moe
