// moe_decode.hip -- gfx950 kernels for the per-token MoE expert path.
//
// Kernels (one launch each, stream-ordered, no grid-wide barriers):
//   k_router : [RMSNorm] + router matvec -> logits[T][E]
//   k_topk   : softmax / top-K / renormalise (for moe_route)
//   k_gateup : every workgroup recomputes top-K from the logits (no host round trip and no
//              grid barrier), stages the activation once in LDS in the order the unpack
//              consumes it, then streams the gate and up rows of all K selected experts in one
//              launch and writes h = silu(g) * u
//   k_down   : down projection of all K experts for a block of output rows, combined with the
//              routing weights (+ residual) in registers before a single cross-lane reduction
//   k_combine: standalone weighted combine
//
// Dequantisation.  The affine form w = q*s + b and its FMA rewrite fma(q, s*x, b*x) come from
// the lilting.ch page "397Bパラメータモデルを48GB MacBookで動かすFlash-MoE", section "Metal
// Compute Shaders".  Summed over the 32 inputs one lane handles (half a group of 64) it becomes
// s * sum(q x) + b * sum(x), and sum(x) is computed once per slot.  Codes become bf16 operands
// without a table (the nzkcom page lists a lookup-table dequant among its rejected experiments)
// by OR-ing them into the mantissa of 128.0: (q | 0x4300) is the bf16 value 128 + q, so two codes
// at the same bit position of the two 16-bit halves of a dword become one packed operand with a
// single AND-OR, and v_dot2_f32_bf16 accumulates (128+q_a) x_a + (128+q_b) x_b in fp32 with exact
// products.  The 128 * sum(x) offset folds into the bias term: s * acc + (b - 128 s) * sum(x).
// Activations that are not exactly bf16 (fp32 inputs, RMSNorm outputs, the SwiGLU output h) are
// split into bf16 hi + lo parts with one more dot2 for the lo part (about 16 significant bits).
//
// Lane geometry.  A lane "slot" is 32 consecutive input columns: 16 bytes of 4-bit codes or 8
// bytes of 2-bit codes, always inside one group of 64.  For rows of >= 64 slots, lane l takes
// slots l, l+64, ... (one coalesced 1 KiB / 512 B load per wave instruction); for shorter rows a
// wave covers several rows at once, lanes grouped by the row's slot count rounded up to a power
// of two.  Both code widths share the geometry, so experts of different widths combine in
// registers, and a lane's activation operands come from LDS once per work unit.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "moe_internal.h"

namespace moe {
namespace {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr uint32_t kMagic = 0x43004300u;  // bf16 128.0 in both 16-bit halves
constexpr int kBlock = 256;               // threads per workgroup (4 wavefronts)
constexpr int kWaves = kBlock / 64;
constexpr int kDPS = 16;                  // activation dwords per slot (32 columns, bf16 pairs)

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c,
                                           false);
}
__device__ __forceinline__ uint32_t bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}
__device__ __forceinline__ float bf16_f32(uint32_t b) { return __uint_as_float(b << 16); }
__device__ __forceinline__ float load_act(const void *x, int dtype, size_t i) {
    return dtype == MOE_BF16 ? bf16_f32(((const uint16_t *)x)[i]) : ((const float *)x)[i];
}
__device__ __forceinline__ float silu(float z) { return z / (1.0f + expf(-z)); }

// Sum over aligned groups of gs lanes (gs a power of two <= 64); every lane gets its group's sum.
__device__ __forceinline__ float group_sum(float v, int gs) {
    for (int off = gs >> 1; off > 0; off >>= 1) v += __shfl_xor(v, off);
    return v;
}

__device__ float block_sum(float v, float *red) {
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

// --------------------------------------------------------------------------- activation layout
// Slot s covers columns 32s..32s+31.  4-bit: the slot's 16 bytes are 4 dwords of 8 codes and the
// AND-OR at shift 4i pairs columns (8k+i, 8k+i+4) of dword k; 2-bit: 8 bytes = 2 dwords of 16
// codes and shift 2i pairs (16k+i, 16k+i+8).  Activation dword d of slot s packs the same pair.
template <int BITS>
__device__ __forceinline__ int arr_col(int d, int hf) {
    const int s = d >> 4, j = d & 15;
    if (BITS == 4) return s * 32 + (j >> 2) * 8 + (j & 3) + 4 * hf;
    return s * 32 + (j >> 3) * 16 + (j & 7) + 8 * hf;
}

struct ActView {
    const uint32_t *hi, *lo;  // [cols/2] packed bf16 pairs (lo: bf16 of the remainder)
    const float *xs;          // [cols/32] sum over the slot of hi + lo
};

template <int BITS, bool SPLIT, typename F>
__device__ void stage_layout(F value, int cols, uint32_t *hi, uint32_t *lo) {
    for (int d = threadIdx.x; d < cols / 2; d += blockDim.x) {
        const float v0 = value(arr_col<BITS>(d, 0)), v1 = value(arr_col<BITS>(d, 1));
        const uint32_t h0 = bf16_rne(v0), h1 = bf16_rne(v1);
        hi[d] = h0 | (h1 << 16);
        if (SPLIT) lo[d] = bf16_rne(v0 - bf16_f32(h0)) | (bf16_rne(v1 - bf16_f32(h1)) << 16);
    }
}
// Per-slot sums of the values the dot products actually see (hi + lo).
template <bool SPLIT>
__device__ void stage_sums(int cols, const uint32_t *hi, const uint32_t *lo, float *xs) {
    for (int s = threadIdx.x; s < cols / 32; s += blockDim.x) {
        float t = 0.f;
        for (int j = 0; j < kDPS; ++j) {
            const uint32_t h = hi[s * kDPS + j];
            t += bf16_f32(h & 0xFFFFu) + bf16_f32(h >> 16);
            if (SPLIT) {
                const uint32_t l = lo[s * kDPS + j];
                t += bf16_f32(l & 0xFFFFu) + bf16_f32(l >> 16);
            }
        }
        xs[s] = t;
    }
}

// --------------------------------------------------------------------------- slot dot products
// s * sum(q x) + b * sum(x) over one slot, given its codes and (scale, bias) dword.
template <int BITS, bool SPLIT>
__device__ __forceinline__ float slot_dot(const u32x4 q, const uint32_t *X, const uint32_t *XL, uint32_t sb,
                                          float xs) {
    float a0 = 0.f, a1 = 0.f, l0 = 0.f, l1 = 0.f;
    constexpr int NW = BITS == 4 ? 4 : 2;     // code dwords per slot
    constexpr int PW = BITS == 4 ? 4 : 8;     // pairs per dword
#pragma unroll
    for (int k = 0; k < NW; ++k) {
        const uint32_t v = q[k];
#pragma unroll
        for (int i = 0; i < PW; ++i) {
            const uint32_t p = BITS == 4 ? (((v >> (4 * i)) & 0x000F000Fu) | kMagic)
                                         : (((v >> (2 * i)) & 0x00030003u) | kMagic);
            const int d = k * PW + i;
            if (d & 1) a1 = dot2(p, X[d], a1); else a0 = dot2(p, X[d], a0);
            if (SPLIT) { if (d & 1) l1 = dot2(p, XL[d], l1); else l0 = dot2(p, XL[d], l0); }
        }
    }
    const float acc = SPLIT ? (a0 + a1) + (l0 + l1) : a0 + a1;
    const float s = bf16_f32(sb & 0xFFFFu), b = bf16_f32(sb >> 16);
    return s * acc + (b - 128.f * s) * xs;
}

template <int BITS>
__device__ __forceinline__ u32x4 load_slot(const uint8_t *row, int slot) {
    if (BITS == 4) return *(const u32x4 *)(row + (size_t)slot * 16);
    const u32x2 v = *(const u32x2 *)(row + (size_t)slot * 8);
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
__device__ __forceinline__ Geo make_geo(int cols) {
    Geo g;
    const int lane = threadIdx.x & 63;
    g.spr = cols / 32;
    if (g.spr >= 64) {
        g.gsz = 64; g.rpi = 1; g.lrow = 0; g.lsl = lane;
    } else {
        g.gsz = next_pow2(g.spr); g.rpi = 64 / g.gsz; g.lrow = lane / g.gsz; g.lsl = lane % g.gsz;
    }
    return g;
}

struct Planes {
    const uint8_t *q; const uint32_t *sb;
};
__device__ __forceinline__ void expert_planes(const uint8_t *blob, int H, int I, int bits, Planes p[3]) {
    const size_t cin = (size_t)I * H * bits / 8, sbin = (size_t)I * (H / 64) * 4;
    const size_t cout = (size_t)H * I * bits / 8;
    size_t off = 0;
    p[0].q = blob + off; off = round256(off + cin);
    p[0].sb = (const uint32_t *)(blob + off); off = round256(off + sbin);
    p[1].q = blob + off; off = round256(off + cin);
    p[1].sb = (const uint32_t *)(blob + off); off = round256(off + sbin);
    p[2].q = blob + off; off = round256(off + cout);
    p[2].sb = (const uint32_t *)(blob + off);
}

// --------------------------------------------------------------------------- top-K (one wave)
// Largest K logits, descending, equal values -> lower index; NaN counts as -inf.  The weights are
// the softmax over the selected logits, which equals the softmax over all E renormalised.
// `lg` is the logit row in LDS (E <= MOE_MAX_EXPERTS, so a lane owns at most 32 entries).
__device__ void wave_topk(const float *lg, int E, int K, int *s_idx, float *s_w) {
    const int lane = threadIdx.x & 63;
    const int nper = (E + 63) / 64;
    uint32_t taken = 0;
    float top[MOE_MAX_TOPK];
    int topi[MOE_MAX_TOPK];
#pragma unroll
    for (int k = 0; k < MOE_MAX_TOPK; ++k) {
        top[k] = -INFINITY;
        topi[k] = 0;
        if (k < K) {
            float bv = -INFINITY;
            int bi = 0x7FFFFFFF;
            for (int t = 0; t < nper; ++t) {
                const int e = lane + 64 * t;
                if (e < E && !((taken >> t) & 1u)) {
                    float v = lg[e];
                    v = (v != v) ? -INFINITY : v;
                    if (v > bv || (v == bv && e < bi)) { bv = v; bi = e; }
                }
            }
            for (int off = 32; off > 0; off >>= 1) {
                const float ov = __shfl_xor(bv, off);
                const int oi = __shfl_xor(bi, off);
                if (ov > bv || (ov == bv && oi < bi)) { bv = ov; bi = oi; }
            }
            if ((bi & 63) == lane) taken |= 1u << (bi >> 6);
            top[k] = bv;
            topi[k] = bi;
        }
    }
    if (lane == 0) {
        float z = 0.f;
        float ex[MOE_MAX_TOPK];
#pragma unroll
        for (int k = 0; k < MOE_MAX_TOPK; ++k) {
            ex[k] = k < K ? expf(top[k] - top[0]) : 0.f;
            z += ex[k];
        }
#pragma unroll
        for (int k = 0; k < MOE_MAX_TOPK; ++k)
            if (k < K) { s_idx[k] = topi[k]; s_w[k] = ex[k] / z; }
    }
}

// Copy one token's logits into LDS (whole workgroup), for wave_topk.
__device__ __forceinline__ void load_logits(const float *g, int E, float *lg) {
    for (int e = threadIdx.x; e < E; e += blockDim.x) lg[e] = g[e];
}

// --------------------------------------------------------------------------- router
template <int RDT>
__global__ void __launch_bounds__(kBlock) k_router(RouterLaunch a, int rows_per_wave) {
    extern __shared__ float s_x[];  // [H] activation fed to the router
    __shared__ float red[kWaves];
    const int t = blockIdx.y;
    const int H = a.H;
    const void *x = (const char *)a.x + (size_t)t * a.x_stride * (a.x_dtype == MOE_BF16 ? 2 : 4);
    float inv = 1.f;
    if (a.norm_w) {
        float ss = 0.f;
        for (int c = threadIdx.x; c < H; c += blockDim.x) { const float v = load_act(x, a.x_dtype, c); ss += v * v; }
        ss = block_sum(ss, red);
        inv = 1.0f / sqrtf(ss / (float)H + a.eps);
    }
    for (int c = threadIdx.x; c < H; c += blockDim.x) {
        float v = load_act(x, a.x_dtype, c);
        if (a.norm_w) v = v * inv * bf16_f32(a.norm_w[c]);
        s_x[c] = v;
    }
    __syncthreads();
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int e0 = (blockIdx.x * kWaves + wave) * rows_per_wave;
    for (int r = 0; r < rows_per_wave; ++r) {
        const int e = e0 + r;
        if (e >= a.E) break;
        float acc = 0.f;
        if (RDT == MOE_BF16) {
            const uint8_t *row = (const uint8_t *)a.router + (size_t)e * H * 2;
            for (int c = lane * 8; c < H; c += 512) {
                const u32x4 v = *(const u32x4 *)(row + (size_t)c * 2);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    acc = fmaf(bf16_f32(v[j] & 0xFFFFu), s_x[c + 2 * j], acc);
                    acc = fmaf(bf16_f32(v[j] >> 16), s_x[c + 2 * j + 1], acc);
                }
            }
        } else {
            const float *row = (const float *)a.router + (size_t)e * H;
            for (int c = lane * 4; c < H; c += 256) {
                const u32x4 v = *(const u32x4 *)(row + c);
#pragma unroll
                for (int j = 0; j < 4; ++j) acc = fmaf(__uint_as_float(v[j]), s_x[c + j], acc);
            }
        }
        acc = group_sum(acc, 64);
        if (lane == 0) a.logits[(size_t)t * a.E + e] = acc + (a.logit_bias ? a.logit_bias[e] : 0.f);
    }
}

__global__ void __launch_bounds__(64) k_topk(TopkLaunch a) {
    __shared__ int s_idx[MOE_MAX_TOPK];
    __shared__ float s_w[MOE_MAX_TOPK];
    __shared__ float s_lg[MOE_MAX_EXPERTS];
    const int t = blockIdx.x;
    load_logits(a.logits + (size_t)t * a.E, a.E, s_lg);
    __syncthreads();
    wave_topk(s_lg, a.E, a.K, s_idx, s_w);
    __syncthreads();
    if ((int)threadIdx.x < a.K) {
        a.idx[(size_t)t * a.K + threadIdx.x] = s_idx[threadIdx.x];
        a.w[(size_t)t * a.K + threadIdx.x] = s_w[threadIdx.x];
    }
}

// --------------------------------------------------------------------------- gate/up + SwiGLU
// Instruction groups per work unit: enough loads in flight per lane (about 16 slots of gate+up).
template <int NJ>
__host__ __device__ constexpr int gu_rg() { return NJ >= 4 ? 2 : 8 / NJ; }

// One work unit: RB consecutive rows of gate and up of one expert.
template <int BITS, int NJ, int RG, bool SPLIT>
__device__ void gateup_unit(const Planes *pl, const Geo &g, int H, int I, int r0, int RB, const ActView &av,
                            float *hout) {
    const int G = H / 64;
    const size_t rowb = (size_t)H * BITS / 8;
    uint32_t X[NJ][kDPS], XL[NJ][SPLIT ? kDPS : 1];
    float XS[NJ];
    bool sok[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        const int slot = g.lsl + 64 * j;
        sok[j] = slot < g.spr;
        const int ss = sok[j] ? slot : 0;
#pragma unroll
        for (int i = 0; i < kDPS; ++i) {
            X[j][i] = sok[j] ? av.hi[ss * kDPS + i] : 0u;
            if (SPLIT) XL[j][i] = sok[j] ? av.lo[ss * kDPS + i] : 0u;
        }
        XS[j] = sok[j] ? av.xs[ss] : 0.f;
    }
    u32x4 qg[RG][NJ], qu[RG][NJ];
    uint32_t sg[RG][NJ], su[RG][NJ];
#pragma unroll
    for (int gi = 0; gi < RG; ++gi) {
        const int rr = gi * g.rpi + g.lrow;
        const int r = r0 + rr;
        const bool rok = rr < RB && r < I;
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            const int slot = g.lsl + 64 * j;
            if (rok && sok[j]) {
                qg[gi][j] = load_slot<BITS>(pl[0].q + (size_t)r * rowb, slot);
                qu[gi][j] = load_slot<BITS>(pl[1].q + (size_t)r * rowb, slot);
                const size_t sbi = (size_t)r * G + (slot >> 1);
                sg[gi][j] = pl[0].sb[sbi];
                su[gi][j] = pl[1].sb[sbi];
            } else {
                qg[gi][j] = qu[gi][j] = u32x4{0u, 0u, 0u, 0u};
                sg[gi][j] = su[gi][j] = 0u;
            }
        }
    }
#pragma unroll
    for (int gi = 0; gi < RG; ++gi) {
        float pg = 0.f, pu = 0.f;
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            pg += slot_dot<BITS, SPLIT>(qg[gi][j], X[j], XL[j], sg[gi][j], XS[j]);
            pu += slot_dot<BITS, SPLIT>(qu[gi][j], X[j], XL[j], su[gi][j], XS[j]);
        }
        pg = group_sum(pg, g.gsz);
        pu = group_sum(pu, g.gsz);
        const int rr = gi * g.rpi + g.lrow;
        if (g.lsl == 0 && rr < RB && r0 + rr < I) hout[r0 + rr] = silu(pg) * pu;
    }
}

template <int NJ, bool SPLIT>
__global__ void __launch_bounds__(kBlock) k_gateup(GateUpLaunch a) {
    extern __shared__ uint32_t lds[];
    __shared__ int s_idx[MOE_MAX_TOPK];
    __shared__ float s_w[MOE_MAX_TOPK];
    __shared__ uint64_t s_blob[MOE_MAX_TOPK];
    __shared__ int s_bits[MOE_MAX_TOPK];
    __shared__ float red[kWaves];
    __shared__ float s_lg[MOE_MAX_EXPERTS];
    const int H = a.H, I = a.I, K = a.K, t = blockIdx.y;
    const int lane = threadIdx.x & 63;

    // 1. routing of this token
    if (!a.idx_in) {
        load_logits(a.logits + (size_t)t * a.E, a.E, s_lg);
        __syncthreads();
    }
    if (a.idx_in) {
        if ((int)threadIdx.x < K) s_idx[threadIdx.x] = a.idx_in[(size_t)t * K + threadIdx.x];
    } else if (threadIdx.x < 64) {
        wave_topk(s_lg, a.E, K, s_idx, s_w);
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
        if (blockIdx.x == 0 && lane < K) {
            const size_t o = (size_t)t * K + lane;
            if (a.idx_out) a.idx_out[o] = s_idx[lane];
            if (a.w_out) a.w_out[o] = s_w[lane];
            if (a.idx_ws) a.idx_ws[o] = s_idx[lane];
            if (a.w_ws) a.w_ws[o] = s_w[lane];
        }
    }

    // 2. activation (RMSNorm when requested), staged in both code-width layouts
    const void *x = (const char *)a.x + (size_t)t * a.x_stride * (a.x_dtype == MOE_BF16 ? 2 : 4);
    float inv = 1.f;
    if (a.norm_w) {
        float ss = 0.f;
        for (int c = threadIdx.x; c < H; c += blockDim.x) { const float v = load_act(x, a.x_dtype, c); ss += v * v; }
        ss = block_sum(ss, red);
        inv = 1.0f / sqrtf(ss / (float)H + a.eps);
    }
    const uint16_t *nw = a.norm_w;
    const int xdt = a.x_dtype;
    auto value = [&](int c) {
        float v = load_act(x, xdt, c);
        if (nw) v = v * inv * bf16_f32(nw[c]);
        return v;
    };
    uint32_t *h4 = lds, *l4 = lds + H / 2, *h2 = lds + H, *l2 = lds + 3 * H / 2;
    float *xs = (float *)(lds + 2 * H);
    stage_layout<4, SPLIT>(value, H, h4, l4);
    stage_layout<2, SPLIT>(value, H, h2, l2);
    __syncthreads();
    stage_sums<SPLIT>(H, h4, l4, xs);
    if ((int)threadIdx.x < K) {
        const int e = s_idx[threadIdx.x];
        if (e >= 0 && e < a.E) {
            const moe_expert_desc d = a.experts[e];
            s_blob[threadIdx.x] = d.blob;
            s_bits[threadIdx.x] = d.bits == 2 ? 2 : 4;
        } else {
            s_blob[threadIdx.x] = 0;
            s_bits[threadIdx.x] = 4;
        }
    }
    __syncthreads();
    const ActView v4{h4, l4, xs}, v2{h2, l2, xs};

    // 3. work units: (expert, block of RB rows)
    const Geo g = make_geo(H);
    constexpr int RG = gu_rg<NJ>();
    const int RB = RG * g.rpi;
    const int nblk = (I + RB - 1) / RB;
    const int units = K * nblk;
    const int wave = threadIdx.x >> 6;
    for (int u = blockIdx.x * kWaves + wave; u < units; u += gridDim.x * kWaves) {
        const int k = u / nblk;
        const int r0 = (u - k * nblk) * RB;
        float *hout = a.h + ((size_t)t * K + k) * I;
        const uint64_t blob = s_blob[k];
        if (!blob) {
            for (int r = r0 + lane; r < r0 + RB && r < I; r += 64) hout[r] = 0.f;
            continue;
        }
        Planes pl[3];
        expert_planes((const uint8_t *)blob, H, I, s_bits[k], pl);
        if (s_bits[k] == 2) gateup_unit<2, NJ, RG, SPLIT>(pl, g, H, I, r0, RB, v2, hout);
        else gateup_unit<4, NJ, RG, SPLIT>(pl, g, H, I, r0, RB, v4, hout);
    }
}

// --------------------------------------------------------------------------- down + combine
template <int NJ>
__host__ __device__ constexpr int dn_rg() { return NJ >= 2 ? 1 : 2; }

// Adds to part[gi] this lane's partial sums of RG instruction rows of one expert's down matrix.
template <int BITS, int NJ, int RG>
__device__ __forceinline__ void down_part(const Planes &pl, const Geo &g, int H, int I, int r0, int RB,
                                          const ActView &av, float *part) {
    const int G = I / 64;
    const size_t rowb = (size_t)I * BITS / 8;
    u32x4 q[RG][NJ];
    uint32_t sb[RG][NJ];
#pragma unroll
    for (int gi = 0; gi < RG; ++gi) {
        const int rr = gi * g.rpi + g.lrow;
        const int r = r0 + rr;
        const bool rok = rr < RB && r < H;
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            const int slot = g.lsl + 64 * j;
            if (rok && slot < g.spr) {
                q[gi][j] = load_slot<BITS>(pl.q + (size_t)r * rowb, slot);
                sb[gi][j] = pl.sb[(size_t)r * G + (slot >> 1)];
            } else {
                q[gi][j] = u32x4{0u, 0u, 0u, 0u};
                sb[gi][j] = 0u;
            }
        }
    }
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        const int slot = g.lsl + 64 * j;
        const bool ok = slot < g.spr;
        const int ss = ok ? slot : 0;
        uint32_t X[kDPS], XL[kDPS];
#pragma unroll
        for (int i = 0; i < kDPS; ++i) {
            X[i] = ok ? av.hi[ss * kDPS + i] : 0u;
            XL[i] = ok ? av.lo[ss * kDPS + i] : 0u;
        }
        const float xs = ok ? av.xs[ss] : 0.f;
#pragma unroll
        for (int gi = 0; gi < RG; ++gi) part[gi] += slot_dot<BITS, true>(q[gi][j], X, XL, sb[gi][j], xs);
    }
}

// LDS per expert: hi [I/2], lo [I/2], xs [I/32].
__host__ __device__ __forceinline__ int down_lds_per_expert(int I) { return I + I / 32; }

template <int NJ, bool COMBINE>
__global__ void __launch_bounds__(kBlock) k_down(DownLaunch a, int E) {
    extern __shared__ uint32_t lds[];
    __shared__ uint64_t s_blob[MOE_MAX_TOPK];
    __shared__ int s_bits[MOE_MAX_TOPK];
    __shared__ float s_w[MOE_MAX_TOPK];
    const int H = a.H, I = a.I, K = a.K, t = blockIdx.y;
    if ((int)threadIdx.x < K) {
        const int e = a.idx[(size_t)t * K + threadIdx.x];
        if (e >= 0 && e < E) {
            const moe_expert_desc d = a.experts[e];
            s_blob[threadIdx.x] = d.blob;
            s_bits[threadIdx.x] = d.bits == 2 ? 2 : 4;
        } else {
            s_blob[threadIdx.x] = 0;
            s_bits[threadIdx.x] = 4;
        }
        s_w[threadIdx.x] = COMBINE ? a.w[(size_t)t * K + threadIdx.x] : 0.f;
    }
    __syncthreads();
    const int per = down_lds_per_expert(I);
    for (int k = 0; k < K; ++k) {
        const float *hk = a.h + ((size_t)t * K + k) * I;
        auto value = [&](int c) { return hk[c]; };
        uint32_t *hi = lds + k * per, *lo = hi + I / 2;
        if (s_bits[k] == 2) stage_layout<2, true>(value, I, hi, lo);
        else stage_layout<4, true>(value, I, hi, lo);
    }
    __syncthreads();
    for (int k = 0; k < K; ++k) {
        uint32_t *hi = lds + k * per;
        stage_sums<true>(I, hi, hi + I / 2, (float *)(hi + I));
    }
    __syncthreads();

    const Geo g = make_geo(I);
    constexpr int RG = dn_rg<NJ>();
    const int RB = RG * g.rpi;
    const int nblk = (H + RB - 1) / RB;
    const int wave = threadIdx.x >> 6;
    const char *res = a.residual ? (const char *)a.residual + (size_t)t * a.residual_stride * (a.residual_dtype == MOE_BF16 ? 2 : 4) : nullptr;
    for (int u = blockIdx.x * kWaves + wave; u < nblk; u += gridDim.x * kWaves) {
        const int r0 = u * RB;
        float acc[RG];
#pragma unroll
        for (int gi = 0; gi < RG; ++gi) acc[gi] = 0.f;
        for (int k = 0; k < K; ++k) {
            const uint64_t blob = s_blob[k];
            float part[RG];
#pragma unroll
            for (int gi = 0; gi < RG; ++gi) part[gi] = 0.f;
            if (blob) {
                Planes pl[3];
                expert_planes((const uint8_t *)blob, H, I, s_bits[k], pl);
                const uint32_t *hi = lds + k * per;
                const ActView v{hi, hi + I / 2, (const float *)(hi + I)};
                if (s_bits[k] == 2) down_part<2, NJ, RG>(pl[2], g, H, I, r0, RB, v, part);
                else down_part<4, NJ, RG>(pl[2], g, H, I, r0, RB, v, part);
            }
            if (COMBINE) {
#pragma unroll
                for (int gi = 0; gi < RG; ++gi) acc[gi] += s_w[k] * part[gi];
            } else {
#pragma unroll
                for (int gi = 0; gi < RG; ++gi) {
                    const float s = group_sum(part[gi], g.gsz);
                    const int rr = gi * g.rpi + g.lrow;
                    if (g.lsl == 0 && rr < RB && r0 + rr < H) a.out[((size_t)t * K + k) * H + r0 + rr] = s;
                }
            }
        }
        if (COMBINE) {
#pragma unroll
            for (int gi = 0; gi < RG; ++gi) {
                const float s = group_sum(acc[gi], g.gsz);
                const int rr = gi * g.rpi + g.lrow;
                const int r = r0 + rr;
                if (g.lsl == 0 && rr < RB && r < H)
                    a.out[(size_t)t * H + r] = s + (res ? load_act(res, a.residual_dtype, r) : 0.f);
            }
        }
    }
}

__global__ void __launch_bounds__(kBlock) k_combine(CombineLaunch a) {
    const size_t n = (size_t)a.T * a.H;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) {
        const size_t t = i / a.H, c = i - t * a.H;
        float acc = 0.f;
        for (int k = 0; k < a.K; ++k) acc += a.w[t * a.K + k] * a.y[(t * a.K + k) * a.H + c];
        a.out[i] = acc + (a.residual ? a.residual[i] : 0.f);
    }
}

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

// --------------------------------------------------------------------------- launchers
int gateup_rows_per_unit(int cols) {
    const int nj = nj_for(cols);
    return (nj == 1 ? gu_rg<1>() : nj == 2 ? gu_rg<2>() : gu_rg<4>()) * rpi_for(cols);
}
int down_rows_per_unit(int cols) {
    const int nj = nj_for(cols);
    return (nj == 1 ? dn_rg<1>() : nj == 2 ? dn_rg<2>() : dn_rg<4>()) * rpi_for(cols);
}
size_t gateup_lds_bytes(int H) { return ((size_t)2 * H + H / 32) * 4; }
size_t down_lds_bytes(int I, int K) { return (size_t)K * down_lds_per_expert(I) * 4; }

hipError_t launch_router(const RouterLaunch &a, hipStream_t s) {
    const int rpw = a.T == 1 ? 1 : 4;
    const int rows_per_block = rpw * kWaves;
    dim3 grid((a.E + rows_per_block - 1) / rows_per_block, a.T);
    const size_t lds = (size_t)a.H * 4;
    if (a.router_dtype == MOE_BF16)
        hipLaunchKernelGGL(k_router<MOE_BF16>, grid, dim3(kBlock), lds, s, a, rpw);
    else
        hipLaunchKernelGGL(k_router<MOE_F32>, grid, dim3(kBlock), lds, s, a, rpw);
    return hipGetLastError();
}

hipError_t launch_topk(const TopkLaunch &a, hipStream_t s) {
    hipLaunchKernelGGL(k_topk, dim3(a.T), dim3(64), 0, s, a);
    return hipGetLastError();
}

template <int NJ, bool SPLIT>
static hipError_t gateup_impl(const GateUpLaunch &a, hipStream_t s) {
    const int RB = gateup_rows_per_unit(a.H);
    const int units = a.K * ((a.I + RB - 1) / RB);
    dim3 grid((units + kWaves - 1) / kWaves, a.T);
    const size_t lds = gateup_lds_bytes(a.H);
    auto fn = k_gateup<NJ, SPLIT>;
    if (lds > 64 * 1024) {
        hipError_t e = hipFuncSetAttribute((const void *)fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(fn, grid, dim3(kBlock), lds, s, a);
    return hipGetLastError();
}

hipError_t launch_gateup(const GateUpLaunch &a, hipStream_t s) {
    const bool split = !(a.x_dtype == MOE_BF16 && a.norm_w == nullptr);
    switch (nj_for(a.H)) {
        case 1: return split ? gateup_impl<1, true>(a, s) : gateup_impl<1, false>(a, s);
        case 2: return split ? gateup_impl<2, true>(a, s) : gateup_impl<2, false>(a, s);
        default: return split ? gateup_impl<4, true>(a, s) : gateup_impl<4, false>(a, s);
    }
}

template <int NJ, bool COMBINE>
static hipError_t down_impl(const DownLaunch &a, int E, hipStream_t s) {
    const int RB = down_rows_per_unit(a.I);
    const int units = (a.H + RB - 1) / RB;
    dim3 grid((units + kWaves - 1) / kWaves, a.T);
    const size_t lds = down_lds_bytes(a.I, a.K);
    auto fn = k_down<NJ, COMBINE>;
    if (lds > 64 * 1024) {
        hipError_t e = hipFuncSetAttribute((const void *)fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(fn, grid, dim3(kBlock), lds, s, a, E);
    return hipGetLastError();
}

hipError_t launch_down(const DownLaunch &a, int E, hipStream_t s) {
    const bool comb = a.w != nullptr;
    switch (nj_for(a.I)) {
        case 1: return comb ? down_impl<1, true>(a, E, s) : down_impl<1, false>(a, E, s);
        case 2: return comb ? down_impl<2, true>(a, E, s) : down_impl<2, false>(a, E, s);
        default: return comb ? down_impl<4, true>(a, E, s) : down_impl<4, false>(a, E, s);
    }
}

hipError_t launch_combine(const CombineLaunch &a, hipStream_t s) {
    const size_t n = (size_t)a.T * a.H;
    size_t blocks = (n + kBlock - 1) / kBlock;
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL(k_combine, dim3((unsigned)blocks), dim3(kBlock), 0, s, a);
    return hipGetLastError();
}

}  // namespace moe
