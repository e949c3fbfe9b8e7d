// moe_decode.hip -- gfx950 kernels for the per-token MoE expert path.
//
// Kernels (one launch each, stream-ordered, no grid-wide barriers):
//   k_router : [RMSNorm] + router matvec -> logits[T][E]
//   k_topk   : softmax / top-K / renormalise (for moe_route)
//   k_gateup : every wavefront recomputes top-K from the logits (no host round trip, no grid
//              barrier), stages the activation once in LDS as digit planes in the code order,
//              and streams the gate and up rows of all K selected experts in one launch,
//              writing h = silu(g) * u
//   k_down   : down projection of all K experts for a block of output rows, combined with the
//              routing weights (+ residual) in registers before a single cross-lane reduction
//   k_combine: standalone weighted combine
//
// Dequantisation.  The affine form w = q*s + b and its FMA rewrite fma(q, s*x, b*x) come from
// the lilting.ch page "397Bパラメータモデルを48GB MacBookで動かすFlash-MoE", section "Metal
// Compute Shaders".  Summed over the 32 inputs one lane handles (half a group of 64) it becomes
// s * sum(q x) + b * sum(x), and sum(x) is computed once per slot.  Codes are never converted to
// floats (the nzkcom page lists a lookup-table dequant among its rejected experiments): the
// activation is staged once per workgroup as 16-bit fixed point per slot, in four planes of signed
// 4-bit digits, so sum(q x) is an exact integer dot product that v_dot8_i32_i4 takes eight codes
// at a time, straight from the code dwords (4-bit codes XOR 8; 2-bit codes spread to nibbles with
// one AND per parity).  The slot's scale turns it back into fp32.  Per weight this costs about a
// quarter of the vector instructions of a bf16 dot2 on unpacked codes, which matters because a
// decode step has the whole GPU's vector units for only a few microseconds.
//
// Lane geometry.  A lane "slot" is 32 consecutive input columns: 16 bytes of 4-bit codes or 8
// bytes of 2-bit codes, always inside one group of 64.  For rows of >= 64 slots, lane l takes
// slots l, l+64, ... (one coalesced 1 KiB / 512 B load per wave instruction); for shorter rows a
// wave covers several rows at once, lanes grouped by the row's slot count rounded up to a power
// of two.  Both code widths share the geometry, so experts of different widths combine in
// registers, and a lane's activation operands come from LDS once per work unit.
//
// Latency.  A decode step moves ~30 MB in a few microseconds, so each kernel is built to pay
// about two memory latencies: all independent loads (logits, descriptor table, activation,
// norm weight) are issued together; the first work unit's weight loads are issued before the
// activation layouts are written to LDS, so they are in flight while the workgroup stages.
#include "moe_device.h"

namespace moe {
namespace {

template <int RDT, bool SPLIT>
__global__ void __launch_bounds__(kBlock) k_router(RouterLaunch a) {
    extern __shared__ __align__(16) uint32_t s_r[];
    __shared__ float red[kWaves];
    float lg;
    if (router_row<RDT, SPLIT>(a, blockIdx.x, blockIdx.y, s_r, red, lg) && (threadIdx.x & 63) == 0)
        a.logits[(size_t)blockIdx.y * a.E + blockIdx.x * kWaves + (threadIdx.x >> 6)] = lg;
}

// NS > 1: the row is first summed from the batched router's NS partial rows (split order, then the
// bias) and written out.
template <int NP, int NS>
__global__ void __launch_bounds__(64) k_topk(TopkLaunch a) {
    const int t = blockIdx.x;
    float lg[NP];
    if constexpr (NS == 1) {
        issue_logits<NP>(a.logits + (size_t)t * a.E, a.E, lg);
    } else {
        const int lane = threadIdx.x & 63;
        float p[NS][NP];
#pragma unroll
        for (int q = 0; q < NS; ++q) issue_logits<NP>(a.part + ((size_t)q * a.T + t) * a.E, a.E, p[q]);
        float b[NP];
#pragma unroll
        for (int i = 0; i < NP; ++i) b[i] = a.bias ? a.bias[min(NP * lane + i, a.E - 1)] : 0.f;
#pragma unroll
        for (int i = 0; i < NP; ++i) {
            float v = p[0][i];
#pragma unroll
            for (int q = 1; q < NS; ++q) v += p[q][i];
            lg[i] = v + b[i];
            if (NP * lane + i < a.E) a.logits_out[(size_t)t * a.E + NP * lane + i] = lg[i];
        }
    }
    uint32_t key[NP];
    logit_keys<NP>(lg, a.E, key);
    int my_idx;
    float my_w;
    wave_topk<NP>(key, a.K, my_idx, my_w);
    if ((int)threadIdx.x < a.K) {
        a.idx[(size_t)t * a.K + threadIdx.x] = my_idx;
        a.w[(size_t)t * a.K + threadIdx.x] = my_w;
    }
}

template <int NJ, int NP>
__global__ void __launch_bounds__(kBlock) k_gateup(GateUpLaunch a) {
    extern __shared__ __align__(16) uint32_t lds[];
    __shared__ uint64_t s_tab[kTabMax];
    __shared__ float red[kWaves];
    constexpr int RG = gu_rg<NJ>();
    const int H = a.H, I = a.I, E = a.E, K = a.K, t = blockIdx.y;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const bool use_tab = E <= kTabMax;

    // 1. independent loads, issued back to back (straight-line code: a loop here would make the
    //    compiler wait for every outstanding load at its header): this lane's logits (first, so the
    //    routing can start when they land), descriptor table, activation chunks
    float lg[NP];
    if (!a.idx_in) issue_logits<NP>(a.logits + (size_t)t * E, E, lg);
    u32x4 dsc[kTabMax / kBlock];
    if (use_tab) {
#pragma unroll
        for (int j = 0; j < kTabMax / kBlock; ++j)
            dsc[j] = *(const GLOBAL_AS u32x4 *)(a.experts + min((int)threadIdx.x + kBlock * j, E - 1));
    }
    const void *x = (const char *)a.x + (size_t)t * a.x_stride * (a.x_dtype == MOE_BF16 ? 2 : 4);
    const int nch = H / 16;
    Chunk16 xc[2], nc[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int m = min((int)threadIdx.x + kBlock * j, nch - 1);   // clamped; extra chunks unused
        issue_chunk16(x, a.x_dtype, m, xc[j]);
        if (a.norm_w) issue_chunk16(a.norm_w, MOE_BF16, m, nc[j]);
    }

    // 2. routing in registers (each wave, identical results)
    int my_idx = 0;
    float my_w = 0.f;
    if (a.idx_in) {
        if (lane < K) my_idx = a.idx_in[(size_t)t * K + lane];
    } else {
        uint32_t key[NP];
        logit_keys<NP>(lg, E, key);
        wave_topk<NP>(key, K, my_idx, my_w);
    }

    // 3. descriptor table and RMSNorm statistics; one barrier publishes the table
    if (use_tab) {
#pragma unroll
        for (int j = 0; j < kTabMax / kBlock; ++j) {
            const int e = threadIdx.x + kBlock * j;
            if (e < E) s_tab[e] = pack_sel(((uint64_t)dsc[j].y << 32) | dsc[j].x, dsc[j].z);
        }
    }
    float v[2][16];
#pragma unroll
    for (int j = 0; j < 2; ++j) chunk16_f32(xc[j], a.x_dtype, v[j]);
    float inv = 1.f;
    if (a.norm_w) {
        float ss = 0.f;
#pragma unroll
        for (int j = 0; j < 2; ++j)
            if ((int)threadIdx.x + kBlock * j < nch) {
#pragma unroll
                for (int i = 0; i < 16; ++i) ss += v[j][i] * v[j][i];
            }
        ss = block_sum(ss, red);   // also makes s_tab visible
        inv = 1.0f / sqrtf(ss / (float)H + a.eps);
    } else {
        __syncthreads();
    }

    // 4. routing outputs and the first unit's weight loads
    if (blockIdx.x == 0 && wave == 0 && lane < K) {
        const size_t o = (size_t)t * K + lane;
        if (a.idx_out) a.idx_out[o] = my_idx;
        if (a.w_out) a.w_out[o] = my_w;
        if (a.w_ws) a.w_ws[o] = my_w;
        a.sel_ws[o] = lookup_sel(my_idx, E, use_tab, s_tab, a.experts);
    }
    const Geo g = make_geo(a.geo);
    const int RB = a.geo.rb;
    const int nblk = a.geo.nblk;
    const int units = K * nblk;
    int u = blockIdx.x * kWaves + wave;
    GULoads<NJ, RG> L;
    uint64_t sel = 0;
    Planes pl[3];
    if (u < units) {
        const int k = blk_of(u, a.geo);
        sel = lookup_sel(__builtin_amdgcn_readlane(my_idx, k), E, use_tab, s_tab, a.experts);
        if (sel) {
            expert_planes(sel_blob(sel), sel_bits(sel), a.pt, pl);
            if (sel_bits(sel) == 2) gu_issue<2, NJ, RG>(pl, g, H, I, (u - k * nblk) * RB, RB, L);
            else gu_issue<4, NJ, RG>(pl, g, H, I, (u - k * nblk) * RB, RB, L);
        }
    }

    // 5. activation digit planes for both code widths, straight from registers
    uint32_t *d4 = lds, *d2 = lds + H / 2;
    float2 *xs = (float2 *)(lds + H);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int m = threadIdx.x + kBlock * j;
        if (a.norm_w && m < nch) {
            float w[16];
            chunk16_f32(nc[j], MOE_BF16, w);
#pragma unroll
            for (int i = 0; i < 16; ++i) v[j][i] = v[j][i] * inv * w[i];
        }
        stage_chunk(m, m < nch, v[j], d4, d2, xs);
    }
    __syncthreads();
    const ActView v4{d4, xs}, v2{d2, xs};

    // 6. work units
    bool first = true;
    for (; u < units; u += gridDim.x * kWaves) {
        const int k = blk_of(u, a.geo);
        const int r0 = (u - k * nblk) * RB;
        float *hout = a.h + ((size_t)t * K + k) * I;
        if (!first) {
            sel = lookup_sel(__builtin_amdgcn_readlane(my_idx, k), E, use_tab, s_tab, a.experts);
            if (sel) {
                expert_planes(sel_blob(sel), sel_bits(sel), a.pt, pl);
                if (sel_bits(sel) == 2) gu_issue<2, NJ, RG>(pl, g, H, I, r0, RB, L);
                else gu_issue<4, NJ, RG>(pl, g, H, I, r0, RB, L);
            }
        }
        first = false;
        if (!sel) {
            for (int r = r0 + lane; r < r0 + RB && r < I; r += 64) hout[r] = 0.f;
            continue;
        }
        if (sel_bits(sel) == 2) gu_finish<2, NJ, RG, true>(g, I, r0, RB, v2, L, hout);
        else gu_finish<4, NJ, RG, true>(g, I, r0, RB, v4, L, hout);
    }
}

template <int NJ, bool COMBINE, int KM>
__global__ void __launch_bounds__(kBlock) k_down(DownLaunch a) {
    extern __shared__ __align__(16) uint32_t lds[];
    constexpr int RG = dn_rg<NJ>();
    const int H = a.H, I = a.I, K = a.K, t = blockIdx.y;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    // 0. two-launch schedule: advance the launch counter (every workgroup of the router + gate/up
    //    launch read it before this kernel started) and pick up its error word
    if (a.seq && blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) {
        const uint32_t nt = a.seq[0] + 1u;
        __hip_atomic_store(a.seq, nt ? nt : 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    // The error word is loaded without a branch (a harmless in-bounds word stands in when there is
    // none) so that its wait falls at the output stores, not here.
    const uint32_t err_word = *(const GLOBAL_AS uint32_t *)(a.err ? a.err : (const uint32_t *)a.sel);
    // 1. the selected experts, then this thread's h chunks (first pass) and the routing weights, all
    //    in flight together (branch-free clamped loads).  Loads complete in issue order, so the
    //    selections can be used -- and the first unit's weight loads issued -- while h is still on
    //    its way.
    const int per = down_lds_per_expert(I);
    const int cpe = I / 16;                         // chunks per expert
    const int nch = K * cpe;
    const float *hrow = a.h + (size_t)t * K * I;
    uint64_t sel[KM];
    float wk[KM];
#pragma unroll
    for (int k = 0; k < KM; ++k) sel[k] = ((const GLOBAL_AS uint64_t *)a.sel)[(size_t)t * K + min(k, K - 1)];
    Chunk16 hc[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) issue_chunk16(hrow, MOE_F32, min((int)threadIdx.x + kBlock * j, nch - 1), hc[j]);
#pragma unroll
    for (int k = 0; k < KM; ++k) wk[k] = COMBINE ? ((const GLOBAL_AS float *)a.w)[(size_t)t * K + min(k, K - 1)] : 0.f;
    uint32_t two_mask = 0;   // bit k: expert k has 2-bit codes
#pragma unroll
    for (int k = 0; k < KM; ++k) {
        sel[k] = k < K ? sel[k] : 0;
        wk[k] = k < K ? wk[k] : 0.f;
        if (sel_bits(sel[k]) == 2) two_mask |= 1u << k;
    }
    // the first unit's load offsets while the selections are in flight, then its weight loads
    const Geo g = make_geo(a.geo);
    const int RB = a.geo.rb;
    const int nblk = a.geo.nblk;
    int u = blockIdx.x * kWaves + wave;
    DNOffs<NJ, RG> o;
    dn_offsets<NJ, RG>(a.pt, g, H, I, min(u, nblk - 1) * RB, o);
    DLoads<NJ, RG, KM> L;
    dn_issue_all_at<NJ, RG, KM>(sel, K, o, a.h, L);    // a wave past the rows re-reads the last unit
    float v[2][16];
#pragma unroll
    for (int j = 0; j < 2; ++j) chunk16_f32(hc[j], MOE_F32, v[j]);

    // 2. stage h of every expert in its code width's digit-plane order.  The first pass works on
    //    registers only, so the weight loads just issued stay in flight meanwhile.
    auto stage = [&](int m, const float (&vv)[16]) {
        const bool valid = m < nch;
        const int kk = valid ? m / cpe : 0;
        const int mm = m - kk * cpe;
        uint32_t *d = lds + kk * per;
        const bool two = (two_mask >> kk) & 1u;
        stage_chunk(mm, valid, vv, two ? nullptr : d, two ? d : nullptr, (float2 *)(d + I / 2));
    };
#pragma unroll
    for (int j = 0; j < 2; ++j) stage(threadIdx.x + kBlock * j, v[j]);
    for (int base = 2 * kBlock; base < nch; base += 2 * kBlock) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int m = base + threadIdx.x + kBlock * j;
            issue_chunk16(hrow, MOE_F32, min(m, nch - 1), hc[j]);
        }
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            chunk16_f32(hc[j], MOE_F32, v[j]);
            stage(base + threadIdx.x + kBlock * j, v[j]);
        }
    }
    __syncthreads();

    // 3. units: all experts of a block of output rows
    const char *res = a.residual ? (const char *)a.residual + (size_t)t * a.residual_stride * (a.residual_dtype == MOE_BF16 ? 2 : 4) : nullptr;
    const bool bad = a.err && err_word != 0;
    bool first = true;
    for (; u < nblk; u += gridDim.x * kWaves) {
        const int r0 = u * RB;
        if (!first) dn_issue_all<NJ, RG, KM>(sel, K, g, H, I, r0, a.pt, L);
        first = false;
        float acc[RG];
#pragma unroll
        for (int gi = 0; gi < RG; ++gi) acc[gi] = 0.f;
#pragma unroll
        for (int k = 0; k < KM; ++k) {
            if (k >= K) break;
            float part[RG];
#pragma unroll
            for (int gi = 0; gi < RG; ++gi) part[gi] = 0.f;
            if (sel[k]) {
                const uint32_t *d = lds + k * per;
                const ActView av{d, (const float2 *)(d + I / 2)};
                const bool two = sel_bits(sel[k]) == 2;
#pragma unroll
                for (int j = 0; j < NJ; ++j) {
                    // idle lanes (slot past the row) read clamped codes against zero operands
                    const int slot = g.lsl + 64 * j;
                    uint32_t D[kSlotDw];
                    float2 xsv;
                    load_act_slot(av, slot, slot < g.spr, D, xsv);
#pragma unroll
                    for (int gi = 0; gi < RG; ++gi)
                        part[gi] += two ? slot_dot<2>(L.q[k][gi][j], D, L.sb[k][gi][j], xsv)
                                        : slot_dot<4>(L.q[k][gi][j], D, L.sb[k][gi][j], xsv);
                }
            }
            if (COMBINE) {
#pragma unroll
                for (int gi = 0; gi < RG; ++gi) acc[gi] += wk[k] * part[gi];
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
                    a.out[(size_t)t * H + r] = bad ? __uint_as_float(0x7FC00000u)
                                                   : s + (res ? load_act(res, a.residual_dtype, r) : 0.f);
            }
        }
    }
}

// Read-stream reference: every thread walks 16-byte chunks with a grid stride, four loads in
// flight, and the XOR of all dwords lands in sink[0] (one atomic per wave).
__global__ void __launch_bounds__(kBlock) k_stream_read(const u32x4 *p, size_t n16, uint32_t *sink) {
    const size_t stride = (size_t)gridDim.x * kBlock;
    size_t i = (size_t)blockIdx.x * kBlock + threadIdx.x;
    uint32_t acc = 0;
    for (; i + 3 * stride < n16; i += 4 * stride) {
        const u32x4 a = __builtin_nontemporal_load((const GLOBAL_AS u32x4 *)(p + i));
        const u32x4 b = __builtin_nontemporal_load((const GLOBAL_AS u32x4 *)(p + i + stride));
        const u32x4 c = __builtin_nontemporal_load((const GLOBAL_AS u32x4 *)(p + i + 2 * stride));
        const u32x4 d = __builtin_nontemporal_load((const GLOBAL_AS u32x4 *)(p + i + 3 * stride));
        acc ^= (a.x ^ a.y ^ a.z ^ a.w) ^ (b.x ^ b.y ^ b.z ^ b.w) ^ (c.x ^ c.y ^ c.z ^ c.w) ^ (d.x ^ d.y ^ d.z ^ d.w);
    }
    for (; i < n16; i += stride) {
        const u32x4 a = __builtin_nontemporal_load((const GLOBAL_AS u32x4 *)(p + i));
        acc ^= a.x ^ a.y ^ a.z ^ a.w;
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, o);
    if ((threadIdx.x & 63) == 0) atomicXor(sink, acc);
}

// out[t][c] = sum_k w[t][k] * y[t][k][c] (+ residual[t][c]), k in order.  k_combine4: one token per
// grid row, four columns per thread with 16-byte loads and stores (H a multiple of 4, buffers 16-byte
// aligned); k_combine: any shape, one element per thread.
typedef float fv4 __attribute__((ext_vector_type(4)));
__global__ void __launch_bounds__(kBlock) k_combine4(CombineLaunch a) {
    const int t = blockIdx.y;
    const int c4 = blockIdx.x * kBlock + threadIdx.x;
    if (c4 * 4 >= a.H) return;
    const size_t row = (size_t)t * a.H;
    fv4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int k = 0; k < a.K; ++k) {
        const float wk = a.w[t * a.K + k];
        const fv4 y = __builtin_nontemporal_load((const fv4 *)(a.y + (row * a.K + (size_t)k * a.H)) + c4);
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[j] += wk * y[j];
    }
    if (a.residual) {
        const fv4 r = ((const fv4 *)(a.residual + row))[c4];
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[j] += r[j];
    }
    ((fv4 *)(a.out + row))[c4] = acc;
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
RowGeo row_geo(int cols, int rows, int rg) {
    RowGeo r;
    r.spr = cols / 32;
    const int gsz = r.spr >= 64 ? 64 : next_pow2(r.spr);
    r.gsh = 0;
    while ((1 << r.gsh) < gsz) ++r.gsh;
    r.rpi = 64 / gsz;
    r.rb = rg * r.rpi;
    r.nblk = (rows + r.rb - 1) / r.rb;
    r.blk_mul = ((uint64_t)1 << 32) / (uint64_t)r.nblk + (((uint64_t)1 << 32) % (uint64_t)r.nblk ? 1 : 0);
    return r;
}
RowGeo gateup_geo(int H, int I) {
    const int nj = nj_for(H);
    return row_geo(H, I, nj == 1 ? gu_rg<1>() : nj == 2 ? gu_rg<2>() : gu_rg<4>());
}
RowGeo down_geo(int H, int I) {
    const int nj = nj_for(I);
    return row_geo(I, H, nj == 1 ? dn_rg<1>() : nj == 2 ? dn_rg<2>() : dn_rg<4>());
}
PlaneTable plane_table(int H, int I) {
    PlaneTable t;
    for (int b = 0; b < 2; ++b) {
        const size_t bits = b == 0 ? 2 : 4;
        const size_t cin = (size_t)I * H * bits / 8, sbin = (size_t)I * (H / 64) * 4, cout = (size_t)H * I * bits / 8;
        const size_t sbout = (size_t)H * (I / 64) * 4;
        const size_t sizes[6] = {cin, sbin, cin, sbin, cout, sbout};
        size_t off = 0;
        for (int p = 0; p < 6; ++p) {
            t.off[b][p] = off;
            off = round256(off + sizes[p]);
        }
    }
    return t;
}
size_t gateup_lds_bytes(int H) { return ((size_t)H + H / 16) * 4; }   // both orders + xs
size_t down_lds_bytes(int I, int K) { return (size_t)K * down_lds_per_expert(I) * 4; }

template <int RDT, bool SPLIT>
static hipError_t router_impl(const RouterLaunch &a, hipStream_t s, const KernelEvents &ev) {
    dim3 grid((a.E + kWaves - 1) / kWaves, a.T);
    const size_t lds = (size_t)a.H * 4;
    auto fn = k_router<RDT, SPLIT>;
    if (hipError_t e = lds_for<k_router<RDT, SPLIT>>(lds)) return e;
    return dispatch(fn, grid, dim3(kBlock), lds, s, ev, a);
}

hipError_t launch_router(const RouterLaunch &a, hipStream_t s, const KernelEvents &ev) {
    if (router_mfma_fits(a) && !ev.start && !ev.stop) return launch_router_mfma(a, s);
    if (a.router_dtype != MOE_BF16) return router_impl<MOE_F32, false>(a, s, ev);
    const bool split = !(a.x_dtype == MOE_BF16 && a.norm_w == nullptr);
    return split ? router_impl<MOE_BF16, true>(a, s, ev) : router_impl<MOE_BF16, false>(a, s, ev);
}

// Partial rows per lane are held in registers: up to 8 splits at E <= 512, 2 above (the split
// count of the batched router keeps to these).
template <int NP, int MAXS>
static hipError_t topk_np(const TopkLaunch &a, hipStream_t s) {
    switch (a.nsplit) {
        case 0:
        case 1: hipLaunchKernelGGL((k_topk<NP, 1>), dim3(a.T), dim3(64), 0, s, a); break;
        case 2: hipLaunchKernelGGL((k_topk<NP, 2>), dim3(a.T), dim3(64), 0, s, a); break;
        case 4:
            if constexpr (MAXS >= 4) { hipLaunchKernelGGL((k_topk<NP, (MAXS >= 4 ? 4 : 1)>), dim3(a.T), dim3(64), 0, s, a); break; }
            return hipErrorInvalidValue;
        case 8:
            if constexpr (MAXS >= 8) { hipLaunchKernelGGL((k_topk<NP, (MAXS >= 8 ? 8 : 1)>), dim3(a.T), dim3(64), 0, s, a); break; }
            return hipErrorInvalidValue;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_topk(const TopkLaunch &a, hipStream_t s) {
    if (a.nsplit > 1 && (!a.part || !a.logits_out)) return hipErrorInvalidValue;
    return a.E <= 512 ? topk_np<8, 8>(a, s) : topk_np<32, 2>(a, s);
}

template <int NJ, int NP>
static hipError_t gateup_impl_np(const GateUpLaunch &a, hipStream_t s, const KernelEvents &ev) {
    const int units = a.K * a.geo.nblk;
    dim3 grid((units + kWaves - 1) / kWaves, a.T);
    const size_t lds = gateup_lds_bytes(a.H);
    auto fn = k_gateup<NJ, NP>;
    if (hipError_t e = lds_for<k_gateup<NJ, NP>>(lds)) return e;
    return dispatch(fn, grid, dim3(kBlock), lds, s, ev, a);
}

template <int NJ>
static hipError_t gateup_impl(const GateUpLaunch &a, hipStream_t s, const KernelEvents &ev) {
    return a.E <= 512 ? gateup_impl_np<NJ, 8>(a, s, ev) : gateup_impl_np<NJ, 32>(a, s, ev);
}

hipError_t launch_gateup(const GateUpLaunch &a_in, hipStream_t s, const KernelEvents &ev) {
    GateUpLaunch a = a_in;
    a.geo = gateup_geo(a.H, a.I);
    a.pt = plane_table(a.H, a.I);
    switch (nj_for(a.H)) {
        case 1: return gateup_impl<1>(a, s, ev);
        case 2: return gateup_impl<2>(a, s, ev);
        default: return gateup_impl<4>(a, s, ev);
    }
}

template <int NJ, bool COMBINE, int KM>
static hipError_t down_impl_k(const DownLaunch &a, hipStream_t s, const KernelEvents &ev) {
    const int units = a.geo.nblk;
    dim3 grid((units + kWaves - 1) / kWaves, a.T);
    const size_t lds = down_lds_bytes(a.I, a.K);
    auto fn = k_down<NJ, COMBINE, KM>;
    if (hipError_t e = lds_for<k_down<NJ, COMBINE, KM>>(lds)) return e;
    return dispatch(fn, grid, dim3(kBlock), lds, s, ev, a);
}

template <int NJ, bool COMBINE>
static hipError_t down_impl(const DownLaunch &a, hipStream_t s, const KernelEvents &ev) {
    if (a.K <= 2) return down_impl_k<NJ, COMBINE, 2>(a, s, ev);
    if (a.K <= 4) return down_impl_k<NJ, COMBINE, 4>(a, s, ev);
    return down_impl_k<NJ, COMBINE, 8>(a, s, ev);
}

hipError_t launch_down(const DownLaunch &a_in, hipStream_t s, const KernelEvents &ev) {
    DownLaunch a = a_in;
    a.geo = down_geo(a.H, a.I);
    a.pt = plane_table(a.H, a.I);
    const bool comb = a.w != nullptr;
    switch (nj_for(a.I)) {
        case 1: return comb ? down_impl<1, true>(a, s, ev) : down_impl<1, false>(a, s, ev);
        case 2: return comb ? down_impl<2, true>(a, s, ev) : down_impl<2, false>(a, s, ev);
        default: return comb ? down_impl<4, true>(a, s, ev) : down_impl<4, false>(a, s, ev);
    }
}

hipError_t launch_stream_read(const void *buf, size_t bytes, uint32_t *sink, hipStream_t s) {
    int dev = 0, cus = 0;
    if (hipError_t e = hipGetDevice(&dev)) return e;
    if (hipError_t e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev)) return e;
    // two workgroups per CU measured fastest (7.06 TB/s against 6.33 with eight, 4 GiB)
    hipLaunchKernelGGL(k_stream_read, dim3((unsigned)(cus * 2)), dim3(kBlock), 0, s, (const u32x4 *)buf, bytes / 16,
                       sink);
    return hipGetLastError();
}

hipError_t launch_combine(const CombineLaunch &a, hipStream_t s) {
    auto al16 = [](const void *p) { return ((uintptr_t)p & 15) == 0; };
    if (a.H % 4 == 0 && al16(a.y) && al16(a.out) && (!a.residual || al16(a.residual)) && a.T <= 65535) {
        const dim3 grid((unsigned)((a.H / 4 + kBlock - 1) / kBlock), (unsigned)a.T);
        hipLaunchKernelGGL(k_combine4, grid, dim3(kBlock), 0, s, a);
        return hipGetLastError();
    }
    const size_t n = (size_t)a.T * a.H;
    size_t blocks = (n + kBlock - 1) / kBlock;
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL(k_combine, dim3((unsigned)blocks), dim3(kBlock), 0, s, a);
    return hipGetLastError();
}

}  // namespace moe
