// moe_grouped.hip -- batched (T > 1) expert FFN: token grouping and MFMA grouped dequant-GEMM.
//
//   k_group    : counting sort of the T*K (token, slot) pairs by expert -- histogram (LDS integer
//                atomics), exclusive prefix sum, and a scatter of the pairs into their experts'
//                ranges through per-expert LDS cursors (the order inside a range is arbitrary: each
//                output row depends on its own token only, so results do not depend on it); also
//                emits the work list of (expert, 32-token tile) and the small-expert records.
//   k_norm_rows: RMSNorm of every token row (only when the layer has a norm weight).
//   k_gu_mfma  : per (expert, token tile, 128 rows of I): G = X W_g^T and U = X W_u^T with
//                v_mfma_f32_32x32x16_bf16, then h = silu(G) * U.
//   k_dn_mfma  : per (expert, token tile, 128 rows of H): Y = h W_d^T, each row written straight
//                to y[token][slot] (the scatter back to token order; the weighted sum is
//                moe_combine).
//
// Exactness.  The B operand is the 4-bit (or 2-bit) code OR-ed into the mantissa of bf16 128.0
// (exact: 128 + q), the A operand is the bf16 activation (split into hi + lo bf16 parts when it
// is not exactly bf16, e.g. h).  Each MFMA K-step stays inside one quantisation group of 64, so
// after the four steps of a group the fp32 accumulator P holds sum_c (128 + q) x; the group's
// scale and bias are then applied in fp32: acc += s * P + (b - 128 s) * S[token][group], with
// S the token's sum of x over the group -- the affine form w = q*s + b summed per group (the FMA
// rewrite on the lilting.ch page "397Bパラメータモデルを48GB MacBookで動かすFlash-MoE", section
// "Metal Compute Shaders").  The dequantised weight is never rounded to bf16.
//
// Operand layout of v_mfma_f32_32x32x16_bf16 (checked on the device): lane l supplies row (A) or
// column (B) l % 32 and the 8 K-values 8*(l/32)..+8; accumulator element v of lane l is row
// 8*(v/4) + 4*(l/32) + v%4, column l % 32.  Within a K-step the order of the 8 K-values only has
// to agree between A and B; it follows the code unpack order (pairs (c, c+4) of a 4-bit dword,
// (c, c+8) of a 2-bit dword), so the A operand is staged in the same pair order.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "moe_internal.h"

namespace moe {
namespace {

#define GLOBAL_AS __attribute__((address_space(1)))
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef const GLOBAL_AS uint8_t *gbytes;
typedef const GLOBAL_AS uint32_t *gwords;

constexpr uint32_t kMagic = 0x43004300u;
constexpr int kTM = 32;          // tokens per tile
constexpr int kTN = 128;         // output rows per workgroup (4 waves x 32)
constexpr int kKC = 256;         // K columns staged per chunk (4 groups)
constexpr int kRowDw = kKC / 2 + 4;   // LDS dwords per token row of a chunk (padded)

__device__ __forceinline__ uint32_t bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}
__device__ __forceinline__ float bf16_f32(uint32_t b) { return __uint_as_float(b << 16); }
__device__ __forceinline__ size_t round256(size_t v) { return (v + 255) & ~(size_t)255; }
__device__ __forceinline__ float silu(float z) { return z / (1.0f + expf(-z)); }

__device__ __forceinline__ f32x16 mfma(const u32x4 a, const u32x4 b, const f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c,
                                                   0, 0, 0);
}

// B operand (8 bf16 = 128 + q) of K-step `step` for this lane's half h.
template <int BITS>
__device__ __forceinline__ u32x4 unpack_b(const u32x4 q, int step, int h) {
    u32x4 r;
    if (BITS == 4) {
        const uint32_t v = q[step];     // lane half h loaded dwords 4h..4h+3 of the group
#pragma unroll
        for (int j = 0; j < 4; ++j) r[j] = ((v >> (4 * j)) & 0x000F000Fu) | kMagic;
    } else {
        const uint32_t v = q[step];     // 2-bit: the whole group (4 dwords); pairs 4h..4h+3 of dword `step`
#pragma unroll
        for (int j = 0; j < 4; ++j) r[j] = ((v >> (2 * (4 * h + j))) & 0x00030003u) | kMagic;
    }
    return r;
}

// LDS dword offset (within a token row of the chunk) of the A operand of group gl, step, half h.
template <int BITS>
__device__ __forceinline__ int a_offset(int gl, int step, int h) {
    if (BITS == 4) return (2 * gl + h) * 16 + 4 * step;
    return (2 * gl + (step >> 1)) * 16 + 8 * (step & 1) + 4 * h;
}

// Column pair packed by activation dword d of a 32-column slot (same orders as the decode path).
template <int BITS>
__device__ __forceinline__ int pair_col(int d, int hf) {
    if (BITS == 4) return (d >> 2) * 8 + (d & 3) + 4 * hf;
    return (d >> 3) * 16 + (d & 7) + 8 * hf;
}

__device__ __forceinline__ void planes_of(uint64_t blob_addr, int R0, int C0, int R2, int C2, int bits,
                                          gbytes *q, gwords *sb) {
    // gate (R0 x C0), up (R0 x C0), down (R2 x C2)
    gbytes blob = (gbytes)blob_addr;
    const size_t c0 = (size_t)R0 * C0 * bits / 8, s0 = (size_t)R0 * (C0 / 64) * 4;
    const size_t c2 = (size_t)R2 * C2 * bits / 8;
    size_t off = 0;
    q[0] = blob + off; off = round256(off + c0);
    sb[0] = (gwords)(blob + off); off = round256(off + s0);
    q[1] = blob + off; off = round256(off + c0);
    sb[1] = (gwords)(blob + off); off = round256(off + s0);
    q[2] = blob + off; off = round256(off + c2);
    sb[2] = (gwords)(blob + off);
}

// --------------------------------------------------------------------------- grouping
__host__ __device__ __forceinline__ int pow2_at_least(int v) {
    int p = 2;
    while (p < v) p <<= 1;
    return p;
}

// Exclusive block scan (1024 threads) of N values per thread: p receives this thread's prefixes and
// tot the totals (the same in every thread).  s_w: 16 * N words of LDS.
template <int N>
__device__ __forceinline__ void block_scan(const uint32_t (&v)[N], uint32_t (&p)[N], uint32_t (&tot)[N], uint32_t *s_w) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    uint32_t inc[N];
#pragma unroll
    for (int i = 0; i < N; ++i) inc[i] = v[i];
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
#pragma unroll
        for (int i = 0; i < N; ++i) {
            const uint32_t u = (uint32_t)__shfl_up((int)inc[i], o);
            if (lane >= o) inc[i] += u;
        }
    }
    if (lane == 63) {
#pragma unroll
        for (int i = 0; i < N; ++i) s_w[16 * i + wave] = inc[i];
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < N; ++i) {
        uint32_t before = 0, t = 0;
        for (int w = 0; w < 16; ++w) {
            const uint32_t x = s_w[16 * i + w];
            before += w < wave ? x : 0u;
            t += x;
        }
        p[i] = before + inc[i] - v[i];
        tot[i] = t;
    }
    __syncthreads();
}

// Count of bin n (1..8) in a word array holding two 16-bit bins per word (bin n in word (n-1)/2).
__device__ __forceinline__ int bin_of(const uint32_t (&w)[4], int n) {
    return (int)((w[(n - 1) >> 1] >> (16 * ((n - 1) & 1))) & 0xFFFFu);
}
static_assert(kSmallTokens <= 8, "the small-list ranking packs eight token-count bins");

// Counting sort of the T*K (token, slot) pairs by expert in one 1024-thread workgroup: an LDS
// histogram, block scans of the counts, of the 32-token MFMA tiles of busy experts and of the small
// experts binned by token count, then a scatter of the pairs into their experts' ranges (through
// per-expert cursors, so the order inside a range is arbitrary: every output row depends on its own
// token only); then the MFMA work list of (expert, tile) and the small-expert records, most tokens
// first, so that the longest workgroups of the small-expert kernels start first.  (A bitonic sort
// of the keys expert * P + pair, which kept each range in pair order, took 8 us more per
// 256-token batch.)
__global__ void __launch_bounds__(1024) k_group(GroupLaunch a) {
    extern __shared__ int s_all[];
    __shared__ uint32_t s_w[64];
    const int P = a.T * a.K, E = a.E, NP2 = pow2_at_least(P);
    uint32_t *s_key = (uint32_t *)s_all;     // [NP2] pair index at each sorted position
    int *s_cnt = s_all + NP2;                // [E]
    int *s_off = s_cnt + E;                  // [E + 1]
    int *s_toff = s_off + E + 1;             // [E + 1]
    const int tid = threadIdx.x;
    for (int e = tid; e < E; e += blockDim.x) s_cnt[e] = 0;
    __syncthreads();
    auto valid = [&](int e) { return e >= 0 && e < E && a.experts[e].blob != 0; };
    for (int p = tid; p < P; p += blockDim.x) {
        const int e = a.idx[p];
        if (valid(e)) {
            atomicAdd(&s_cnt[e], 1);
        } else {
            // an index outside [0, E) or an absent expert (blob 0, e.g. not resident in an expert
            // cache) gets a zero output row, as in the decode path
            for (int c = 0; c < a.H; ++c) a.y[(size_t)p * a.H + c] = 0.f;
        }
    }
    __syncthreads();
    // thread t owns experts 2t and 2t+1 (E <= 2048)
    const int e0 = 2 * tid, e1 = 2 * tid + 1;
    const int c0 = e0 < E ? s_cnt[e0] : 0, c1 = e1 < E ? s_cnt[e1] : 0;
    const int cap = a.small_cap;
    const bool sm0 = c0 >= 1 && c0 <= cap, sm1 = c1 >= 1 && c1 <= cap;
    const int t0 = sm0 ? 0 : (c0 + kTM - 1) / kTM, t1 = sm1 ? 0 : (c1 + kTM - 1) / kTM;
    // offsets and MFMA tile offsets
    {
        const uint32_t v[2] = {(uint32_t)(c0 + c1), (uint32_t)(t0 + t1)};
        uint32_t p[2], tot[2];
        block_scan<2>(v, p, tot, s_w);
        if (e0 < E) { s_off[e0] = (int)p[0]; s_toff[e0] = (int)p[1]; }
        if (e1 < E) { s_off[e1] = (int)p[0] + c0; s_toff[e1] = (int)p[1] + t0; }
        if (tid == 0) { s_off[E] = (int)tot[0]; s_toff[E] = (int)tot[1]; *a.ntiles = (int)tot[1]; }
    }
    // small-expert list positions: bins by token count (two 16-bit bins per word), bin n starting
    // after every bin with more tokens, experts in index order inside a bin
    int pos0 = -1, pos1 = -1;
    {
        uint32_t v[4] = {0u, 0u, 0u, 0u}, p[4], tot[4];
        if (sm0) v[(c0 - 1) >> 1] += 1u << (16 * ((c0 - 1) & 1));
        if (sm1) v[(c1 - 1) >> 1] += 1u << (16 * ((c1 - 1) & 1));
        block_scan<4>(v, p, tot, s_w);
        int start[9], nsm = 0;
        for (int n = kSmallTokens; n >= 1; --n) {
            start[n] = nsm;
            nsm += n <= cap ? bin_of(tot, n) : 0;
        }
        if (sm0) pos0 = start[c0] + bin_of(p, c0);
        if (sm1) pos1 = start[c1] + bin_of(p, c1) + (sm0 && c0 == c1 ? 1 : 0);
        if (tid == 0) *a.nsmall = nsm;
    }
    // scatter: each valid pair takes the next position of its expert's range (the order inside an
    // expert's range does not matter: every output row depends on its own token only)
    __syncthreads();
    for (int e = tid; e < E; e += blockDim.x) s_cnt[e] = 0;
    __syncthreads();
    for (int p = tid; p < P; p += blockDim.x) {
        const int e = a.idx[p];
        if (valid(e)) s_key[s_off[e] + atomicAdd(&s_cnt[e], 1)] = (uint32_t)p;
    }
    __syncthreads();
    const int nv = s_off[E];
    for (int i = tid; i < nv; i += blockDim.x) a.perm[i] = (int)s_key[i];
    for (int e = tid; e <= E; e += blockDim.x) a.off[e] = s_off[e];
    for (int e = tid; e < E; e += blockDim.x) {
        const int nt = s_toff[e + 1] - s_toff[e];
        for (int j = 0; j < nt; ++j) {
            a.tiles[2 * (s_toff[e] + j)] = e;
            a.tiles[2 * (s_toff[e] + j) + 1] = j * kTM;
        }
    }
    auto small_rec = [&](int e, int n, int pos) {
        const moe_expert_desc d = a.experts[e];
        SmallRec r;
        r.blob = d.blob;
        r.e = e;
        r.n = n;
        r.base = s_off[e];
        r.bits = d.bits == 2 ? 2 : 4;
        r.pad[0] = r.pad[1] = 0;
#pragma unroll
        for (int t = 0; t < kSmallTokens; ++t) r.pair[t] = (int)s_key[r.base + min(t, n - 1)];
        a.small[pos] = r;
    };
    if (sm0) small_rec(e0, c0, pos0);
    if (sm1) small_rec(e1, c1, pos1);
}

__global__ void __launch_bounds__(256) k_norm_rows(const void *x, int x_dtype, const uint16_t *norm_w, float eps,
                                                   int H, float *out) {
    __shared__ float red[4];
    const int t = blockIdx.x;
    float ss = 0.f;
    for (int c = threadIdx.x; c < H; c += blockDim.x) {
        const float v = x_dtype == MOE_BF16 ? bf16_f32(((const uint16_t *)x)[(size_t)t * H + c])
                                             : ((const float *)x)[(size_t)t * H + c];
        ss += v * v;
    }
    for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
    __syncthreads();
    const float tot = red[0] + red[1] + red[2] + red[3];
    const float inv = 1.0f / sqrtf(tot / (float)H + eps);
    for (int c = threadIdx.x; c < H; c += blockDim.x) {
        const float v = x_dtype == MOE_BF16 ? bf16_f32(((const uint16_t *)x)[(size_t)t * H + c])
                                             : ((const float *)x)[(size_t)t * H + c];
        out[(size_t)t * H + c] = v * inv * bf16_f32(norm_w[c]);
    }
}

// --------------------------------------------------------------------------- shared GEMM pieces
// Staging of K columns [kc, kc+kKC) of the tile's tokens: each of the 256 threads owns 32 columns
// (one slot) of one token row.  The loads (16 bytes each: 4 for bf16, 8 for fp32, none for a row
// that is absent or a slot past K) are issued by xload one chunk ahead, together with that chunk's
// weight loads, and converted by xstage into the pair order of BITS (hi, and lo when SPLIT) plus
// the group sums.
template <int DT>
struct XChunk {
    u32x4 q[DT == MOE_BF16 ? 4 : 8];
};
template <int DT>
__device__ __forceinline__ void xload(const void *rowp, int kc, int K, XChunk<DT> &xc) {
    constexpr int NB = DT == MOE_BF16 ? 4 : 8;
    const int c0 = kc + 32 * (threadIdx.x & 7);
    const bool ok = rowp != nullptr && c0 < K;                 // K is a multiple of 64: all or none
    const GLOBAL_AS u32x4 *p = (const GLOBAL_AS u32x4 *)((const char *)rowp + (size_t)c0 * (DT == MOE_BF16 ? 2 : 4));
#pragma unroll
    for (int i = 0; i < NB; ++i) xc.q[i] = ok ? p[i] : u32x4{0u, 0u, 0u, 0u};
}
template <int BITS, bool SPLIT, int DT>
__device__ __forceinline__ void xstage(const XChunk<DT> &xc, uint32_t *s_hi, uint32_t *s_lo, float *s_sum) {
    const int row = threadIdx.x >> 3, slot = threadIdx.x & 7;     // 32 rows x 8 slots of 32 columns
    float v[32];
    if constexpr (DT == MOE_BF16) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const uint32_t w = xc.q[i >> 2][i & 3];
            v[2 * i] = bf16_f32(w & 0xFFFFu);
            v[2 * i + 1] = bf16_f32(w >> 16);
        }
    } else {
#pragma unroll
        for (int i = 0; i < 32; ++i) v[i] = __uint_as_float(xc.q[i >> 2][i & 3]);
    }
    uint32_t hv[32], lv[32];
    float sum = 0.f;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
        hv[i] = bf16_rne(v[i]);
        lv[i] = SPLIT ? bf16_rne(v[i] - bf16_f32(hv[i])) : 0u;
        sum += bf16_f32(hv[i]) + (SPLIT ? bf16_f32(lv[i]) : 0.f);
    }
    uint32_t *hi = s_hi + row * kRowDw + slot * 16, *lo = s_lo + row * kRowDw + slot * 16;
#pragma unroll
    for (int d = 0; d < 16; d += 4) {
        u32x4 H4, L4;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            H4[j] = hv[pair_col<BITS>(d + j, 0)] | (hv[pair_col<BITS>(d + j, 1)] << 16);
            L4[j] = lv[pair_col<BITS>(d + j, 0)] | (lv[pair_col<BITS>(d + j, 1)] << 16);
        }
        *(u32x4 *)(hi + d) = H4;
        if (SPLIT) *(u32x4 *)(lo + d) = L4;
    }
    sum += __shfl_xor(sum, 1);                                // two slots per group of 64
    if (!(slot & 1)) s_sum[row * 5 + (slot >> 1)] = sum;      // [kTM][4 groups] (row stride 5)
}

// Loads of one chunk (4 groups) of weight row `r` for this lane half: codes and (scale, bias).
template <int BITS>
__device__ __forceinline__ void load_chunk_w(gbytes q, gwords sb, int r, int cols, int kc, int h, u32x4 (&qv)[4],
                                             uint32_t (&sv)[4]) {
    const size_t rowb = (size_t)cols * BITS / 8;
    const int G = cols / 64;
#pragma unroll
    for (int gl = 0; gl < 4; ++gl) {
        const int g = min(kc / 64 + gl, G - 1);
        if (BITS == 4) qv[gl] = *(const GLOBAL_AS u32x4 *)(q + (size_t)r * rowb + (size_t)g * 32 + 16 * h);
        else qv[gl] = *(const GLOBAL_AS u32x4 *)(q + (size_t)r * rowb + (size_t)g * 16);
        sv[gl] = sb[(size_t)r * G + g];
    }
}

// acc += s * P + (b - 128 s) * S[row][gl] over this lane's 16 accumulator rows.
__device__ __forceinline__ void apply_group(f32x16 &acc, const f32x16 &P, uint32_t sbw, const float *s_sum, int gl,
                                            int h) {
    const float s = bf16_f32(sbw & 0xFFFFu), c = bf16_f32(sbw >> 16) - 128.f * s;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
        const int m = 8 * (v >> 2) + 4 * h + (v & 3);
        acc[v] += s * P[v] + c * s_sum[m * 5 + gl];
    }
}

// Tile bookkeeping shared by both GEMM kernels.
struct TileInfo {
    int e, m0, n, base;   // expert, first token of the tile within the expert, tokens in tile, offset of expert
};
__device__ __forceinline__ bool tile_info(const GroupedLaunch &a, TileInfo &ti) {
    const int tile = blockIdx.y;
    if (tile >= *a.ntiles) return false;
    ti.e = a.tiles[2 * tile];
    ti.m0 = a.tiles[2 * tile + 1];
    ti.base = a.off[ti.e];
    ti.n = min(kTM, a.off[ti.e + 1] - ti.base - ti.m0);
    return true;
}

// --------------------------------------------------------------------------- gate/up
// Activations and weights of chunk kc + kKC are requested before chunk kc is staged and multiplied
// (branch-free: past the last chunk the activation loads are off and the weight loads re-read the
// last group), so one chunk of both is always in flight behind the MFMA work.
template <int BITS, bool SPLIT>
__device__ void gu_tile(const GroupedLaunch &a, const TileInfo &ti, gbytes qg, gwords sg, gbytes qu, gwords su,
                        const int *s_tok, uint32_t *s_hi, uint32_t *s_lo, float *s_sum) {
    constexpr int DT = SPLIT ? MOE_F32 : MOE_BF16;     // the launcher picks SPLIT from the dtype
    const int H = a.H, I = a.I, lane = threadIdx.x & 63, wave = threadIdx.x >> 6, h = lane >> 5;
    const int r = blockIdx.x * kTN + wave * 32 + (lane & 31);
    const int rc = min(r, I - 1);
    f32x16 accG = {}, accU = {};
    const int trow = s_tok[threadIdx.x >> 3];
    const void *xrow = trow < 0 ? nullptr : (const char *)a.x + (size_t)trow * H * (DT == MOE_BF16 ? 2 : 4);
    XChunk<DT> xc[2];
    u32x4 q_g[2][4], q_u[2][4];
    uint32_t s_g[2][4], s_u[2][4];
    xload<DT>(xrow, 0, H, xc[0]);
    load_chunk_w<BITS>(qg, sg, rc, H, 0, h, q_g[0], s_g[0]);
    load_chunk_w<BITS>(qu, su, rc, H, 0, h, q_u[0], s_u[0]);
    auto chunk = [&](int kc, int cur) {
        xload<DT>(xrow, kc + kKC, H, xc[cur ^ 1]);
        load_chunk_w<BITS>(qg, sg, rc, H, kc + kKC, h, q_g[cur ^ 1], s_g[cur ^ 1]);
        load_chunk_w<BITS>(qu, su, rc, H, kc + kKC, h, q_u[cur ^ 1], s_u[cur ^ 1]);
        __syncthreads();                        // previous chunk fully consumed
        xstage<BITS, SPLIT, DT>(xc[cur], s_hi, s_lo, s_sum);
        __syncthreads();
        const int m = lane & 31;
#pragma unroll
        for (int gl = 0; gl < 4; ++gl) {
            if (kc + 64 * gl >= H) break;
            f32x16 Pg = {}, Pu = {};
#pragma unroll
            for (int st = 0; st < 4; ++st) {
                const int off = m * kRowDw + a_offset<BITS>(gl, st, h);
                const u32x4 A = *(const u32x4 *)(s_hi + off);
                const u32x4 Bg = unpack_b<BITS>(q_g[cur][gl], st, h), Bu = unpack_b<BITS>(q_u[cur][gl], st, h);
                Pg = mfma(A, Bg, Pg);
                Pu = mfma(A, Bu, Pu);
                if (SPLIT) {
                    const u32x4 Al = *(const u32x4 *)(s_lo + off);
                    Pg = mfma(Al, Bg, Pg);
                    Pu = mfma(Al, Bu, Pu);
                }
            }
            apply_group(accG, Pg, s_g[cur][gl], s_sum, gl, h);
            apply_group(accU, Pu, s_u[cur][gl], s_sum, gl, h);
        }
    };
    for (int kc = 0; kc < H; kc += 2 * kKC) {
        chunk(kc, 0);
        chunk(kc + kKC, 1);                     // past H: nothing to multiply, loads clamped or off
    }
    if (r < I) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int m = 8 * (v >> 2) + 4 * h + (v & 3);
            if (m < ti.n) a.hbuf[(size_t)(ti.base + ti.m0 + m) * I + r] = silu(accG[v]) * accU[v];
        }
    }
}

template <bool SPLIT>
__global__ void __launch_bounds__(256) k_gu_mfma(GroupedLaunch a) {
    __shared__ __align__(16) uint32_t s_hi[kTM * kRowDw];
    __shared__ __align__(16) uint32_t s_lo[SPLIT ? kTM * kRowDw : 4];
    __shared__ float s_sum[kTM * 5];
    __shared__ int s_tok[kTM];
    TileInfo ti;
    if (!tile_info(a, ti)) return;
    if (threadIdx.x < kTM) s_tok[threadIdx.x] = (int)threadIdx.x < ti.n ? a.perm[ti.base + ti.m0 + threadIdx.x] / a.K : -1;
    const moe_expert_desc d = a.experts[ti.e];
    gbytes q[3];
    gwords sb[3];
    const int bits = d.bits == 2 ? 2 : 4;
    planes_of(d.blob, a.I, a.H, a.H, a.I, bits, q, sb);
    __syncthreads();
    if (bits == 2) gu_tile<2, SPLIT>(a, ti, q[0], sb[0], q[1], sb[1], s_tok, s_hi, s_lo, s_sum);
    else gu_tile<4, SPLIT>(a, ti, q[0], sb[0], q[1], sb[1], s_tok, s_hi, s_lo, s_sum);
}

// --------------------------------------------------------------------------- down
template <int BITS>
__device__ void dn_tile(const GroupedLaunch &a, const TileInfo &ti, gbytes qd, gwords sd, const int *s_pair,
                        uint32_t *s_hi, uint32_t *s_lo, float *s_sum) {
    const int H = a.H, I = a.I, lane = threadIdx.x & 63, wave = threadIdx.x >> 6, h = lane >> 5;
    const int r = blockIdx.x * kTN + wave * 32 + (lane & 31);
    const int rc = min(r, H - 1);
    f32x16 acc = {};
    const int n = ti.n;
    const int hr = threadIdx.x >> 3;
    const void *hrow = hr < n ? (const void *)(a.hbuf + (size_t)(ti.base + ti.m0 + hr) * I) : nullptr;
    XChunk<MOE_F32> xc[2];
    u32x4 qv[2][4];
    uint32_t sv[2][4];
    xload<MOE_F32>(hrow, 0, I, xc[0]);
    load_chunk_w<BITS>(qd, sd, rc, I, 0, h, qv[0], sv[0]);
    auto chunk = [&](int kc, int cur) {
        xload<MOE_F32>(hrow, kc + kKC, I, xc[cur ^ 1]);
        load_chunk_w<BITS>(qd, sd, rc, I, kc + kKC, h, qv[cur ^ 1], sv[cur ^ 1]);
        __syncthreads();
        xstage<BITS, true, MOE_F32>(xc[cur], s_hi, s_lo, s_sum);
        __syncthreads();
        const int m = lane & 31;
#pragma unroll
        for (int gl = 0; gl < 4; ++gl) {
            if (kc + 64 * gl >= I) break;
            f32x16 P = {};
#pragma unroll
            for (int st = 0; st < 4; ++st) {
                const int off = m * kRowDw + a_offset<BITS>(gl, st, h);
                const u32x4 B = unpack_b<BITS>(qv[cur][gl], st, h);
                P = mfma(*(const u32x4 *)(s_hi + off), B, P);
                P = mfma(*(const u32x4 *)(s_lo + off), B, P);
            }
            apply_group(acc, P, sv[cur][gl], s_sum, gl, h);
        }
    };
    for (int kc = 0; kc < I; kc += 2 * kKC) {
        chunk(kc, 0);
        chunk(kc + kKC, 1);
    }
    if (r < H) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int m = 8 * (v >> 2) + 4 * h + (v & 3);
            if (m < n) a.y[(size_t)s_pair[m] * H + r] = acc[v];
        }
    }
}

__global__ void __launch_bounds__(256) k_dn_mfma(GroupedLaunch a) {
    __shared__ __align__(16) uint32_t s_hi[kTM * kRowDw];
    __shared__ __align__(16) uint32_t s_lo[kTM * kRowDw];
    __shared__ float s_sum[kTM * 5];
    __shared__ int s_pair[kTM];
    TileInfo ti;
    if (!tile_info(a, ti)) return;
    if (threadIdx.x < kTM) s_pair[threadIdx.x] = (int)threadIdx.x < ti.n ? a.perm[ti.base + ti.m0 + threadIdx.x] : 0;
    const moe_expert_desc d = a.experts[ti.e];
    gbytes q[3];
    gwords sb[3];
    const int bits = d.bits == 2 ? 2 : 4;
    planes_of(d.blob, a.I, a.H, a.H, a.I, bits, q, sb);
    __syncthreads();
    if (bits == 2) dn_tile<2>(a, ti, q[2], sb[2], s_pair, s_hi, s_lo, s_sum);
    else dn_tile<4>(a, ti, q[2], sb[2], s_pair, s_hi, s_lo, s_sum);
}

// --------------------------------------------------------------------------- down, h resident
// When a tile's whole h fits in LDS (I <= kDnResI), a workgroup stages it once -- bf16 hi/lo in the
// pair order of the expert's code width, plus the group sums -- and then covers kDnRB blocks of
// 128 output rows with no further barrier, the next row block's weights (all its chunks) loading
// while the current one is multiplied.  Against the chunked kernel this stages h once per 1024
// output rows instead of once per 128 and keeps two row blocks of weights in flight per wave.
constexpr int kDnResI = 1024;              // largest I staged whole (LDS ~132 KiB)
constexpr int kDnRB = 4;                   // 128-row blocks per workgroup
constexpr int kDnCh = kDnResI / kKC;       // chunks of kKC columns per row

__host__ __device__ __forceinline__ int dn_res_rowdw(int I) { return ((I + kKC - 1) / kKC) * (kKC / 2) + 4; }
size_t dn_res_lds_bytes(int I) {
    return ((size_t)2 * kTM * dn_res_rowdw(I) + (size_t)kTM * ((I + 63) / 64)) * 4;
}

template <int BITS>
__device__ void dn_res_tile(const GroupedLaunch &a, const TileInfo &ti, gbytes qd, gwords sd, const int *s_pair,
                            uint32_t *s_hi, uint32_t *s_lo, float *s_sum) {
    const int H = a.H, I = a.I, lane = threadIdx.x & 63, wave = threadIdx.x >> 6, h = lane >> 5;
    const int rs = dn_res_rowdw(I), G = (I + 63) / 64, nch = (I + kKC - 1) / kKC;
    const int n = ti.n, m = lane & 31;
    // 1. stage the tile's h: thread (row, slot) converts slot `slot` of every chunk of its token row
    {
        const int hr = threadIdx.x >> 3, slot = threadIdx.x & 7;
        const void *hrow = hr < n ? (const void *)(a.hbuf + (size_t)(ti.base + ti.m0 + hr) * I) : nullptr;
        for (int c = 0; c < nch; ++c) {
            XChunk<MOE_F32> xc;
            xload<MOE_F32>(hrow, c * kKC, I, xc);
            float v[32];
#pragma unroll
            for (int i = 0; i < 32; ++i) v[i] = __uint_as_float(xc.q[i >> 2][i & 3]);
            uint32_t hv[32], lv[32];
            float sum = 0.f;
#pragma unroll
            for (int i = 0; i < 32; ++i) {
                hv[i] = bf16_rne(v[i]);
                lv[i] = bf16_rne(v[i] - bf16_f32(hv[i]));
                sum += bf16_f32(hv[i]) + bf16_f32(lv[i]);
            }
            uint32_t *hi = s_hi + hr * rs + c * (kKC / 2) + slot * 16, *lo = s_lo + hr * rs + c * (kKC / 2) + slot * 16;
#pragma unroll
            for (int d = 0; d < 16; d += 4) {
                u32x4 H4, L4;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    H4[j] = hv[pair_col<BITS>(d + j, 0)] | (hv[pair_col<BITS>(d + j, 1)] << 16);
                    L4[j] = lv[pair_col<BITS>(d + j, 0)] | (lv[pair_col<BITS>(d + j, 1)] << 16);
                }
                *(u32x4 *)(hi + d) = H4;
                *(u32x4 *)(lo + d) = L4;
            }
            sum += __shfl_xor(sum, 1);
            const int g = c * (kKC / 64) + (slot >> 1);
            if (!(slot & 1) && g < G) s_sum[hr * G + g] = sum;
        }
    }
    __syncthreads();
    // 2. row blocks: weights of block rb+1 in flight while block rb is multiplied
    u32x4 qA[kDnCh][4], qB[kDnCh][4];
    uint32_t sA[kDnCh][4], sB[kDnCh][4];
    const int rb0 = blockIdx.x * kDnRB;
    auto rowof = [&](int rb) { return rb * kTN + wave * 32 + m; };
    auto load_rb = [&](int rb, u32x4 (&q)[kDnCh][4], uint32_t (&sv)[kDnCh][4]) {
        const int rc = min(rowof(rb), H - 1);
#pragma unroll
        for (int c = 0; c < kDnCh; ++c)
            if (c < nch) load_chunk_w<BITS>(qd, sd, rc, I, c * kKC, h, q[c], sv[c]);
    };
    auto compute_rb = [&](int rb, const u32x4 (&q)[kDnCh][4], const uint32_t (&sv)[kDnCh][4]) {
        f32x16 acc = {};
#pragma unroll
        for (int c = 0; c < kDnCh; ++c) {
            if (c >= nch) break;
#pragma unroll
            for (int gl = 0; gl < 4; ++gl) {
                const int g = c * (kKC / 64) + gl;
                if (g >= G) break;
                f32x16 P = {};
#pragma unroll
                for (int st = 0; st < 4; ++st) {
                    const int off = m * rs + c * (kKC / 2) + a_offset<BITS>(gl, st, h);
                    const u32x4 B = unpack_b<BITS>(q[c][gl], st, h);
                    P = mfma(*(const u32x4 *)(s_hi + off), B, P);
                    P = mfma(*(const u32x4 *)(s_lo + off), B, P);
                }
                const float sc = bf16_f32(sv[c][gl] & 0xFFFFu), bc = bf16_f32(sv[c][gl] >> 16) - 128.f * sc;
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int mm = 8 * (v >> 2) + 4 * h + (v & 3);
                    acc[v] += sc * P[v] + bc * s_sum[mm * G + g];
                }
            }
        }
        const int r = rowof(rb);
        if (r < H) {
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int mm = 8 * (v >> 2) + 4 * h + (v & 3);
                if (mm < n) a.y[(size_t)s_pair[mm] * H + r] = acc[v];
            }
        }
    };
    const int nrb = min(kDnRB, (H + kTN - 1) / kTN - rb0);
    load_rb(rb0, qA, sA);
    for (int i = 0; i < nrb; i += 2) {
        if (i + 1 < nrb) load_rb(rb0 + i + 1, qB, sB);
        compute_rb(rb0 + i, qA, sA);
        if (i + 2 < nrb) load_rb(rb0 + i + 2, qA, sA);
        if (i + 1 < nrb) compute_rb(rb0 + i + 1, qB, sB);
    }
}

__global__ void __launch_bounds__(256) k_dn_res(GroupedLaunch a) {
    extern __shared__ __align__(16) uint32_t s_dyn[];
    __shared__ int s_pair[kTM];
    TileInfo ti;
    if (!tile_info(a, ti)) return;
    const int rs = dn_res_rowdw(a.I);
    uint32_t *s_hi = s_dyn, *s_lo = s_dyn + kTM * rs;
    float *s_sum = (float *)(s_lo + kTM * rs);
    if (threadIdx.x < kTM) s_pair[threadIdx.x] = (int)threadIdx.x < ti.n ? a.perm[ti.base + ti.m0 + threadIdx.x] : 0;
    const moe_expert_desc d = a.experts[ti.e];
    gbytes q[3];
    gwords sb[3];
    const int bits = d.bits == 2 ? 2 : 4;
    planes_of(d.blob, a.I, a.H, a.H, a.I, bits, q, sb);
    __syncthreads();
    if (bits == 2) dn_res_tile<2>(a, ti, q[2], sb[2], s_pair, s_hi, s_lo, s_sum);
    else dn_res_tile<4>(a, ti, q[2], sb[2], s_pair, s_hi, s_lo, s_sum);
}

// --------------------------------------------------------------------------- batched router
// logits[t][e] = sum_c x[t][c] R[e][c] (+ bias[e]) for a bf16 router R, as v_mfma_f32_32x32x16_bf16
// tiles of 32 tokens (A rows) by 32 experts (B columns).  With K splits (grid z) each workgroup
// takes an equal part of the K range and writes a partial row for the top-K kernel to sum; the
// kRtWaves waves of a workgroup take equal parts of its range and meet in LDS in a fixed order
// (8 waves measured slower than 4).  Both operands come straight from
// memory with cached loads (the router rows of an expert tile are re-read by the tiles of the other
// tokens, which run on the same XCD since the grid has 16 expert tiles per token tile, and the
// token rows by the other expert tiles; 26.7 -> 22.2 us at 256 tokens against non-temporal loads):
// inside each
// block of 64 columns lane half h takes columns 32h .. 32h+31, 8 per MFMA step, for A and B alike
// (the order of the K-values inside a step only has to agree between the operands), so each lane
// reads 64 contiguous bytes of its router row per block.  Activations that are not exactly bf16
// are split into hi + lo bf16 parts, two MFMAs per step, as in the matvec router.
constexpr int kRtTile = 32;
constexpr int kRtWaves = 4;                            // waves per workgroup, each a 1/kRtWaves of K
constexpr int kRtMaxSplit = 8;                         // K splits across workgroups, at most
constexpr long kRtTargetWg = 256;                      // workgroups the splits aim for
template <bool SPLIT, int NB>
__global__ void __launch_bounds__(64 * kRtWaves) k_router_mfma(RouterLaunch a) {
    __shared__ float s_red[kRtWaves - 1][16][64];
    constexpr int XB = SPLIT ? 4 : 2;                  // activation bytes
    constexpr int XQ = SPLIT ? 8 : 4;                  // 16-byte loads of activations per block and lane
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, h = lane >> 5, m = lane & 31;
    const int H = a.H, E = a.E, T = a.T;
    // Tile of this workgroup.  Workgroup b of the grid runs on XCD b mod 8, and each XCD has its own
    // L2, so when the grid divides by 8 XCD c takes the c-th eighth of the tiles in (split, expert
    // tile, token tile) order, token tiles fastest: its workgroups share a few expert tiles' router
    // rows and one split's token rows, and every XCD fetches 1/8 of the router and a share of the
    // tokens instead of every token row (HBM fetch per launch at 256 tokens 21.1 -> 12.7 MB; the
    // kernel is latency-bound, 13.0 and 13.7 us per launch, batch time unchanged).
    const int tx = gridDim.x, ty = gridDim.y, ns = gridDim.z;
    const int nwg = tx * ty * ns;
    int L = blockIdx.x + tx * (blockIdx.y + ty * blockIdx.z);
    if (nwg % 8 == 0) L = (L % 8) * (nwg / 8) + L / 8;
    const int by = (nwg % 8 == 0) ? L % ty : blockIdx.y;
    const int bx = (nwg % 8 == 0) ? (L / ty) % tx : blockIdx.x;
    const int bz = (nwg % 8 == 0) ? L / (ty * tx) : blockIdx.z;
    const int t0 = by * kRtTile, e0 = bx * kRtTile;
    const int tok = min(t0 + m, T - 1), ex = min(e0 + m, E - 1);      // clamped rows are not written
    const int kq = H / (kRtWaves * ns), k0 = (bz * kRtWaves + wave) * kq, nblk = kq / 64;   // split bz of K
    const GLOBAL_AS uint8_t *rrow = (const GLOBAL_AS uint8_t *)a.router + ((size_t)ex * H + k0 + 32 * h) * 2;
    const GLOBAL_AS uint8_t *xrow = (const GLOBAL_AS uint8_t *)a.x + ((size_t)tok * a.x_stride + k0 + 32 * h) * XB;
    // NB blocks in flight per wave; NB divides nblk, so no load runs past the wave's range
    u32x4 bq[NB][4], xq[NB][XQ];
    auto load = [&](int blk, int buf) {
#pragma unroll
        for (int i = 0; i < 4; ++i) bq[buf][i] = *(const GLOBAL_AS u32x4 *)(rrow + (size_t)blk * 128 + 16 * i);
#pragma unroll
        for (int i = 0; i < XQ; ++i) xq[buf][i] = *(const GLOBAL_AS u32x4 *)(xrow + (size_t)blk * 64 * XB + 16 * i);
    };
    f32x16 acc = {};
    auto compute = [&](int buf) {
#pragma unroll
        for (int st = 0; st < 4; ++st) {
            if constexpr (SPLIT) {
                u32x4 hi, lo;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const uint32_t w0 = xq[buf][2 * st + (j >> 1)][2 * (j & 1)], w1 = xq[buf][2 * st + (j >> 1)][2 * (j & 1) + 1];
                    const float f0 = __uint_as_float(w0), f1 = __uint_as_float(w1);
                    const uint32_t h0 = bf16_rne(f0), h1 = bf16_rne(f1);
                    hi[j] = h0 | (h1 << 16);
                    lo[j] = bf16_rne(f0 - bf16_f32(h0)) | (bf16_rne(f1 - bf16_f32(h1)) << 16);
                }
                acc = mfma(hi, bq[buf][st], acc);
                acc = mfma(lo, bq[buf][st], acc);
            } else {
                acc = mfma(xq[buf][st], bq[buf][st], acc);
            }
        }
    };
#pragma unroll
    for (int i = 0; i < NB; ++i) load(i, i);
    for (int b = 0; b < nblk; b += NB) {
        if (b + NB < nblk) {
#pragma unroll
            for (int i = 0; i < NB; ++i) {
                compute(i);
                load(b + NB + i, i);
            }
        } else {
#pragma unroll
            for (int i = 0; i < NB; ++i) compute(i);
        }
    }
    if (wave > 0) {
#pragma unroll
        for (int v = 0; v < 16; ++v) s_red[wave - 1][v][lane] = acc[v];
    }
    __syncthreads();
    if (wave == 0) {
        const int e = e0 + m;
        const bool part = ns > 1;                      // partial row of this split, no bias
        const float bias = (!part && a.logit_bias && e < E) ? a.logit_bias[e] : 0.f;
        float *out = part ? a.part_ws + (size_t)bz * T * E : a.logits;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            float sum = acc[v];
#pragma unroll
            for (int q = 0; q < kRtWaves - 1; ++q) sum += s_red[q][v][lane];
            const int t = t0 + 8 * (v >> 2) + 4 * h + (v & 3);
            if (t < T && e < E) out[(size_t)t * E + e] = sum + bias;
        }
    }
}

}  // namespace

// --------------------------------------------------------------------------- launchers
int grouped_max_tiles(int T, int K, int E) {
    const int P = T * K;
    return (P + kTM - 1) / kTM + (E < P ? E : P);
}

size_t group_lds_bytes(int T, int K, int E) { return ((size_t)pow2_at_least(T * K) + 3 * (size_t)E + 2) * 4; }

hipError_t launch_group(const GroupLaunch &a, hipStream_t s) {
    if (grouped_max_tiles(a.T, a.K, a.E) >= (1 << 16)) return hipErrorInvalidValue;   // packed scan word
    const size_t lds = group_lds_bytes(a.T, a.K, a.E);
    if (hipError_t e = lds_for<k_group>(lds)) return e;
    hipLaunchKernelGGL(k_group, dim3(1), dim3(1024), lds, s, a);
    return hipGetLastError();
}

hipError_t launch_norm_rows(const void *x, int x_dtype, const uint16_t *norm_w, float eps, int H, int T, float *out,
                            hipStream_t s) {
    hipLaunchKernelGGL(k_norm_rows, dim3(T), dim3(256), 0, s, x, x_dtype, norm_w, eps, H, out);
    return hipGetLastError();
}

int router_mfma_splits(int H, int E, int T) {
    // a workgroup per CU at least: a 32 x 32 tile over the whole K range reads 512 KiB at H = 4096,
    // and with 128 tiles (256 tokens) half the CUs would carry it (21.5 -> 17.7 us for the route call
    // of 256 tokens of 512 experts with two splits; four and eight measured the same within 0.5 %)
    const long tiles = (long)((E + kRtTile - 1) / kRtTile) * ((T + kRtTile - 1) / kRtTile);
    const int maxs = E <= 512 ? kRtMaxSplit : 2;       // the top-K kernel's registers per partial row
    int ns = 1;
    while (ns < maxs && tiles * ns < kRtTargetWg && H % (64 * kRtWaves * ns * 2) == 0) ns *= 2;
    return ns;
}

bool router_mfma_fits(const RouterLaunch &a) {
    return a.router_dtype == MOE_BF16 && a.T >= kRouterMfmaMinT && a.H % (64 * kRtWaves) == 0 &&
           (a.norm_w == nullptr || a.xn_ws != nullptr);
}

hipError_t launch_router_mfma(const RouterLaunch &a_in, hipStream_t s) {
    RouterLaunch a = a_in;
    if (a.norm_w) {
        // RMSNorm of every row into the workspace, then the fp32 rows feed the MFMA tiles
        if (hipError_t e = launch_norm_rows(a.x, a.x_dtype, a.norm_w, a.eps, a.H, a.T, a.xn_ws, s)) return e;
        a.x = a.xn_ws;
        a.x_dtype = MOE_F32;
        a.x_stride = a.H;
        a.norm_w = nullptr;
    }
    const int ns = a.part_ws ? router_mfma_splits(a.H, a.E, a.T) : 1;
    const dim3 grid((a.E + kRtTile - 1) / kRtTile, (a.T + kRtTile - 1) / kRtTile, ns);
    const int nblk = a.H / (64 * kRtWaves * ns);       // 64-column blocks per wave
    const dim3 blk(64 * kRtWaves);
    const bool bf = a.x_dtype == MOE_BF16;
    if (nblk % 4 == 0) {
        if (bf) hipLaunchKernelGGL((k_router_mfma<false, 4>), grid, blk, 0, s, a);
        else hipLaunchKernelGGL((k_router_mfma<true, 4>), grid, blk, 0, s, a);
    } else if (nblk % 2 == 0) {
        if (bf) hipLaunchKernelGGL((k_router_mfma<false, 2>), grid, blk, 0, s, a);
        else hipLaunchKernelGGL((k_router_mfma<true, 2>), grid, blk, 0, s, a);
    } else {
        if (bf) hipLaunchKernelGGL((k_router_mfma<false, 1>), grid, blk, 0, s, a);
        else hipLaunchKernelGGL((k_router_mfma<true, 1>), grid, blk, 0, s, a);
    }
    return hipGetLastError();
}

static hipError_t grouped_down_mfma(const GroupedLaunch &a, int max_tiles, hipStream_t s);

// The MFMA chain (busy experts) and the small-expert chain touch disjoint rows of h and y, so with a
// side stream they run concurrently: the MFMA kernels have few, long, latency-bound workgroups and
// the small-expert kernels fill the rest of the machine.  Without one they run in sequence.
hipError_t launch_grouped_ffn(const GroupedLaunch &a, int max_tiles, int max_small, hipStream_t s,
                              const SideStream *side) {
    const bool fork = side != nullptr && max_small > 0;
    // Which chain goes to the side stream, and first: issued eagerly, the MFMA chain on the side
    // stream, enqueued first (548 us per 256-token batch, against 581-583 us for the other two
    // arrangements); captured into a graph, whose replay dispatches the branches in another order,
    // the small-expert chain on the side stream, enqueued first (553 us, against 580-581 us).
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    if (fork)
        if (hipError_t e = hipStreamIsCapturing(s, &cap)) return e;
    const bool small_first = cap == hipStreamCaptureStatusActive;
    hipStream_t sm = s, ss = s;
    if (fork) {
        if (hipError_t e = hipEventRecord(side->fork, s)) return e;
        if (hipError_t e = hipStreamWaitEvent(side->stream, side->fork, 0)) return e;
        (small_first ? ss : sm) = side->stream;
    }
    auto small_chain = [&]() -> hipError_t {
        if (max_small > 0) {
            if (hipError_t e = launch_small_gateup(a, max_small, ss)) return e;
            if (hipError_t e = launch_small_down(a, max_small, ss)) return e;
        }
        return hipSuccess;
    };
    if (small_first)
        if (hipError_t e = small_chain()) return e;
    const bool split = a.x_dtype != MOE_BF16;
    dim3 g1((a.I + kTN - 1) / kTN, max_tiles);
    if (split) hipLaunchKernelGGL(k_gu_mfma<true>, g1, dim3(256), 0, sm, a);
    else hipLaunchKernelGGL(k_gu_mfma<false>, g1, dim3(256), 0, sm, a);
    if (hipError_t e = hipGetLastError()) return e;
    if (hipError_t e = grouped_down_mfma(a, max_tiles, sm)) return e;
    if (!small_first)
        if (hipError_t e = small_chain()) return e;
    if (fork) {
        if (hipError_t e = hipEventRecord(side->join, side->stream)) return e;
        if (hipError_t e = hipStreamWaitEvent(s, side->join, 0)) return e;
    }
    return hipSuccess;
}

static hipError_t grouped_down_mfma(const GroupedLaunch &a, int max_tiles, hipStream_t s) {
    if (a.I <= kDnResI) {
        const size_t lds = dn_res_lds_bytes(a.I);
        if (hipError_t e = lds_for<k_dn_res>(lds)) return e;
        dim3 g2(((a.H + kTN - 1) / kTN + kDnRB - 1) / kDnRB, max_tiles);
        hipLaunchKernelGGL(k_dn_res, g2, dim3(256), lds, s, a);
        return hipGetLastError();
    }
    dim3 g2((a.H + kTN - 1) / kTN, max_tiles);
    hipLaunchKernelGGL(k_dn_mfma, g2, dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace moe
