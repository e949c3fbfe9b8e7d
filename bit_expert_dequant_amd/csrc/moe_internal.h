// moe_internal.h -- launchers shared between the C-ABI layer and the HIP kernels.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

#include <atomic>
#include <mutex>

#include "moe_dequant.h"

namespace moe {

constexpr int kGroup = 64;

// Optional start/stop events of one launch.  When either is set the kernel goes out through
// hipExtLaunchKernel, which stamps the events with the dispatch's own start and end times, so
// hipEventElapsedTime(start, stop) is the kernel's execution time alone.
struct KernelEvents {
    hipEvent_t start = nullptr, stop = nullptr;
};

// Dynamic LDS beyond the default 64 KiB: the kernel's limit is raised only when a launch needs more
// than it was last raised to on this device (a per-kernel, per-device high-water mark), so repeated
// launches -- those recorded under stream capture included -- make no attribute call.
constexpr size_t kCuLds = 160 * 1024;
template <auto FN>
inline hipError_t lds_for(size_t lds) {
    if (lds <= 64 * 1024) return hipSuccess;
    static std::atomic<uint32_t> mark[64];
    int dev = 0;
    if (hipError_t e = hipGetDevice(&dev)) return e;
    if (dev >= 0 && dev < 64 && mark[dev].load(std::memory_order_acquire) >= lds) return hipSuccess;
    static std::mutex mu;                         // raises are serialised: the limit only grows
    std::lock_guard<std::mutex> lock(mu);
    if (dev >= 0 && dev < 64 && mark[dev].load(std::memory_order_relaxed) >= lds) return hipSuccess;
    if (hipError_t e = hipFuncSetAttribute((const void *)FN, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds))
        return e;
    if (dev >= 0 && dev < 64) mark[dev].store((uint32_t)lds, std::memory_order_release);
    return hipSuccess;
}

template <typename F, typename A>
inline hipError_t dispatch(F fn, dim3 grid, dim3 block, size_t lds, hipStream_t s, const KernelEvents &ev,
                           const A &a) {
    if (ev.start || ev.stop) hipExtLaunchKernelGGL(fn, grid, block, (uint32_t)lds, s, ev.start, ev.stop, 0u, a);
    else hipLaunchKernelGGL(fn, grid, block, lds, s, a);
    return hipGetLastError();
}

// Lane geometry of one matrix family (rows of `cols` inputs), computed on the host so that the
// kernels do no integer division: 32-column slots per row, lanes per row group (2^gsh), rows per
// wave instruction, rows per work unit, row blocks per matrix, and the multiplier with which
// (u * blk_mul) >> 32 == u / nblk for every unit index u < 2^16.
struct RowGeo {
    int spr, gsh, rpi, rb, nblk;
    uint64_t blk_mul;
};
// Byte offsets of the six planes of an expert blob, for 2-bit ([0]) and 4-bit ([1]) experts.
struct PlaneTable {
    uint64_t off[2][6];
};
RowGeo row_geo(int cols, int rows, int rg);   // rg: wave instructions (row groups) per unit
RowGeo gateup_geo(int H, int I);   // gate/up rows: I rows of H inputs
RowGeo down_geo(int H, int I);     // down rows: H rows of I inputs
PlaneTable plane_table(int H, int I);

// Rows of the gate/up matrices one wavefront handles per work unit, for a given
// input width (cols) at 4-bit; the 2-bit path covers the same rows.
int gateup_rows_per_unit(int cols);
// Output rows of the down projection one wavefront handles per work unit.
int down_rows_per_unit(int cols);
size_t gateup_lds_bytes(int H);
size_t down_lds_bytes(int I, int K);

struct RouterLaunch {
    const void *x; int x_dtype; int x_stride;     // x [T][x_stride]
    const uint16_t *norm_w; float eps;
    const void *router; int router_dtype;
    const float *logit_bias;
    float *logits;                                 // [T][E]
    int H, E, T;
    float *xn_ws;                                  // [T][H] workspace for normalised rows, or NULL
    float *part_ws;                                // [splits][T][E] partial logits of the MFMA router's K
                                                   // splits (then summed by the top-K kernel), or NULL
};
hipError_t launch_router(const RouterLaunch &a, hipStream_t s, const KernelEvents &ev = {});
// Batched bf16 router as MFMA tiles (moe_grouped.hip); false when the shape does not fit it.  From
// kRouterMfmaMinT tokens on: below that the tiles are too few to fill the GPU (16 workgroups up to
// 32 tokens at E = 512) and the matvec router, whose workgroups each take 4 experts of one token,
// is faster.
constexpr int kRouterMfmaMinT = 64;
bool router_mfma_fits(const RouterLaunch &a);
// K splits of the MFMA router for T tokens (1: one workgroup per 32 x 32 tile sums the whole K range
// and writes the logits itself).  With more than one, each split writes a partial row and the top-K
// kernel adds them in split order.
int router_mfma_splits(int H, int E, int T);
hipError_t launch_router_mfma(const RouterLaunch &a, hipStream_t s);

struct TopkLaunch {
    const float *logits; int E, K, T;
    int32_t *idx; float *w;                        // [T][K]
    // nsplit > 1: the logits are the sum of nsplit partial rows part[s][T][E] (in split order) plus
    // bias (nullable), written to logits_out; `logits` is not read
    const float *part; int nsplit; const float *bias; float *logits_out;
};
hipError_t launch_topk(const TopkLaunch &a, hipStream_t s);

struct GateUpLaunch {
    const void *x; int x_dtype; int x_stride;      // activation source [T][x_stride]
    const uint16_t *norm_w; float eps;             // RMSNorm applied to x when norm_w != NULL
    const float *logits;                           // [T][E]: top-K computed here when idx_in == NULL
    const int32_t *idx_in;                         // [T][K] given routing, or NULL
    int32_t *idx_out; float *w_out;                // [T][K] routing results (nullable)
    uint64_t *sel_ws;                              // [T][K] selected blob address | code width, for down
    float *w_ws;                                   // [T][K] routing weights for down (nullable)
    const moe_expert_desc *experts;
    float *h;                                      // [T][K][I]
    int H, I, E, K, T;
    RowGeo geo; PlaneTable pt;                     // set by launch_gateup
};
hipError_t launch_gateup(const GateUpLaunch &a, hipStream_t s, const KernelEvents &ev = {});

struct DownLaunch {
    const float *h;                                // [T][K][I]
    uint32_t *seq;                                 // two-launch schedule: advance this launch counter, or NULL
    const uint32_t *err;                           // two-launch schedule: nonzero -> NaN outputs, or NULL
    const uint64_t *sel;                           // [T][K] blob address | code width (0: no expert)
    const float *w;                                // [T][K] (combine) or NULL (per-expert output)
    const void *residual; int residual_dtype; int residual_stride;   // [T][stride] or NULL
    float *out;                                    // combine: [T][H]; else y [T][K][H]
    int H, I, K, T;
    RowGeo geo; PlaneTable pt;                     // set by launch_down
};
hipError_t launch_down(const DownLaunch &a, hipStream_t s, const KernelEvents &ev = {});

// Batched path (T > 1): grouping of the T*K (token, slot) pairs by expert, then grouped GEMMs.
// Experts with at most kSmallTokens tokens in a batch take the integer dot-product kernels (work
// proportional to their tokens); busier experts take the MFMA tiles of 32 tokens.
constexpr int kSmallTokens = 8;

// Work of one workgroup row of the integer dot-product kernels: an expert and up to CAP of its
// (token, slot) pairs.  The small-expert list holds CAP = kSmallTokens records (one 64-byte load
// each); the shared-read path builds CAP = kSharedCap records inside the kernels.
template <int CAP>
struct TokRec {
    uint64_t blob;                                 // the expert's blob address
    int32_t e, n, base, bits;                      // expert, pairs (1..CAP), first sorted position, code width
    int32_t pad[2];
    int32_t pair[CAP];                             // pair index (t*K + k) of its tokens, in expert order
};
using SmallRec = TokRec<kSmallTokens>;
static_assert(sizeof(SmallRec) == 64, "SmallRec is one 64-byte record");

// Shared-read path for a few tokens (2 <= T <= kSharedMaxT, T*K <= 64): the kernels derive the
// distinct experts of the call from idx themselves (no grouping pass) and every workgroup stages
// the activation rows of all pairs that chose its expert, so each selected expert's weights are
// streamed once per call whatever the overlap between the tokens' selections.
constexpr int kSharedMaxT = 16;
constexpr int kSharedCap = 16;                     // pairs of one expert per workgroup record
constexpr int kSharedMaxPairs = 64;                // T*K: one wavefront derives the records

struct GroupLaunch {
    const int32_t *idx; int T, K, E;
    const moe_expert_desc *experts;
    int32_t *off;                                  // [E+1] first sorted position of each expert
    int32_t *perm;                                 // [T*K] pair index (t*K+k) in expert order
    int32_t *tiles;                                // [2*max_tiles] (expert, first token) per MFMA tile
    int32_t *ntiles;                               // [1]
    SmallRec *small;                               // [min(E, T*K)] experts with 1..small_cap tokens,
                                                   // most tokens first (ties: lower expert first)
    int32_t *nsmall;                               // [1]
    int small_cap;                                 // kSmallTokens, or 0: every expert takes MFMA tiles
    float *y; int H;                               // rows of out-of-range pairs are zeroed
};
int grouped_max_tiles(int T, int K, int E);
size_t group_lds_bytes(int T, int K, int E);
hipError_t launch_group(const GroupLaunch &a, hipStream_t s);
hipError_t launch_norm_rows(const void *x, int x_dtype, const uint16_t *norm_w, float eps, int H, int T, float *out,
                            hipStream_t s);

struct GroupedLaunch {
    const void *x; int x_dtype;                    // [T][H] activation fed to the experts
    int H, I, K;
    const moe_expert_desc *experts;
    const int32_t *off, *perm, *tiles, *ntiles;
    const SmallRec *small; const int32_t *nsmall;
    float *hbuf;                                   // [T*K][I] SwiGLU outputs in expert order
    float *y;                                      // [T*K][H]
    RowGeo geo; PlaneTable pt;                     // set by the small-expert launchers
    int upw;                                       // work units per wavefront (1..8), set by the launchers
    // shared-read path only: the routing, the rows a gate/up (4 or 8) and a down (cap or 2 cap)
    // workgroup stages at a time, the
    // layer's norm weight, and the pre-staged rows [T][H + H/16]
    const int32_t *idx; int T, E, cap, cap_dn;
    const uint16_t *norm_w; float norm_eps;
    uint32_t *planes;
};
// A second stream of the device with its fork and join events (see launch_grouped_ffn).
struct SideStream {
    hipStream_t stream;
    hipEvent_t fork, join;
};
hipError_t launch_grouped_ffn(const GroupedLaunch &a, int max_tiles, int max_small, hipStream_t s,
                              const SideStream *side);
// Integer dot-product kernels for the small experts (moe_batched8.hip); false when the shapes do
// not fit them (everything then takes the MFMA tiles).
bool small_path_fits(int H, int I);
hipError_t launch_small_gateup(const GroupedLaunch &a, int max_small, hipStream_t s);
// Shared-read path (moe_batched8.hip): gate/up then down for T*K <= kSharedMaxPairs pairs; false
// from shared_path_fits when the staged rows and the record table do not fit in LDS.
bool shared_path_fits(int H, int I, int E, int T);
// The staging and gate/up launches of the path (moe_shared_gu.hip), or the gate/up launch staging its
// rows from x (moe_shared_gux.hip: no norm weight); a.cap, a.geo and a.pt set.
hipError_t launch_shared_gateup(const GroupedLaunch &a, hipStream_t s, const KernelEvents &ev);
hipError_t launch_shared_gateup_direct(const GroupedLaunch &a, hipStream_t s, const KernelEvents &ev);
hipError_t launch_shared_ffn(const GroupedLaunch &a, hipStream_t s, const KernelEvents &gu_ev = {},
                             const KernelEvents &dn_ev = {});
hipError_t launch_small_down(const GroupedLaunch &a, int max_small, hipStream_t s);

// Router + gate/up of one decode token in one launch (two groups of workgroups; the logits pass
// through tagged workspace words, see moe_layer.hip).  The down kernel follows on the stream.
struct LayerLaunch {
    RouterLaunch r;                                // x, norm, router, logit bias (logits unused), T = 1
    const moe_expert_desc *experts;
    int32_t *idx_out; float *w_out;                // [K] routing results, or NULL
    uint64_t *sel_ws; float *w_ws;                 // [K] selections and weights for the down kernel
    float *h;                                      // [K][I] SwiGLU outputs
    int H, I, E, K;
    int split;                                     // router activation not exactly bf16: hi/lo split
    const uint32_t *seq;                           // launch counter (advanced by the down kernel)
    uint64_t *slots;                               // [layer_logit_copies()][E] tag << 32 | logit bits
    uint32_t *err;                                 // timed-out waits (nonzero: the down kernel writes NaN)
    int clear_err;                                 // nonzero: the first workgroup zeroes *err first (per-call errors)
    int nr, ng;                                    // workgroups per group (set by launch_layer)
    RowGeo geo; PlaneTable pt;                     // gate/up geometry (set by launch_layer)
};
void layer_grid(int H, int I, int E, int K, int *nr, int *ng);
int layer_logit_copies();
size_t layer_lds_bytes(int H, int E);
hipError_t launch_layer(const LayerLaunch &a, hipStream_t s, const KernelEvents &ev = {});

// One decode layer in a single launch of a persistent grid (moe_fused.hip): nw workgroups, all
// resident at once, each computing router rows, its gate/up and down units; the logits and h pass
// between them through tagged workspace words.
struct FusedLaunch {
    LayerLaunch L;                                 // router + gate/up part (nr, ng, sel_ws, w_ws unused)
    const void *residual; int residual_dtype;      // [H] added to the output, or NULL
    float *out;                                    // [H]
    uint32_t *flags;                               // [fused_flag_copies()][fused_max_workgroups()]
    uint32_t *seq;                                 // the launch counter (L.seq), advanced by workgroup 0
    int nw;                                        // workgroups (fused_workgroups)
    RowGeo dgeo;                                   // down geometry (set by launch_layer_fused)
};
int fused_flag_copies();
int fused_max_workgroups();
// Workgroups for a layer of this shape on the current device: as many as the layer has router rows
// or units of four waves, at most as many as can be resident at once.
hipError_t fused_workgroups(int H, int I, int E, int K, int *nw);
hipError_t launch_layer_fused(const FusedLaunch &a, hipStream_t s, const KernelEvents &ev = {});

// moe_layer_decode behind its argument checks, on a given workspace.  per_call_errors: a timed-out
// wait makes only the call it happens in write NaN (the error word is cleared at each call's start)
// instead of every later call on the workspace.
int layer_decode_entry(const moe_dims *dims, const moe_layer *layers, int n_layers, const void *x, int x_dtype,
                       unsigned flags, float *out, int32_t *idx, float *w, void *ws, size_t ws_bytes, void *stream,
                       void *const *events, bool per_call_errors);
size_t layer_decode_ws_bytes(const moe_dims *dims);   // 0 for invalid dims
int set_error(int status, const char *msg);           // records the thread's error message, returns status

struct CombineLaunch {
    const float *y; const float *w; const float *residual; float *out;
    int T, K, H;
};
hipError_t launch_combine(const CombineLaunch &a, hipStream_t s);

// Quantise-from-float of an R x C matrix into the packed code and (scale, bias) planes.
struct QuantLaunch {
    const void *w; int w_dtype;                    // [rows][cols] fp32 or bf16
    int rows, cols, bits;
    uint8_t *codes;                                // packed code plane
    uint16_t *sb;                                  // (scale, bias) plane
};
hipError_t launch_quantize(const QuantLaunch &a, hipStream_t s);

// Tiered store policy: usage histogram, hot order, re-tiering (moe_tier.hip).
hipError_t launch_usage(const int32_t *idx, size_t n, int E, uint32_t *counts, hipStream_t s);
hipError_t launch_hot_order(const uint32_t *counts, int E, int32_t *order, hipStream_t s);
struct RetierLaunch {
    const moe_expert_desc *base;                   // [E] the base table (blobs read)
    const int32_t *order;                          // [E] experts by rank; the first n_hot are hot
    int E, H, I, n_hot, cold_bits;
    void *store;                                   // (E - n_hot) cold blobs, cold_bytes apart
    size_t cold_bytes;
    moe_expert_desc *tiered;                       // [E] written last (may be base)
};
hipError_t launch_retier(const RetierLaunch &r, hipStream_t s);

// Expert cache: descriptor-table writes (moe_cache.hip).  An update list names each expert at most
// once; entries with blob 0 mark absent experts.
hipError_t launch_table_absent(moe_expert_desc *table, int E, hipStream_t s);
hipError_t launch_table_update(moe_expert_desc *table, int n, const int32_t *expert, const uint64_t *blob,
                               const uint32_t *bits, hipStream_t s);

// Device-side cache policy (moe_cache.hip).  The state is one device buffer of 32-bit words:
//   header [kCacheHdr]: n_used, head, tail (LRU list ends, -1 when empty), n_copy, refused steps,
//                       then hits, misses, bytes as 64-bit counters
//   slot_of [E] (slot of each expert or -1), expert_of [S], prev [S], next [S] (the LRU list of
//   occupied slots, least recent first), copy [2 S] (slot, expert of this step's loads),
//   src [E] 64-bit device addresses of the pinned host blobs, nbytes [E], bits [E].
constexpr int kCacheHdr = 16;
constexpr int kCacheMaxSlots = 2048;
struct CacheLayout {
    size_t slot_of, expert_of, prev, next, copy, src, nbytes, bits, words;
};
__host__ __device__ inline CacheLayout cache_layout(int E, int S) {
    CacheLayout l;
    size_t o = kCacheHdr;
    l.slot_of = o; o += (size_t)E;
    l.expert_of = o; o += (size_t)S;
    l.prev = o; o += (size_t)S;
    l.next = o; o += (size_t)S;
    l.copy = o; o += 2 * (size_t)S;
    o = (o + 1) & ~(size_t)1;                      // 8-byte alignment of the addresses
    l.src = o; o += 2 * (size_t)E;
    l.nbytes = o; o += (size_t)E;
    l.bits = o; o += (size_t)E;
    l.words = o;
    return l;
}
struct CacheDevLaunch {
    uint32_t *state;
    int E, S;
    moe_expert_desc *table;
    uint8_t *slots;
    uint64_t slot_bytes;
};
size_t cache_policy_lds_bytes(int E, int S);
hipError_t launch_cache_fetch_device(const CacheDevLaunch &c, const int32_t *idx, int n, hipStream_t s);

// Read-stream reference kernel (XOR of every dword of buf into *sink).
hipError_t launch_stream_read(const void *buf, size_t bytes, uint32_t *sink, hipStream_t s);

}  // namespace moe
