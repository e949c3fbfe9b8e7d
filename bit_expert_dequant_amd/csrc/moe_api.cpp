// moe_api.cpp -- C ABI entry points: argument validation, the packed-format packer, workspace
// sizing and kernel dispatch.  Every check runs before anything is enqueued, so a failing call
// leaves the stream untouched.
#include <hip/hip_runtime_api.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <algorithm>
#include <atomic>
#include <cstring>
#include <map>
#include <mutex>
#include <set>
#include <tuple>
#include <string>
#include <utility>
#include <vector>

#include "moe_dequant.h"
#include "moe_internal.h"

namespace {

thread_local std::string g_err;

int fail(int status, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = std::string(moe_status_string(status)) + ": " + buf;
    return status;
}
int ok() {
    g_err.clear();
    return MOE_OK;
}

size_t r256(size_t v) { return (v + 255) & ~(size_t)255; }
bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }
bool bits_ok(int b) { return b == 2 || b == 4; }
bool dim_ok(int v) { return v >= 64 && v <= MOE_MAX_DIM && v % MOE_GROUP == 0; }

int check_dims(const moe_dims *d) {
    if (!d) return fail(MOE_ERR_NULL, "dims is NULL");
    if (!dim_ok(d->hidden)) return fail(MOE_ERR_SHAPE, "hidden=%d must be a multiple of 64 in [64, %d]", d->hidden, MOE_MAX_DIM);
    if (!dim_ok(d->inter)) return fail(MOE_ERR_SHAPE, "inter=%d must be a multiple of 64 in [64, %d]", d->inter, MOE_MAX_DIM);
    if (d->n_experts < 1 || d->n_experts > MOE_MAX_EXPERTS)
        return fail(MOE_ERR_SHAPE, "n_experts=%d outside [1, %d]", d->n_experts, MOE_MAX_EXPERTS);
    if (d->top_k < 1 || d->top_k > MOE_MAX_TOPK || d->top_k > d->n_experts)
        return fail(MOE_ERR_SHAPE, "top_k=%d outside [1, min(n_experts, %d)]", d->top_k, MOE_MAX_TOPK);
    if ((long)d->top_k * d->inter > MOE_MAX_K_TIMES_I)
        return fail(MOE_ERR_UNSUPPORTED, "top_k*inter=%ld exceeds %d (LDS staging of the down projection)",
                    (long)d->top_k * d->inter, MOE_MAX_K_TIMES_I);
    return MOE_OK;
}

int check_dtype(int dt, const char *what) {
    if (dt != MOE_F32 && dt != MOE_BF16) return fail(MOE_ERR_DTYPE, "%s dtype %d is not MOE_F32 or MOE_BF16", what, dt);
    return MOE_OK;
}

int check_layer(const moe_layer *L, int idx) {
    if (!L) return fail(MOE_ERR_NULL, "layer %d is NULL", idx);
    if (!L->router) return fail(MOE_ERR_NULL, "layer %d router is NULL", idx);
    if (!L->experts) return fail(MOE_ERR_NULL, "layer %d experts is NULL", idx);
    if (int s = check_dtype(L->router_dtype, "router")) return s;
    if (!aligned(L->router, 16)) return fail(MOE_ERR_ALIGN, "layer %d router not 16-byte aligned", idx);
    if (!aligned(L->experts, 16)) return fail(MOE_ERR_ALIGN, "layer %d experts table not 16-byte aligned", idx);
    if (L->logit_bias && !aligned(L->logit_bias, 4)) return fail(MOE_ERR_ALIGN, "layer %d logit_bias not 4-byte aligned", idx);
    if (L->norm_w && !aligned(L->norm_w, 2)) return fail(MOE_ERR_ALIGN, "layer %d norm_w not 2-byte aligned", idx);
    if (L->norm_w && !(L->norm_eps >= 0.f && std::isfinite(L->norm_eps)))
        return fail(MOE_ERR_SHAPE, "layer %d norm_eps must be finite and >= 0", idx);
    return MOE_OK;
}

int check_ws(void *ws, size_t have, size_t need) {
    if (need && !ws) return fail(MOE_ERR_WORKSPACE, "workspace is NULL (need %zu bytes)", need);
    if (have < need) return fail(MOE_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", have, need);
    if (ws && !aligned(ws, 256)) return fail(MOE_ERR_ALIGN, "workspace not 256-byte aligned");
    return MOE_OK;
}

int launched(hipError_t e, const char *what) {
    if (e != hipSuccess) return fail(MOE_ERR_LAUNCH, "%s: %s", what, hipGetErrorString(e));
    return MOE_OK;
}

// Test hook (moe_debug_inject_launch_failure): the next g_pass launch steps proceed, then g_fail are
// refused before anything is enqueued, as if the runtime had rejected them.
std::mutex g_inject_mu;
int g_pass = 0, g_fail = 0;
std::atomic<bool> g_armed{false};       // lets unarmed launches skip the lock
bool injected(const char *what) {
    if (!g_armed.load(std::memory_order_acquire)) return false;
    std::lock_guard<std::mutex> lock(g_inject_mu);
    if (g_fail <= 0) return false;
    if (g_pass > 0) {
        --g_pass;
        return false;
    }
    if (--g_fail == 0) g_armed.store(false, std::memory_order_release);
    fail(MOE_ERR_LAUNCH, "%s: injected launch failure (test hook)", what);
    return true;
}
#define MOE_LAUNCH(expr, what) (injected(what) ? MOE_ERR_LAUNCH : launched((expr), (what)))

// Workspace carving (each region 256-byte aligned).
struct Carve {
    char *base;
    size_t off = 0;
    template <typename T>
    T *take(size_t n) {
        T *p = base ? (T *)(base + off) : nullptr;
        off = r256(off + n * sizeof(T));
        return p;
    }
};

// Per-device side stream of the batched path (created on first use, kept until the process ends;
// default priority, non-blocking with respect to the null stream).
std::mutex g_side_mu;
std::vector<moe::SideStream> g_side;
int side_stream(const moe::SideStream **out) {
    int dev = 0;
    if (hipError_t e = hipGetDevice(&dev)) return fail(MOE_ERR_LAUNCH, "hipGetDevice: %s", hipGetErrorString(e));
    std::lock_guard<std::mutex> lock(g_side_mu);
    if ((int)g_side.size() <= dev) g_side.resize(dev + 1, moe::SideStream{nullptr, nullptr, nullptr});
    moe::SideStream &ss = g_side[dev];
    if (!ss.stream) {
        moe::SideStream n{nullptr, nullptr, nullptr};
        hipError_t e = hipStreamCreateWithFlags(&n.stream, hipStreamNonBlocking);
        if (e == hipSuccess) e = hipEventCreateWithFlags(&n.fork, hipEventDisableTiming);
        if (e == hipSuccess) e = hipEventCreateWithFlags(&n.join, hipEventDisableTiming);
        if (e != hipSuccess) return fail(MOE_ERR_LAUNCH, "side stream: %s", hipGetErrorString(e));
        ss = n;
    }
    *out = &ss;
    return MOE_OK;
}

// Router workspace: logits (when the caller passes none), then for T >= kRouterMfmaMinT the
// normalised rows that the MFMA router reads and the partial logits of its K splits (both optional:
// without room for the rows the matvec router normalises in place, without room for the partials
// the MFMA router runs unsplit).
size_t route_split_bytes(const moe_dims *d, int T) {
    const int ns = moe::router_mfma_splits(d->hidden, d->n_experts, T);
    return ns > 1 ? r256((size_t)ns * T * d->n_experts * 4) : 0;
}
size_t route_ws(const moe_dims *d, int T) {
    return r256((size_t)T * d->n_experts * 4) +
           (T >= moe::kRouterMfmaMinT ? r256((size_t)T * d->hidden * 4) + route_split_bytes(d, T) : 0);
}
// Batched path workspace: grouping tables, SwiGLU outputs in expert order, normalised rows.
struct GroupedWs {
    int32_t *off, *ntiles, *perm, *tiles, *nsmall;
    moe::SmallRec *small;
    float *hbuf, *xn;
    size_t bytes;
};
int grouped_max_small(const moe_dims *d, int T) { return std::min(d->n_experts, T * d->top_k); }
GroupedWs grouped_ws(const moe_dims *d, int T, void *base) {
    const int P = T * d->top_k;
    Carve c{(char *)base};
    GroupedWs g;
    g.off = c.take<int32_t>((size_t)d->n_experts + 1);
    g.ntiles = c.take<int32_t>(1);
    g.perm = c.take<int32_t>(P);
    g.tiles = c.take<int32_t>(2 * (size_t)moe::grouped_max_tiles(T, d->top_k, d->n_experts));
    g.small = c.take<moe::SmallRec>((size_t)grouped_max_small(d, T));
    g.nsmall = c.take<int32_t>(1);
    g.hbuf = c.take<float>((size_t)P * d->inter);
    g.xn = c.take<float>((size_t)T * d->hidden);
    g.bytes = c.off;
    return g;
}
constexpr int kMaxGroupedPairs = 32768;   // the grouping kernel keeps every pair in LDS
// Up to this many tokens per call the expert FFN runs the decode kernels with one grid row per
// token: with few tokens almost every selected expert is distinct, so sharing weight reads saves
// little, while grouping costs a fixed ~40 us (grouping, two kernel chains).  Measured on the
// config-1 layer: 29 against 78 us at 2 tokens, 114 against 133 at 16, 206 against 195 at 32.
constexpr int kPerTokenMaxT = 24;
bool grouped_ffn(int T) { return T > kPerTokenMaxT; }
// From 2 to kSharedMaxT tokens (T*K <= kSharedMaxPairs) the shared-read kernels stream each
// selected expert once for all the pairs that chose it; the automatic choice takes them from
// kSharedAutoMinT tokens.  Measured on the config-1 layer (H4096 I1024 E512 K4), per call, shared-read
// against per-token: 23.1 / 19.7 us at 2 tokens (router's choice), 29.0 / 29.8 at 4 (all tokens on
// the same 4 experts), 53.2 / 53.7 at 8 (router), 52.5 / 51.3 at 8 (three experts shared), 46.4 /
// 50.5 at 8 (same experts), 65.5 / 64.6 at 10 (router), 58.0 / 61.9 at 10 (three shared), 73.2 / 75.3
// at 12 (router), 82.6 / 98.8 at 16 (router): below 8 tokens the per-token kernels' shorter prologue
// wins even with overlap; at 8-10 the two are within 2 % on distinct experts and shared experts favour
// the shared-read kernels by up to 9 %; from 12 tokens these win on every routing measured.
constexpr int kSharedAutoMinT = 8;
bool shared_ffn(const moe_dims *d, int T) {
    return T >= 2 && T <= moe::kSharedMaxT && T * d->top_k <= moe::kSharedMaxPairs &&
           moe::shared_path_fits(d->hidden, d->inter, d->n_experts, T);
}
// Shared-read workspace: SwiGLU outputs of every pair in expert order, then the activation rows
// staged as digit planes in both code widths.
struct SharedWs {
    float *hbuf;
    uint32_t *planes;
    size_t bytes;
};
SharedWs shared_ws(const moe_dims *d, int T, void *base) {
    Carve c{(char *)base};
    SharedWs r;
    r.hbuf = c.take<float>((size_t)T * d->top_k * d->inter);
    r.planes = c.take<uint32_t>((size_t)T * (d->hidden + d->hidden / 16));
    r.bytes = c.off;
    return r;
}

size_t per_token_ws(const moe_dims *d, int T) {
    Carve c{nullptr};
    c.take<float>((size_t)T * d->top_k * d->inter);
    c.take<uint64_t>((size_t)T * d->top_k);
    return c.off;
}
// Which kernels run a call (MOE_FFN_AUTO resolved), or -1 when the forced path cannot take T.
int ffn_path(const moe_dims *d, int T, int path) {
    switch (path) {
        case MOE_FFN_AUTO:
            if (grouped_ffn(T)) return T * d->top_k <= kMaxGroupedPairs ? MOE_FFN_GROUPED : -1;
            return T >= kSharedAutoMinT && shared_ffn(d, T) ? MOE_FFN_SHARED : MOE_FFN_PER_TOKEN;
        case MOE_FFN_PER_TOKEN: return T <= kPerTokenMaxT ? path : -1;
        case MOE_FFN_SHARED: return shared_ffn(d, T) ? path : -1;
        case MOE_FFN_GROUPED: return T >= 2 && T * d->top_k <= kMaxGroupedPairs ? path : -1;
        default: return -1;
    }
}
size_t path_ws(const moe_dims *d, int T, int path) {
    switch (path) {
        case MOE_FFN_GROUPED: return grouped_ws(d, T, nullptr).bytes;
        case MOE_FFN_SHARED: return shared_ws(d, T, nullptr).bytes;
        case MOE_FFN_PER_TOKEN: return per_token_ws(d, T);
        default: return 0;
    }
}
// Enough for every path that can take T.
size_t ffn_ws(const moe_dims *d, int T) {
    size_t b = 0;
    for (int p : {MOE_FFN_PER_TOKEN, MOE_FFN_SHARED, MOE_FFN_GROUPED})
        if (ffn_path(d, T, p) == p) b = std::max(b, path_ws(d, T, p));
    return b;
}
// Layer-decode workspace: the two-launch schedule's hand-over words first (they must start
// zeroed), then the buffers both schedules use.
struct DecodeWs {
    uint32_t *sync;      // [0] launch counter, [1] error word
    uint64_t *slots;     // [copies][E] tagged logits
    uint32_t *flags;     // single launch: [copies][max workgroups] "h stored" flags
    float *logits;
    uint64_t *sel;
    float *w;
    float *h;
    float *xbuf;
    size_t bytes;
};
DecodeWs decode_layout(const moe_dims *d, void *ws) {
    Carve c{(char *)ws};
    DecodeWs r;
    r.sync = c.take<uint32_t>(2);
    r.slots = c.take<uint64_t>((size_t)moe::layer_logit_copies() * d->n_experts);
    r.flags = c.take<uint32_t>((size_t)moe::fused_flag_copies() * moe::fused_max_workgroups());
    r.logits = c.take<float>(d->n_experts);
    r.sel = c.take<uint64_t>(d->top_k);
    r.w = c.take<float>(d->top_k);
    r.h = c.take<float>((size_t)d->top_k * d->inter);
    r.xbuf = c.take<float>(2 * (size_t)d->hidden);
    r.bytes = c.off;
    return r;
}

// Workgroups of the single-launch layer kernel for a shape on the current device (an occupancy query
// the first time, then remembered).
std::mutex g_nw_mu;
std::map<std::tuple<int, int, int, int, int>, int> g_nw;
int fused_workgroups_cached(const moe_dims *d, int *nw) {
    int dev = 0;
    if (hipError_t e = hipGetDevice(&dev)) return fail(MOE_ERR_DEVICE, "hipGetDevice: %s", hipGetErrorString(e));
    const auto key = std::make_tuple(dev, d->hidden, d->inter, d->n_experts, d->top_k);
    {
        std::lock_guard<std::mutex> lock(g_nw_mu);
        const auto it = g_nw.find(key);
        if (it != g_nw.end()) {
            *nw = it->second;
            return MOE_OK;
        }
    }
    int n = 0;
    if (hipError_t e = moe::fused_workgroups(d->hidden, d->inter, d->n_experts, d->top_k, &n))
        return fail(MOE_ERR_DEVICE, "occupancy of the layer kernel: %s", hipGetErrorString(e));
    if (n < 1) return fail(MOE_ERR_UNSUPPORTED, "the single-launch layer kernel does not fit this shape on this "
                                                "device; use the default schedule");
    std::lock_guard<std::mutex> lock(g_nw_mu);
    g_nw[key] = n;
    *nw = n;
    return MOE_OK;
}

size_t decode_ws(const moe_dims *d) {
    return decode_layout(d, nullptr).bytes;
}


}  // namespace

extern "C" {

const char *moe_status_string(int s) {
    switch (s) {
        case MOE_OK: return "MOE_OK";
        case MOE_ERR_NULL: return "MOE_ERR_NULL";
        case MOE_ERR_SHAPE: return "MOE_ERR_SHAPE";
        case MOE_ERR_DTYPE: return "MOE_ERR_DTYPE";
        case MOE_ERR_BITS: return "MOE_ERR_BITS";
        case MOE_ERR_ALIGN: return "MOE_ERR_ALIGN";
        case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE";
        case MOE_ERR_LAUNCH: return "MOE_ERR_LAUNCH";
        case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
        case MOE_ERR_BUFFER: return "MOE_ERR_BUFFER";
        case MOE_ERR_DEVICE: return "MOE_ERR_DEVICE";
        default: return "MOE_ERR_UNKNOWN";
    }
}

const char *moe_last_error(void) { return g_err.c_str(); }

const char *moe_version(void) { return "moe_dequant 0.1 (gfx950)"; }

// ------------------------------------------------------------------------------- format
size_t moe_packed_codes_bytes(int rows, int cols, int bits) {
    if (rows < 1 || cols < 64 || cols % MOE_GROUP || !bits_ok(bits)) return 0;
    return (size_t)rows * cols * bits / 8;
}

size_t moe_packed_sb_bytes(int rows, int cols) {
    if (rows < 1 || cols < 64 || cols % MOE_GROUP) return 0;
    return (size_t)rows * (cols / MOE_GROUP) * 4;
}

int moe_expert_plane_offsets(int hidden, int inter, int bits, size_t off[6]) {
    if (!off) return fail(MOE_ERR_NULL, "off is NULL");
    if (!bits_ok(bits)) return fail(MOE_ERR_BITS, "bits=%d", bits);
    if (hidden < 64 || hidden % 64 || inter < 64 || inter % 64)
        return fail(MOE_ERR_SHAPE, "hidden=%d inter=%d must be positive multiples of 64", hidden, inter);
    const size_t sz[6] = {moe_packed_codes_bytes(inter, hidden, bits), moe_packed_sb_bytes(inter, hidden),
                          moe_packed_codes_bytes(inter, hidden, bits), moe_packed_sb_bytes(inter, hidden),
                          moe_packed_codes_bytes(hidden, inter, bits), moe_packed_sb_bytes(hidden, inter)};
    size_t p = 0;
    for (int i = 0; i < 6; ++i) {
        off[i] = p;
        p = r256(p + sz[i]);
    }
    return ok();
}

size_t moe_packed_expert_bytes(int hidden, int inter, int bits) {
    size_t off[6];
    if (moe_expert_plane_offsets(hidden, inter, bits, off) != MOE_OK) return 0;
    return r256(off[5] + moe_packed_sb_bytes(hidden, inter));
}

int moe_pack_matrix(const uint8_t *codes, const uint16_t *scale, const uint16_t *bias, int rows, int cols,
                    int bits, uint8_t *codes_out, size_t codes_out_bytes, uint16_t *sb_out, size_t sb_out_bytes) {
    if (!codes || !scale || !bias || !codes_out || !sb_out) return fail(MOE_ERR_NULL, "NULL argument");
    if (!bits_ok(bits)) return fail(MOE_ERR_BITS, "bits=%d", bits);
    const size_t cb = moe_packed_codes_bytes(rows, cols, bits), sb = moe_packed_sb_bytes(rows, cols);
    if (!cb || !sb) return fail(MOE_ERR_SHAPE, "rows=%d cols=%d", rows, cols);
    if (codes_out_bytes < cb || sb_out_bytes < sb) return fail(MOE_ERR_BUFFER, "need %zu + %zu bytes", cb, sb);
    const size_t n = (size_t)rows * cols;
    const unsigned lim = 1u << bits;
    for (size_t i = 0; i < n; ++i)
        if (codes[i] >= lim) return fail(MOE_ERR_BITS, "code %u at %zu does not fit in %d bits", codes[i], i, bits);
    std::memset(codes_out, 0, cb);
    const size_t rowb = (size_t)cols * bits / 8;
    for (int r = 0; r < rows; ++r)
        for (int c = 0; c < cols; ++c) {
            const size_t bit = (size_t)c * bits;
            codes_out[(size_t)r * rowb + bit / 8] |= (uint8_t)(codes[(size_t)r * cols + c] << (bit % 8));
        }
    const size_t ng = (size_t)rows * (cols / MOE_GROUP);
    for (size_t g = 0; g < ng; ++g) {
        sb_out[2 * g] = scale[g];
        sb_out[2 * g + 1] = bias[g];
    }
    return ok();
}

int moe_unpack_matrix(const uint8_t *codes_in, const uint16_t *sb_in, int rows, int cols, int bits, uint8_t *codes,
                      uint16_t *scale, uint16_t *bias) {
    if (!codes_in || !sb_in || !codes || !scale || !bias) return fail(MOE_ERR_NULL, "NULL argument");
    if (!bits_ok(bits)) return fail(MOE_ERR_BITS, "bits=%d", bits);
    if (!moe_packed_codes_bytes(rows, cols, bits)) return fail(MOE_ERR_SHAPE, "rows=%d cols=%d", rows, cols);
    const size_t rowb = (size_t)cols * bits / 8;
    for (int r = 0; r < rows; ++r)
        for (int c = 0; c < cols; ++c) {
            const size_t bit = (size_t)c * bits;
            codes[(size_t)r * cols + c] = (codes_in[(size_t)r * rowb + bit / 8] >> (bit % 8)) & ((1u << bits) - 1);
        }
    const size_t ng = (size_t)rows * (cols / MOE_GROUP);
    for (size_t g = 0; g < ng; ++g) {
        scale[g] = sb_in[2 * g];
        bias[g] = sb_in[2 * g + 1];
    }
    return ok();
}

int moe_pack_expert(const uint8_t *const codes[3], const uint16_t *const scale[3], const uint16_t *const bias[3],
                    int hidden, int inter, int bits, void *blob_out, size_t blob_out_bytes) {
    if (!codes || !scale || !bias || !blob_out) return fail(MOE_ERR_NULL, "NULL argument");
    size_t off[6];
    if (int s = moe_expert_plane_offsets(hidden, inter, bits, off)) return s;
    const size_t total = moe_packed_expert_bytes(hidden, inter, bits);
    if (blob_out_bytes < total) return fail(MOE_ERR_BUFFER, "blob needs %zu bytes", total);
    std::memset(blob_out, 0, total);
    uint8_t *b = (uint8_t *)blob_out;
    const int R[3] = {inter, inter, hidden}, C[3] = {hidden, hidden, inter};
    for (int m = 0; m < 3; ++m) {
        if (!codes[m] || !scale[m] || !bias[m]) return fail(MOE_ERR_NULL, "matrix %d has a NULL array", m);
        const size_t cb = moe_packed_codes_bytes(R[m], C[m], bits), sb = moe_packed_sb_bytes(R[m], C[m]);
        if (int s = moe_pack_matrix(codes[m], scale[m], bias[m], R[m], C[m], bits, b + off[2 * m], cb,
                                    (uint16_t *)(b + off[2 * m + 1]), sb))
            return s;
    }
    return ok();
}

int moe_check_experts(const moe_expert_desc *experts_dev, int n_experts) {
    if (!experts_dev) return fail(MOE_ERR_NULL, "experts is NULL");
    if (n_experts < 1 || n_experts > MOE_MAX_EXPERTS) return fail(MOE_ERR_SHAPE, "n_experts=%d", n_experts);
    std::vector<moe_expert_desc> h(n_experts);
    hipError_t e = hipMemcpy(h.data(), experts_dev, sizeof(moe_expert_desc) * n_experts, hipMemcpyDeviceToHost);
    if (e != hipSuccess) return fail(MOE_ERR_DEVICE, "copying the descriptor table: %s", hipGetErrorString(e));
    for (int i = 0; i < n_experts; ++i) {
        if (!h[i].blob) return fail(MOE_ERR_NULL, "expert %d blob is NULL", i);
        if (h[i].blob % MOE_BLOB_ALIGN) return fail(MOE_ERR_ALIGN, "expert %d blob not 256-byte aligned", i);
        if (!bits_ok((int)h[i].bits)) return fail(MOE_ERR_BITS, "expert %d bits=%u", i, h[i].bits);
        if (h[i].reserved) return fail(MOE_ERR_SHAPE, "expert %d reserved field is not 0", i);
    }
    return ok();
}

int moe_stream_read(const void *buf, size_t bytes, uint32_t *sink, void *stream) {
    if (!buf || !sink) return fail(MOE_ERR_NULL, "buf and sink are required");
    if (!aligned(buf, 16) || !aligned(sink, 4)) return fail(MOE_ERR_ALIGN, "buf must be 16-byte, sink 4-byte aligned");
    if (bytes == 0 || bytes % 16) return fail(MOE_ERR_SHAPE, "bytes=%zu is not a positive multiple of 16", bytes);
    if (int s = MOE_LAUNCH(moe::launch_stream_read(buf, bytes, sink, (hipStream_t)stream), "stream read")) return s;
    return ok();
}

// ------------------------------------------------------------------------------- workspace
size_t moe_workspace_bytes(int op, const moe_dims *dims, int T, int n_layers) {
    if (!dims || check_dims(dims) != MOE_OK || T < 1) return 0;
    switch (op) {
        case MOE_OP_ROUTE: return route_ws(dims, T);
        case MOE_OP_EXPERT_FFN: return ffn_ws(dims, T);
        case MOE_OP_LAYER_DECODE: return (n_layers >= 1 && T == 1) ? decode_ws(dims) : 0;
        default: return 0;
    }
}

// ------------------------------------------------------------------------------- compute
int moe_route(const moe_dims *dims, const moe_layer *layer, const void *x, int x_dtype, int T, int32_t *idx,
              float *w, float *logits, void *ws, size_t ws_bytes, void *stream) {
    if (int s = check_dims(dims)) return s;
    if (int s = check_layer(layer, 0)) return s;
    if (int s = check_dtype(x_dtype, "x")) return s;
    if (!x || !idx || !w) return fail(MOE_ERR_NULL, "x, idx and w are required");
    if (T < 1 || T > 65535) return fail(MOE_ERR_SHAPE, "T=%d outside [1, 65535]", T);
    if (!aligned(x, 16)) return fail(MOE_ERR_ALIGN, "x not 16-byte aligned");
    if (!aligned(idx, 4) || !aligned(w, 4) || (logits && !aligned(logits, 4)))
        return fail(MOE_ERR_ALIGN, "idx/w/logits not 4-byte aligned");
    Carve c{(char *)ws};
    float *lg = logits ? logits : c.take<float>((size_t)T * dims->n_experts);
    if (int s = check_ws(ws, ws_bytes, c.off)) return s;
    float *xn = nullptr, *part = nullptr;
    if (T >= moe::kRouterMfmaMinT && ws) {
        float *p = c.take<float>((size_t)T * dims->hidden);
        if (ws_bytes >= c.off) xn = p;
        if (const size_t pb = route_split_bytes(dims, T)) {
            float *q = (float *)c.take<char>(pb);
            if (ws_bytes >= c.off) part = q;
        }
    }
    hipStream_t st = (hipStream_t)stream;
    moe::RouterLaunch ra{x, x_dtype, dims->hidden, layer->norm_w, layer->norm_eps, layer->router,
                         layer->router_dtype, layer->logit_bias, lg, dims->hidden, dims->n_experts, T, xn, part};
    if (!moe::router_mfma_fits(ra)) ra.part_ws = nullptr;       // partial rows only from the MFMA router
    if (int s = MOE_LAUNCH(moe::launch_router(ra, st), "router")) return s;
    const int ns = ra.part_ws ? moe::router_mfma_splits(dims->hidden, dims->n_experts, T) : 1;
    moe::TopkLaunch ta{lg, dims->n_experts, dims->top_k, T, idx, w, ra.part_ws, ns, layer->logit_bias, lg};
    if (int s = MOE_LAUNCH(moe::launch_topk(ta, st), "top-k")) return s;
    return ok();
}

int moe_expert_ffn_path(const moe_dims *dims, const moe_layer *layer, const void *x, int x_dtype, int T,
                        const int32_t *idx, float *y, void *ws, size_t ws_bytes, int path, void *stream) {
    if (int s = check_dims(dims)) return s;
    if (int s = check_layer(layer, 0)) return s;
    if (int s = check_dtype(x_dtype, "x")) return s;
    if (!x || !idx || !y) return fail(MOE_ERR_NULL, "x, idx and y are required");
    if (T < 1 || T > 65535) return fail(MOE_ERR_SHAPE, "T=%d outside [1, 65535]", T);
    if (!aligned(x, 16)) return fail(MOE_ERR_ALIGN, "x not 16-byte aligned");
    if (!aligned(idx, 4) || !aligned(y, 4)) return fail(MOE_ERR_ALIGN, "idx/y not 4-byte aligned");
    if (path < MOE_FFN_AUTO || path > MOE_FFN_GROUPED) return fail(MOE_ERR_UNSUPPORTED, "unknown path %d", path);
    const int run = ffn_path(dims, T, path);
    if (run < 0) {
        if (path == MOE_FFN_AUTO || path == MOE_FFN_GROUPED)
            return fail(MOE_ERR_UNSUPPORTED, "T*top_k=%d: the grouped path takes 2 <= T and T*top_k <= %d",
                        T * dims->top_k, kMaxGroupedPairs);
        if (path == MOE_FFN_PER_TOKEN)
            return fail(MOE_ERR_UNSUPPORTED, "T=%d: the per-token path takes T <= %d", T, kPerTokenMaxT);
        return fail(MOE_ERR_UNSUPPORTED, "T=%d top_k=%d: the shared-read path takes 2 <= T <= %d, T*top_k <= %d "
                    "and staged rows that fit in LDS", T, dims->top_k, moe::kSharedMaxT, moe::kSharedMaxPairs);
    }
    if (int s = check_ws(ws, ws_bytes, path_ws(dims, T, run))) return s;
    hipStream_t st = (hipStream_t)stream;
    if (run == MOE_FFN_GROUPED) {
        // batched: group the (token, slot) pairs by expert, then the grouped kernels
        GroupedWs g = grouped_ws(dims, T, ws);
        const void *xa = x;
        int xdt = x_dtype;
        if (layer->norm_w) {
            if (int s = MOE_LAUNCH(moe::launch_norm_rows(x, x_dtype, layer->norm_w, layer->norm_eps, dims->hidden, T,
                                                       g.xn, st), "norm"))
                return s;
            xa = g.xn;
            xdt = MOE_F32;
        }
        const bool small = moe::small_path_fits(dims->hidden, dims->inter);
        moe::GroupLaunch gl{idx, T, dims->top_k, dims->n_experts, layer->experts, g.off, g.perm, g.tiles, g.ntiles,
                            g.small, g.nsmall, small ? moe::kSmallTokens : 0, y, dims->hidden};
        if (int s = MOE_LAUNCH(moe::launch_group(gl, st), "group")) return s;
        moe::GroupedLaunch ga{xa, xdt, dims->hidden, dims->inter, dims->top_k, layer->experts, g.off, g.perm,
                              g.tiles, g.ntiles, g.small, g.nsmall, g.hbuf, y, {}, {}};
        const moe::SideStream *side = nullptr;
        if (small)
            if (int s = side_stream(&side)) return s;
        // the fork/join events are shared per device: enqueue the forked section under the lock
        std::lock_guard<std::mutex> lock(g_side_mu);
        if (int s = MOE_LAUNCH(moe::launch_grouped_ffn(ga, moe::grouped_max_tiles(T, dims->top_k, dims->n_experts),
                                                     small ? grouped_max_small(dims, T) : 0, st, side),
                             "grouped ffn"))
            return s;
        return ok();
    }
    if (run == MOE_FFN_SHARED) {
        SharedWs sw = shared_ws(dims, T, ws);
        moe::GroupedLaunch ga{x, x_dtype, dims->hidden, dims->inter, dims->top_k, layer->experts, nullptr, nullptr,
                              nullptr, nullptr, nullptr, nullptr, sw.hbuf, y, {}, {}, 0, idx, T, dims->n_experts, 0, 0,
                              layer->norm_w, layer->norm_eps, sw.planes};
        if (int s = MOE_LAUNCH(moe::launch_shared_ffn(ga, st), "shared-read ffn")) return s;
        return ok();
    }
    Carve c{(char *)ws};
    float *h = c.take<float>((size_t)T * dims->top_k * dims->inter);
    uint64_t *sel = c.take<uint64_t>((size_t)T * dims->top_k);
    moe::GateUpLaunch ga{x, x_dtype, dims->hidden, layer->norm_w, layer->norm_eps, nullptr, idx, nullptr, nullptr,
                         sel, nullptr, layer->experts, h, dims->hidden, dims->inter, dims->n_experts, dims->top_k, T};
    if (int s = MOE_LAUNCH(moe::launch_gateup(ga, st), "gate/up")) return s;
    moe::DownLaunch da{h, nullptr, nullptr, sel, nullptr, nullptr, MOE_F32, 0, y, dims->hidden, dims->inter, dims->top_k, T};
    if (int s = MOE_LAUNCH(moe::launch_down(da, st), "down")) return s;
    return ok();
}

int moe_expert_ffn(const moe_dims *dims, const moe_layer *layer, const void *x, int x_dtype, int T,
                   const int32_t *idx, float *y, void *ws, size_t ws_bytes, void *stream) {
    return moe_expert_ffn_path(dims, layer, x, x_dtype, T, idx, y, ws, ws_bytes, MOE_FFN_AUTO, stream);
}

int moe_combine(const float *y, const float *w, int T, int K, int H, const float *residual, float *out,
                void *stream) {
    if (!y || !w || !out) return fail(MOE_ERR_NULL, "y, w and out are required");
    if (T < 1 || K < 1 || K > MOE_MAX_TOPK || H < 1) return fail(MOE_ERR_SHAPE, "T=%d K=%d H=%d", T, K, H);
    if (!aligned(y, 4) || !aligned(w, 4) || !aligned(out, 4) || (residual && !aligned(residual, 4)))
        return fail(MOE_ERR_ALIGN, "arrays must be 4-byte aligned");
    moe::CombineLaunch ca{y, w, residual, out, T, K, H};
    if (int s = MOE_LAUNCH(moe::launch_combine(ca, (hipStream_t)stream), "combine")) return s;
    return ok();
}

int moe_quantize_matrix(const void *w, int w_dtype, int rows, int cols, int bits, uint8_t *codes, uint16_t *sb,
                        void *stream) {
    if (!w || !codes || !sb) return fail(MOE_ERR_NULL, "w, codes and sb are required");
    if (int s = check_dtype(w_dtype, "w")) return s;
    if (rows < 1 || cols < 64 || cols % 64 != 0 || (uint64_t)rows * (uint64_t)cols > ((uint64_t)1 << 40))
        return fail(MOE_ERR_SHAPE, "rows=%d cols=%d (cols a positive multiple of 64)", rows, cols);
    if (bits != 2 && bits != 4) return fail(MOE_ERR_BITS, "bits=%d (2 or 4)", bits);
    if (!aligned(w, 16) || !aligned(codes, 16) || !aligned(sb, 4))
        return fail(MOE_ERR_ALIGN, "w and codes must be 16-byte aligned, sb 4-byte aligned");
    moe::QuantLaunch qa{w, w_dtype, rows, cols, bits, codes, sb};
    if (int s = MOE_LAUNCH(moe::launch_quantize(qa, (hipStream_t)stream), "quantize")) return s;
    return ok();
}

int moe_expert_usage(const int32_t *idx, int n, int n_experts, uint32_t *counts, void *stream) {
    if (!counts || (n > 0 && !idx)) return fail(MOE_ERR_NULL, "counts (and idx when n > 0) are required");
    if (n < 0) return fail(MOE_ERR_SHAPE, "n=%d is negative", n);
    if (n_experts < 1 || n_experts > MOE_MAX_EXPERTS)
        return fail(MOE_ERR_SHAPE, "n_experts=%d outside [1, %d]", n_experts, MOE_MAX_EXPERTS);
    if (!aligned(counts, 4) || (idx && !aligned(idx, 4))) return fail(MOE_ERR_ALIGN, "idx and counts must be 4-byte aligned");
    if (int s = MOE_LAUNCH(moe::launch_usage(idx, (size_t)n, n_experts, counts, (hipStream_t)stream), "usage")) return s;
    return ok();
}

int moe_hot_order(const uint32_t *counts, int n_experts, int32_t *order, void *stream) {
    if (!counts || !order) return fail(MOE_ERR_NULL, "counts and order are required");
    if (n_experts < 1 || n_experts > MOE_MAX_EXPERTS)
        return fail(MOE_ERR_SHAPE, "n_experts=%d outside [1, %d]", n_experts, MOE_MAX_EXPERTS);
    if (!aligned(counts, 4) || !aligned(order, 4)) return fail(MOE_ERR_ALIGN, "counts and order must be 4-byte aligned");
    if (int s = MOE_LAUNCH(moe::launch_hot_order(counts, n_experts, order, (hipStream_t)stream), "hot order")) return s;
    return ok();
}

int moe_retier(const moe_dims *dims, const moe_expert_desc *base, const int32_t *order, int n_hot, int cold_bits,
               void *store, size_t store_bytes, moe_expert_desc *tiered, void *stream) {
    if (int s = check_dims(dims)) return s;
    if (!base || !order || !tiered) return fail(MOE_ERR_NULL, "base, order and tiered are required");
    const int E = dims->n_experts;
    if (n_hot < 0 || n_hot > E) return fail(MOE_ERR_SHAPE, "n_hot=%d outside [0, n_experts=%d]", n_hot, E);
    if (!bits_ok(cold_bits)) return fail(MOE_ERR_BITS, "cold_bits=%d (2 or 4)", cold_bits);
    if (!aligned(base, 16) || !aligned(tiered, 16) || !aligned(order, 4))
        return fail(MOE_ERR_ALIGN, "base and tiered must be 16-byte aligned, order 4-byte aligned");
    const size_t cold = moe_packed_expert_bytes(dims->hidden, dims->inter, cold_bits);
    const size_t need = (size_t)(E - n_hot) * cold;
    if (need) {
        if (!store) return fail(MOE_ERR_NULL, "store is NULL (%d cold experts need %zu bytes)", E - n_hot, need);
        if (!aligned(store, MOE_BLOB_ALIGN)) return fail(MOE_ERR_ALIGN, "store must be %d-byte aligned", MOE_BLOB_ALIGN);
        if (store_bytes < need)
            return fail(MOE_ERR_BUFFER, "store_bytes=%zu < %zu (%d cold experts of %zu bytes)", store_bytes, need,
                        E - n_hot, cold);
    }
    moe::RetierLaunch r{base, order, E, dims->hidden, dims->inter, n_hot, cold_bits, store, cold, tiered};
    if (int s = MOE_LAUNCH(moe::launch_retier(r, (hipStream_t)stream), "retier")) return s;
    return ok();
}

// ----------------------------------------------------------------------------- expert cache
// Least recently used replacement over n_slots device slots; a call touches its distinct experts
// first (hits), then loads each missing one into the lowest free slot or, with none free, into the
// slot used least recently among those the call has not touched (equal times: the lower slot).
struct moe_expert_cache {
    int E = 0, n_slots = 0;
    unsigned flags = 0;
    std::vector<moe_expert_desc> host;            // host blob address and width per expert
    std::vector<size_t> bytes;                    // blob bytes per expert
    uint8_t *slots = nullptr;
    size_t slot_bytes = 0;
    moe_expert_desc *table = nullptr;
    std::vector<int> slot_of, expert_of;
    std::vector<uint64_t> last_use, mark;
    std::set<std::pair<uint64_t, int>> lru;       // (last use, slot) of occupied slots
    std::set<int> free_slots;
    uint64_t tick = 0, epoch = 0;
    uint64_t hits = 0, misses = 0, copied = 0;
    bool broken = false;
    uint32_t *dev_state = nullptr;                // device-side policy state once attached
    int dev_device = -1;
    // per-call scratch
    std::vector<int> req;
    std::vector<int32_t> upd_e;
    std::vector<uint64_t> upd_blob;
    std::vector<uint32_t> upd_bits;
};

int moe_cache_create(const moe_dims *dims, const moe_expert_desc *host_experts, void *slots, size_t slot_bytes,
                     int n_slots, moe_expert_desc *table, unsigned flags, void *stream, moe_expert_cache **cache) {
    if (!cache) return fail(MOE_ERR_NULL, "cache is NULL");
    *cache = nullptr;
    if (int s = check_dims(dims)) return s;
    if (flags & ~MOE_CACHE_DRY_RUN) return fail(MOE_ERR_UNSUPPORTED, "unknown flags 0x%x", flags);
    const bool dry = flags & MOE_CACHE_DRY_RUN;
    if (!host_experts) return fail(MOE_ERR_NULL, "host_experts is NULL");
    const int E = dims->n_experts;
    if (n_slots < dims->top_k || n_slots > (1 << 20))
        return fail(MOE_ERR_SHAPE, "n_slots=%d outside [top_k=%d, 2^20]", n_slots, dims->top_k);
    if (!dry) {
        if (!slots || !table) return fail(MOE_ERR_NULL, "slots and table are required");
        if (!aligned(slots, MOE_BLOB_ALIGN) || slot_bytes % MOE_BLOB_ALIGN != 0)
            return fail(MOE_ERR_ALIGN, "slots and slot_bytes must be multiples of %d", MOE_BLOB_ALIGN);
        if (!aligned(table, 16)) return fail(MOE_ERR_ALIGN, "table must be 16-byte aligned");
    }
    auto c = new moe_expert_cache;
    c->E = E;
    c->n_slots = n_slots;
    c->flags = flags;
    c->host.assign(host_experts, host_experts + E);
    c->bytes.resize(E);
    for (int e = 0; e < E; ++e) {
        const moe_expert_desc &d = c->host[e];
        int st = MOE_OK;
        if (!d.blob) st = fail(MOE_ERR_NULL, "host_experts[%d].blob is NULL", e);
        else if (!bits_ok((int)d.bits)) st = fail(MOE_ERR_BITS, "host_experts[%d].bits=%u (2 or 4)", e, d.bits);
        else if (d.reserved) st = fail(MOE_ERR_SHAPE, "host_experts[%d].reserved must be 0", e);
        else if ((c->bytes[e] = moe_packed_expert_bytes(dims->hidden, dims->inter, (int)d.bits)) > slot_bytes && !dry)
            st = fail(MOE_ERR_BUFFER, "slot_bytes=%zu < expert %d's blob of %zu bytes", slot_bytes, e, c->bytes[e]);
        if (st) {
            delete c;
            return st;
        }
    }
    c->slots = (uint8_t *)slots;
    c->slot_bytes = slot_bytes;
    c->table = table;
    c->slot_of.assign(E, -1);
    c->mark.assign(E, 0);
    c->expert_of.assign(n_slots, -1);
    c->last_use.assign(n_slots, 0);
    for (int s = 0; s < n_slots; ++s) c->free_slots.insert(s);
    if (!dry) {
        if (int st = MOE_LAUNCH(moe::launch_table_absent(table, E, (hipStream_t)stream), "cache table")) {
            delete c;
            return st;
        }
    }
    *cache = c;
    return ok();
}

int moe_cache_fetch(moe_expert_cache *c, const int32_t *idx, int n, void *stream, int *misses_out) {
    if (!c) return fail(MOE_ERR_NULL, "cache is NULL");
    if (c->dev_state) return fail(MOE_ERR_UNSUPPORTED, "the cache's policy runs on the device: use moe_cache_fetch_device");
    if (c->broken) return fail(MOE_ERR_LAUNCH, "an earlier enqueue on this cache failed; destroy it");
    if (n < 0) return fail(MOE_ERR_SHAPE, "n=%d is negative", n);
    if (n > 0 && !idx) return fail(MOE_ERR_NULL, "idx is NULL");
    const uint64_t ep = ++c->epoch;
    c->req.clear();
    for (int i = 0; i < n; ++i) {
        const int e = idx[i];
        if (e >= 0 && e < c->E && c->mark[e] != ep) {
            c->mark[e] = ep;
            c->req.push_back(e);
        }
    }
    if ((int)c->req.size() > c->n_slots)
        return fail(MOE_ERR_SHAPE, "%zu distinct experts exceed the %d slots", c->req.size(), c->n_slots);
    const uint64_t t = ++c->tick;
    int hit = 0;
    for (int e : c->req) {
        const int s = c->slot_of[e];
        if (s < 0) continue;
        ++hit;
        c->lru.erase({c->last_use[s], s});
        c->last_use[s] = t;
        c->lru.insert({t, s});
    }
    c->upd_e.clear();
    c->upd_blob.clear();
    c->upd_bits.clear();
    const bool dry = c->flags & MOE_CACHE_DRY_RUN;
    int miss = 0;
    for (int e : c->req) {
        if (c->slot_of[e] >= 0) continue;
        ++miss;
        int s;
        if (!c->free_slots.empty()) {
            s = *c->free_slots.begin();
            c->free_slots.erase(c->free_slots.begin());
        } else {
            // the least recent (last use, slot); a slot touched by this call has last use t and is
            // never first while an untouched one exists, which the slot count guarantees
            const auto it = c->lru.begin();
            s = it->second;
            c->lru.erase(it);
            const int old = c->expert_of[s];
            c->slot_of[old] = -1;
            c->upd_e.push_back(old);
            c->upd_blob.push_back(0);
            c->upd_bits.push_back(4);
        }
        c->slot_of[e] = s;
        c->expert_of[s] = e;
        c->last_use[s] = t;
        c->lru.insert({t, s});
        uint8_t *dst = c->slots + (size_t)s * c->slot_bytes;
        c->upd_e.push_back(e);
        c->upd_blob.push_back((uint64_t)(uintptr_t)dst);
        c->upd_bits.push_back(c->host[e].bits);
        c->copied += c->bytes[e];
        if (!dry) {
            const hipError_t err = hipMemcpyAsync(dst, (const void *)(uintptr_t)c->host[e].blob, c->bytes[e],
                                                  hipMemcpyHostToDevice, (hipStream_t)stream);
            if (err != hipSuccess) {
                c->broken = true;
                return fail(MOE_ERR_LAUNCH, "copy of expert %d: %s", e, hipGetErrorString(err));
            }
        }
    }
    c->hits += hit;
    c->misses += miss;
    if (!dry && !c->upd_e.empty()) {
        const hipError_t err = moe::launch_table_update(c->table, (int)c->upd_e.size(), c->upd_e.data(),
                                                        c->upd_blob.data(), c->upd_bits.data(), (hipStream_t)stream);
        if (err != hipSuccess) {
            c->broken = true;
            return fail(MOE_ERR_LAUNCH, "cache table update: %s", hipGetErrorString(err));
        }
    }
    if (misses_out) *misses_out = miss;
    return ok();
}

int moe_cache_stats(const moe_expert_cache *c, uint64_t *hits, uint64_t *misses, uint64_t *bytes) {
    if (!c) return fail(MOE_ERR_NULL, "cache is NULL");
    uint64_t h = c->hits, m = c->misses, b = c->copied;
    if (c->dev_state) {
        uint32_t hdr[moe::kCacheHdr];
        if (hipError_t e = hipMemcpy(hdr, c->dev_state, sizeof(hdr), hipMemcpyDeviceToHost))
            return fail(MOE_ERR_DEVICE, "reading the device cache state: %s", hipGetErrorString(e));
        h = hdr[6] | ((uint64_t)hdr[7] << 32);
        m = hdr[8] | ((uint64_t)hdr[9] << 32);
        b = hdr[10] | ((uint64_t)hdr[11] << 32);
    }
    if (hits) *hits = h;
    if (misses) *misses = m;
    if (bytes) *bytes = b;
    return ok();
}

int moe_cache_slot(const moe_expert_cache *c, int expert) {
    if (!c || expert < 0 || expert >= c->E) return -2;
    if (c->dev_state) {
        int32_t v = -2;
        const moe::CacheLayout L = moe::cache_layout(c->E, c->n_slots);
        if (hipMemcpy(&v, c->dev_state + L.slot_of + expert, 4, hipMemcpyDeviceToHost) != hipSuccess) return -2;
        return v;
    }
    return c->slot_of[expert];
}

size_t moe_cache_device_state_bytes(const moe_expert_cache *c) {
    if (!c || (c->flags & MOE_CACHE_DRY_RUN) || c->n_slots > moe::kCacheMaxSlots) return 0;
    return moe::cache_layout(c->E, c->n_slots).words * 4;
}

int moe_cache_attach_device(moe_expert_cache *c, void *state, size_t state_bytes, void *stream) {
    if (!c) return fail(MOE_ERR_NULL, "cache is NULL");
    if (c->dev_state) return fail(MOE_ERR_UNSUPPORTED, "the cache is already attached to a device state");
    if (c->flags & MOE_CACHE_DRY_RUN) return fail(MOE_ERR_UNSUPPORTED, "a dry-run cache has no device side");
    if (c->broken) return fail(MOE_ERR_LAUNCH, "an earlier enqueue on this cache failed; destroy it");
    if (c->n_slots > moe::kCacheMaxSlots)
        return fail(MOE_ERR_UNSUPPORTED, "n_slots=%d exceeds the device policy's %d", c->n_slots, moe::kCacheMaxSlots);
    if (!state) return fail(MOE_ERR_NULL, "state is NULL");
    if (!aligned(state, 256)) return fail(MOE_ERR_ALIGN, "state must be 256-byte aligned");
    const moe::CacheLayout L = moe::cache_layout(c->E, c->n_slots);
    if (state_bytes < L.words * 4) return fail(MOE_ERR_WORKSPACE, "state_bytes=%zu < %zu", state_bytes, L.words * 4);
    // every host blob must be pinned memory the device can read
    std::vector<uint32_t> w(L.words, 0u);
    for (int e = 0; e < c->E; ++e) {
        void *dp = nullptr;
        if (hipHostGetDevicePointer(&dp, (void *)(uintptr_t)c->host[e].blob, 0) != hipSuccess || !dp) {
            (void)hipGetLastError();
            return fail(MOE_ERR_UNSUPPORTED, "expert %d's host blob is not pinned device-accessible memory "
                                             "(allocate the store with hipHostMalloc)", e);
        }
        const uint64_t a = (uint64_t)(uintptr_t)dp;
        w[L.src + 2 * (size_t)e] = (uint32_t)a;
        w[L.src + 2 * (size_t)e + 1] = (uint32_t)(a >> 32);
        w[L.nbytes + e] = (uint32_t)c->bytes[e];
        w[L.bits + e] = c->host[e].bits;
    }
    // the host state so far: occupied slots are 0 .. n_used - 1 (the lowest free slot is always taken)
    int n_used = 0;
    for (int s = 0; s < c->n_slots; ++s) n_used += c->expert_of[s] >= 0 ? 1 : 0;
    w[0] = (uint32_t)n_used;
    int prev = -1, head = -1;
    for (const auto &ls : c->lru) {                 // least recent first
        const int s = ls.second;
        w[L.prev + s] = (uint32_t)prev;
        if (prev >= 0) w[L.next + prev] = (uint32_t)s; else head = s;
        prev = s;
    }
    if (prev >= 0) w[L.next + prev] = (uint32_t)-1;
    w[1] = (uint32_t)head;
    w[2] = (uint32_t)prev;
    for (int s = 0; s < c->n_slots; ++s) {
        w[L.expert_of + s] = (uint32_t)c->expert_of[s];
        if (c->expert_of[s] < 0) w[L.prev + s] = w[L.next + s] = (uint32_t)-1;
    }
    for (int e = 0; e < c->E; ++e) w[L.slot_of + e] = (uint32_t)c->slot_of[e];
    w[6] = (uint32_t)c->hits; w[7] = (uint32_t)(c->hits >> 32);
    w[8] = (uint32_t)c->misses; w[9] = (uint32_t)(c->misses >> 32);
    w[10] = (uint32_t)c->copied; w[11] = (uint32_t)(c->copied >> 32);
    hipStream_t st = (hipStream_t)stream;
    if (hipError_t e = hipMemcpyAsync(state, w.data(), L.words * 4, hipMemcpyHostToDevice, st))
        return fail(MOE_ERR_DEVICE, "state upload: %s", hipGetErrorString(e));
    if (hipError_t e = hipStreamSynchronize(st)) return fail(MOE_ERR_DEVICE, "state upload: %s", hipGetErrorString(e));
    int dev = 0;
    if (hipError_t e = hipGetDevice(&dev)) return fail(MOE_ERR_DEVICE, "hipGetDevice: %s", hipGetErrorString(e));
    c->dev_state = (uint32_t *)state;
    c->dev_device = dev;
    return ok();
}

int moe_cache_fetch_device(moe_expert_cache *c, const int32_t *idx, int n, void *stream) {
    if (!c) return fail(MOE_ERR_NULL, "cache is NULL");
    if (!c->dev_state) return fail(MOE_ERR_UNSUPPORTED, "the cache has no device state: call moe_cache_attach_device");
    if (n < 0) return fail(MOE_ERR_SHAPE, "n=%d is negative", n);
    if (n > 0 && !idx) return fail(MOE_ERR_NULL, "idx is NULL");
    if (idx && !aligned(idx, 4)) return fail(MOE_ERR_ALIGN, "idx must be 4-byte aligned");
    moe::CacheDevLaunch cl{c->dev_state, c->E, c->n_slots, c->table, c->slots, c->slot_bytes};
    if (int st = MOE_LAUNCH(moe::launch_cache_fetch_device(cl, idx, n, (hipStream_t)stream), "device cache fetch"))
        return st;
    return ok();
}

int moe_cache_device_refused(const moe_expert_cache *c) {
    if (!c || !c->dev_state) return -1;
    uint32_t v = 0;
    if (hipMemcpy(&v, c->dev_state + 4, 4, hipMemcpyDeviceToHost) != hipSuccess) return -1;
    return (int)v;
}

void moe_cache_destroy(moe_expert_cache *c) { delete c; }

int moe_debug_inject_launch_failure(int after, int count) {
    if (after < 0 || count < 0) return fail(MOE_ERR_SHAPE, "after=%d count=%d must be >= 0", after, count);
    std::lock_guard<std::mutex> lock(g_inject_mu);
    g_pass = after;
    g_fail = count;
    g_armed.store(count > 0, std::memory_order_release);
    return ok();
}

// Start/stop events of kernel j of a timed call: events[2j], events[2j+1].
static moe::KernelEvents kernel_events(void *const *events, int j) {
    moe::KernelEvents ev;
    if (events) {
        ev.start = (hipEvent_t)events[2 * j];
        ev.stop = (hipEvent_t)events[2 * j + 1];
    }
    return ev;
}

static int layer_decode_impl(const moe_dims *dims, const moe_layer *layers, int n_layers, const void *x,
                             int x_dtype, unsigned flags, float *out, int32_t *idx, float *w, void *ws,
                             size_t ws_bytes, void *stream, void *const *events, bool per_call_errors) {
    if (int s = check_dims(dims)) return s;
    if (!layers) return fail(MOE_ERR_NULL, "layers is NULL");
    if (n_layers < 1 || n_layers > 4096) return fail(MOE_ERR_SHAPE, "n_layers=%d outside [1, 4096]", n_layers);
    for (int l = 0; l < n_layers; ++l)
        if (int s = check_layer(&layers[l], l)) return s;
    if (int s = check_dtype(x_dtype, "x")) return s;
    if (!x || !out) return fail(MOE_ERR_NULL, "x and out are required");
    if ((idx == nullptr) != (w == nullptr)) return fail(MOE_ERR_NULL, "idx and w must both be given or both NULL");
    if (flags & ~(MOE_FLAG_RESIDUAL | MOE_FLAG_SEPARATE_KERNELS | MOE_FLAG_SINGLE_LAUNCH))
        return fail(MOE_ERR_UNSUPPORTED, "unknown flags 0x%x", flags);
    if ((flags & MOE_FLAG_SEPARATE_KERNELS) && (flags & MOE_FLAG_SINGLE_LAUNCH))
        return fail(MOE_ERR_UNSUPPORTED, "MOE_FLAG_SEPARATE_KERNELS and MOE_FLAG_SINGLE_LAUNCH exclude each other");
    if (!aligned(x, 16) || !aligned(out, 16)) return fail(MOE_ERR_ALIGN, "x and out must be 16-byte aligned");
    if ((idx && !aligned(idx, 4)) || (w && !aligned(w, 4))) return fail(MOE_ERR_ALIGN, "idx/w not 4-byte aligned");
    if (out == x) return fail(MOE_ERR_SHAPE, "out must not alias x");
    if (int s = check_ws(ws, ws_bytes, decode_ws(dims))) return s;

    const int H = dims->hidden, I = dims->inter, E = dims->n_experts, K = dims->top_k;
    const DecodeWs W = decode_layout(dims, ws);
    hipStream_t st = (hipStream_t)stream;
    const bool residual = flags & MOE_FLAG_RESIDUAL;
    const bool separate = flags & MOE_FLAG_SEPARATE_KERNELS;
    const bool single = flags & MOE_FLAG_SINGLE_LAUNCH;
    int nw = 0;
    if (single)
        if (int s = fused_workgroups_cached(dims, &nw)) return s;
    for (int l = 0; l < n_layers; ++l) {
        const moe_layer &L = layers[l];
        const void *xl = l == 0 ? x : (const void *)(W.xbuf + (size_t)((l - 1) & 1) * H);
        const int xdt = l == 0 ? x_dtype : MOE_F32;
        float *ol = l == n_layers - 1 ? out : W.xbuf + (size_t)(l & 1) * H;
        int32_t *idx_l = idx ? idx + (size_t)l * K : nullptr;
        float *w_l = w ? w + (size_t)l * K : nullptr;
        moe::RouterLaunch ra{xl, xdt, H, L.norm_w, L.norm_eps, L.router, L.router_dtype, L.logit_bias, W.logits, H, E, 1,
                             nullptr};
        if (!separate) {
            moe::LayerLaunch la{};
            la.r = ra;
            la.experts = L.experts;
            la.idx_out = idx_l;
            la.w_out = w_l;
            la.sel_ws = W.sel;
            la.w_ws = W.w;
            la.h = W.h;
            la.H = H; la.I = I; la.E = E; la.K = K;
            la.split = !(xdt == MOE_BF16 && L.norm_w == nullptr);
            la.seq = W.sync;
            la.err = W.sync + 1;
            la.clear_err = per_call_errors && l == 0;
            la.slots = W.slots;
            if (single) {
                moe::FusedLaunch fa{};
                fa.L = la;
                fa.residual = residual ? xl : nullptr;
                fa.residual_dtype = xdt;
                fa.out = ol;
                fa.flags = W.flags;
                fa.seq = W.sync;
                fa.nw = nw;
                if (int s = MOE_LAUNCH(moe::launch_layer_fused(fa, st, kernel_events(events, l)), "layer")) return s;
                continue;
            }
            if (int s = MOE_LAUNCH(moe::launch_layer(la, st, kernel_events(events, 2 * l)), "router + gate/up")) return s;
            moe::DownLaunch da{W.h, W.sync, W.sync + 1, W.sel, W.w, residual ? xl : nullptr, xdt, H, ol, H, I, K, 1};
            if (int s = MOE_LAUNCH(moe::launch_down(da, st, kernel_events(events, 2 * l + 1)), "down")) return s;
            continue;
        }
        if (int s = MOE_LAUNCH(moe::launch_router(ra, st, kernel_events(events, 3 * l)), "router")) return s;
        moe::GateUpLaunch ga{xl, xdt, H, L.norm_w, L.norm_eps, W.logits, nullptr, idx_l, w_l, W.sel, W.w,
                             L.experts, W.h, H, I, E, K, 1};
        if (int s = MOE_LAUNCH(moe::launch_gateup(ga, st, kernel_events(events, 3 * l + 1)), "gate/up")) return s;
        moe::DownLaunch da{W.h, nullptr, nullptr, W.sel, W.w, residual ? xl : nullptr, xdt, H, ol, H, I, K, 1};
        if (int s = MOE_LAUNCH(moe::launch_down(da, st, kernel_events(events, 3 * l + 2)), "down")) return s;
    }
    return ok();
}

int moe_layer_decode(const moe_dims *dims, const moe_layer *layers, int n_layers, const void *x, int x_dtype,
                     unsigned flags, float *out, int32_t *idx, float *w, void *ws, size_t ws_bytes, void *stream) {
    return layer_decode_impl(dims, layers, n_layers, x, x_dtype, flags, out, idx, w, ws, ws_bytes, stream, nullptr,
                             false);
}

int moe_layer_decode_timed(const moe_dims *dims, const moe_layer *layers, int n_layers, const void *x, int x_dtype,
                           unsigned flags, float *out, int32_t *idx, float *w, void *ws, size_t ws_bytes,
                           void *stream, void *const *events) {
    if (!events) return fail(MOE_ERR_NULL, "events is NULL");
    if (n_layers < 1 || n_layers > 4096) return fail(MOE_ERR_SHAPE, "n_layers=%d outside [1, 4096]", n_layers);
    const int per_layer = (flags & MOE_FLAG_SEPARATE_KERNELS) ? 3 : (flags & MOE_FLAG_SINGLE_LAUNCH) ? 1 : 2;
    for (int i = 0; i < 2 * per_layer * n_layers; ++i)
        if (!events[i]) return fail(MOE_ERR_NULL, "events[%d] is NULL", i);
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing((hipStream_t)stream, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone)
        return fail(MOE_ERR_UNSUPPORTED, "moe_layer_decode_timed cannot be captured into a graph");
    return layer_decode_impl(dims, layers, n_layers, x, x_dtype, flags, out, idx, w, ws, ws_bytes, stream, events,
                             false);
}

}  // extern "C"

namespace moe {
int layer_decode_entry(const moe_dims *dims, const moe_layer *layers, int n_layers, const void *x, int x_dtype,
                       unsigned flags, float *out, int32_t *idx, float *w, void *ws, size_t ws_bytes, void *stream,
                       void *const *events, bool per_call_errors) {
    return layer_decode_impl(dims, layers, n_layers, x, x_dtype, flags, out, idx, w, ws, ws_bytes, stream, events,
                             per_call_errors);
}
size_t layer_decode_ws_bytes(const moe_dims *dims) {
    return check_dims(dims) == MOE_OK ? decode_ws(dims) : 0;
}
int set_error(int status, const char *msg) { return fail(status, "%s", msg); }
}  // namespace moe
