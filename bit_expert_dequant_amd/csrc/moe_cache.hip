// moe_cache.hip -- device side of the expert cache: writes of the descriptor table that the expert
// kernels read.  The pages stream each selected expert from SSD once routing is known and rely on
// the OS page cache for reuse (lilting.ch, "397Bパラメータモデルを48GB MacBookで動かすFlash-MoE",
// section "コア技術: SSDエキスパートストリーミング"); here the store is in host memory and a cache of
// slots in device memory plays the page cache's part.  With the host policy (moe_api.cpp) these
// kernels only rewrite table entries, with the new entries passed by value as kernel arguments, so
// no host buffer has to outlive the enqueue; the device-side policy runs the same policy in a kernel
// and copies the missing blobs with a kernel reading the pinned host memory directly.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kUpdMax = 64;                   // table entries per update kernel

struct TableUpdates {
    int32_t n;
    int32_t expert[kUpdMax];
    uint32_t bits[kUpdMax];
    uint64_t blob[kUpdMax];                   // 0: the expert is absent
};

__global__ void __launch_bounds__(kUpdMax) k_table_update(moe_expert_desc *table, TableUpdates u) {
    const int i = threadIdx.x;
    if (i >= u.n) return;
    moe_expert_desc d;
    d.blob = u.blob[i];
    d.bits = u.bits[i];
    d.reserved = 0;
    table[u.expert[i]] = d;
}

__global__ void __launch_bounds__(256) k_table_absent(moe_expert_desc *table, int E) {
    const int e = blockIdx.x * 256 + threadIdx.x;
    if (e >= E) return;
    moe_expert_desc d;
    d.blob = 0;
    d.bits = 4;
    d.reserved = 0;
    table[e] = d;
}

// --------------------------------------------------------------------------- device-side policy
// The policy of the host cache (hits first become most recent; each missing expert, in first
// occurrence order, takes the lowest never-used slot or else the least recently used slot the step
// has not touched, equal times by lower slot) on device indices, so a routing step needs no host
// round trip.  The least-recent order is a doubly linked list of occupied slots; the slots a step
// touches (all given that step's time) are appended in slot order, which keeps the list sorted by
// (last use, slot) -- the host cache's order.  One workgroup: every thread loads the state into LDS
// and finds the step's distinct experts in first-occurrence order (LDS atomic minimum of the
// position per expert, then an ordered compaction); thread 0 walks them through the list; every
// thread writes the state back.  Table entries change in the same kernel: the copy kernel after it
// and the expert kernels after that run in stream order.
__device__ __forceinline__ uint64_t ld64(const uint32_t *p) { return (uint64_t)p[0] | ((uint64_t)p[1] << 32); }
__device__ __forceinline__ void st64(uint32_t *p, uint64_t v) {
    p[0] = (uint32_t)v;
    p[1] = (uint32_t)(v >> 32);
}

__global__ void __launch_bounds__(256) k_cache_policy(CacheDevLaunch c, const int32_t *idx, int n) {
    extern __shared__ int32_t sm[];
    const int E = c.E, S = c.S, tid = threadIdx.x, TW = (S + 31) / 32;
    const CacheLayout L = cache_layout(E, S);
    uint32_t *st = c.state;
    int *s_first = sm, *s_slot = s_first + E, *s_exp = s_slot + E, *s_prev = s_exp + S, *s_next = s_prev + S;
    uint32_t *s_touch = (uint32_t *)(s_next + S);
    int *s_req = (int *)(s_touch + TW), *s_cnt = s_req + E;
    for (int i = tid; i < E; i += 256) {
        s_first[i] = 0x7FFFFFFF;
        s_slot[i] = (int)st[L.slot_of + i];
    }
    for (int i = tid; i < S; i += 256) {
        s_exp[i] = (int)st[L.expert_of + i];
        s_prev[i] = (int)st[L.prev + i];
        s_next[i] = (int)st[L.next + i];
    }
    for (int i = tid; i < TW; i += 256) s_touch[i] = 0u;
    __syncthreads();
    for (int p = tid; p < n; p += 256) {
        const int e = idx[p];
        if (e >= 0 && e < E) atomicMin(&s_first[e], p);
    }
    __syncthreads();
    // ordered compaction of the first occurrences: thread t takes positions [t * ch, (t + 1) * ch)
    const int ch = (n + 255) / 256, p0 = tid * ch, p1 = min(n, p0 + ch);
    int cnt = 0;
    for (int p = p0; p < p1; ++p) {
        const int e = idx[p];
        cnt += (e >= 0 && e < E && s_first[e] == p) ? 1 : 0;
    }
    s_cnt[tid] = cnt;
    __syncthreads();
    if (tid == 0) {
        int acc = 0;
        for (int t = 0; t < 256; ++t) {
            const int v = s_cnt[t];
            s_cnt[t] = acc;
            acc += v;
        }
        s_cnt[256] = acc;
    }
    __syncthreads();
    int o = s_cnt[tid];
    for (int p = p0; p < p1; ++p) {
        const int e = idx[p];
        if (e >= 0 && e < E && s_first[e] == p) s_req[o++] = e;
    }
    __syncthreads();
    if (tid == 0) {
        const int nreq = s_cnt[256];
        int n_used = (int)st[0], head = (int)st[1], tail = (int)st[2], nc = 0;
        if (nreq > S) {
            st[4] += 1u;                                   // refused: nothing changes
        } else {
            uint64_t hits = ld64(st + 6), misses = ld64(st + 8), bytes = ld64(st + 10);
            auto unlink = [&](int s) {
                const int pv = s_prev[s], nx = s_next[s];
                if (pv >= 0) s_next[pv] = nx; else head = nx;
                if (nx >= 0) s_prev[nx] = pv; else tail = pv;
            };
            for (int i = 0; i < nreq; ++i) {
                const int s = s_slot[s_req[i]];
                if (s < 0) continue;
                ++hits;
                unlink(s);
                s_touch[s >> 5] |= 1u << (s & 31);
            }
            for (int i = 0; i < nreq; ++i) {
                const int e = s_req[i];
                if (s_slot[e] >= 0) continue;
                int s;
                if (n_used < S) {
                    s = n_used++;
                } else {
                    s = head;                              // least recent untouched slot
                    unlink(s);
                    const int old = s_exp[s];
                    s_slot[old] = -1;
                    c.table[old] = moe_expert_desc{0, 4u, 0u};
                }
                s_slot[e] = s;
                s_exp[s] = e;
                s_touch[s >> 5] |= 1u << (s & 31);
                st[L.copy + 2 * nc] = (uint32_t)s;
                st[L.copy + 2 * nc + 1] = (uint32_t)e;
                ++nc;
                ++misses;
                bytes += st[L.nbytes + e];
                c.table[e] = moe_expert_desc{(uint64_t)(c.slots + (size_t)s * c.slot_bytes), st[L.bits + e], 0u};
            }
            for (int w = 0; w < TW; ++w) {                 // touched slots become most recent, in slot order
                for (uint32_t b = s_touch[w]; b; b &= b - 1) {
                    const int s = w * 32 + __builtin_ctz(b);
                    s_prev[s] = tail;
                    s_next[s] = -1;
                    if (tail >= 0) s_next[tail] = s; else head = s;
                    tail = s;
                }
            }
            st64(st + 6, hits);
            st64(st + 8, misses);
            st64(st + 10, bytes);
        }
        st[0] = (uint32_t)n_used;
        st[1] = (uint32_t)head;
        st[2] = (uint32_t)tail;
        st[3] = (uint32_t)nc;
    }
    __syncthreads();
    for (int i = tid; i < E; i += 256) st[L.slot_of + i] = (uint32_t)s_slot[i];
    for (int i = tid; i < S; i += 256) {
        st[L.expert_of + i] = (uint32_t)s_exp[i];
        st[L.prev + i] = (uint32_t)s_prev[i];
        st[L.next + i] = (uint32_t)s_next[i];
    }
}

// The step's loads: every workgroup takes a grid-stride share of each missing blob, read straight
// from pinned host memory (16-byte loads, no L2 allocation) into its slot.
typedef uint32_t u32x4c __attribute__((ext_vector_type(4)));
__global__ void __launch_bounds__(256) k_cache_copy(CacheDevLaunch c) {
    const CacheLayout L = cache_layout(c.E, c.S);
    const uint32_t *st = c.state;
    const int nc = (int)st[3];
    for (int j = 0; j < nc; ++j) {
        const int s = (int)st[L.copy + 2 * j], e = (int)st[L.copy + 2 * j + 1];
        const u32x4c *src = (const u32x4c *)ld64(st + L.src + 2 * (size_t)e);
        u32x4c *dst = (u32x4c *)(c.slots + (size_t)s * c.slot_bytes);
        const size_t n16 = st[L.nbytes + e] / 16;
        for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += (size_t)gridDim.x * 256)
            dst[i] = __builtin_nontemporal_load(src + i);
    }
}

}  // namespace

size_t cache_policy_lds_bytes(int E, int S) {
    return ((size_t)2 * E + 3 * (size_t)S + (S + 31) / 32 + E + 257) * 4;
}

hipError_t launch_cache_fetch_device(const CacheDevLaunch &c, const int32_t *idx, int n, hipStream_t s) {
    const size_t lds = cache_policy_lds_bytes(c.E, c.S);
    if (hipError_t e = lds_for<k_cache_policy>(lds)) return e;
    hipLaunchKernelGGL(k_cache_policy, dim3(1), dim3(256), lds, s, c, idx, n);
    if (hipError_t e = hipGetLastError()) return e;
    // 256 workgroups: measured at the link's rate (57 GB/s) for 64 to 512 of them
    hipLaunchKernelGGL(k_cache_copy, dim3(256), dim3(256), 0, s, c);
    return hipGetLastError();
}

hipError_t launch_table_absent(moe_expert_desc *table, int E, hipStream_t s) {
    hipLaunchKernelGGL(k_table_absent, dim3((unsigned)((E + 255) / 256)), dim3(256), 0, s, table, E);
    return hipGetLastError();
}

hipError_t launch_table_update(moe_expert_desc *table, int n, const int32_t *expert, const uint64_t *blob,
                               const uint32_t *bits, hipStream_t s) {
    for (int i0 = 0; i0 < n; i0 += kUpdMax) {
        TableUpdates u;
        u.n = n - i0 < kUpdMax ? n - i0 : kUpdMax;
        for (int i = 0; i < u.n; ++i) {
            u.expert[i] = expert[i0 + i];
            u.blob[i] = blob[i0 + i];
            u.bits[i] = bits[i0 + i];
        }
        hipLaunchKernelGGL(k_table_update, dim3(1), dim3(kUpdMax), 0, s, table, u);
        if (hipError_t e = hipGetLastError()) return e;
    }
    return hipSuccess;
}

}  // namespace moe
