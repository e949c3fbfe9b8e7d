// moe_cache.hip -- device side of the expert cache: writes of the descriptor table that the expert
// kernels read.  The pages stream each selected expert from SSD once routing is known and rely on
// the OS page cache for reuse (lilting.ch, "397Bパラメータモデルを48GB MacBookで動かすFlash-MoE",
// section "コア技術: SSDエキスパートストリーミング"); here the store is in host memory and a cache of
// slots in device memory plays the page cache's part.  The policy and the copies are host code in
// moe_api.cpp; these kernels only rewrite table entries, with the new entries passed by value as
// kernel arguments, so no host buffer has to outlive the enqueue.
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

}  // namespace

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
