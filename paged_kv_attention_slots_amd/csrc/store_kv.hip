// store_kv: scatter the step's new K/V rows into the paged pools at out_loc.
//
// The KV-write custom kernel of the Stage 4 milestone ("What each chapter
// adds"): a pure copy, one [kv_heads, head_dim] row per new token, for K and
// V.  Source and destination rows are contiguous (2 KiB for 8 kv heads x 128
// bf16), so each thread moves one 16-byte vector of K and the same vector of
// V; a row is covered by consecutive threads, which makes every wave's reads
// and writes whole 128-byte lines.  HBM-bound: 2 x row bytes read + written
// per token, plus the 4-byte slot id.
#include "common.h"
#include "launch.h"

namespace msgl {

__global__ __launch_bounds__(256) void store_kv_kernel(StoreKvArgs a) {
    const int64_t nvec = a.row_vec16;
    const int64_t total = (int64_t)a.num_tokens * nvec;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t t = i / nvec;
        const int64_t v = i - t * nvec;
        const int64_t slot = a.out_loc[t];
        if (slot < 0 || slot >= a.num_slots) continue;  // malformed id: never write out of bounds
        const int64_t dst = slot * nvec + v;
        const uint4 kv = ld16_nt(reinterpret_cast<const uint4 *>(a.k_new) + i);
        const uint4 vv = ld16_nt(reinterpret_cast<const uint4 *>(a.v_new) + i);
        reinterpret_cast<uint4 *>(a.k_pool)[dst] = kv;
        reinterpret_cast<uint4 *>(a.v_pool)[dst] = vv;
    }
}

hipError_t launch_store_kv(const StoreKvArgs &a, hipStream_t stream) {
    if (a.num_tokens == 0) return hipSuccess;
    const int64_t total = (int64_t)a.num_tokens * a.row_vec16;
    int64_t blocks = (total + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL(store_kv_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace msgl
