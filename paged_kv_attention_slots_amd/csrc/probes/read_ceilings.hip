// Read-bandwidth probes for the ceilings the decode attention kernel is held
// against (measurement only; not part of libmsgl): how fast this GPU streams a
// large buffer, and how fast it reads a KV pool in the decode kernel's access
// patterns (random rows read as 256-byte per-head slices, and random 16-row
// pages read the same way).  Each kernel folds what it reads into one word and
// writes it when a runtime flag (always 0 from the launchers) is set, so that
// the compiler keeps every load.
// Every index is in bounds by construction: grid-stride loops over [0, n) and
// row ids the caller checked to lie in [0, rows).
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Sequential stream of 16-byte nontemporal loads, 4 in flight per lane.
__global__ __launch_bounds__(256) void stream_read(const u32x4 *__restrict__ p, int64_t n, unsigned *sink,
                                                   int keep) {
    unsigned acc = 0;
    const int64_t step = (int64_t)gridDim.x * 256 * 4;
    for (int64_t i = (int64_t)blockIdx.x * 256 * 4 + threadIdx.x; i < n; i += step) {
        u32x4 v[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int64_t j = i + (int64_t)k * 256;
            v[k] = j < n ? __builtin_nontemporal_load(p + j) : u32x4{0, 0, 0, 0};
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) acc ^= v[k].x ^ v[k].y ^ v[k].z ^ v[k].w;
    }
    if (keep) sink[blockIdx.x & 3] = acc;
}

// Rows of `row_vec` 16-byte vectors (kv heads x 256 bytes); head h = blockIdx.y.
// Each group of 16 lanes reads one row's 256-byte slice of head h; a wave holds
// 4 rows per load and NF loads in flight.  PAGE: ids name pages of 16
// consecutive rows, and a wave reads the 16 rows of NF / 4 pages per round (the
// page-size-16 pattern); otherwise each row id is a random row (page size 1).
template <bool PAGE, int NF>
__global__ __launch_bounds__(256) void gather_heads(const u32x4 *__restrict__ pool, const int *__restrict__ ids,
                                                    int n_ids, int row_vec, unsigned *sink, int keep) {
    static_assert(NF % 4 == 0, "whole pages per round");
    const int lane = threadIdx.x & 63, grp = lane >> 4, l = lane & 15;
    const int wave = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int nwaves = gridDim.x * 4;
    const int h = blockIdx.y;
    unsigned acc = 0;
    const int per_wave = PAGE ? NF / 4 : 4 * NF;  // ids a wave consumes per round
    for (int r0 = wave * per_wave; r0 < n_ids; r0 += nwaves * per_wave) {
        u32x4 v[NF];
#pragma unroll
        for (int k = 0; k < NF; ++k) {
            int64_t row;
            bool ok;
            if (PAGE) {
                const int r = r0 + k / 4;
                ok = r < n_ids;
                row = ok ? (int64_t)ids[r] * 16 + 4 * (k % 4) + grp : 0;
            } else {
                const int r = r0 + 4 * k + grp;
                ok = r < n_ids;
                row = ok ? ids[r] : 0;
            }
            v[k] = ok ? __builtin_nontemporal_load(pool + row * row_vec + h * 16 + l) : u32x4{0, 0, 0, 0};
        }
#pragma unroll
        for (int k = 0; k < NF; ++k) acc ^= v[k].x ^ v[k].w;
    }
    if (keep) sink[blockIdx.x & 3] = acc;
}

}  // namespace

// bytes: a multiple of 16.  Returns a hipError_t.
extern "C" int msglp_stream_read(const void *buf, int64_t bytes, unsigned *sink, int blocks, void *stream) {
    if (bytes % 16 != 0 || blocks < 1) return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(stream_read, dim3(blocks), dim3(256), 0, (hipStream_t)stream, (const u32x4 *)buf, bytes / 16,
                       sink, 0);
    return (int)hipGetLastError();
}

// pool: rows of heads x 256 bytes.  page == 0: ids are n_ids row ids in [0, rows);
// page == 1: ids are n_ids page ids in [0, rows / 16).  Reads every head's slice of
// every named row: n_ids x heads x 256 bytes (x 16 for pages).  inflight: 4 or 8
// loads per lane in flight.
extern "C" int msglp_gather_heads(const void *pool, const int *ids, int n_ids, int heads, int page, unsigned *sink,
                                  int blocks, int inflight, void *stream) {
    if (heads < 1 || heads > 64 || n_ids < 0 || blocks < 1 || (inflight != 4 && inflight != 8))
        return (int)hipErrorInvalidValue;
    const dim3 grid(blocks, heads);
    const hipStream_t st = (hipStream_t)stream;
    const u32x4 *p = (const u32x4 *)pool;
    if (page && inflight == 4) hipLaunchKernelGGL((gather_heads<true, 4>), grid, dim3(256), 0, st, p, ids, n_ids, heads * 16, sink, 0);
    if (page && inflight == 8) hipLaunchKernelGGL((gather_heads<true, 8>), grid, dim3(256), 0, st, p, ids, n_ids, heads * 16, sink, 0);
    if (!page && inflight == 4) hipLaunchKernelGGL((gather_heads<false, 4>), grid, dim3(256), 0, st, p, ids, n_ids, heads * 16, sink, 0);
    if (!page && inflight == 8) hipLaunchKernelGGL((gather_heads<false, 8>), grid, dim3(256), 0, st, p, ids, n_ids, heads * 16, sink, 0);
    return (int)hipGetLastError();
}
