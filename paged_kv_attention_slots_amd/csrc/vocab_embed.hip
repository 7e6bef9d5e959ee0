// vocab_embed: vocabulary indexing, the embedding rows of the step's token ids.
//
// The Stage 4 milestone's table names vocabulary indexing, beside the KV
// write, as a small operation worth its own kernel (launch overhead and
// memory traffic).  Under tensor parallelism a rank holds the table rows of
// the ids vocab_start .. vocab_start + rows - 1; an id outside that range
// gives a zero row, so the ranks' outputs sum to the full table's rows.
//
// A pure gather: one block per token (grid-stride over tokens), its threads
// striding over the row's 16-byte vectors, so every wave reads and writes
// whole 128-byte lines; each thread issues all its loads before its stores.
// The id is checked against the shard before any read.  HBM-bound: per token
// one row read and one row written (nothing read for an id outside the
// shard), plus the 4-byte id.
#include "common.h"
#include "launch.h"

namespace msgl {

constexpr int kEmbedThreads = 256;
constexpr int kEmbedVecs = 4;  // vectors per thread kept in flight (rows up to 16 KiB in one pass)

__global__ __launch_bounds__(kEmbedThreads) void vocab_embed_kernel(VocabEmbedArgs a) {
    const int tid = threadIdx.x;
    const uint4 zero = make_uint4(0u, 0u, 0u, 0u);
    for (int t = blockIdx.x; t < a.num_tokens; t += gridDim.x) {
        const int64_t r = (int64_t)a.ids[t] - a.vocab_start;
        const bool hit = r >= 0 && r < a.rows;
        const uint4 *src = static_cast<const uint4 *>(a.weight) + (hit ? r : 0) * a.row_vec;
        uint4 *dst = static_cast<uint4 *>(a.out) + (int64_t)t * a.row_vec;
        for (int v0 = 0; v0 < a.row_vec; v0 += kEmbedThreads * kEmbedVecs) {
            uint4 x[kEmbedVecs];
#pragma unroll
            for (int k = 0; k < kEmbedVecs; ++k) {
                const int v = v0 + tid + kEmbedThreads * k;
                x[k] = (hit && v < a.row_vec) ? ld16_nt(src + v) : zero;
            }
#pragma unroll
            for (int k = 0; k < kEmbedVecs; ++k) {
                const int v = v0 + tid + kEmbedThreads * k;
                if (v < a.row_vec) dst[v] = x[k];
            }
        }
    }
}

hipError_t launch_vocab_embed(const VocabEmbedArgs &a, hipStream_t stream) {
    if (a.num_tokens == 0) return hipSuccess;
    const unsigned blocks = (unsigned)(a.num_tokens < 65536 ? a.num_tokens : 65536);
    hipLaunchKernelGGL(vocab_embed_kernel, dim3(blocks), dim3(kEmbedThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace msgl
