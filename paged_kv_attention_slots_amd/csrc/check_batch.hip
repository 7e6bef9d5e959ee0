// Device-side check of a batch's metadata: the invariants msgl_validate_batch
// checks on host copies, checked on the device arrays the attention calls
// read, so that a debug step can run (or be captured) right before them with
// no host copy and no synchronisation.
//
// The invariants are the ones the pages' engine builds into its metadata
// (Mini-SGLang tag page, Engine article, the per-batch metadata step: a
// request's keys are its page-table row up to its length, its new tokens are
// the row's entries from its cached length on, and they are what store_kv
// writes; KV-cache article: slots index the pools, page_size consecutive
// slots per page).
//
// One wave per request.  Every read is in bounds whatever the metadata hold:
// a request's page-table row is read only once its table index is known to
// be in [0, rows), up to min(seq_len, row_stride) entries; out_loc only at
// token indices in [0, num_tokens); the repeat bitmap only at slots in
// [0, num_slots).  Violations are recorded with vector atomics into `result`.
#include <algorithm>
#include <climits>

#include "common.h"
#include "check_batch.h"

namespace msgl {

namespace {

constexpr int kCheckWaves = 4;

__global__ __launch_bounds__(256) void check_init_kernel(CheckBatchArgs a) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < a.seen_words; i += stride) a.seen[i] = 0u;
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        a.result[0] = 0;
        a.result[1] = 0;
        a.result[2] = INT_MAX;
        a.result[3] = INT_MAX;
    }
}

MSGL_DEV int wave_or(int v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v |= __shfl_xor(v, off);
    return v;
}

__global__ __launch_bounds__(64 * kCheckWaves) void check_batch_kernel(CheckBatchArgs a) {
    const int lane = threadIdx.x & 63;
    const int b = blockIdx.x * kCheckWaves + (int)(threadIdx.x >> 6);
    if (b >= a.batch) return;
    const int lim = min(a.max_seq_len, a.row_stride);
    const int r = a.table_idx[b];
    const int L = a.seq_lens[b];
    const int C = a.cached_lens != nullptr ? a.cached_lens[b] : L - 1;
    int code = 0;
    if (r < 0 || r >= a.rows) code |= kCheckTableIdx;
    if (L < 1 || L > lim) code |= kCheckSeqLen;
    if (C < 0 || C >= L) code |= kCheckCachedLen;
    int t0 = b;  // decode without cu_q: one new token per request, in batch order
    if (a.cu_q != nullptr) {
        const int q0 = a.cu_q[b], q1 = a.cu_q[b + 1];
        if ((b == 0 && q0 != 0) || (int64_t)q1 - q0 != (int64_t)L - C) code |= kCheckCuQ;
        if (a.out_loc != nullptr && b == a.batch - 1 && q1 != a.num_tokens) code |= kCheckTokenCount;
        t0 = q0;
    }
    // the request's keys: slot ids in range, pages of consecutive slots starting at multiples of page_size
    int lane_code = 0;
    if (!(code & kCheckTableIdx)) {
        const int32_t *row = a.page_table + (int64_t)r * a.row_stride;
        const int n = min(max(L, 0), a.row_stride);
        for (int j = lane; j < n; j += 64) {
            const int s = row[j];
            if (s < 0 || s >= a.num_slots) lane_code |= kCheckSlot;
            if (a.page_size > 1) {
                const int off = j % a.page_size;
                if (off == 0 ? s % a.page_size != 0 : s != row[j - 1] + 1) lane_code |= kCheckPage;
            }
        }
        // the new tokens: out_loc[t0 + i - C] == row[i] for C <= i < L, each slot once (but the dummy)
        if (a.out_loc != nullptr && code == 0) {
            int first_bad = INT_MAX;
            for (int i = C + lane; i < L; i += 64) {
                const int64_t t = (int64_t)t0 + (i - C);
                int c = 0;
                if (t < 0 || t >= a.num_tokens) {
                    c = kCheckTokenCount;
                } else {
                    const int s = a.out_loc[t];
                    if (s < 0 || s >= a.num_slots) {
                        c = kCheckOutLoc;
                    } else {
                        if (s != row[i]) c = kCheckOutLoc;
                        if (a.seen != nullptr) {
                            const uint32_t bit = 1u << (s & 31);
                            const uint32_t old = atomicOr(a.seen + (s >> 5), bit);
                            if ((old & bit) && s != a.dummy_slot) c |= kCheckRepeat;
                        }
                    }
                    if (c != 0) first_bad = min(first_bad, (int)t);
                }
                lane_code |= c;
            }
            if (first_bad != INT_MAX) atomicMin(a.result + 3, first_bad);
        }
    }
    code = wave_or(code | lane_code);
    if (code != 0 && lane == 0) {
        atomicOr(a.result, code);
        atomicAdd(a.result + 1, 1);
        atomicMin(a.result + 2, b);
    }
}

}  // namespace

hipError_t launch_check_batch(const CheckBatchArgs &a, hipStream_t stream) {
    const int64_t init_blocks = std::min<int64_t>(1024, std::max<int64_t>(1, (a.seen_words + 255) / 256));
    hipLaunchKernelGGL(check_init_kernel, dim3((unsigned)init_blocks), dim3(256), 0, stream, a);
    if (a.batch > 0) {
        const unsigned blocks = (unsigned)((a.batch + kCheckWaves - 1) / kCheckWaves);
        hipLaunchKernelGGL(check_batch_kernel, dim3(blocks), dim3(64 * kCheckWaves), 0, stream, a);
    }
    return hipGetLastError();
}

}  // namespace msgl
