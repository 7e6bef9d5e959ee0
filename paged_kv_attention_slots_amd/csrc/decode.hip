// Decode attention: split-K over each request's gathered page list.
//
// Decode has one query token per request at position seq_len - 1 (the token
// just written by store_kv).  The step is HBM-bound: each visible token's K
// and V slices are read once per kv head, and everything else (q, out,
// partials, page-table ids) is small beside them.
//
// Work decomposition.  A request's keys are cut into chunks of `chunk`
// tokens; a work item is (request, chunk, group of HPW kv heads).  The grid
// is persistent (about as many 256-thread blocks as fit on the chip at once)
// and blocks pull items from a device-side counter, so the grid does not
// depend on the lengths: a graph captured once stays valid for any batch
// whose lengths stay within max_seq_len, and the long tail of a lognormal
// length mix is balanced dynamically.  Each block derives the item list from
// seq_lens itself (a prefix sum of chunks per request in LDS).  The last
// block to finish resets the counters, so they are zero between calls
// without a memset.
//
// Inside an item, the 4 waves of the block split as HPW kv heads x (4 / HPW)
// token streams; see attend_valu.h for the lane layout.  A request whose keys
// fit in one chunk writes its normalised output directly; longer ones write
// per-chunk partial states (m, l, unnormalised o) that decode_merge_kernel
// combines with the usual log-sum-exp rescaling.
#include "attend_valu.h"
#include "launch.h"

namespace msgl {

template <typename T, int D, int GQ, int HPW>
__global__ __launch_bounds__(256) void decode_split_kernel(DecodeArgs a) {
    using Geo = Geometry<T, D>;
    constexpr int E = Geo::kEpl;
    constexpr int LPR = Geo::kLpr;
    constexpr int NSTREAM = 4 / HPW;
    extern __shared__ int s_prefix[];  // [batch + 1] chunks before each request
    __shared__ float s_buf[4 * GQ * (D + 2)];
    __shared__ int s_item;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int hw = wave % HPW;
    const int stream = wave / HPW;
    const int rg = lane / LPR;
    const int lr = lane % LPR;
    const int nhg = a.kv_heads / HPW;
    const int64_t row_elems = (int64_t)a.kv_heads * D;

    // chunk counts -> exclusive prefix in LDS (wave 0, 64 requests at a time)
    if (wave == 0) {
        int carry = 0;
        if (lane == 0) s_prefix[0] = 0;
        for (int base = 0; base < a.batch; base += 64) {
            const int b = base + lane;
            int n = 0;
            if (b < a.batch) {
                const int L = a.seq_lens[b];
                n = L > 0 ? min((L + a.chunk - 1) / a.chunk, a.max_splits) : 0;
            }
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const int y = __shfl_up(n, off);
                if (lane >= off) n += y;
            }
            if (b < a.batch) s_prefix[b + 1] = carry + n;
            carry += __shfl(n, 63);
        }
    }
    __syncthreads();
    const int total_items = s_prefix[a.batch] * nhg;

    for (;;) {
        if (tid == 0) s_item = (int)atomicAdd(&a.ctrl[0], 1u);
        __syncthreads();
        const int item = s_item;
        __syncthreads();
        if (item >= total_items) break;

        const int hg = item % nhg;
        const int pair = item / nhg;
        int lo = 0, hi = a.batch;  // s_prefix[lo] <= pair < s_prefix[hi]
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (s_prefix[mid] <= pair) lo = mid; else hi = mid;
        }
        const int b = lo;
        const int split = pair - s_prefix[b];
        const int nsplit = s_prefix[b + 1] - s_prefix[b];
        // lengths beyond the table row or the workspace's split count are cut
        // there (malformed input must not read or write out of bounds)
        const int L = min(a.seq_lens[b], (int)min(a.row_stride, (int64_t)a.max_splits * a.chunk));
        const int t0 = split * a.chunk;
        const int t1 = min(L, t0 + a.chunk);
        const int kvh = hg * HPW + hw;
        const int32_t *pt = a.page_table + (int64_t)a.table_idx[b] * a.row_stride;

        QSlice<T> q[GQ];
        const T *qp = reinterpret_cast<const T *>(a.q) +
                      ((int64_t)b * a.q_heads + (int64_t)kvh * GQ) * D + lr * E;
#pragma unroll
        for (int h = 0; h < GQ; ++h) q[h].load(qp + h * D);

        SoftmaxState<T, D, GQ> st;
        st.init();
        const T *kb = reinterpret_cast<const T *>(a.k_pool) + (int64_t)kvh * D + lr * E;
        const T *vb = reinterpret_cast<const T *>(a.v_pool) + (int64_t)kvh * D + lr * E;
        attend_range<T, D, GQ>(pt, t0, t1, stream, NSTREAM, kb, vb, row_elems, (uint32_t)a.num_slots, q,
                               a.scale_log2, rg, st);
        st.template reduce_wave<LPR>();
        merge_streams<T, D, GQ>(st, s_buf, wave, stream, NSTREAM, lane, lr, rg);

        if (stream == 0 && rg == 0) {
            const int qh0 = kvh * GQ;
            if (nsplit == 1) {
#pragma unroll
                for (int h = 0; h < GQ; ++h) {
                    const float inv = 1.0f / st.l[h];
                    float f[E];
#pragma unroll
                    for (int e = 0; e < E; ++e) f[e] = st.o[h][e] * inv;
                    T *op = reinterpret_cast<T *>(a.out) + ((int64_t)b * a.q_heads + qh0 + h) * D +
                            lr * E;
                    st16(op, Store<T>::narrow(f));
                    if (a.lse != nullptr && lr == 0)
                        a.lse[(int64_t)b * a.q_heads + qh0 + h] = (st.m[h] + __log2f(st.l[h])) * kLn2;
                }
            } else {
                const int64_t base = ((int64_t)b * a.max_splits + split) * a.q_heads + qh0;
#pragma unroll
                for (int h = 0; h < GQ; ++h) {
                    float *po = a.part_o + (base + h) * D + lr * E;
#pragma unroll
                    for (int e = 0; e < E; e += 4)
                        *reinterpret_cast<float4 *>(po + e) =
                            make_float4(st.o[h][e], st.o[h][e + 1], st.o[h][e + 2], st.o[h][e + 3]);
                    if (lr == 0) {
                        a.part_ml[(base + h) * 2] = st.m[h];
                        a.part_ml[(base + h) * 2 + 1] = st.l[h];
                    }
                }
            }
        }
    }

    // every block has taken its last item: the last one out resets the counters
    if (tid == 0) {
        const unsigned done = atomicAdd(&a.ctrl[1], 1u);
        if (done == gridDim.x - 1) {
            atomicExch(&a.ctrl[0], 0u);
            atomicExch(&a.ctrl[1], 0u);
        }
    }
}

// Combine the chunk partials of every request with more than one chunk.
// One wave per (request, q head); each lane owns D / 64 output elements.
template <typename T, int D>
__global__ __launch_bounds__(256) void decode_merge_kernel(DecodeArgs a) {
    constexpr int PER = D / 64;
    const int b = blockIdx.x;
    const int h = blockIdx.y * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (h >= a.q_heads) return;
    const int L = a.seq_lens[b];
    const int nsplit = L > 0 ? min((L + a.chunk - 1) / a.chunk, a.max_splits) : 0;
    if (nsplit <= 1) return;
    const int64_t base = (int64_t)b * a.max_splits * a.q_heads + h;
    const int64_t sstride = a.q_heads;
    float mx = -INFINITY;
    for (int s = 0; s < nsplit; ++s) mx = fmaxf(mx, a.part_ml[(base + s * sstride) * 2]);
    float l = 0.0f;
    float acc[PER];
#pragma unroll
    for (int e = 0; e < PER; ++e) acc[e] = 0.0f;
    for (int s = 0; s < nsplit; ++s) {
        const int64_t idx = base + s * sstride;
        const float w = fast_exp2(a.part_ml[idx * 2] - mx);
        l = fmaf(a.part_ml[idx * 2 + 1], w, l);
        const float *po = a.part_o + idx * D + lane * PER;
#pragma unroll
        for (int e = 0; e < PER; ++e) acc[e] = fmaf(po[e], w, acc[e]);
    }
    const float inv = 1.0f / l;
    T *op = reinterpret_cast<T *>(a.out) + ((int64_t)b * a.q_heads + h) * D + lane * PER;
    if constexpr (sizeof(T) == 2) {
        if constexpr (PER == 2) {
            *reinterpret_cast<uint32_t *>(op) = pack_bf16x2(acc[0] * inv, acc[1] * inv);
        } else {
            *reinterpret_cast<uint16_t *>(op) = (uint16_t)f32_to_bf16_bits(acc[0] * inv);
        }
    } else {
#pragma unroll
        for (int e = 0; e < PER; ++e) reinterpret_cast<float *>(op)[e] = acc[e] * inv;
    }
    if (a.lse != nullptr && lane == 0) a.lse[(int64_t)b * a.q_heads + h] = (mx + __log2f(l)) * kLn2;
}

// ---------------------------------------------------------------------------
// host side

namespace {

int device_cu_count() {
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cached[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            n = 256;
        cached[dev] = n;
    }
    return cached[dev];
}

template <typename T, int D, int GQ, int HPW>
int decode_occupancy(int batch) {
    static int occ = 0;  // blocks per CU at this instantiation's resource use
    if (occ == 0) {
        const size_t smem = sizeof(int) * (size_t)(batch + 1);
        int n = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, decode_split_kernel<T, D, GQ, HPW>, 256,
                                                         smem + 4096) != hipSuccess || n <= 0)
            n = 1;
        occ = n;
    }
    return occ;
}

// prepare_only: resolve the cached device queries (CU count, occupancy) and
// launch nothing; used before stream capture.
template <typename T, int D, int GQ, int HPW>
hipError_t run_decode(const DecodeArgs &a, hipStream_t stream, bool prepare_only) {
    const int occ = decode_occupancy<T, D, GQ, HPW>(a.batch);
    const int cus = device_cu_count();
    if (prepare_only) return hipSuccess;
    const size_t smem = sizeof(int) * (size_t)(a.batch + 1);
    const int64_t max_items = (int64_t)a.batch * a.max_splits * (a.kv_heads / HPW);
    int64_t grid = (int64_t)cus * occ;
    if (grid > max_items) grid = max_items;
    if (grid < 1) grid = 1;
    hipLaunchKernelGGL((decode_split_kernel<T, D, GQ, HPW>), dim3((unsigned)grid), dim3(256), smem, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (a.max_splits > 1) {
        hipLaunchKernelGGL((decode_merge_kernel<T, D>), dim3(a.batch, (a.q_heads + 3) / 4), dim3(256), 0,
                           stream, a);
        e = hipGetLastError();
    }
    return e;
}

template <typename T, int D>
hipError_t run_decode_g(const DecodeArgs &a, hipStream_t stream, bool prep) {
    const int g = a.q_heads / a.kv_heads;
    const bool two = (a.kv_heads % 2) == 0;
    switch (g) {
        case 1: return two ? run_decode<T, D, 1, 2>(a, stream, prep) : run_decode<T, D, 1, 1>(a, stream, prep);
        case 2: return two ? run_decode<T, D, 2, 2>(a, stream, prep) : run_decode<T, D, 2, 1>(a, stream, prep);
        case 4: return two ? run_decode<T, D, 4, 2>(a, stream, prep) : run_decode<T, D, 4, 1>(a, stream, prep);
        case 8: return two ? run_decode<T, D, 8, 2>(a, stream, prep) : run_decode<T, D, 8, 1>(a, stream, prep);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

size_t decode_workspace_bytes(int batch, int q_heads, int head_dim, int max_seq_len, int chunk) {
    if (chunk <= 0) chunk = kDefaultChunk;
    const size_t max_splits = ((size_t)max_seq_len + chunk - 1) / chunk;
    const size_t parts = (size_t)batch * max_splits * q_heads;
    return kCtrlBytes + parts * head_dim * sizeof(float) + parts * 2 * sizeof(float);
}

hipError_t launch_decode(const DecodeArgs &a, DType dtype, int head_dim, hipStream_t stream,
                         bool prepare_only) {
    if (dtype == kBF16) {
        if (head_dim == 128) return run_decode_g<bf16_t, 128>(a, stream, prepare_only);
        if (head_dim == 64) return run_decode_g<bf16_t, 64>(a, stream, prepare_only);
    } else {
        if (head_dim == 128) return run_decode_g<float, 128>(a, stream, prepare_only);
        if (head_dim == 64) return run_decode_g<float, 64>(a, stream, prepare_only);
    }
    return hipErrorInvalidValue;
}

}  // namespace msgl
