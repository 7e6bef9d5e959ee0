// Decode attention: split-K over each request's gathered page list.
//
// Decode has one query token per request at position seq_len - 1 (the token
// just written by store_kv).  The step is HBM-bound: each visible token's K
// and V slices are read once per kv head, and everything else (q, out,
// partials, page-table ids) is small beside them.
//
// Work decomposition (balanced split).  Concatenate every request's keys into
// one sequence of sum(seq_lens) tokens (per group of kv heads when there are
// more kv heads than waves in a block) and give each block of the persistent
// grid an equal, contiguous share of it.  A block has one wave per kv head;
// each wave streams its share of tokens for its head with a software pipeline
// (attend_valu.h) and no barriers.  Where a block's share covers a request
// whole, the wave writes the normalised output; where a request straddles
// block boundaries, each piece writes its partial softmax state (m, l,
// unnormalised o) and decode_merge_kernel combines the pieces with the usual
// log-sum-exp rescaling.  Equal shares balance any length mix (a lognormal tail
// included) without a work queue, the grid does not depend on the lengths
// (so a graph captured once serves any batch within max_seq_len), and the
// workspace carries no state between calls.  Each block derives the prefix of
// lengths from seq_lens itself; block 0 also leaves it (and the share) in the
// workspace for the merge.
#include "attend_valu.h"
#include "launch.h"

namespace msgl {

// Workspace layout (offsets in bytes):
//   [0, 256)            control: int64 total tokens, int64 share per block
//   [256, 256 + P)      int32 prefix of lengths [batch + 1], P rounded up to 256
//   then                float part_o [batch + kMaxDecodeGrid][q_heads][head_dim]
//   then                float part_ml[batch + kMaxDecodeGrid][q_heads][2]
// A piece (request b, block j) is stored at index b + j: pieces are
// contiguous in both orders, so no two (b, j) pairs of real pieces collide.

template <typename T, int D, int GQ, int U>
__global__ __launch_bounds__(512) void decode_split_kernel(DecodeArgs a) {
    using Geo = Geometry<T, D>;
    constexpr int E = Geo::kEpl;
    constexpr int LPR = Geo::kLpr;
    extern __shared__ int s_tok[];  // [batch + 1] tokens before each request

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int wpb = blockDim.x >> 6;  // kv heads per block
    const int rg = lane / LPR;
    const int lr = lane % LPR;
    const int nhg = a.kv_heads / wpb;
    const int64_t row_elems = (int64_t)a.kv_heads * D;
    // lengths beyond the table row or max_seq_len are cut there, and
    // non-positive ones count as empty (malformed input never leaves bounds)
    const int lmax = (int)min(a.row_stride, (int64_t)a.max_seq_len);

    if (wave == 0) {
        int carry = 0;
        if (lane == 0) s_tok[0] = 0;
        for (int base = 0; base < a.batch; base += 64) {
            const int b = base + lane;
            int n = b < a.batch ? max(0, min(a.seq_lens[b], lmax) - (a.key_start ? max(0, a.key_start[b]) : 0)) : 0;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const int y = __shfl_up(n, off);
                if (lane >= off) n += y;
            }
            if (b < a.batch) s_tok[b + 1] = carry + n;
            carry += __shfl(n, 63);
        }
    }
    __syncthreads();
    const int64_t total = s_tok[a.batch];
    const int64_t work = total * nhg;
    int64_t share = (work + gridDim.x - 1) / gridDim.x;
    if (share < a.chunk) share = a.chunk;
    if (blockIdx.x == 0) {
        for (int i = threadIdx.x; i <= a.batch; i += blockDim.x) a.prefix[i] = s_tok[i];
        if (threadIdx.x == 0) {
            a.ctrl[0] = total;
            a.ctrl[1] = share;
        }
    }
    int64_t cur = (int64_t)blockIdx.x * share;
    const int64_t end = min(cur + share, work);
    if (cur >= end) return;

    int hg = (int)(cur / total);
    const int64_t off = cur - (int64_t)hg * total;
    int lo = 0, hi = a.batch;  // last b with s_tok[b] <= off
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (s_tok[mid] <= off) lo = mid; else hi = mid;
    }
    int b = lo;
    int j = (int)(off - s_tok[b]);

    while (cur < end) {
        const int L = s_tok[b + 1] - s_tok[b];
        const int je = (int)min((int64_t)L, (int64_t)j + (end - cur));
        if (je > j) {
            const int kvh = hg * wpb + wave;
            const int32_t *pt = a.page_table + (int64_t)a.table_idx[b] * a.row_stride +
                                (a.key_start ? max(0, a.key_start[b]) : 0);
            QSlice<T> q[GQ];
            const T *qp = reinterpret_cast<const T *>(a.q) +
                          ((int64_t)b * a.q_heads + (int64_t)kvh * GQ) * D + lr * E;
#pragma unroll
            for (int h = 0; h < GQ; ++h) q[h].load(qp + h * D);
            SoftmaxState<T, D, GQ> st;
            st.init();
            const T *kb = reinterpret_cast<const T *>(a.k_pool) + (int64_t)kvh * D + lr * E;
            const T *vb = reinterpret_cast<const T *>(a.v_pool) + (int64_t)kvh * D + lr * E;
            attend_pipelined<T, D, GQ, U>(pt, j, je, kb, vb, row_elems, (uint32_t)a.num_slots, q,
                                          a.scale_log2, rg, st);
            st.template reduce_wave<LPR>();
            if (rg == 0) {
                const int qh0 = kvh * GQ;
                if (j == 0 && je == L) {
#pragma unroll
                    for (int h = 0; h < GQ; ++h) {
                        const float inv = 1.0f / st.l[h];
                        float f[E];
#pragma unroll
                        for (int e = 0; e < E; ++e) f[e] = st.o[h][e] * inv;
                        const int64_t oi = ((int64_t)b * a.q_heads + qh0 + h) * D + lr * E;
                        if (a.out_f32) {
#pragma unroll
                            for (int e = 0; e < E; e += 4)
                                *reinterpret_cast<float4 *>(static_cast<float *>(a.out) + oi + e) =
                                    make_float4(f[e], f[e + 1], f[e + 2], f[e + 3]);
                        } else {
                            st16(reinterpret_cast<T *>(a.out) + oi, Store<T>::narrow(f));
                        }
                        if (a.lse != nullptr && lr == 0)
                            a.lse[(int64_t)b * a.q_heads + qh0 + h] = (st.m[h] + __log2f(st.l[h])) * kLn2;
                    }
                } else {
                    const int64_t base = ((int64_t)b + blockIdx.x) * a.q_heads + qh0;
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
        cur += je - j;
        j = je;
        if (j >= L) {
            j = 0;
            if (++b == a.batch) {
                b = 0;
                ++hg;
            }
        }
    }
}

// Combine the pieces of every request that straddles block boundaries.
// One wave per (request, q head); each lane owns D / 64 output elements.
template <typename T, int D, int GQ>
__global__ __launch_bounds__(256) void decode_merge_kernel(DecodeArgs a) {
    constexpr int PER = D / 64;
    const int b = blockIdx.x;
    const int h = blockIdx.y * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (h >= a.q_heads) return;
    const int64_t total = a.ctrl[0];
    const int64_t share = a.ctrl[1];
    const int L = a.prefix[b + 1] - a.prefix[b];
    if (L <= 0) return;
    const int hg = (h / GQ) / a.wpb;
    const int64_t first_tok = (int64_t)hg * total + a.prefix[b];
    const int first = (int)(first_tok / share);
    const int last = (int)((first_tok + L - 1) / share);
    if (first == last) return;  // one piece: the split kernel wrote the output
    float mx = -INFINITY;
    for (int j = first; j <= last; ++j) mx = fmaxf(mx, a.part_ml[(((int64_t)b + j) * a.q_heads + h) * 2]);
    float l = 0.0f;
    float acc[PER];
#pragma unroll
    for (int e = 0; e < PER; ++e) acc[e] = 0.0f;
#pragma unroll 4
    for (int j = first; j <= last; ++j) {
        const int64_t idx = ((int64_t)b + j) * a.q_heads + h;
        const float w = fast_exp2(a.part_ml[idx * 2] - mx);
        l = fmaf(a.part_ml[idx * 2 + 1], w, l);
        const float *po = a.part_o + idx * D + lane * PER;
#pragma unroll
        for (int e = 0; e < PER; ++e) acc[e] = fmaf(po[e], w, acc[e]);
    }
    const float inv = 1.0f / l;
    T *op = reinterpret_cast<T *>(a.out) + ((int64_t)b * a.q_heads + h) * D + lane * PER;
    if (a.out_f32) {
        float *fo = static_cast<float *>(a.out) + ((int64_t)b * a.q_heads + h) * D + lane * PER;
#pragma unroll
        for (int e = 0; e < PER; ++e) fo[e] = acc[e] * inv;
    } else if constexpr (sizeof(T) == 2) {
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

namespace {

// Loads per wave-iteration of the decode pipeline (4 tokens per load for
// 256-byte head slices: 16 tokens per iteration).
template <typename T, int D>
constexpr int decode_unroll() {
#ifdef MSGL_DECODE_UNROLL  // tuning builds only
    return MSGL_DECODE_UNROLL;
#else
    return Geometry<T, D>::kU;
#endif
}

template <typename T, int D, int GQ>
int decode_occupancy(int threads, int batch) {
    static int occ[17] = {0};  // blocks per CU, by waves per block
    const int w = threads / 64;
    if (occ[w] == 0) {
        const size_t smem = sizeof(int) * (size_t)(batch + 1);
        int n = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
                &n, decode_split_kernel<T, D, GQ, decode_unroll<T, D>()>, threads, smem + 4096) != hipSuccess ||
            n <= 0)
            n = 1;
        occ[w] = n;
    }
    return occ[w];
}

// prepare_only: resolve the cached device queries (CU count, occupancy) and
// launch nothing; used before stream capture.
// Waves (kv heads) per decode block: the largest power of two up to
// kDecodeWaves that divides kv_heads.
int decode_waves(int kv_heads) {
#ifdef MSGL_DECODE_WPB  // tuning builds only
    constexpr int kDecodeWaves = MSGL_DECODE_WPB;
#else
    constexpr int kDecodeWaves = 4;
#endif
    int w = kDecodeWaves;
    while (w > 1 && kv_heads % w != 0) w >>= 1;
    return w;
}

template <typename T, int D, int GQ>
hipError_t run_decode(const DecodeArgs &a_in, hipStream_t stream, bool prepare_only) {
    DecodeArgs a = a_in;
    a.wpb = decode_waves(a.kv_heads);
    const int threads = 64 * a.wpb;
#ifdef MSGL_DECODE_BLOCKS_PER_CU  // tuning builds only
    const int occ = MSGL_DECODE_BLOCKS_PER_CU;
#else
    const int occ = decode_occupancy<T, D, GQ>(threads, a.batch);
#endif
    const int cus = device_cu_count();
    if (prepare_only) return hipSuccess;
    int64_t grid = (int64_t)cus * occ;
    if (grid > kMaxDecodeGrid) grid = kMaxDecodeGrid;
    const size_t smem = sizeof(int) * (size_t)(a.batch + 1);
    hipLaunchKernelGGL((decode_split_kernel<T, D, GQ, decode_unroll<T, D>()>), dim3((unsigned)grid),
                       dim3(threads), smem, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((decode_merge_kernel<T, D, GQ>), dim3(a.batch, (a.q_heads + 3) / 4), dim3(256), 0, stream,
                       a);
    return hipGetLastError();
}

template <typename T, int D>
hipError_t run_decode_g(const DecodeArgs &a, hipStream_t stream, bool prep) {
    switch (a.q_heads / a.kv_heads) {
        case 1: return run_decode<T, D, 1>(a, stream, prep);
        case 2: return run_decode<T, D, 2>(a, stream, prep);
        case 4: return run_decode<T, D, 4>(a, stream, prep);
        case 8: return run_decode<T, D, 8>(a, stream, prep);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

size_t decode_workspace_bytes(int batch, int q_heads, int head_dim, int max_seq_len, int chunk) {
    (void)max_seq_len;
    (void)chunk;
    const size_t pieces = (size_t)batch + kMaxDecodeGrid;
    return kCtrlBytes + decode_prefix_bytes(batch) + pieces * q_heads * ((size_t)head_dim + 2) * sizeof(float);
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
