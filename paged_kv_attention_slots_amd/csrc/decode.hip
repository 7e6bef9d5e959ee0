// Decode attention: split-K over each request's gathered page list.
//
// Decode has one query token per request at position seq_len - 1 (the token
// just written by store_kv).  The step is HBM-bound: each visible token's K
// and V slices are read once per kv head, and everything else (q, out,
// partials, page-table ids) is small beside them.
//
// Work decomposition (balanced split).  Concatenate every request's keys into
// one sequence (per group of kv heads when there are more kv heads than waves
// in a block), each request preceded by kPieceUnits units of fixed cost, and
// give each block of the persistent grid an equal, contiguous share of it.
// The fixed cost stands for what a piece costs beyond its keys (its q, page
// table and K/V round trips, the reductions, the write), so a run of
// one-key requests (padded rows of a captured batch) spreads over blocks
// instead of queueing in one.  A block has one wave per kv head;
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

// Batches up to this size merge with four waves per (request, q head).
constexpr int kMergeSplitBatch = 64;

// Workspace layout (offsets in bytes):
//   [0, 256)            control: int64 total work units, int64 share per block
//   [256, 256 + P)      int32 prefix of work units [batch + 1], P rounded up to 256
//   then                float part_o [batch + kMaxDecodeGrid][q_heads][head_dim]
//   then                float part_ml[batch + kMaxDecodeGrid][q_heads][2]
// A piece (request b, block j) is stored at index b + j: pieces are
// contiguous in both orders, so no two (b, j) pairs of real pieces collide.

template <typename T, int D, int GQ, int U>
__global__ __launch_bounds__(512) void decode_split_kernel(DecodeArgs a) {
    using Geo = Geometry<T, D>;
    constexpr int E = Geo::kEpl;
    constexpr int LPR = Geo::kLpr;
    extern __shared__ int s_tok[];  // [batch + 1] work units before each request

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
            n = n > 0 ? n + kPieceUnits : 0;  // a request's work: its keys plus a fixed cost
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
    int u = (int)(off - s_tok[b]);  // work unit within request b

    while (cur < end) {
        // request b's units: kPieceUnits of fixed cost, then one per key
        const int W = s_tok[b + 1] - s_tok[b];
        const int L = W > 0 ? W - kPieceUnits : 0;
        const int ue = (int)min((int64_t)W, (int64_t)u + (end - cur));
        const int j = max(u - kPieceUnits, 0);
        const int je = max(ue - kPieceUnits, 0);
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
            if (a.fuse_store && je == L && rg == 0) {
                // the KV write of this request's new token (its last key), this
                // wave's head: only the piece holding that key reads it, and it
                // reads it after this store, from the same wave
                const int64_t slot = a.out_loc[b];
                if (slot >= 0 && slot < a.num_slots) {
                    const int64_t src = ((int64_t)b * a.kv_heads + kvh) * D + lr * E;
                    const int64_t dst = slot * row_elems + (int64_t)kvh * D + lr * E;
                    st16(static_cast<T *>(a.k_pool_w) + dst, ld16(static_cast<const T *>(a.k_new) + src));
                    st16(static_cast<T *>(a.v_pool_w) + dst, ld16(static_cast<const T *>(a.v_new) + src));
                }
            }
            if (a.fuse_store && je == L)  // the row is written before any lane of the wave reads it
                asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
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
        cur += ue - u;
        u = ue;
        if (u >= W) {
            u = 0;
            if (++b == a.batch) {
                b = 0;
                ++hg;
            }
        }
    }
}

MSGL_DEV float wave_max64(float x) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x = fmaxf(x, __shfl_xor(x, off));
    return x;
}

MSGL_DEV float wave_sum64(float x) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off);
    return x;
}

// Combine the pieces of every request that straddles block boundaries.
// The pieces' (max, sum) states are read lanes-over-pieces, 64 at a time, so a
// long request costs a few round trips rather than one per piece.  For the
// outputs a wave splits into four groups of 16 lanes; each lane owns D / 16
// consecutive elements.  PW waves share one (request, q head): wave w's group
// g takes the pieces k with k % (4 PW) == 4 w + g, so that 4 PW pieces' loads
// are in flight; with PW > 1 the waves' sums meet in LDS.  PW = 1 (a block
// serves 4 q heads of a request) suits large batches, whose requests are cut
// into few pieces; PW = 4 suits small ones, where one long request can span
// tens of pieces and sets the kernel's time.
template <typename T, int D, int GQ, int PW>
__global__ __launch_bounds__(256) void decode_merge_kernel(DecodeArgs a) {
    constexpr int DPL = D / 16;  // elements per lane (a multiple of 4)
    constexpr int S = 4 * PW;    // piece stride of a group
    __shared__ float s_acc[PW > 1 ? PW - 1 : 1][D];
    const int b = blockIdx.x;
    const int wave = threadIdx.x >> 6;
    const int h = PW > 1 ? (int)blockIdx.y : blockIdx.y * 4 + wave;
    const int lane = threadIdx.x & 63;
    const int grp = lane >> 4;
    const int slot = (PW > 1 ? 4 * wave : 0) + grp;
    const int col = (lane & 15) * DPL;
    if (h >= a.q_heads) return;  // uniform over the block when PW > 1
    const int64_t total = a.ctrl[0];
    const int64_t share = a.ctrl[1];
    const int W = a.prefix[b + 1] - a.prefix[b];
    const int L = W - kPieceUnits;  // its keys
    if (L <= 0) return;
    const int hg = (h / GQ) / a.wpb;
    const int64_t first_tok = (int64_t)hg * total + a.prefix[b] + kPieceUnits;  // its first key's unit
    const int first = (int)(first_tok / share);
    const int last = (int)((first_tok + L - 1) / share);
    if (first == last) return;  // one piece: the split kernel wrote the output
    const int n = last - first + 1;
    // piece k of this request (block first + k) keeps its state at index (b + first + k) * q_heads + h
    const int64_t i0 = ((int64_t)b + first) * a.q_heads + h;
    const int64_t pstride = (int64_t)a.q_heads * D;  // floats between consecutive pieces' outputs
    // (max, sum) of the lane's first piece, kept for the weights below
    float m0 = -INFINITY, l0 = 0.0f;
    if (lane < n) {
        const float2 v = *reinterpret_cast<const float2 *>(a.part_ml + (i0 + (int64_t)lane * a.q_heads) * 2);
        m0 = v.x;
        l0 = v.y;
    }
    float mx = m0;
    for (int k = lane + 64; k < n; k += 64) mx = fmaxf(mx, a.part_ml[(i0 + (int64_t)k * a.q_heads) * 2]);
    mx = wave_max64(mx);
    float l = 0.0f;
    float acc[DPL];
#pragma unroll
    for (int e = 0; e < DPL; ++e) acc[e] = 0.0f;
    for (int c0 = 0; c0 < n; c0 += 64) {
        const int k = c0 + lane;
        float wk = 0.0f;
        if (k < n) {
            float mk = m0, lk = l0;
            if (c0 != 0) {
                const float2 v = *reinterpret_cast<const float2 *>(a.part_ml + (i0 + (int64_t)k * a.q_heads) * 2);
                mk = v.x;
                lk = v.y;
            }
            wk = fast_exp2(mk - mx);
            l = fmaf(lk, wk, l);
        }
        const int cn = min(64, n - c0);
        const float *po = a.part_o + i0 * D + (int64_t)c0 * pstride + col;
#pragma unroll 4
        for (int t0 = 0; t0 < cn; t0 += S) {
            const int t = t0 + slot;
            const float w = __shfl(wk, t & 63);  // every lane takes part; past the end w is unused
            if (t < cn) {
                const float *pp = po + (int64_t)t * pstride;
#pragma unroll
                for (int e = 0; e < DPL; e += 4) {
                    const float4 v = *reinterpret_cast<const float4 *>(pp + e);
                    acc[e] = fmaf(v.x, w, acc[e]);
                    acc[e + 1] = fmaf(v.y, w, acc[e + 1]);
                    acc[e + 2] = fmaf(v.z, w, acc[e + 2]);
                    acc[e + 3] = fmaf(v.w, w, acc[e + 3]);
                }
            }
        }
    }
#pragma unroll
    for (int e = 0; e < DPL; ++e) {
        acc[e] += __shfl_xor(acc[e], 16);
        acc[e] += __shfl_xor(acc[e], 32);
    }
    l = wave_sum64(l);
    if constexpr (PW > 1) {  // waves 1.. hand their sums to wave 0
        if (wave > 0 && grp == 0)
#pragma unroll
            for (int e = 0; e < DPL; ++e) s_acc[wave - 1][col + e] = acc[e];
        __syncthreads();
        if (wave > 0) return;
#pragma unroll
        for (int v = 0; v < PW - 1; ++v)
#pragma unroll
            for (int e = 0; e < DPL; ++e) acc[e] += s_acc[v][col + e];
    }
    if (grp != 0) return;
    const float inv = 1.0f / l;
    const int64_t oi = ((int64_t)b * a.q_heads + h) * D + col;
    if (a.out_f32) {
        float *fo = static_cast<float *>(a.out) + oi;
#pragma unroll
        for (int e = 0; e < DPL; e += 4)
            *reinterpret_cast<float4 *>(fo + e) =
                make_float4(acc[e] * inv, acc[e + 1] * inv, acc[e + 2] * inv, acc[e + 3] * inv);
    } else if constexpr (sizeof(T) == 2) {
#pragma unroll
        for (int e = 0; e < DPL; e += 4)
            *reinterpret_cast<uint2 *>(reinterpret_cast<T *>(a.out) + oi + e) =
                make_uint2(pack_bf16x2(acc[e] * inv, acc[e + 1] * inv), pack_bf16x2(acc[e + 2] * inv, acc[e + 3] * inv));
    } else {
#pragma unroll
        for (int e = 0; e < DPL; e += 4)
            *reinterpret_cast<float4 *>(reinterpret_cast<float *>(a.out) + oi + e) =
                make_float4(acc[e] * inv, acc[e + 1] * inv, acc[e + 2] * inv, acc[e + 3] * inv);
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
// launch nothing; used before stream capture.  split_only: the split kernel
// alone (the cascade merges the pieces itself).
template <typename T, int D, int GQ>
hipError_t run_decode(const DecodeArgs &a_in, hipStream_t stream, bool prepare_only, bool split_only) {
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
    if (e != hipSuccess || split_only) return e;
    if (a.batch <= kMergeSplitBatch)
        hipLaunchKernelGGL((decode_merge_kernel<T, D, GQ, 4>), dim3(a.batch, a.q_heads), dim3(256), 0, stream, a);
    else
        hipLaunchKernelGGL((decode_merge_kernel<T, D, GQ, 1>), dim3(a.batch, (a.q_heads + 3) / 4), dim3(256), 0,
                           stream, a);
    return hipGetLastError();
}

template <typename T, int D>
hipError_t run_decode_g(const DecodeArgs &a, hipStream_t stream, bool prep, bool split_only) {
    switch (a.q_heads / a.kv_heads) {
        case 1: return run_decode<T, D, 1>(a, stream, prep, split_only);
        case 2: return run_decode<T, D, 2>(a, stream, prep, split_only);
        case 4: return run_decode<T, D, 4>(a, stream, prep, split_only);
        case 8: return run_decode<T, D, 8>(a, stream, prep, split_only);
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
                         bool prepare_only, bool split_only) {
    if (dtype == kBF16) {
        if (head_dim == 128) return run_decode_g<bf16_t, 128>(a, stream, prepare_only, split_only);
        if (head_dim == 64) return run_decode_g<bf16_t, 64>(a, stream, prepare_only, split_only);
    } else {
        if (head_dim == 128) return run_decode_g<float, 128>(a, stream, prepare_only, split_only);
        if (head_dim == 64) return run_decode_g<float, 64>(a, stream, prepare_only, split_only);
    }
    return hipErrorInvalidValue;
}

}  // namespace msgl
