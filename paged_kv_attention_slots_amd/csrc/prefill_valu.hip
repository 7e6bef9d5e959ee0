// Prefill / extend attention on the vector ALUs (fp32 storage, and a
// reference-grade path for bf16).
//
// Each new token t of request b sits at position p = cached_len + (t - cu_q[b])
// and attends keys 0..p of its page-table row (the causal mask is offset by
// the cached prefix).  A work item is (token, group of HPW kv heads); it runs
// the same per-query core as decode (attend_valu.h) over the whole visible
// range and writes the normalised output.  Throughput is bounded by the
// re-reading of K/V per query row, so bf16 prefill normally takes the matrix
// core kernel instead; this path is the fp32 one.
#include "attend_valu.h"
#include "launch.h"

namespace msgl {

template <typename T, int D, int GQ, int HPW>
__global__ __launch_bounds__(256) void prefill_valu_kernel(PrefillArgs a) {
    using Geo = Geometry<T, D>;
    constexpr int E = Geo::kEpl;
    constexpr int LPR = Geo::kLpr;
    constexpr int NSTREAM = 4 / HPW;
    __shared__ float s_buf[4 * GQ * (D + 2)];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int hw = wave % HPW;
    const int stream = wave / HPW;
    const int rg = lane / LPR;
    const int lr = lane % LPR;
    const int nhg = a.kv_heads / HPW;
    const int64_t row_elems = (int64_t)a.kv_heads * D;
    const int64_t total = (int64_t)a.total_q * nhg;

    for (int64_t item = blockIdx.x; item < total; item += gridDim.x) {
        const int t = (int)(item / nhg);
        const int hg = (int)(item % nhg);
        int lo = 0, hi = a.batch;  // cu_q[lo] <= t < cu_q[hi]
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (a.cu_q[mid] <= t) lo = mid; else hi = mid;
        }
        const int b = lo;
        const int lim = (int)min((int64_t)a.seq_lens[b], a.row_stride);
        const int p = max(0, min(a.cached_lens[b] + (t - a.cu_q[b]), lim - 1));
        const int kvh = hg * HPW + hw;
        const int32_t *pt = a.page_table + (int64_t)a.table_idx[b] * a.row_stride;

        QSlice<T> q[GQ];
        const T *qp = reinterpret_cast<const T *>(a.q) +
                      ((int64_t)t * a.q_heads + (int64_t)kvh * GQ) * D + lr * E;
#pragma unroll
        for (int h = 0; h < GQ; ++h) q[h].load(qp + h * D);

        SoftmaxState<T, D, GQ> st;
        st.init();
        const T *kb = reinterpret_cast<const T *>(a.k_pool) + (int64_t)kvh * D + lr * E;
        const T *vb = reinterpret_cast<const T *>(a.v_pool) + (int64_t)kvh * D + lr * E;
        attend_range<T, D, GQ>(pt, 0, p + 1, stream, NSTREAM, kb, vb, row_elems, (uint32_t)a.num_slots, q,
                               a.scale_log2, rg, st);
        st.template reduce_wave<LPR>();
        merge_streams<T, D, GQ>(st, s_buf, wave, stream, NSTREAM, lane, lr, rg);

        if (stream == 0 && rg == 0) {
            const int qh0 = kvh * GQ;
#pragma unroll
            for (int h = 0; h < GQ; ++h) {
                const float inv = 1.0f / st.l[h];
                float f[E];
#pragma unroll
                for (int e = 0; e < E; ++e) f[e] = st.o[h][e] * inv;
                T *op = reinterpret_cast<T *>(a.out) + ((int64_t)t * a.q_heads + qh0 + h) * D + lr * E;
                st16(op, Store<T>::narrow(f));
                if (a.lse != nullptr && lr == 0)
                    a.lse[(int64_t)t * a.q_heads + qh0 + h] = (st.m[h] + __log2f(st.l[h])) * kLn2;
            }
        }
    }
}

namespace {

template <typename T, int D, int GQ, int HPW>
hipError_t run_prefill_valu(const PrefillArgs &a, hipStream_t stream) {
    const int64_t items = (int64_t)a.total_q * (a.kv_heads / HPW);
    int64_t grid = items < 4096 ? items : 4096;
    if (grid < 1) return hipSuccess;
    hipLaunchKernelGGL((prefill_valu_kernel<T, D, GQ, HPW>), dim3((unsigned)grid), dim3(256), 0, stream, a);
    return hipGetLastError();
}

template <typename T, int D>
hipError_t run_prefill_valu_g(const PrefillArgs &a, hipStream_t stream) {
    const int g = a.q_heads / a.kv_heads;
    const bool two = (a.kv_heads % 2) == 0;
    switch (g) {
        case 1: return two ? run_prefill_valu<T, D, 1, 2>(a, stream) : run_prefill_valu<T, D, 1, 1>(a, stream);
        case 2: return two ? run_prefill_valu<T, D, 2, 2>(a, stream) : run_prefill_valu<T, D, 2, 1>(a, stream);
        case 4: return two ? run_prefill_valu<T, D, 4, 2>(a, stream) : run_prefill_valu<T, D, 4, 1>(a, stream);
        case 8: return two ? run_prefill_valu<T, D, 8, 2>(a, stream) : run_prefill_valu<T, D, 8, 1>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_prefill_valu(const PrefillArgs &a, DType dtype, int head_dim, hipStream_t stream) {
    if (dtype == kBF16) {
        if (head_dim == 128) return run_prefill_valu_g<bf16_t, 128>(a, stream);
        if (head_dim == 64) return run_prefill_valu_g<bf16_t, 64>(a, stream);
    } else {
        if (head_dim == 128) return run_prefill_valu_g<float, 128>(a, stream);
        if (head_dim == 64) return run_prefill_valu_g<float, 64>(a, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace msgl
