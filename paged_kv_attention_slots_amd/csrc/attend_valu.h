// One query token against a range of its request's keys, on the vector ALUs.
//
// Used by the decode split kernel (one key chunk per work item) and by the
// VALU prefill kernel (the whole visible range).  A wave owns one kv head and
// GQ q heads (the query heads that share it).  A [kv_heads, head_dim] pool row
// is contiguous; one head's slice is head_dim * sizeof(T) bytes = 256 B for
// bf16 x 128 (or fp32 x 64), read as LPR lanes x 16 B.  A wave therefore
// gathers RPW tokens per load instruction (4 for 256-byte slices), each token's
// slice a whole pair of 128-byte lines, and U loads per iteration keep
// RPW*U tokens of K and V in flight per wave.
//
// Scores are q.k partial dot products per lane (v_dot2_f32_bf16 for bf16,
// fma for fp32) summed across the LPR lanes of a token with DPP row moves.
// Each lane group (the LPR lanes of one token slot) keeps its own online
// softmax state (running max m in log2 units, running sum l, unnormalised
// output slice o); groups and waves are merged at the end of the range.
#pragma once

#include "common.h"

namespace msgl {

template <typename T>
struct QSlice;

template <>
struct QSlice<bf16_t> {
    uint32_t w[4];
    MSGL_DEV void load(const bf16_t *p) {
        const uint4 v = ld16(p);
        w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
    }
    MSGL_DEV float dot(const uint4 &k) const {
        float acc = dot2_bf16(k.x, w[0], 0.0f);
        acc = dot2_bf16(k.y, w[1], acc);
        acc = dot2_bf16(k.z, w[2], acc);
        return dot2_bf16(k.w, w[3], acc);
    }
};

template <>
struct QSlice<float> {
    float f[4];
    MSGL_DEV void load(const float *p) {
        const uint4 v = ld16(p);
        f[0] = __uint_as_float(v.x); f[1] = __uint_as_float(v.y);
        f[2] = __uint_as_float(v.z); f[3] = __uint_as_float(v.w);
    }
    MSGL_DEV float dot(const uint4 &k) const {
        float acc = f[0] * __uint_as_float(k.x);
        acc = fmaf(f[1], __uint_as_float(k.y), acc);
        acc = fmaf(f[2], __uint_as_float(k.z), acc);
        return fmaf(f[3], __uint_as_float(k.w), acc);
    }
};

template <typename T, int D>
struct Geometry {
    static constexpr int kEpl = Store<T>::kEpl;       // elements per lane per load
    static constexpr int kLpr = D / kEpl;             // lanes per token slice
    static constexpr int kRpw = 64 / kLpr;            // tokens per wave per load
    static constexpr int kU = (16 / kRpw) > 0 ? 16 / kRpw : 1;  // loads per iteration
    static constexpr int kTpi = kRpw * kU;            // tokens per wave iteration
    static_assert(kLpr >= 2 && kLpr <= 32 && 64 % kLpr == 0, "unsupported head geometry");
};

template <typename T, int D, int GQ>
struct SoftmaxState {
    static constexpr int E = Store<T>::kEpl;
    float m[GQ];
    float l[GQ];
    float o[GQ][E];
    MSGL_DEV void init() {
#pragma unroll
        for (int h = 0; h < GQ; ++h) {
            m[h] = -INFINITY;
            l[h] = 0.0f;
#pragma unroll
            for (int e = 0; e < E; ++e) o[h][e] = 0.0f;
        }
    }
    // Merge another state (m2, l2, o2) of the same heads and dims into this one.
    MSGL_DEV void merge_one(int h, float m2, float l2, const float *o2) {
        const float mn = fmaxf(m[h], m2);
        const float mu = (mn == -INFINITY) ? 0.0f : mn;
        const float a1 = fast_exp2(m[h] - mu);
        const float a2 = fast_exp2(m2 - mu);
        l[h] = l[h] * a1 + l2 * a2;
#pragma unroll
        for (int e = 0; e < E; ++e) o[h][e] = o[h][e] * a1 + o2[e] * a2;
        m[h] = mn;
    }
    // Fold the lane groups of a wave together (lanes differing in the bits
    // above the row group); afterwards every group holds the wave's state.
    template <int LPR>
    MSGL_DEV void reduce_wave() {
#pragma unroll
        for (int off = LPR; off < 64; off <<= 1) {
#pragma unroll
            for (int h = 0; h < GQ; ++h) {
                const float m2 = __shfl_xor(m[h], off);
                const float l2 = __shfl_xor(l[h], off);
                float o2[E];
#pragma unroll
                for (int e = 0; e < E; ++e) o2[e] = __shfl_xor(o[h][e], off);
                merge_one(h, m2, l2, o2);
            }
        }
    }
};

// Page-table ids of one iteration's tokens (base + u*RPW + rg), -1 past te.
template <int U, int RPW>
MSGL_DEV void load_slots(int (&slot)[U], const int32_t *__restrict__ pt, int base, int te, int rg) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int tok = base + u * RPW + rg;
        slot[u] = tok < te ? pt[tok] : -1;
    }
}

// Issue the K and V loads of one iteration.  Slot ids outside [0, num_slots)
// (malformed input) read slot 0, so no access leaves the pools; a -1 slot
// (past the range) loads nothing.
template <typename T, int U>
MSGL_DEV void issue_kv(uint4 (&kv)[U], uint4 (&vv)[U], const int (&slot)[U], const T *__restrict__ kbase,
                       const T *__restrict__ vbase, int64_t row_elems, uint32_t num_slots) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
        if (slot[u] >= 0) {
            const int64_t off = (int64_t)((uint32_t)slot[u] < num_slots ? slot[u] : 0) * row_elems;
            kv[u] = ld16_nt(kbase + off);
            vv[u] = ld16_nt(vbase + off);
        } else {
            kv[u] = make_uint4(0, 0, 0, 0);
            vv[u] = make_uint4(0, 0, 0, 0);
        }
    }
}

// Scores, online-softmax update and P.V of one iteration's tokens.
template <typename T, int D, int GQ, int U>
MSGL_DEV void consume_iter(const uint4 (&kv)[U], const uint4 (&vv)[U], const int (&slot)[U],
                           const QSlice<T> (&q)[GQ], float scale_log2, SoftmaxState<T, D, GQ> &st) {
    constexpr int E = Store<T>::kEpl;
    constexpr int LPR = Geometry<T, D>::kLpr;
    float s[U][GQ];
#pragma unroll
    for (int u = 0; u < U; ++u) {
#pragma unroll
        for (int h = 0; h < GQ; ++h) {
            const float d = group_sum<LPR>(q[h].dot(kv[u]));
            s[u][h] = slot[u] >= 0 ? d * scale_log2 : -INFINITY;
        }
    }
    float p[U][GQ];
#pragma unroll
    for (int h = 0; h < GQ; ++h) {
        float mx = s[0][h];
#pragma unroll
        for (int u = 1; u < U; ++u) mx = fmaxf(mx, s[u][h]);
        const float mn = fmaxf(st.m[h], mx);
        const float mu = (mn == -INFINITY) ? 0.0f : mn;
        const float alpha = fast_exp2(st.m[h] - mu);
        float psum = 0.0f;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            p[u][h] = fast_exp2(s[u][h] - mu);
            psum += p[u][h];
        }
        st.l[h] = st.l[h] * alpha + psum;
#pragma unroll
        for (int e = 0; e < E; ++e) st.o[h][e] *= alpha;
        st.m[h] = mn;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
        float vf[E];
        Store<T>::widen(vv[u], vf);
#pragma unroll
        for (int h = 0; h < GQ; ++h) {
#pragma unroll
            for (int e = 0; e < E; ++e) st.o[h][e] = fmaf(p[u][h], vf[e], st.o[h][e]);
        }
    }
}

// Attend tokens [tb, te) of page-table row `pt`, taking wave-iterations
// stream, stream + nstream, ... of TPI tokens each (one iteration's loads in
// flight per wave).  kbase / vbase point at this lane's 16-byte slice of slot
// 0's kv head.
template <typename T, int D, int GQ>
MSGL_DEV void attend_range(const int32_t *__restrict__ pt, int tb, int te, int stream, int nstream,
                           const T *__restrict__ kbase, const T *__restrict__ vbase,
                           int64_t row_elems, uint32_t num_slots, const QSlice<T> (&q)[GQ],
                           float scale_log2, int rg, SoftmaxState<T, D, GQ> &st) {
    using Geo = Geometry<T, D>;
    constexpr int RPW = Geo::kRpw;
    constexpr int U = Geo::kU;
    constexpr int TPI = Geo::kTpi;
    const int step = nstream * TPI;
    int base = tb + stream * TPI;
    if (base >= te) return;
    int slot[U];
    load_slots<U, RPW>(slot, pt, base, te, rg);
    for (;;) {
        uint4 kv[U], vv[U];
        issue_kv<T, U>(kv, vv, slot, kbase, vbase, row_elems, num_slots);
        const int nbase = base + step;
        int nslot[U];
        load_slots<U, RPW>(nslot, pt, nbase, te, rg);  // ahead of use
        consume_iter<T, D, GQ, U>(kv, vv, slot, q, scale_log2, st);
        if (nbase >= te) break;
        base = nbase;
#pragma unroll
        for (int u = 0; u < U; ++u) slot[u] = nslot[u];
    }
}

// Attend tokens [tb, te) with a software pipeline: page-table ids three
// iterations ahead and K/V data two iterations ahead of the compute, so every
// wave keeps two iterations of loads in flight while it works on the previous
// tokens.  (One iteration ahead fits three 4-wave blocks per CU instead of
// two, but measured 1.5% slower at batch 256 and 4-6% at batch 32-64.)
template <typename T, int D, int GQ, int U>
MSGL_DEV void attend_pipelined(const int32_t *__restrict__ pt, int tb, int te,
                               const T *__restrict__ kbase, const T *__restrict__ vbase,
                               int64_t row_elems, uint32_t num_slots, const QSlice<T> (&q)[GQ],
                               float scale_log2, int rg, SoftmaxState<T, D, GQ> &st) {
    constexpr int RPW = Geometry<T, D>::kRpw;
    constexpr int TPI = RPW * U;
    if (tb >= te) return;
    int s0[U], s1[U], s2[U];
    load_slots<U, RPW>(s0, pt, tb, te, rg);
    load_slots<U, RPW>(s1, pt, tb + TPI, te, rg);
    int s3[U];
    load_slots<U, RPW>(s2, pt, tb + 2 * TPI, te, rg);
    uint4 k0[U], v0[U], k1[U], v1[U], k2[U], v2[U];
    issue_kv<T, U>(k0, v0, s0, kbase, vbase, row_elems, num_slots);
    issue_kv<T, U>(k1, v1, s1, kbase, vbase, row_elems, num_slots);
    for (int base = tb; base < te; base += TPI) {
        load_slots<U, RPW>(s3, pt, base + 3 * TPI, te, rg);
        issue_kv<T, U>(k2, v2, s2, kbase, vbase, row_elems, num_slots);
        consume_iter<T, D, GQ, U>(k0, v0, s0, q, scale_log2, st);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            k0[u] = k1[u];
            v0[u] = v1[u];
            k1[u] = k2[u];
            v1[u] = v2[u];
            s0[u] = s1[u];
            s1[u] = s2[u];
            s2[u] = s3[u];
        }
    }
}

// Cross-wave merge through LDS: waves 1..nstream-1 of a head hand their
// (already wave-reduced) state to wave 0 of that head.  `buf` holds
// [4 waves][GQ][D + 2] floats.  Must be called by every thread of the block.
template <typename T, int D, int GQ>
MSGL_DEV void merge_streams(SoftmaxState<T, D, GQ> &st, float *buf, int wave, int stream,
                            int nstream, int lane, int lr, int rg) {
    constexpr int E = Store<T>::kEpl;
    constexpr int ROW = D + 2;
    if (nstream > 1) {
        if (stream > 0 && rg == 0) {
            float *w = buf + wave * GQ * ROW;
#pragma unroll
            for (int h = 0; h < GQ; ++h) {
#pragma unroll
                for (int e = 0; e < E; ++e) w[h * ROW + lr * E + e] = st.o[h][e];
                if (lr == 0) {
                    w[h * ROW + D] = st.m[h];
                    w[h * ROW + D + 1] = st.l[h];
                }
            }
        }
        __syncthreads();
        if (stream == 0 && rg == 0) {
            const int hpw = 4 / nstream;  // waves of one stream
            for (int s2 = 1; s2 < nstream; ++s2) {
                const float *r = buf + (wave + s2 * hpw) * GQ * ROW;
#pragma unroll
                for (int h = 0; h < GQ; ++h) {
                    float o2[E];
#pragma unroll
                    for (int e = 0; e < E; ++e) o2[e] = r[h * ROW + lr * E + e];
                    st.merge_one(h, r[h * ROW + D], r[h * ROW + D + 1], o2);
                }
            }
        }
        __syncthreads();
    }
    (void)lane;
}

}  // namespace msgl
