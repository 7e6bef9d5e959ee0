// Prefill / extend attention on matrix cores (bf16 MFMA, fp32 accumulate).
//
// New token i of request b sits at position p = cached_len + i and attends
// keys 0..p of its page-table row: a causal mask offset by the cached prefix.
//
// Block = one kv head x one block of query tokens.  Its 128 "columns" are
// (token, q head) pairs of the q heads that share the kv head (token-major),
// so every gathered K/V tile serves all of them.  Each of the 4 waves owns 32
// columns.  Keys stream through LDS in tiles of 64, double-buffered, with the
// gathers pipelined: page-table slot ids are read two tiles ahead and the
// 256-byte K and V rows of the next tile are in flight while the current tile
// computes.  K and V tiles are stored row-major; V feeds the A operand below
// through gfx950's transposing LDS read.
//
// Per 32 keys a wave computes S^T = K Q^T with v_mfma_f32_32x32x16_bf16
// (A = 32 keys x 16 dims from LDS, B = Q^T held in registers, 8 steps over
// head_dim 128).  The MFMA result layout leaves each lane with 16 scores of
// one column; after the softmax update they are rounded to bf16 and are,
// unchanged, the B operand (P^T) of O^T += V^T P^T, because the order of the
// contraction index inside an MFMA is free as long as both operands agree:
// the V^T reads (ds_read_b64_tr_b16 on the row-major V tile) pick the keys in
// the order the scores arrived in.  Nothing is shuffled between lanes except
// one exchange for the column max (v_permlane32_swap, no LDS round trip).
//
// Softmax: log2 domain (scale times log2 e folded into one fma before exp2),
// running max per column and lazy rescaling: the output is only rescaled when
// a column's max grows by more than 2^8, which keeps exp2 arguments bounded
// and skips almost every rescale.  The output is normalised by the sum of the
// bf16-rounded probabilities that the P.V product uses, so the applied weights
// sum to one; that sum is itself two more MFMAs (an all-ones A operand times
// P^T gives the column sums in every row).  The returned lse comes from a
// lane-partial fp32 sum of the unrounded weights, reduced once at the end.
//
// Blocks are ordered longest-first (last query blocks, which see the most
// keys, get the lowest block ids) so the ragged tail balances.
#include "common.h"
#include "launch.h"

namespace msgl {

typedef __attribute__((__vector_size__(16 * sizeof(float)))) float floatx16_t;

namespace pf {
constexpr int kD = 128;
constexpr int kKT = 64;                        // keys per LDS tile
constexpr int kWaves = 4;
constexpr int kColsW = 32;                     // query columns per wave
constexpr int kCols = kWaves * kColsW;         // query columns per block
constexpr int kKStride = kD * 2 + 16;          // bytes per key row of the K tile (padded)
constexpr int kVStride = kD * 2 + 32;          // bytes per key row of the V tile (padded)
constexpr int kKBytes = kKT * kKStride;
constexpr int kVBytes = kKT * kVStride;
constexpr int kStage = kKBytes + kVBytes;
constexpr float kRescaleLog2 = 8.0f;
}  // namespace pf

MSGL_DEV floatx16_t mfma_32x32x16(const bf16x8_t &a, const bf16x8_t &b, const floatx16_t &c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// A tile's gathers for one thread: keys 4*grp .. 4*grp+3, dims 8*sl .. 8*sl+7.
struct TileRegs {
    uint4 k[4];
    uint4 v[4];
};

// Slot ids of a thread's 4 keys in the tile starting at k0 (-1 past nkeys).
MSGL_DEV void tile_slots(int (&slot)[4], const int32_t *__restrict__ pt, int k0, int nkeys, int tid) {
    const int grp = tid >> 4;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int key = k0 + 4 * grp + i;
        slot[i] = key < nkeys ? pt[key] : -1;
    }
}

MSGL_DEV void tile_fetch(TileRegs &r, const int (&slot)[4], const bf16_t *__restrict__ kh,
                         const bf16_t *__restrict__ vh, int64_t row_elems, uint32_t num_slots, int tid) {
    const int sl = tid & 15;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        if (slot[i] >= 0) {
            const int64_t s = (uint32_t)slot[i] < num_slots ? slot[i] : 0;  // malformed id: stay in the pool
            const int64_t off = s * row_elems + sl * 8;
            r.k[i] = ld16(kh + off);
            r.v[i] = ld16(vh + off);
        } else {
            r.k[i] = make_uint4(0, 0, 0, 0);  // keys past the end: zero rows (masked anyway)
            r.v[i] = make_uint4(0, 0, 0, 0);
        }
    }
}

MSGL_DEV void tile_store(const TileRegs &r, char *stage, int tid) {
    const int grp = tid >> 4;
    const int sl = tid & 15;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        *reinterpret_cast<uint4 *>(stage + (4 * grp + i) * pf::kKStride + sl * 16) = r.k[i];
        *reinterpret_cast<uint4 *>(stage + pf::kKBytes + (4 * grp + i) * pf::kVStride + sl * 16) = r.v[i];
    }
}

// Combine a value with the one held by lane l ^ 32 (v_permlane32_swap: after
// swapping the upper half of a copy with the lower half of another copy, each
// lane holds its own value in one result and its partner's in the other).
MSGL_DEV float max_with_other_half(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

MSGL_DEV float add_with_other_half(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

typedef short shortx4_t __attribute__((ext_vector_type(4)));

// Transposing LDS read (ds_read_b64_tr_b16).  Within each group of 16 lanes,
// lane 4j+a names 4 consecutive 16-bit values; lane l receives value l%4 of
// the lanes l/4, 4+l/4, 8+l/4 and 12+l/4.  When lanes 4j..4j+3 point at key
// j's row at dims +0, +4, +8, +12, lane l therefore gets dim l of keys 0..3.
MSGL_DEV uint2 lds_read_tr16(const char *p) {
    const shortx4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) shortx4_t *)(const_cast<char *>(p)));
    return __builtin_bit_cast(uint2, v);
}

template <int GQ>
__global__ __launch_bounds__(256, 2) void prefill_mfma_kernel(PrefillArgs a, int nqb) {
    constexpr int BQ = pf::kCols / GQ;  // query tokens per block
    __shared__ __attribute__((aligned(16))) char smem[2 * pf::kStage];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int jj = lane >> 5;
    const int G = a.kv_heads;

    int idx = blockIdx.x;  // longest first: query block index descends with the block id
    const int kvh = idx % G;
    idx /= G;
    const int b = idx % a.batch;
    idx /= a.batch;
    const int qb = nqb - 1 - idx;
    const int L = (int)min((int64_t)a.seq_lens[b], a.row_stride);
    const int C = a.cached_lens[b];
    const int E = L - C;
    const int t0 = qb * BQ;
    if (qb < 0 || C < 0 || t0 >= E) return;  // uniform over the block, before any barrier
    const int row0 = a.cu_q[b] + t0;
    const int ntok = min(min(BQ, E - t0), a.total_q - row0);
    if (ntok <= 0) return;
    const int pos0 = C + t0;         // position of the block's first token
    const int nkeys = pos0 + ntok;   // keys 0 .. position of its last token

    // this lane's query column
    const int col = wave * pf::kColsW + (lane & 31);
    const int tl = col / GQ;
    const int hq = kvh * GQ + col % GQ;
    const bool valid = tl < ntok;
    const int tok = valid ? tl : ntok - 1;
    const int pos = pos0 + tok;

    // Q^T operands: d-chunk dc holds dims 16*dc + 8*jj .. +7 of this column
    bf16x8_t qv[8];
    const bf16_t *qp = reinterpret_cast<const bf16_t *>(a.q) +
                       ((int64_t)(row0 + tok) * a.q_heads + hq) * pf::kD + 8 * jj;
#pragma unroll
    for (int dc = 0; dc < 8; ++dc) qv[dc] = __builtin_bit_cast(bf16x8_t, ld16(qp + 16 * dc));

    floatx16_t acc[4];
#pragma unroll
    for (int db = 0; db < 4; ++db) acc[db] = floatx16_t{};
    float m = -INFINITY;  // running column max (log2 units; may lag by < 2^8)
    float lt = 0.0f;      // this lane's share of the running sum of the weights (for lse)
    floatx16_t acc_l = floatx16_t{};  // running sum of the bf16-rounded weights (any element)
    const bf16x8_t ones = __builtin_bit_cast(bf16x8_t, make_uint4(0x3f803f80u, 0x3f803f80u, 0x3f803f80u,
                                                                  0x3f803f80u));

    const int32_t *pt = a.page_table + (int64_t)a.table_idx[b] * a.row_stride;
    const bf16_t *kh = reinterpret_cast<const bf16_t *>(a.k_pool) + (int64_t)kvh * pf::kD;
    const bf16_t *vh = reinterpret_cast<const bf16_t *>(a.v_pool) + (int64_t)kvh * pf::kD;
    const int64_t row_elems = (int64_t)G * pf::kD;
    const uint32_t num_slots = (uint32_t)a.num_slots;
    const int ntiles = (nkeys + pf::kKT - 1) / pf::kKT;

    // pipeline: slot ids two tiles ahead, K/V rows one tile ahead, LDS double-buffered
    TileRegs r;
    int slot0[4], slot1[4], slot2[4];
    tile_slots(slot0, pt, 0, nkeys, tid);
    tile_slots(slot1, pt, pf::kKT, nkeys, tid);
    tile_fetch(r, slot0, kh, vh, row_elems, num_slots, tid);
    tile_store(r, smem, tid);
    __syncthreads();

    for (int t = 0; t < ntiles; ++t) {
        const char *st = smem + (t & 1) * pf::kStage;
        const bool more = t + 1 < ntiles;
        tile_slots(slot2, pt, (t + 2) * pf::kKT, nkeys, tid);
        if (more) tile_fetch(r, slot1, kh, vh, row_elems, num_slots, tid);
        const int k0 = t * pf::kKT;
        const bool need_mask = k0 + pf::kKT - 1 > pos0;
        // scores of both 32-key halves first, so that the second half's MFMAs
        // (and then the first half's P.V) overlap the softmax arithmetic
        floatx16_t sc[2] = {floatx16_t{}, floatx16_t{}};
        {
            const char *krow = st + (lane & 31) * pf::kKStride + 16 * jj;
#pragma unroll
            for (int dc = 0; dc < 8; ++dc)  // two independent accumulation chains, interleaved
#pragma unroll
                for (int half = 0; half < 2; ++half)
                    sc[half] = mfma_32x32x16(
                        *reinterpret_cast<const bf16x8_t *>(krow + half * 32 * pf::kKStride + 32 * dc), qv[dc],
                        sc[half]);
        }
        // causal mask, only on tiles that reach past the block's first position
        if (need_mask) {
#pragma unroll
            for (int half = 0; half < 2; ++half)
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int key = k0 + half * 32 + 8 * (e >> 2) + 4 * jj + (e & 3);
                    sc[half][e] = key > pos ? -INFINITY : sc[half][e];
                }
        }
        // one column max per 64-key tile (raw scores; the scale is positive)
        float mx = fmaxf(sc[0][0], sc[1][0]);
#pragma unroll
        for (int e = 1; e < 16; ++e) mx = fmaxf(mx, fmaxf(sc[0][e], sc[1][e]));
        mx = max_with_other_half(mx) * a.scale_log2;
        if (__any(mx > m + pf::kRescaleLog2)) {
            const float mn = fmaxf(m, mx);
            const float alpha = (mn == -INFINITY) ? 1.0f : fast_exp2(m - mn);
            lt *= alpha;
#pragma unroll
            for (int e = 0; e < 16; ++e) acc_l[e] *= alpha;
#pragma unroll
            for (int db = 0; db < 4; ++db)
#pragma unroll
                for (int e = 0; e < 16; ++e) acc[db][e] *= alpha;
            m = mn;
        }
        const float nmu = (m == -INFINITY) ? 0.0f : -m;

        // weights of both halves, then the row sums and P.V: one straight-line
        // region, so the MFMAs of one half overlap the arithmetic of the other
        bf16x8_t pb[2][2];
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            uint32_t pw[8];
#pragma unroll
            for (int e = 0; e < 16; e += 2) {
                const float p0 = fast_exp2(fmaf(sc[half][e], a.scale_log2, nmu));
                const float p1 = fast_exp2(fmaf(sc[half][e + 1], a.scale_log2, nmu));
                pw[e >> 1] = pack_bf16x2(p0, p1);
                lt += p0 + p1;
            }
            pb[half][0] = __builtin_bit_cast(bf16x8_t, make_uint4(pw[0], pw[1], pw[2], pw[3]));
            pb[half][1] = __builtin_bit_cast(bf16x8_t, make_uint4(pw[4], pw[5], pw[6], pw[7]));
        }
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            // running sum of the rounded weights: every row of ones . P^T is the column sum
            acc_l = mfma_32x32x16(ones, pb[half][0], acc_l);
            acc_l = mfma_32x32x16(ones, pb[half][1], acc_l);
            // V^T operands straight from the row-major V tile: lane L reads the
            // rows of keys kb + 16*mm + 4*jj + (L/4)%4 (+8), dims 16*((L/16)%2) + 4*(L%4)
            const char *vt = st + pf::kKBytes + (half * 32 + 4 * jj + ((lane >> 2) & 3)) * pf::kVStride +
                             (16 * ((lane >> 4) & 1) + 4 * (lane & 3)) * 2;
#pragma unroll
            for (int db = 0; db < 4; ++db) {
                const char *vrow = vt + db * 32 * 2;
                const uint2 a0 = lds_read_tr16(vrow);
                const uint2 a1 = lds_read_tr16(vrow + 8 * pf::kVStride);
                const uint2 a2 = lds_read_tr16(vrow + 16 * pf::kVStride);
                const uint2 a3 = lds_read_tr16(vrow + 24 * pf::kVStride);
                acc[db] = mfma_32x32x16(__builtin_bit_cast(bf16x8_t, make_uint4(a0.x, a0.y, a1.x, a1.y)),
                                        pb[half][0], acc[db]);
                acc[db] = mfma_32x32x16(__builtin_bit_cast(bf16x8_t, make_uint4(a2.x, a2.y, a3.x, a3.y)),
                                        pb[half][1], acc[db]);
            }
        }
        if (more) tile_store(r, smem + ((t + 1) & 1) * pf::kStage, tid);
        __syncthreads();
#pragma unroll
        for (int i = 0; i < 4; ++i) slot1[i] = slot2[i];
    }

    lt = add_with_other_half(lt);
    if (valid) {
        const float inv = 1.0f / acc_l[0];
        bf16_t *op = reinterpret_cast<bf16_t *>(a.out) + ((int64_t)(row0 + tl) * a.q_heads + hq) * pf::kD;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int d0 = db * 32 + 8 * i + 4 * jj;
                *reinterpret_cast<uint2 *>(op + d0) =
                    make_uint2(pack_bf16x2(acc[db][4 * i] * inv, acc[db][4 * i + 1] * inv),
                               pack_bf16x2(acc[db][4 * i + 2] * inv, acc[db][4 * i + 3] * inv));
            }
        if (a.lse != nullptr && jj == 0) a.lse[(int64_t)(row0 + tl) * a.q_heads + hq] = (m + __log2f(lt)) * kLn2;
    }
}

namespace {

template <int GQ>
hipError_t run_prefill_mfma(const PrefillArgs &a, hipStream_t stream) {
    constexpr int BQ = pf::kCols / GQ;
    const int nqb = (a.max_extend + BQ - 1) / BQ;
    const int64_t grid = (int64_t)nqb * a.batch * a.kv_heads;
    if (grid < 1) return hipSuccess;
    if (grid > 0x7fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL((prefill_mfma_kernel<GQ>), dim3((unsigned)grid), dim3(256), 0, stream, a, nqb);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs &a, DType dtype, int head_dim, hipStream_t stream) {
    if (dtype == kBF16 && head_dim == pf::kD) {
        switch (a.q_heads / a.kv_heads) {
            case 1: return run_prefill_mfma<1>(a, stream);
            case 2: return run_prefill_mfma<2>(a, stream);
            case 4: return run_prefill_mfma<4>(a, stream);
            case 8: return run_prefill_mfma<8>(a, stream);
            default: break;
        }
    }
    return launch_prefill_valu(a, dtype, head_dim, stream);
}

}  // namespace msgl
