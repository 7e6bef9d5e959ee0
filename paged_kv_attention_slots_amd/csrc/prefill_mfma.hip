// Prefill / extend attention on matrix cores (bf16 MFMA, fp32 accumulate).
//
// New token i of request b sits at position p = cached_len + i and attends
// keys 0..p of its page-table row: a causal mask offset by the cached prefix.
//
// Block = one kv head x 256 query "columns", one block per CU.  A column is a
// (token, q head) pair of the q heads that share the kv head (token-major), so
// every gathered K/V tile serves the whole group; each of the 8 waves owns 32
// columns.  Keys stream through a ring of 4 LDS stages of 64 keys (K rows, then
// V rows, 256 bytes each, their 16-byte chunks permuted per row so that the
// column-wise reads below hit every bank once).  The gathers go straight from
// the pools into LDS (global_load_lds_dwordx4: lane l's 16 bytes land at the
// destination + 16 l), three tiles ahead of the compute; the page-table ids
// are scalar loads five tiles ahead.  Every iteration issues the same four
// vector memory instructions per wave, so one vmcnt wait plus one barrier per
// tile is exact.
//
// Per 32 keys a wave computes S^T = K Q^T with v_mfma_f32_32x32x16_bf16
// (A = 32 keys x 16 dims from LDS, B = Q^T held in registers, 8 steps over
// head_dim 128).  The MFMA result layout leaves each lane with 16 scores of
// one column; after the softmax update they are rounded to bf16 and are,
// unchanged, the B operand (P^T) of O^T += V^T P^T, because the order of the
// contraction index inside an MFMA is free as long as both operands agree:
// the V^T reads (ds_read_b64_tr_b16 on the row-major V rows) pick the keys in
// the order the scores arrived in.  Nothing is shuffled between lanes except
// one exchange for the column max (v_permlane32_swap, no LDS round trip).
//
// Softmax: log2 domain (scale times log2 e folded into one fma before exp2),
// one running max per column per 64-key tile and lazy rescaling: the output is
// only rescaled when a column's max grows by more than 2^8, which keeps exp2
// arguments bounded and skips almost every rescale.  The output is normalised
// by the sum of the bf16-rounded probabilities that the P.V product uses, so
// the applied weights sum to one; that sum is itself two more MFMAs (an
// all-ones A operand times P^T gives the column sums in every row).  The
// returned lse comes from a lane-partial fp32 sum of the unrounded weights,
// reduced once at the end.
//
// Block ids enumerate the query blocks of all requests densely, in decreasing
// order of the keys they see (computed in the kernel from the lengths), so the
// longest work starts first and no id is left idle: an idle id still holds a
// dispatch slot, and the in-order dispatcher would queue the rest behind it.
#include <algorithm>

#include "common.h"
#include "launch.h"

namespace msgl {

typedef __attribute__((__vector_size__(16 * sizeof(float)))) float floatx16_t;
typedef short shortx4_t __attribute__((ext_vector_type(4)));

namespace pf {
constexpr int kD = 128;
constexpr int kKT = 64;                    // keys per tile
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kColsW = 32;                 // query columns per wave
constexpr int kCols = kWaves * kColsW;     // query columns per block
constexpr int kRow = kD * 2;               // bytes per K or V row in LDS
constexpr int kHalf = kKT * kRow;          // the K rows of a stage, then its V rows
constexpr int kStage = 2 * kHalf;
constexpr int kStages = 4;
constexpr int kAhead = kStages - 1;        // tiles gathered ahead of the compute
constexpr int kGathersPerTile = 16;        // vector memory instructions per wave per tile
constexpr float kRescaleLog2 = 8.0f;
}  // namespace pf

MSGL_DEV floatx16_t mfma_32x32x16(const bf16x8_t &a, const bf16x8_t &b, const floatx16_t &c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
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

// Transposing LDS read (ds_read_b64_tr_b16).  Within each group of 16 lanes,
// lane 4j+a names 4 consecutive 16-bit values; lane l receives value l%4 of
// the lanes l/4, 4+l/4, 8+l/4 and 12+l/4.  When lanes 4j..4j+3 point at key
// j's row at dims +0, +4, +8, +12, lane l therefore gets dim l of keys 0..3.
MSGL_DEV uint2 lds_read_tr16(const char *p) {
    const shortx4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) shortx4_t *)(const_cast<char *>(p)));
    return __builtin_bit_cast(uint2, v);
}

// Row permutation code: chunk c of row r sits at chunk position c ^ code(r).
// code is a bijection on r % 16, so 16 (or 8) consecutive rows read at one
// chunk spread over all positions (the K reads), and its bits 1..3 give 4
// consecutive rows distinct chunk groups (the transposing V reads, 4 chunks
// of 4 rows at once).
MSGL_DEV int row_code(int r) {
    return ((r >> 2) & 1) | ((r & 1) << 1) | (((r >> 1) & 1) << 2) | (((r ^ (r >> 3)) & 1) << 3);
}

// The 8 page-table ids of rows 8w..8w+7 of a tile (uniform per wave, scalar
// loads, left unchecked until they are used).  Keys past the block's last one
// read key 0's id: a real row whose scores the causal mask removes.
typedef int TileIds __attribute__((ext_vector_type(8)));

MSGL_DEV void load_ids(TileIds &ids, const __attribute__((address_space(4))) int32_t *pt, int key0, int nkeys) {
    if (key0 + 8 <= nkeys) {
#pragma unroll
        for (int j = 0; j < 8; ++j) ids[j] = pt[key0 + j];
    } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) ids[j] = pt[key0 + j < nkeys ? key0 + j : 0];
    }
}

// One gather of 4 bytes per lane straight into LDS (global_load_lds_dword):
// lane l's bytes land at LDS address lds + 4 l (lds is wave-uniform, in M0);
// the source is a wave-uniform row address plus a per-lane offset.  Issued as
// inline assembly so that the compiler neither counts it nor holds later LDS
// reads back for it: the kernel orders it itself (vmcnt + barrier).
MSGL_DEV void gather_row_to_lds(const char *row, uint32_t lane_off, uint32_t lds) {
    asm volatile("s_nop 0\n\tglobal_load_lds_dword %0, %1" ::"v"(lane_off), "s"(row), "{m0}"(lds) : "memory");
}

// Gathers of one tile by one wave to LDS address `dst` (the stage + this
// wave's first row): K rows, then V rows 8w..8w+7, one instruction per row.
// Lane l fills bytes 4l..4l+3 of its row, i.e. chunk position l/4, so it
// reads the chunk that the row permutation puts there.
MSGL_DEV void issue_tile(uint32_t dst, TileIds ids, int wave, const char *kbase, int64_t v_minus_k,
                         int64_t row_bytes, uint32_t lane4, uint32_t num_slots) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int s = (uint32_t)ids[j] < num_slots ? ids[j] : 0;  // a malformed id stays inside the pool
        const char *krow = kbase + (int64_t)s * row_bytes;
        const uint32_t off = lane4 ^ (row_code(8 * wave + j) << 4);
        gather_row_to_lds(krow, off, dst + j * pf::kRow);
        gather_row_to_lds(krow + v_minus_k, off, dst + pf::kHalf + j * pf::kRow);
    }
}

template <int N>
MSGL_DEV void wait_vmcnt() {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Workgroup barrier that orders LDS only (the gathers are ordered by the
// explicit vmcnt waits before it).
MSGL_DEV void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Instruction order hint for one unit's main block: the first LDS reads up
// front, then one MFMA, a few VALU instructions and the next LDS read in
// turn, so that the matrix core and the vector ALU work side by side instead
// of in phases, and every MFMA finds its LDS operand already loaded.
#ifndef MSGL_PREFILL_SCHED
#define MSGL_PREFILL_SCHED 2
#endif
template <int I, int N>
MSGL_DEV void interleave_unit() {
    if constexpr (MSGL_PREFILL_SCHED == 1 && I < N) {
        __builtin_amdgcn_sched_group_barrier(0x100, I < 6 ? 2 : 1, 0);  // LDS reads
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);              // MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);              // VALU
        interleave_unit<I + 1, N>();
    } else if constexpr (MSGL_PREFILL_SCHED >= 2 && I < N) {
        constexpr int kValu = MSGL_PREFILL_SCHED == 2 ? 6 : 4;
        if constexpr (I == 0) __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, kValu, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        interleave_unit<I + 1, N>();
    }
}

// Sum over the 64 lanes of a wave (every lane gets the total).
MSGL_DEV int wave_sum(int v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
    return v;
}

// The query blocks of all requests, in decreasing order of the number of key
// tiles they see (ties: by request, then by query block), so that the block
// ids form a dense list with the longest work first.  Query block q of
// request b holds new tokens q*BQ .. q*BQ+BQ-1 of its E_b and sees
// C_b + min((q+1) BQ, E_b) keys.  Returns the request and query block of
// list entry r (b = -1 past the end).  Every lane of the wave returns the same.
struct BlockItem {
    int b;
    int qb;
};

template <int BQ>
MSGL_DEV BlockItem sorted_block(const PrefillArgs &a, int r, int lane) {
    // new and cached tokens of request b (no blocks when the request is malformed)
    auto extend = [&](int b, int &E, int &C) __attribute__((always_inline)) {
        const int L = (int)min((int64_t)a.seq_lens[b], a.row_stride);
        C = a.cached_lens[b];
        E = C < 0 ? 0 : L - C;
    };
    // first query block of a request with more than x key tiles (nb if none)
    auto first_above = [&](int E, int C, int x) __attribute__((always_inline)) {
        const int y = pf::kKT * x - C;  // needs min((q+1) BQ, E) > y
        const int nb = (E + BQ - 1) / BQ;
        return E > y ? (y < 0 ? 0 : y / BQ) : nb;
    };
    // number of query blocks with more than x key tiles
    auto count_above = [&](int x) __attribute__((always_inline)) {
        int n = 0;
        for (int b = lane; b < a.batch; b += 64) {
            int E, C;
            extend(b, E, C);
            if (E > 0) n += (E + BQ - 1) / BQ - first_above(E, C, x);
        }
        return wave_sum(n);
    };
    const int xmax = (int)min((a.row_stride + pf::kKT - 1) / pf::kKT, (int64_t)1 << 24);
    if (count_above(0) <= r) return {-1, 0};
    // tile count x of entry r: the largest x with more than r blocks of >= x tiles
    int lo = 1, hi = xmax + 1;
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (count_above(mid - 1) > r) lo = mid;
        else hi = mid;
    }
    // the k-th block with exactly lo tiles, in request order
    int k = r - count_above(lo);
    for (int base = 0; base < a.batch; base += 64) {
        const int b = base + lane;
        int c = 0, q0 = 0;
        if (b < a.batch) {
            int E, C;
            extend(b, E, C);
            if (E > 0) {
                q0 = first_above(E, C, lo - 1);
                c = first_above(E, C, lo) - q0;
            }
        }
        int incl = c;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int t = __shfl_up(incl, off);
            if (lane >= off) incl += t;
        }
        const unsigned long long hit = __ballot(k >= incl - c && k < incl);
        if (hit != 0) {
            const int src = __builtin_ctzll(hit);
            return {__shfl(b, src), __shfl(q0 + k - (incl - c), src)};
        }
        k -= __shfl(incl, 63);
    }
    return {-1, 0};
}

template <int GQ>
__global__ __launch_bounds__(pf::kThreads, 2) void prefill_mfma_kernel(PrefillArgs a) {
    constexpr int BQ = pf::kCols / GQ;  // query tokens per block
    constexpr int S = pf::kStages;
    __shared__ __attribute__((aligned(1024))) char smem[S * pf::kStage];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int jj = lane >> 5;
    const int G = a.kv_heads;

    // block id = list entry * G + kv head: the query blocks longest first, no gaps
    const int kvh = blockIdx.x % G;
    const BlockItem item = sorted_block<BQ>(a, blockIdx.x / G, lane);
    const int b = __builtin_amdgcn_readfirstlane(item.b);
    const int qb = __builtin_amdgcn_readfirstlane(item.qb);
    if (b < 0) return;  // past the last query block: uniform over the block, before any barrier
    const int L = (int)min((int64_t)a.seq_lens[b], a.row_stride);
    const int C = a.cached_lens[b];
    const int E = L - C;
    const int t0 = qb * BQ;
    if (qb < 0 || C < 0 || t0 >= E) return;
    const int row0 = a.cu_q[b] + t0;
    const int ntok = min(min(BQ, E - t0), a.total_q - row0);
    if (ntok <= 0) return;
    const int pos0 = C + t0;         // position of the block's first token
    const int nkeys = pos0 + ntok;   // keys 0 .. position of its last token
    const int ntiles = (nkeys + pf::kKT - 1) / pf::kKT;

    // this lane's query column
    const int col = wave * pf::kColsW + (lane & 31);
    const int tl = col / GQ;
    const int hq = kvh * GQ + col % GQ;
    const bool valid = tl < ntok;
    const int tok = valid ? tl : ntok - 1;
    const int pos = pos0 + tok;

    // gather sources: page-table row, pools at this kv head, per-lane chunk offsets
    const auto *pt = (const __attribute__((address_space(4))) int32_t *)(
        a.page_table + (int64_t)a.table_idx[b] * a.row_stride);
    const uint32_t num_slots = (uint32_t)a.num_slots;
    const int64_t row_bytes = (int64_t)G * pf::kD * 2;
    const char *kbase = reinterpret_cast<const char *>(a.k_pool) + (int64_t)kvh * pf::kRow;
    const int64_t v_minus_k = reinterpret_cast<const char *>(a.v_pool) - reinterpret_cast<const char *>(a.k_pool);
    const uint32_t lane4 = 4 * lane;
    const uint32_t lds_wave = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char *)smem +
                              8 * wave * pf::kRow;  // this wave's first row of stage 0

    // pipeline prologue: gathers of tiles 0..S-2, then Q, then the ids of tiles S-1 and S
    TileIds ids_use, ids_next;
#pragma unroll
    for (int t = 0; t < S - 1; ++t) {
        load_ids(ids_use, pt, t * pf::kKT + 8 * wave, nkeys);
        issue_tile(lds_wave + t * pf::kStage, ids_use, wave, kbase, v_minus_k, row_bytes, lane4, num_slots);
    }
    // Q^T operands: d-chunk dc holds dims 16*dc + 8*jj .. +7 of this column.
    // The empty asm below makes the compiler wait for them here, once; the
    // gathers it cannot see are older, so they are complete then as well.
    bf16x8_t qv[8];
    const bf16_t *qp = reinterpret_cast<const bf16_t *>(a.q) +
                       ((int64_t)(row0 + tok) * a.q_heads + hq) * pf::kD + 8 * jj;
#pragma unroll
    for (int dc = 0; dc < 8; ++dc) qv[dc] = __builtin_bit_cast(bf16x8_t, ld16(qp + 16 * dc));
#pragma unroll
    for (int dc = 0; dc < 8; ++dc) asm volatile("" ::"v"(qv[dc]));
    load_ids(ids_use, pt, (S - 1) * pf::kKT + 8 * wave, nkeys);
    load_ids(ids_next, pt, S * pf::kKT + 8 * wave, nkeys);

    // LDS read offsets within a stage.  K (A of S^T): row (lane%32) [+32 for
    // the second half], chunk 2*dc + jj.  V (A of O^T, transposing reads):
    // lane L reads row 4*jj + (L/4)%4 [+8*qq, +32 for the second half] at
    // dims 32*db + 16*((L/16)%2) + 4*(L%4), i.e. chunk 4*db + vch, byte 8*(L%2).
    const int kx = row_code(lane & 15) ^ jj;
    const int krow = (lane & 31) * pf::kRow;
    const int vrow = 4 * jj + ((lane >> 2) & 3);
    const int vch = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
    const int vx0 = vrow * pf::kRow + ((vch ^ row_code(vrow)) << 4) + (lane & 1) * 8;      // qq even
    const int vx1 = vrow * pf::kRow + ((vch ^ row_code(vrow + 8)) << 4) + (lane & 1) * 8;  // qq odd

    // The key sequence is processed in units of 32 keys (half a tile).  Unit
    // u's scores are computed two units ahead of its P.V and its softmax one
    // unit ahead, so that every unit's MFMAs (scores of u+2, P.V of u) and its
    // VALU work (softmax of u+1) are independent and can overlap.
    floatx16_t acc[4];
#pragma unroll
    for (int db = 0; db < 4; ++db) acc[db] = floatx16_t{};
 float ls = 0.0f;                  // this lane's share of the running sum of the bf16-rounded weights
    float m;                          // running column max (log2 units; may lag by < 2^8)
    float lt = 0.0f;                  // this lane's share of the running sum of the weights (for lse)
    floatx16_t sc;                    // raw scores of the unit whose softmax is next
    bf16x8_t pb[2];                   // weights of the unit whose P.V is next

    auto scores = [&](int u) __attribute__((always_inline)) {
        const char *kr = smem + ((u >> 1) % S) * pf::kStage + (u & 1) * 32 * pf::kRow + krow;
        floatx16_t s = floatx16_t{};
#pragma unroll
        for (int dc = 0; dc < 8; ++dc)
            s = mfma_32x32x16(*reinterpret_cast<const bf16x8_t *>(kr + (((2 * dc) ^ kx) << 4)), qv[dc], s);
        return s;
    };
    auto mask = [&](floatx16_t &s, int u) __attribute__((always_inline)) {
        if (32 * u + 31 > pos0) {  // causal mask, only on units that reach past the block's first position
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int key = 32 * u + 8 * (e >> 2) + 4 * jj + (e & 3);
                s[e] = key > pos ? -INFINITY : s[e];
            }
        }
    };
    auto column_max = [&](const floatx16_t &s) __attribute__((always_inline)) {
        float mx = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
#pragma unroll
        for (int e = 4; e < 16; e += 4) mx = fmaxf(mx, fmaxf(fmaxf(s[e], s[e + 1]), fmaxf(s[e + 2], s[e + 3])));
        return max_with_other_half(mx) * a.scale_log2;  // raw scores: the scale is positive
    };
    auto weights = [&](const floatx16_t &s, bf16x8_t (&out)[2]) __attribute__((always_inline)) {
        const float nmu = -m;
        uint32_t pw[8];
#pragma unroll
        for (int e = 0; e < 16; e += 2) {
            const float p0 = fast_exp2(fmaf(s[e], a.scale_log2, nmu));
            const float p1 = fast_exp2(fmaf(s[e + 1], a.scale_log2, nmu));
            pw[e >> 1] = pack_bf16x2(p0, p1);
            lt += p0 + p1;
            ls = dot2_bf16(pw[e >> 1], 0x3f803f80u, ls);  // the rounded pair, as P.V will use it
        }
        out[0] = __builtin_bit_cast(bf16x8_t, make_uint4(pw[0], pw[1], pw[2], pw[3]));
        out[1] = __builtin_bit_cast(bf16x8_t, make_uint4(pw[4], pw[5], pw[6], pw[7]));
    };
    auto pv = [&](int u) __attribute__((always_inline)) {
        const char *vs = smem + ((u >> 1) % S) * pf::kStage + pf::kHalf + (u & 1) * 32 * pf::kRow;
#pragma unroll
        for (int db = 0; db < 4; ++db) {
            uint2 av[4];
#pragma unroll
            for (int qq = 0; qq < 4; ++qq)
                av[qq] = lds_read_tr16(vs + 8 * qq * pf::kRow + ((qq & 1 ? vx1 : vx0) ^ (db << 6)));
            acc[db] = mfma_32x32x16(__builtin_bit_cast(bf16x8_t, make_uint4(av[0].x, av[0].y, av[1].x, av[1].y)),
                                    pb[0], acc[db]);
            acc[db] = mfma_32x32x16(__builtin_bit_cast(bf16x8_t, make_uint4(av[2].x, av[2].y, av[3].x, av[3].y)),
                                    pb[1], acc[db]);
        }
    };
    // One unit: P.V of unit u, the softmax of unit u+1 (whose scores are in
    // sc) and, if there is one, the scores of unit u+2.
    auto unit = [&](int u, bool has_scores, bool has_softmax) __attribute__((always_inline)) {
        if (has_softmax) mask(sc, u + 1);
        floatx16_t s_new;
        if (has_scores) s_new = scores(u + 2);
        pv(u);
        float alpha = 1.0f;
        bf16x8_t pb_new[2];
        if (has_softmax) {
            const float mx = column_max(sc);
            const float mn = mx > m + pf::kRescaleLog2 ? mx : m;  // lazy: move the max only by more than 2^8
            alpha = fast_exp2(m - mn);
            m = mn;
            lt *= alpha;
            ls *= alpha;
            weights(sc, pb_new);
            // keep the weights in this block (the compiler would otherwise sink
            // them past the rescale branch, away from the MFMAs they overlap)
            asm volatile("" ::"v"(pb_new[0]), "v"(pb_new[1]), "v"(lt), "v"(ls));
        }
        if (has_scores && has_softmax) interleave_unit<0, 16>();
        if (has_softmax && __any(alpha != 1.0f)) {  // rare: rescale what P.V of units <= u accumulated
#pragma unroll
            for (int db = 0; db < 4; ++db)
#pragma unroll
                for (int e = 0; e < 16; ++e) acc[db][e] *= alpha;
        }
        if (has_softmax) {
            pb[0] = pb_new[0];
            pb[1] = pb_new[1];
        }
        if (has_scores) sc = s_new;
    };

    // scores and weights of unit 0, scores of unit 1 (tile 0)
    wait_vmcnt<(S - 2) * pf::kGathersPerTile>();
    lds_barrier();
    {
        floatx16_t s0 = scores(0);
        sc = scores(1);
        mask(s0, 0);
        m = column_max(s0);  // key 0 is visible to every column: finite
        weights(s0, pb);
    }
    for (int t = 0; t + 1 < ntiles; ++t) {
        // this wave's gathers of tile t+1 are done (the later tiles' may still
        // be in flight); after the barrier everyone's are, and every wave has
        // finished reading tile t-1's stage, which is refilled with tile t+S-1
        wait_vmcnt<(S - 3) * pf::kGathersPerTile>();
        lds_barrier();
        {
            TileIds ids_new;
            load_ids(ids_new, pt, (t + S + 1) * pf::kKT + 8 * wave, nkeys);
            issue_tile(lds_wave + ((t + S - 1) % S) * pf::kStage, ids_use, wave, kbase, v_minus_k, row_bytes,
                       lane4, num_slots);  // past the end: harmless reloads
            ids_use = ids_next;
            ids_next = ids_new;
        }
        unit(2 * t, true, true);
        unit(2 * t + 1, true, true);
    }
    // the last tile: it is resident since the previous iteration (or the prologue)
    unit(2 * ntiles - 2, false, true);
    unit(2 * ntiles - 1, false, false);
    // the gathers issued past the last tile must land before the block's LDS is released
    wait_vmcnt<0>();

    lt = add_with_other_half(lt);
    ls = add_with_other_half(ls);
    if (valid) {
        const float inv = 1.0f / ls;
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
    // at most sum over requests of ceil(E_b / BQ) query blocks
    const int64_t nqb = (a.max_extend + BQ - 1) / BQ;
    const int64_t blocks = std::min(nqb * a.batch, ((int64_t)a.total_q + (int64_t)a.batch * (BQ - 1)) / BQ);
    const int64_t grid = blocks * a.kv_heads;
    if (grid < 1) return hipSuccess;
    if (grid > 0x7fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL((prefill_mfma_kernel<GQ>), dim3((unsigned)grid), dim3(pf::kThreads), 0, stream, a);
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
