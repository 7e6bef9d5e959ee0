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
// Blocks are ordered longest-first (last query blocks, which see the most
// keys, get the lowest block ids) so the ragged tail balances.
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
constexpr int kGathersPerTile = 4;         // vector memory instructions per wave per tile
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

// One gather of 16 bytes per lane straight into LDS (global_load_lds_dwordx4):
// lane l's bytes land at LDS address lds + 16 l (lds is wave-uniform, in M0).
// Issued as inline assembly so that the compiler neither counts it nor holds
// later LDS reads back for it: the kernel orders it itself (vmcnt + barrier).
MSGL_DEV void gather_to_lds(const void *src, uint32_t lds) {
    asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "{m0}"(lds) : "memory");
}

// Gathers of one tile by one wave to LDS address `dst` (the stage + this
// wave's first row): K rows then V rows 8w + 4i + l/16 (i = 0, 1).  Lane l
// writes chunk position l%16 of its row, so gofs names the chunk the row
// permutation puts there.
MSGL_DEV void issue_tile(uint32_t dst, TileIds ids, int grp, const char *kbase, int64_t v_minus_k, int64_t row_bytes,
                         uint2 gofs, uint32_t num_slots) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        int s = ids[4 * i];
        s = grp == 1 ? ids[4 * i + 1] : s;
        s = grp == 2 ? ids[4 * i + 2] : s;
        s = grp == 3 ? ids[4 * i + 3] : s;
        s = (uint32_t)s < num_slots ? s : 0;  // a malformed id stays inside the pool
        const char *ksrc = kbase + (int64_t)s * row_bytes + (i == 0 ? gofs.x : gofs.y);
        gather_to_lds(ksrc, dst + 4 * i * pf::kRow);
        gather_to_lds(ksrc + v_minus_k, dst + pf::kHalf + 4 * i * pf::kRow);
    }
}

template <int GQ>
__global__ __launch_bounds__(pf::kThreads, 2) void prefill_mfma_kernel(PrefillArgs a, int nqb) {
    constexpr int BQ = pf::kCols / GQ;  // query tokens per block
    __shared__ __attribute__((aligned(1024))) char smem[pf::kStages * pf::kStage];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
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
    const int ntiles = (nkeys + pf::kKT - 1) / pf::kKT;

    // this lane's query column
    const int col = wave * pf::kColsW + (lane & 31);
    const int tl = col / GQ;
    const int hq = kvh * GQ + col % GQ;
    const bool valid = tl < ntok;
    const int tok = valid ? tl : ntok - 1;
    const int pos = pos0 + tok;
    // the wave's last position: tiles that start beyond it are skipped by this wave
    const int wave_last = pos0 + min((wave * pf::kColsW + pf::kColsW - 1) / GQ, ntok - 1);

    // gather sources: page-table row, pools at this kv head, per-lane chunk offsets
    const auto *pt = (const __attribute__((address_space(4))) int32_t *)(
        a.page_table + (int64_t)a.table_idx[b] * a.row_stride);
    const uint32_t num_slots = (uint32_t)a.num_slots;
    const int64_t row_bytes = (int64_t)G * pf::kD * 2;
    const char *kbase = reinterpret_cast<const char *>(a.k_pool) + (int64_t)kvh * pf::kRow;
    const int64_t v_minus_k = reinterpret_cast<const char *>(a.v_pool) - reinterpret_cast<const char *>(a.k_pool);
    const int grp = lane >> 4;
    const uint32_t lds_wave = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char *)smem +
                              8 * wave * pf::kRow;  // this wave's first row of stage 0
    const uint2 gofs = make_uint2(((lane & 15) ^ row_code(8 * wave + grp)) << 4,
                                  ((lane & 15) ^ row_code(8 * wave + 4 + grp)) << 4);

    // pipeline prologue: gathers of tiles 0..2, then Q, then the ids of tiles 3 and 4
    TileIds ids3, ids4;
#pragma unroll
    for (int t = 0; t < pf::kAhead; ++t) {
        load_ids(ids3, pt, t * pf::kKT + 8 * wave, nkeys);
        issue_tile(lds_wave + t * pf::kStage, ids3, grp, kbase, v_minus_k, row_bytes, gofs, num_slots);
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
    load_ids(ids3, pt, 3 * pf::kKT + 8 * wave, nkeys);
    load_ids(ids4, pt, 4 * pf::kKT + 8 * wave, nkeys);

    floatx16_t acc[4];
#pragma unroll
    for (int db = 0; db < 4; ++db) acc[db] = floatx16_t{};
    float m = -INFINITY;  // running column max (log2 units; may lag by < 2^8)
    float lt = 0.0f;      // this lane's share of the running sum of the weights (for lse)
    floatx16_t acc_l = floatx16_t{};  // running sum of the bf16-rounded weights (any element)
    const bf16x8_t ones = __builtin_bit_cast(bf16x8_t, make_uint4(0x3f803f80u, 0x3f803f80u, 0x3f803f80u,
                                                                  0x3f803f80u));

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

    for (int t = 0; t < ntiles; ++t) {
        // this wave's gathers of tile t are done (the two later tiles' are
        // still allowed in flight); after the barrier everyone's are, and every
        // wave has finished reading tile t-1's stage
        asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
        static_assert(2 * pf::kGathersPerTile == 8, "vmcnt above counts the gathers of two tiles");
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
        {
            TileIds ids5;
            load_ids(ids5, pt, (t + 5) * pf::kKT + 8 * wave, nkeys);
            issue_tile(lds_wave + ((t + pf::kAhead) % pf::kStages) * pf::kStage, ids3, grp, kbase, v_minus_k,
                       row_bytes, gofs, num_slots);  // past the end: harmless reloads
            ids3 = ids4;
            ids4 = ids5;
        }
        const int k0 = t * pf::kKT;
        if (k0 > wave_last) continue;  // every key of the tile is masked for this wave
        const char *st = smem + (t % pf::kStages) * pf::kStage;
        const bool need_mask = k0 + pf::kKT - 1 > pos0;

        // scores of both 32-key halves: two independent accumulation chains
        floatx16_t sc[2] = {floatx16_t{}, floatx16_t{}};
#pragma unroll
        for (int dc = 0; dc < 8; ++dc)
#pragma unroll
            for (int half = 0; half < 2; ++half)
                sc[half] = mfma_32x32x16(
                    *reinterpret_cast<const bf16x8_t *>(st + half * 32 * pf::kRow + krow + (((2 * dc) ^ kx) << 4)),
                    qv[dc], sc[half]);
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
        // one column max per tile (raw scores; the scale is positive)
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
        const char *vs = st + pf::kHalf;
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            // running sum of the rounded weights: every row of ones . P^T is the column sum
            acc_l = mfma_32x32x16(ones, pb[half][0], acc_l);
            acc_l = mfma_32x32x16(ones, pb[half][1], acc_l);
#pragma unroll
            for (int db = 0; db < 4; ++db) {
                uint2 av[4];
#pragma unroll
                for (int qq = 0; qq < 4; ++qq)
                    av[qq] = lds_read_tr16(vs + (half * 32 + 8 * qq) * pf::kRow +
                                           ((qq & 1 ? vx1 : vx0) ^ (db << 6)));
                acc[db] = mfma_32x32x16(__builtin_bit_cast(bf16x8_t, make_uint4(av[0].x, av[0].y, av[1].x, av[1].y)),
                                        pb[half][0], acc[db]);
                acc[db] = mfma_32x32x16(__builtin_bit_cast(bf16x8_t, make_uint4(av[2].x, av[2].y, av[3].x, av[3].y)),
                                        pb[half][1], acc[db]);
            }
        }
    }
    // the gathers issued past the last tile must land before the block's LDS is released
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

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
    hipLaunchKernelGGL((prefill_mfma_kernel<GQ>), dim3((unsigned)grid), dim3(pf::kThreads), 0, stream, a, nqb);
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
