// Prefill / extend attention on matrix cores (bf16 MFMA, fp32 accumulate).
//
// New token i of request b sits at position p = cached_len + i and attends
// keys 0..p of its page-table row: a causal mask offset by the cached prefix.
//
// A block covers one kv head and a set of query "columns".  A column is a
// (token, q head) pair of the q heads that share the kv head (token-major), so
// every gathered K/V tile serves the whole group; each wave owns 32 columns.
// Keys stream through LDS in 64-key tiles (K rows and V rows of 256 bytes,
// their 16-byte chunks permuted per row so that the column-wise reads below
// hit every bank once).  The gathers go straight from the pools into LDS
// (global_load_lds_dwordx4: lane l's 16 bytes land at the destination + 16 l,
// so one instruction fills 4 rows), and so do the page-table ids of a tile
// (global_load_lds_dword) ahead of its gathers.  Two layouts:
//
//  - prefill_mfma_kernel: 4 waves (128 columns), K and V rings of two tiles,
//    68 KB of LDS, so two blocks share a CU and one computes while the other
//    starts up or waits.  At each tile the wave waits for all its copies (K of
//    the next tile, V of this one, issued one tile earlier) and a barrier
//    makes everyone's visible.
//  - prefill_mfma_long_kernel: 8 waves (256 columns), one ring of 4 tiles,
//    gathers three tiles ahead, one block per CU.  Every iteration issues the
//    same five vector memory instructions per wave (fewer near the end: no
//    gathers past the last tile), so one vmcnt wait that leaves the last
//    tile's copies in flight plus one barrier per tile is exact.  It serves
//    long uniform chunks (2048 or more new tokens per request on average),
//    where its deeper ring beats the other layout's hiding of block starts.
//
// Both unroll the main loop over the ring's stages so that every LDS read
// address is a per-lane register plus an immediate.

// Keys are processed in units of 32 (half a tile).  For unit u a wave
// computes S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (A = 32 keys x 16 dims
// from LDS, B = Q^T held in registers, 8 steps over head_dim 128) two units
// ahead of its P.V and its softmax one unit ahead, so that the MFMAs of a unit
// (scores of u+2, P.V of u) and its VALU work (softmax of u+1) are independent
// and overlap.  The MFMA result layout leaves each lane with 16 scores of one
// column; after the softmax update they are rounded to bf16 and are,
// unchanged, the B operand (P^T) of O^T += V^T P^T, because the order of the
// contraction index inside an MFMA is free as long as both operands agree:
// the V^T reads (ds_read_b64_tr_b16 on the row-major V rows) pick the keys in
// the order the scores arrived in.  Nothing is shuffled between lanes except
// one exchange for the column max (v_permlane32_swap, no LDS round trip).
//
// Softmax: log2 domain (scale times log2 e folded into one fma before exp2),
// one running max per column per unit and lazy rescaling: the max only moves
// when a unit's max exceeds it by more than 2^8, which keeps exp2 arguments
// bounded and skips almost every rescale.  The P.V product applies the
// weights rounded to bf16, so the output is normalised by the fp32 sum of
// those rounded weights (a v_dot2 with a pair of ones per pair): the applied
// weights then sum to one up to float32 rounding (V = 1 gives exactly 1),
// whatever the size of the weights.  The returned lse comes from a second
// fp32 sum, of the unrounded weights, kept only when an lse is asked for (the
// instances without it save 16 adds per 32 keys).  Both sums are lane-partial
// and are reduced once at the end.
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

namespace pf {  // shared by both layouts
constexpr int kD = 128;
constexpr int kKT = 64;                          // keys per tile
constexpr int kColsW = 32;                       // query columns per wave
constexpr int kRow = kD * 2;                     // bytes per K or V row in LDS
constexpr int kTile = kKT * kRow;                // the K (or V) rows of one tile
constexpr int kIdSlots = 4;                      // page-table id slots per wave
constexpr float kRescaleLog2 = 8.0f;
constexpr int kMaxBatch = 1024;                  // requests per call on the MFMA path
}  // namespace pf
// Two bf16 ones (v_dot2 with it sums a pair of weights).
constexpr uint32_t kBf16OnesPair = 0x3f803f80u;
// A unit whose weights exceed this somewhere raises the softmax reference (2^64).
constexpr float kPrefillWeightBound = 18446744073709551616.0f;
static_assert(pf::kKT == kPlanKeyTile, "the host plan orders blocks by this kernel's key tiles");

namespace pfc {  // two blocks per CU: 4 waves, K and V rings of two tiles each
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kCols = kWaves * pf::kColsW;       // query columns per block
constexpr int kKBase = 0;                        // K ring
constexpr int kVBase = 2 * pf::kTile;            // V ring
constexpr int kIdsBase = 4 * pf::kTile;          // per wave, kIdSlots tiles of ids
constexpr int kLds = kIdsBase + kWaves * pf::kIdSlots * pf::kKT * 4;
constexpr int kRowsW = pf::kKT / kWaves;         // rows of a tile this wave gathers
static_assert(2 * kLds <= 160 * 1024, "two blocks must fit one CU's LDS");
static_assert(kRowsW == 16, "a wave's gathers of a tile: 4 instructions of 4 rows");
}  // namespace pfc

namespace pfl {  // long chunks: one block per CU, 8 waves, a ring of 4 tiles
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kCols = kWaves * pf::kColsW;       // query columns per block
constexpr int kStages = 4;
constexpr int kKBase = 0;                        // K tiles of the stages
constexpr int kVBase = kStages * pf::kTile;      // V tiles of the stages
constexpr int kIdsBase = 2 * kStages * pf::kTile;  // page-table ids: per wave, kIdSlots tiles
constexpr int kLds = kIdsBase + kWaves * pf::kIdSlots * pf::kKT * 4;
constexpr int kAhead = kStages - 1;              // tiles gathered ahead of the compute
constexpr int kIdsAhead = kStages + 1;           // tiles whose ids are copied ahead
constexpr int kIdsPerTile = 1;                   // per wave and tile: 1 id copy ...
constexpr int kVmemPerTile = kIdsPerTile + 4;    // ... and 4 gathers (none past the last tile)
static_assert(kIdsAhead - kAhead < pf::kIdSlots && kIdsAhead == pf::kIdSlots + 1 && kAhead >= 2,
              "an id slot is refilled only after its gathers were issued (the prologue relies on these values)");
}  // namespace pfl

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

typedef __attribute__((address_space(3))) char lds_char;

// Transposing LDS read (ds_read_b64_tr_b16).  Within each group of 16 lanes,
// lane 4j+a names 4 consecutive 16-bit values; lane l receives value l%4 of
// the lanes l/4, 4+l/4, 8+l/4 and 12+l/4.  When lanes 4j..4j+3 point at key
// j's row at dims +0, +4, +8, +12, lane l therefore gets dim l of keys 0..3.
MSGL_DEV uint2 lds_read_tr16(uint32_t addr) {
    const shortx4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) shortx4_t *)(uintptr_t)addr);
    return __builtin_bit_cast(uint2, v);
}

MSGL_DEV bf16x8_t lds_read16(uint32_t addr) {
    return *(const __attribute__((address_space(3))) bf16x8_t *)(uintptr_t)addr;
}

MSGL_DEV int lds_read_i32(uint32_t addr) { return *(const __attribute__((address_space(3))) int *)(uintptr_t)addr; }

// Row permutation code: chunk c of row r sits at chunk position c ^ code(r).
// code is a bijection on r % 16, so 16 (or 8) consecutive rows read at one
// chunk spread over all positions (the K reads), and its bits 1..3 give 4
// consecutive rows distinct chunk groups (the transposing V reads, 4 chunks
// of 4 rows at once).
MSGL_DEV int row_code(int r) {
    return ((r >> 2) & 1) | ((r & 1) << 1) | (((r >> 1) & 1) << 2) | (((r ^ (r >> 3)) & 1) << 3);
}

// Copies straight into LDS (global_load_lds_dword / _dwordx4): lane l's 4 or
// 16 bytes land at LDS address lds + 4 l or + 16 l; lds is wave-uniform (M0).
// Issued as inline assembly so that the compiler neither counts them nor holds
// later LDS reads back for them: the kernel orders them itself (vmcnt waits
// and barriers).  The compiler does not see the memory instruction inside, so
// it cannot insert the wait states the hardware needs between a VALU write of
// a scalar register (a readfirstlane of the base, or M0) or of an address
// register and this read of it: the s_nop 4 (5 wait states) covers them.
MSGL_DEV void copy4_to_lds(const void *base, uint32_t lane_off, uint32_t lds) {
    // the base must live in scalar registers: make its uniformity explicit
    const uint64_t b = (uint64_t)base;
    const uint64_t ub = ((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32)) << 32) |
                        (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b);
    asm volatile("s_nop 4\n\tglobal_load_lds_dword %0, %1" ::"v"(lane_off), "s"((const void *)ub), "{m0}"(lds)
                 : "memory");
}

MSGL_DEV void copy16_to_lds(const void *src, uint32_t lds) {
    asm volatile("s_nop 4\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "{m0}"(lds) : "memory");
}

// The same with the source as a 32-bit byte offset from a wave-uniform base
// (pools below 4 GiB): the address is base + off, with no 64-bit arithmetic.
MSGL_DEV void copy16_to_lds_at(const void *base, uint32_t off, uint32_t lds) {
    asm volatile("s_nop 4\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(base), "{m0}"(lds) : "memory");
}

template <int N>
MSGL_DEV void wait_vmcnt() {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Workgroup barrier that orders LDS only (the copies into LDS are ordered by
// the explicit vmcnt waits before it).
MSGL_DEV void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Instruction order hint for one unit's main block: D0 LDS reads up front,
// then groups of M MFMAs, V VALU instructions and D LDS reads in turn, so
// that the matrix core and the vector ALU work side by side instead of in
// phases, and every MFMA finds its LDS operand already loaded.
template <int M, int V, int D, int D0, int I = 0, int N = 16>
MSGL_DEV void interleave_unit() {
    if constexpr (I * M < N) {
        if constexpr (I == 0) __builtin_amdgcn_sched_group_barrier(0x100, D0, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, M, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, V, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, D, 0);
        interleave_unit<M, V, D, D0, I + 1, N>();
    }
}

// Sum over the 64 lanes of a wave (every lane gets the total).
MSGL_DEV int wave_sum(int v) {
    v += __builtin_amdgcn_update_dpp(0, v, kDppXor1, 0xF, 0xF, false);       // pairs
    v += __builtin_amdgcn_update_dpp(0, v, kDppXor2, 0xF, 0xF, false);       // quads
    v += __builtin_amdgcn_update_dpp(0, v, kDppHalfMirror, 0xF, 0xF, false); // 8 lanes
    v += __builtin_amdgcn_update_dpp(0, v, kDppMirror, 0xF, 0xF, false);     // 16-lane rows
    return __builtin_amdgcn_readlane(v, 0) + __builtin_amdgcn_readlane(v, 16) + __builtin_amdgcn_readlane(v, 32) +
           __builtin_amdgcn_readlane(v, 48);
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
    int E;      // new tokens of request b
    int C;      // its cached tokens
    int q0;     // its first q row (cu_q[b])
    int row;    // its page-table row (table_idx[b])
};

// NB = number of requests each lane keeps in registers (batch <= 64 NB); the
// per-request values are read once, and the found request's are handed over
// from the lane that holds them.  Up to 4 requests per lane the first q row
// and page-table row come in the same round trip as the lengths; beyond, they
// are read once the request is known (registers are scarcer there).
//
// Shared-prefix mode (SH): "request" b is a group of decode requests, rows
// cu_q[b] .. cu_q[b+1]-1 of q, that share the first cached_lens[cu_q[b]]
// keys of their page-table rows; its "new tokens" are the group's queries and
// its cached tokens that shared prefix, read through the first member's row.
template <int BQ, int NB, bool SH = false>
MSGL_DEV BlockItem sorted_block(const PrefillArgs &a, int r, int lane) {
    constexpr bool kAll = NB <= 4;
    constexpr int NX = kAll ? NB : 1;
    // new and cached tokens of the lane's requests (no blocks when a request is
    // malformed), their first q rows and page-table rows
    int E[NB], C[NB], Q0[NX], TI[NX];
#pragma unroll
    for (int k = 0; k < NB; ++k) {
        const int b = lane + 64 * k;
        E[k] = 0;
        C[k] = 0;
        if (kAll) {
            Q0[k % NX] = 0;
            TI[k % NX] = 0;
        }
        if (SH && b < a.batch) {
            const int q0 = a.cu_q[b], q1 = a.cu_q[b + 1];
            if (q0 >= 0 && q1 > q0 && q1 <= a.total_q) {  // a malformed group gets no blocks
                C[k] = (int)min((int64_t)a.cached_lens[q0], a.row_stride);
                E[k] = C[k] <= 0 ? 0 : q1 - q0;
                if (kAll) {
                    Q0[k % NX] = q0;
                    TI[k % NX] = a.table_idx[q0];
                }
            }
        } else if (b < a.batch) {
            const int L = (int)min((int64_t)a.seq_lens[b], a.row_stride);
            C[k] = a.cached_lens[b];
            E[k] = C[k] < 0 ? 0 : L - C[k];
            if (kAll) {
                Q0[k % NX] = a.cu_q[b];
                TI[k % NX] = a.table_idx[b];
            }
        }
    }
    // first query block of a request with more than x key tiles (nb if none)
    auto first_above = [&](int e, int c, int x) __attribute__((always_inline)) {
        const int y = pf::kKT * x - c;  // needs min((q+1) BQ, E) > y
        const int nb = (e + BQ - 1) / BQ;
        return e > y ? (y < 0 ? 0 : y / BQ) : nb;
    };
    // number of query blocks with more than x key tiles
    auto count_above = [&](int x) __attribute__((always_inline)) {
        int n = 0;
#pragma unroll
        for (int k = 0; k < NB; ++k)
            if (E[k] > 0) n += (E[k] + BQ - 1) / BQ - first_above(E[k], C[k], x);
        return wave_sum(n);
    };
    if (count_above(0) <= r) return {-1, 0, 0, 0, 0, 0};
    // tile count x of entry r: the largest x with more than r blocks of >= x tiles
    int most = 0;  // the most key tiles any block sees
#pragma unroll
    for (int k = 0; k < NB; ++k)
        if (E[k] > 0) most = max(most, (C[k] + E[k] + pf::kKT - 1) / pf::kKT);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) most = max(most, __shfl_xor(most, off));
    int lo = 1, hi = most + 1;
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (count_above(mid - 1) > r) lo = mid;
        else hi = mid;
    }
    // the k-th block with exactly lo tiles, in request order
    int k = r - count_above(lo);
#pragma unroll
    for (int j = 0; j < NB; ++j) {
        int c = 0, q0 = 0;
        if (E[j] > 0) {
            q0 = first_above(E[j], C[j], lo - 1);
            c = first_above(E[j], C[j], lo) - q0;
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
            const int b = __shfl(lane + 64 * j, src);
            if constexpr (kAll)
                return {b, __shfl(q0 + k - (incl - c), src), __shfl(E[j], src), __shfl(C[j], src),
                        __shfl(Q0[j % NX], src), __shfl(TI[j % NX], src)};
            else if constexpr (SH) {
                const int qr = a.cu_q[__builtin_amdgcn_readfirstlane(b)];
                return {b, __shfl(q0 + k - (incl - c), src), __shfl(E[j], src), __shfl(C[j], src), qr,
                        a.table_idx[qr]};
            } else
                return {b, __shfl(q0 + k - (incl - c), src), __shfl(E[j], src), __shfl(C[j], src),
                        a.cu_q[__builtin_amdgcn_readfirstlane(b)], a.table_idx[__builtin_amdgcn_readfirstlane(b)]};
        }
        k -= __shfl(incl, 63);
    }
    return {-1, 0, 0, 0, 0, 0};
}

// A block's work item read from the host plan (entry i of its block list).
MSGL_DEV BlockItem planned_block(const PrefillArgs &a, int i) {
    const int32_t *e = a.plan + (int64_t)i * kPlanEntryInts;
    return {e[0], e[1], e[2], e[3], e[4], e[5]};
}

template <int GQ, bool PL, bool LSE>
__global__ __launch_bounds__(pfl::kThreads, 2) void prefill_mfma_long_kernel(PrefillArgs a) {
    constexpr int BQ = pfl::kCols / GQ;  // query tokens per block
    constexpr int S = pfl::kStages;
    __shared__ __attribute__((aligned(1024))) char smem[pfl::kLds];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int jj = lane >> 5;
    const int G = a.kv_heads;

    // block id = list entry * G + kv head: the query blocks longest first, no gaps
    const int kvh = blockIdx.x % G;
    const BlockItem item = PL                ? planned_block(a, blockIdx.x / G)
                           : a.batch <= 64  ? sorted_block<BQ, 1>(a, blockIdx.x / G, lane)
                           : a.batch <= 256 ? sorted_block<BQ, 4>(a, blockIdx.x / G, lane)
                                            : sorted_block<BQ, pf::kMaxBatch / 64>(a, blockIdx.x / G, lane);
    const int b = __builtin_amdgcn_readfirstlane(item.b);
    const int qb = __builtin_amdgcn_readfirstlane(item.qb);
    if (b < 0) return;  // past the last query block: uniform over the block, before any barrier
    const int C = __builtin_amdgcn_readfirstlane(item.C);
    const int E = __builtin_amdgcn_readfirstlane(item.E);
    const int t0 = qb * BQ;
    if (qb < 0 || C < 0 || t0 >= E) return;
    if (PL && (int64_t)C + E > a.row_stride) return;  // an entry whose keys pass the table row runs nothing
    const int row0 = __builtin_amdgcn_readfirstlane(item.q0) + t0;
    const int ntok = min(min(BQ, E - t0), a.total_q - row0);
    if (ntok <= 0 || row0 < 0) return;
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

    const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_char *)smem;
    // page-table ids: each wave copies all 64 ids of a tile into its own slot
    // (keys past the block's last one read key 0's id: a real row whose scores
    // the causal mask removes)
    const int32_t *pt = a.page_table + (int64_t)__builtin_amdgcn_readfirstlane(item.row) * a.row_stride;
    const uint32_t ids_wave = lds0 + pfl::kIdsBase + wave * pf::kIdSlots * pf::kKT * 4;
    auto copy_ids = [&](int t) __attribute__((always_inline)) {
        const int key = t * pf::kKT + lane;
        copy4_to_lds(pt, 4u * (uint32_t)(key < nkeys ? key : 0), ids_wave + (t % pf::kIdSlots) * pf::kKT * 4);
    };
    // gathers: per tile this wave fills rows 8w + 4i + l/16 (i = 0, 1) of K and
    // V; lane l writes chunk position l%16 of its row, so it loads the chunk
    // that the permutation puts there
    const uint32_t last_slot = (uint32_t)(min(a.num_slots, (int64_t)1 << 31) - 1);
    const uint32_t row_bytes = (uint32_t)G * pf::kRow;
    const int grp = lane >> 4;
    const char *kb[2], *vb[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const uint32_t off = (uint32_t)kvh * pf::kRow + (((lane & 15) ^ row_code(8 * wave + 4 * i + grp)) << 4);
        kb[i] = reinterpret_cast<const char *>(a.k_pool) + off;
        vb[i] = reinterpret_cast<const char *>(a.v_pool) + off;
    }
    auto gather = [&](int t, int stage) __attribute__((always_inline)) {
        const uint32_t ids = ids_wave + (t % pf::kIdSlots) * pf::kKT * 4 + (8 * wave + grp) * 4;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            int s = lds_read_i32(ids + 16 * i);
            s = (int)min((uint32_t)s, last_slot);  // a malformed id (negative or too large) reads the last slot
            const uint32_t dst = lds0 + stage * pf::kTile + (8 * wave + 4 * i) * pf::kRow;
            copy16_to_lds(kb[i] + (uint64_t)(uint32_t)s * row_bytes, dst + pfl::kKBase);
            copy16_to_lds(vb[i] + (uint64_t)(uint32_t)s * row_bytes, dst + pfl::kVBase);
        }
    };

    // pipeline prologue: ids of tiles 0..3, gathers of tiles 0..2 with the
    // ids of tile 4 copied once the slot of tile 0 has been read, then Q
#pragma unroll
    for (int t = 0; t < pf::kIdSlots; ++t) copy_ids(t);
    wait_vmcnt<pf::kIdSlots - pfl::kAhead>();  // this wave's ids of tiles 0..2 (its own slots)
    gather(0, 0);
    copy_ids(pf::kIdSlots);
#pragma unroll
    for (int t = 1; t < pfl::kAhead; ++t)
        if (t < ntiles) gather(t, t);
    // Q^T operands: d-chunk dc holds dims 16*dc + 8*jj .. +7 of this column.
    // The empty asm below makes the compiler wait for them here, once; the
    // copies it cannot see are older, so they are complete then as well.
    bf16x8_t qv[8];
    const bf16_t *qp = reinterpret_cast<const bf16_t *>(a.q) +
                       ((int64_t)(row0 + tok) * a.q_heads + hq) * pf::kD + 8 * jj;
#pragma unroll
    for (int dc = 0; dc < 8; ++dc) qv[dc] = __builtin_bit_cast(bf16x8_t, ld16(qp + 16 * dc));
#pragma unroll
    for (int dc = 0; dc < 8; ++dc) asm volatile("" ::"v"(qv[dc]));

    // LDS read addresses, per lane, of stage 0's first half (stages and halves
    // are immediate offsets).  K (A of S^T): row lane%32, chunk 2*dc + jj.
    // V (A of O^T, transposing reads): lane L reads row 4*jj + (L/4)%4 [+8*qq]
    // at dims 32*db + 16*((L/16)%2) + 4*(L%4), i.e. chunk 4*db + vch, byte 8*(L%2).
    uint32_t kaddr[8], vaddr[4][2];
    {
        const int kx = row_code(lane & 15) ^ jj;
        const int vrow = 4 * jj + ((lane >> 2) & 3);
        const int vch = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
#pragma unroll
        for (int dc = 0; dc < 8; ++dc) kaddr[dc] = lds0 + pfl::kKBase + (lane & 31) * pf::kRow + (((2 * dc) ^ kx) << 4);
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int par = 0; par < 2; ++par)
                vaddr[db][par] = lds0 + pfl::kVBase + vrow * pf::kRow +
                                 (((4 * db + vch) ^ row_code(vrow + 8 * par)) << 4) + (lane & 1) * 8;
    }

    floatx16_t acc[4];
#pragma unroll
    for (int db = 0; db < 4; ++db) acc[db] = floatx16_t{};
    float m;                          // running column max (log2 units; may lag by < 2^8)
    float lt = 0.0f;                  // this lane's share of the running sum of the weights: the lse
    float lr = 0.0f;                  // ... of the weights rounded to bf16, as P.V applies them: the normalisation
    floatx16_t sc;                    // raw scores of the unit whose softmax is next
    bf16x8_t pb[2];                   // weights of the unit whose P.V is next

    auto scores = [&](int stage, int half) __attribute__((always_inline)) {
        floatx16_t s = floatx16_t{};
#pragma unroll
        for (int dc = 0; dc < 8; ++dc)
            s = mfma_32x32x16(lds_read16(kaddr[dc] + stage * pf::kTile + half * 32 * pf::kRow), qv[dc], s);
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
        float mx = fmaxf(fmaxf(s[0], s[1]), s[2]);  // a chain of three-input maxes
#pragma unroll
        for (int e = 3; e < 15; e += 2) mx = fmaxf(fmaxf(mx, s[e]), s[e + 1]);
        mx = fmaxf(mx, s[15]);
        return max_with_other_half(mx) * a.scale_log2;  // raw scores: the scale is positive
    };
    // weights exp2(s * scale - mu), rounded pairs for P.V, the sum of the
    // weights and the sum of the rounded weights
    auto weights = [&](const floatx16_t &s, float mu, bf16x8_t (&out)[2], float &sum, float &rsum)
                       __attribute__((always_inline)) {
        uint32_t pw[8];
        sum = 0.0f;
        rsum = 0.0f;
#pragma unroll
        for (int e = 0; e < 16; e += 2) {
            const float p0 = fast_exp2(fmaf(s[e], a.scale_log2, -mu));
            const float p1 = fast_exp2(fmaf(s[e + 1], a.scale_log2, -mu));
            pw[e >> 1] = pack_bf16x2(p0, p1);
            if constexpr (LSE) sum += p0 + p1;  // the unrounded sum serves only the lse
            rsum = dot2_bf16(pw[e >> 1], kBf16OnesPair, rsum);
        }
        out[0] = __builtin_bit_cast(bf16x8_t, make_uint4(pw[0], pw[1], pw[2], pw[3]));
        out[1] = __builtin_bit_cast(bf16x8_t, make_uint4(pw[4], pw[5], pw[6], pw[7]));
    };
    auto pv = [&](int stage, int half) __attribute__((always_inline)) {
#pragma unroll
        for (int db = 0; db < 4; ++db) {
            uint2 av[4];
#pragma unroll
            for (int qq = 0; qq < 4; ++qq)
                av[qq] = lds_read_tr16(vaddr[db][qq & 1] + stage * pf::kTile + half * 32 * pf::kRow +
                                       8 * qq * pf::kRow);
            acc[db] = mfma_32x32x16(__builtin_bit_cast(bf16x8_t, make_uint4(av[0].x, av[0].y, av[1].x, av[1].y)),
                                    pb[0], acc[db]);
            acc[db] = mfma_32x32x16(__builtin_bit_cast(bf16x8_t, make_uint4(av[2].x, av[2].y, av[3].x, av[3].y)),
                                    pb[1], acc[db]);
        }
    };
    // One unit: P.V of unit u (tile stage `stage`, half u%2), the softmax of
    // unit u+1 (its scores are in sc) and, if there is one, the scores of
    // unit u+2 (the same half of the next tile, stage `next`).
    auto unit = [&](int u, int stage, int next, bool has_scores, bool has_softmax) __attribute__((always_inline)) {
        const int half = u & 1;
        if (has_softmax) mask(sc, u + 1);
        floatx16_t s_new;
        if (has_scores) s_new = scores(next, half);
        pv(stage, half);
        float mn = m, lt_u = 0.0f, lr_u = 0.0f;
        bf16x8_t pb_new[2];
        if (has_softmax) {
            const float mx = column_max(sc);
            mn = mx > m + pf::kRescaleLog2 ? mx : m;  // lazy: move the max only by more than 2^8
            weights(sc, mn, pb_new, lt_u, lr_u);
            // keep the weights in this block (the compiler would otherwise sink
            // them past the rescale branch, away from the MFMAs they overlap)
            asm volatile("" ::"v"(pb_new[0]), "v"(pb_new[1]), "v"(lt_u), "v"(lr_u));
        }
        if (has_scores && has_softmax) interleave_unit<2, 10, 3, 8>();
        if (has_softmax && __any(mn != m)) {  // rare: rescale what units <= u accumulated
            const float alpha = fast_exp2(m - mn);
            lt *= alpha;
            lr *= alpha;
#pragma unroll
            for (int db = 0; db < 4; ++db)
#pragma unroll
                for (int e = 0; e < 16; ++e) acc[db][e] *= alpha;
        }
        if (has_softmax) {
            m = mn;
            lt += lt_u;
            lr += lr_u;
            pb[0] = pb_new[0];
            pb[1] = pb_new[1];
        }
        if (has_scores) sc = s_new;
    };
    // Tile t < ntiles-1 (its stage is t % S): refill the stage of tile t-1
    // with tile t+S-1, copy the ids of tile t+S+1, then units 2t and 2t+1.
    auto tile = [&](int t, int stage) __attribute__((always_inline)) {
        // this wave's copies of tile t+1 (and of the ids of tile t+S-1) are
        // done, the later ones may still be in flight; after the barrier
        // everyone's are, and every wave has finished reading tile t-1's stage
        if (t + S - 2 < ntiles) wait_vmcnt<(S - 3) * pfl::kVmemPerTile>();
        else wait_vmcnt<(S - 3) * pfl::kIdsPerTile>();  // some later tiles had no gathers: count only the id copies
        lds_barrier();
        copy_ids(t + pfl::kIdsAhead);  // past the end: a harmless copy of key 0's id
        if (t + pfl::kAhead < ntiles) gather(t + pfl::kAhead, (stage + pfl::kAhead) % S);
        const int next = (stage + 1) % S;
        unit(2 * t, stage, next, true, true);
        unit(2 * t + 1, stage, next, true, true);
    };

    // scores and weights of unit 0, scores of unit 1 (tile 0)
    lds_barrier();
    {
        floatx16_t s0 = scores(0, 0);
        sc = scores(0, 1);
        mask(s0, 0);
        m = column_max(s0);  // key 0 is visible to every column: finite
        weights(s0, m, pb, lt, lr);
    }
    int t = 0;
    for (; t + S <= ntiles - 1; t += S) {
        tile(t, 0);
        tile(t + 1, 1);
        tile(t + 2, 2);
        tile(t + 3, 3);
    }
    for (; t < ntiles - 1; ++t) tile(t, t % S);
    // the last tile: resident since the previous iteration (or the prologue)
    const int last = (ntiles - 1) % S;
    unit(2 * ntiles - 2, last, 0, false, true);
    unit(2 * ntiles - 1, last, 0, false, false);
    // the id copies issued past the last tile must land before the block's LDS is released
    wait_vmcnt<0>();

    // normalised by the sum of the weights P.V applied (V = 1 gives 1 exactly);
    // lse from the sum of the unrounded weights
    if constexpr (LSE) lt = add_with_other_half(lt);
    lr = add_with_other_half(lr);
    if (valid) {
        const float inv = 1.0f / lr;
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
        if constexpr (LSE)
            if (a.lse != nullptr && jj == 0) a.lse[(int64_t)(row0 + tl) * a.q_heads + hq] = (m + __log2f(lt)) * kLn2;
    }
}

// Two blocks per CU: 4 waves (128 query columns) and K and V rings of two
// 64-key tiles each (68 KB of LDS), so that while one block waits (its
// start, its gathers, the dispatch of the next block) the other computes.
// At tile t the wave waits for all its copies and a barrier makes everyone's
// visible (K of t+1 and V of t, issued in tile t-1); then it refills the
// stages tile t-1 used, K of t+2 and V of t+1 (from ids it read into
// registers in tile t-1), copies the ids of t+4, reads the ids of the next
// tile's gathers, and runs units 2t and 2t+1.
//
// Differences from the single-block layout:
//  - Gathers: wave w's instruction i writes LDS rows 16w + 4i + lane/16, each
//    the row of key 16w + 4(lane/16) + i of the tile, so a lane's 4 ids are
//    adjacent (one 16-byte LDS read).  With O32 (pools below 4 GiB) the rows
//    are addressed as 32-bit offsets from the pool base.
//  - Each unit runs P.V first, then the scores of the unit two ahead.
//  - Softmax without a per-unit maximum: the weights are taken against the
//    first unit's column maximum m.  A unit whose weights pass 2^64 in some
//    lane (or are not finite) raises m to its own column maximum and rescales
//    what came before; this branch is rare and, so that none of it runs on
//    the common path, its inputs go through an opaque copy.
//  - Each wave stops computing after its last tile (the one holding its last
//    query's key), and skips that tile's second half when every key there
//    lies past its queries; it still takes part in every tile's copies and
//    barrier.
//  - The page-table ids of a tile are copied four tiles ahead, and a wave
//    reads the ids of its next tile's gathers into registers a tile early, so
//    the gathers issue right after the barrier without waiting on LDS.
//
// In shared-prefix mode (SH, decode requests grouped by a shared radix prefix)
// the block id also carries a key split s < a.splits: the block attends its
// group's queries to split s of the shared prefix (no causal mask: every
// query sits after the prefix) and writes the normalised partial output and
// its lse, in float32, to split s of the partial arrays.
template <int GQ, bool SH, bool PL, bool O32, bool LSE>
__global__ __launch_bounds__(pfc::kThreads, 2) void prefill_mfma_kernel(PrefillArgs a) {
    constexpr int BQ = pfc::kCols / GQ;  // query tokens per block
    __shared__ __attribute__((aligned(1024))) char smem[pfc::kLds];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int jj = lane >> 5;
    const int grp = lane >> 4;
    const int G = a.kv_heads;

    // block id = (list entry * G + kv head) [* splits + split]: the query blocks
    // longest first, no gaps
    const int split = SH ? (int)(blockIdx.x % a.splits) : 0;
    const int bid = SH ? (int)(blockIdx.x / a.splits) : (int)blockIdx.x;
    const int kvh = bid % G;
    const BlockItem item = PL                ? planned_block(a, bid / G)
                           : a.batch <= 64  ? sorted_block<BQ, 1, SH>(a, bid / G, lane)
                           : a.batch <= 256 ? sorted_block<BQ, 4, SH>(a, bid / G, lane)
                                            : sorted_block<BQ, pf::kMaxBatch / 64, SH>(a, bid / G, lane);
    const int b = __builtin_amdgcn_readfirstlane(item.b);
    const int qb = __builtin_amdgcn_readfirstlane(item.qb);
    if (b < 0) return;  // past the last query block: uniform over the block, before any barrier
    const int C = __builtin_amdgcn_readfirstlane(item.C);
    const int E = __builtin_amdgcn_readfirstlane(item.E);
    const int t0 = qb * BQ;
    if (qb < 0 || C < 0 || t0 >= E) return;
    if (PL && (int64_t)C + E > a.row_stride) return;  // an entry whose keys pass the table row runs nothing
    const int row0 = __builtin_amdgcn_readfirstlane(item.q0) + t0;
    const int ntok = min(min(BQ, E - t0), a.total_q - row0);
    if (ntok <= 0 || row0 < 0) return;
    // SH: keys k0 .. k0 + span - 1 of the shared prefix (splits of whole tiles)
    const int span = SH ? (((C + a.splits - 1) / a.splits + pf::kKT - 1) / pf::kKT) * pf::kKT : 0;
    const int k0 = SH ? min(C, split * span) : 0;
    const int pos0 = SH ? min(C, k0 + span) - k0 - 1 : C + t0;  // SH: every query sees the whole split
    const int nkeys = SH ? pos0 + 1 : pos0 + ntok;  // keys 0 .. position of its last token
    const int ntiles = (nkeys + pf::kKT - 1) / pf::kKT;

    // this lane's query column
    const int col = wave * pf::kColsW + (lane & 31);
    const int tl = col / GQ;
    const int hq = kvh * GQ + col % GQ;
    const bool valid = tl < ntok;
    const int tok = valid ? tl : ntok - 1;
    const int pos = SH ? pos0 : pos0 + tok;
    // this wave's last tile: the one holding its last valid query's last key (-1: no valid query)
    const int wfirst = (wave * pf::kColsW) / GQ;
    // this wave's last key (the position of its last valid query) and the tile holding it
    const int wlast = SH ? pos0 : pos0 + min(ntok - 1, (wave * pf::kColsW + pf::kColsW - 1) / GQ);
    const int tw = wfirst >= ntok ? -1 : wlast / pf::kKT;

    if constexpr (SH) {
        if (nkeys <= 0) {  // an empty split: an empty softmax state, marked by lse = -inf
            if (valid && jj == 0)
                a.part_lse[((int64_t)split * a.total_q + row0 + tl) * a.q_heads + hq] = -INFINITY;
            return;
        }
    }

    const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_char *)smem;
    // page-table ids: each wave copies all 64 ids of a tile into its own slot
    // (keys past the block's last one read key 0's id: a real row whose scores
    // the causal mask removes)
    const int32_t *pt = a.page_table + (int64_t)__builtin_amdgcn_readfirstlane(item.row) * a.row_stride + k0;
    const uint32_t ids_wave = lds0 + pfc::kIdsBase + wave * pf::kIdSlots * pf::kKT * 4;
    auto copy_ids = [&](int t) __attribute__((always_inline)) {
        const int key = t * pf::kKT + lane;
        copy4_to_lds(pt, 4u * (uint32_t)(key < nkeys ? key : 0), ids_wave + (t % pf::kIdSlots) * pf::kKT * 4);
    };
    const uint32_t last_slot = (uint32_t)(min(a.num_slots, (int64_t)1 << 31) - 1);
    const uint32_t row_bytes = (uint32_t)G * pf::kRow;
    // byte offset, within a pool row, of the chunk lane l loads for gather i (it writes chunk
    // position l%16 of its LDS row, so it loads the chunk the row permutation puts there)
    uint32_t lane_off[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
        lane_off[i] = (uint32_t)kvh * pf::kRow + (((lane & 15) ^ row_code(pfc::kRowsW * wave + 4 * i + grp)) << 4);
    // this wave's 4 ids of tile t (its rows' slots), read from the tile's id slot
    auto read_ids = [&](int t) __attribute__((always_inline)) {
        return *(const __attribute__((address_space(3))) u32x4_t *)(uintptr_t)(
            ids_wave + (t % pf::kIdSlots) * pf::kKT * 4 + (pfc::kRowsW * wave + 4 * grp) * 4);
    };
    // gathers of tile t into ring stage t % 2: this wave's 4 instructions
    auto gather = [&](int t, bool is_v, const u32x4_t ids) __attribute__((always_inline)) {
        const uint32_t base = lds0 + (t & 1) * pf::kTile + (is_v ? pfc::kVBase : pfc::kKBase) + pfc::kRowsW * wave * pf::kRow;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t s = min(ids[i], last_slot);  // a malformed id (negative or too large) reads the last slot
            if constexpr (O32)
                copy16_to_lds_at(is_v ? a.v_pool : a.k_pool, __umul24(s, row_bytes) + lane_off[i],
                                 base + 4 * i * pf::kRow);
            else
                copy16_to_lds(reinterpret_cast<const char *>(is_v ? a.v_pool : a.k_pool) +
                                  ((uint64_t)s * row_bytes + lane_off[i]),
                              base + 4 * i * pf::kRow);
        }
    };

    // prologue: ids of tiles 0..3, K of tiles 0 and 1, V of tile 0, then Q and a full wait; the
    // ids of the first tile's gathers (K of 2, V of 1) go to registers
#pragma unroll
    for (int t = 0; t < 4; ++t) copy_ids(t);
    wait_vmcnt<0>();
    {
        const u32x4_t id0 = read_ids(0);
        gather(0, false, id0);
        if (ntiles > 1) gather(1, false, read_ids(1));
        gather(0, true, id0);
    }
    u32x4_t kid = read_ids(2), vid = read_ids(1);
    // Q^T operands as in the single-block layout; the empty asm makes the
    // compiler wait for them here, and the explicit wait covers the copies
    bf16x8_t qv[8];
    const bf16_t *qp = reinterpret_cast<const bf16_t *>(a.q) +
                       ((int64_t)(row0 + tok) * a.q_heads + hq) * pf::kD + 8 * jj;
#pragma unroll
    for (int dc = 0; dc < 8; ++dc) qv[dc] = __builtin_bit_cast(bf16x8_t, ld16(qp + 16 * dc));
#pragma unroll
    for (int dc = 0; dc < 8; ++dc) asm volatile("" ::"v"(qv[dc]));
    wait_vmcnt<0>();

    // LDS read addresses of ring stage 0's first half, as in the single-block
    // layout (stages and halves are immediate offsets)
    uint32_t kaddr[8], vaddr[4][2];
    {
        const int kx = row_code(lane & 15) ^ jj;
        const int vrow = 4 * jj + ((lane >> 2) & 3);
        const int vch = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
#pragma unroll
        for (int dc = 0; dc < 8; ++dc) kaddr[dc] = lds0 + pfc::kKBase + (lane & 31) * pf::kRow + (((2 * dc) ^ kx) << 4);
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int par = 0; par < 2; ++par)
                vaddr[db][par] = lds0 + pfc::kVBase + vrow * pf::kRow +
                                 (((4 * db + vch) ^ row_code(vrow + 8 * par)) << 4) + (lane & 1) * 8;
    }

    floatx16_t acc[4];
#pragma unroll
    for (int db = 0; db < 4; ++db) acc[db] = floatx16_t{};
    float m;           // reference of the weights (log2 units)
    float lt = 0.0f;   // lane's share of the sum of the weights: the lse
    float lr = 0.0f;   // ... of the weights rounded to bf16, as P.V applies them: the normalisation
    floatx16_t sc;
    bf16x8_t pb[2];

    auto scores = [&](int stage, int half) __attribute__((always_inline)) {
        floatx16_t s = floatx16_t{};
#pragma unroll
        for (int dc = 0; dc < 8; ++dc)
            s = mfma_32x32x16(lds_read16(kaddr[dc] + stage * pf::kTile + half * 32 * pf::kRow), qv[dc], s);
        return s;
    };
    // element e of a unit's S^T tile is LDS row 8(e/4) + 4jj + e%4 of the unit, which holds the
    // unit's key 16(e/8) + 4(e%4) + 2((e/4)%2) + jj (see the gathers)
    auto mask = [&](floatx16_t &s, int u) __attribute__((always_inline)) {
        if (32 * u + 31 > pos0) {
            const int thr = pos - 32 * u - jj;  // element e is masked when its key offset exceeds this
#pragma unroll
            for (int e = 0; e < 16; ++e) s[e] = 16 * (e >> 3) + 4 * (e & 3) + 2 * ((e >> 2) & 1) > thr ? -INFINITY : s[e];
        }
    };
    auto column_max = [&](const floatx16_t &s) __attribute__((always_inline)) {
        float mx = fmaxf(fmaxf(s[0], s[1]), s[2]);  // a chain of three-input maxes
#pragma unroll
        for (int e = 3; e < 15; e += 2) mx = fmaxf(fmaxf(mx, s[e]), s[e + 1]);
        mx = fmaxf(mx, s[15]);
        return max_with_other_half(mx) * a.scale_log2;
    };
    auto weights = [&](const floatx16_t &s, float mu, bf16x8_t (&out)[2], float &sum, float &rsum)
                       __attribute__((always_inline)) {
        uint32_t pw[8];
        sum = 0.0f;
        rsum = 0.0f;
#pragma unroll
        for (int e = 0; e < 16; e += 2) {
            const float p0 = fast_exp2(fmaf(s[e], a.scale_log2, -mu));
            const float p1 = fast_exp2(fmaf(s[e + 1], a.scale_log2, -mu));
            pw[e >> 1] = pack_bf16x2(p0, p1);
            if constexpr (LSE) sum += p0 + p1;  // the unrounded sum serves only the lse
            rsum = dot2_bf16(pw[e >> 1], kBf16OnesPair, rsum);
        }
        out[0] = __builtin_bit_cast(bf16x8_t, make_uint4(pw[0], pw[1], pw[2], pw[3]));
        out[1] = __builtin_bit_cast(bf16x8_t, make_uint4(pw[4], pw[5], pw[6], pw[7]));
    };
    auto pv = [&](int stage, int half) __attribute__((always_inline)) {
#pragma unroll
        for (int db = 0; db < 4; ++db) {
            uint2 av[4];
#pragma unroll
            for (int qq = 0; qq < 4; ++qq)
                av[qq] = lds_read_tr16(vaddr[db][qq & 1] + stage * pf::kTile + half * 32 * pf::kRow +
                                       8 * qq * pf::kRow);
            acc[db] = mfma_32x32x16(__builtin_bit_cast(bf16x8_t, make_uint4(av[0].x, av[0].y, av[1].x, av[1].y)),
                                    pb[0], acc[db]);
            acc[db] = mfma_32x32x16(__builtin_bit_cast(bf16x8_t, make_uint4(av[2].x, av[2].y, av[3].x, av[3].y)),
                                    pb[1], acc[db]);
        }
    };
    // One unit: P.V of unit u (tile stage `stage`, half u%2), the scores of
    // unit u+2 (the same half of the next tile, stage `next`) and the softmax
    // of unit u+1 (its raw scores are in sc).
    auto unit = [&](int u, int stage, int next, bool has_scores, bool has_softmax) __attribute__((always_inline)) {
        const int half = u & 1;
        if (has_softmax) mask(sc, u + 1);
        floatx16_t s_new;
        pv(stage, half);
        if (has_scores) s_new = scores(next, half);
        float lt_u = 0.0f, lr_u = 0.0f;
        bf16x8_t pb_new[2];
        if (has_softmax) {
            weights(sc, m, pb_new, lt_u, lr_u);
            // keep the weights in this block (the compiler would otherwise sink
            // them past the rescale branch, away from the MFMAs they overlap)
            asm volatile("" ::"v"(pb_new[0]), "v"(pb_new[1]), "v"(lt_u), "v"(lr_u));
        }
        if (has_scores && has_softmax) interleave_unit<1, 4, 2, 8>();
        if (has_softmax && __any(!(lr_u <= kPrefillWeightBound))) {  // rare
            floatx16_t sr = sc;
            asm volatile("" : "+v"(sr));
            const float mn = fmaxf(m, column_max(sr));
            const float alpha = fast_exp2(m - mn);
            lt *= alpha;
            lr *= alpha;
#pragma unroll
            for (int db = 0; db < 4; ++db)
#pragma unroll
                for (int e = 0; e < 16; ++e) acc[db][e] *= alpha;
            m = mn;
            weights(sr, m, pb_new, lt_u, lr_u);
        }
        if (has_softmax) {
            lt += lt_u;
            lr += lr_u;
            pb[0] = pb_new[0];
            pb[1] = pb_new[1];
        }
        if (has_scores) sc = s_new;
    };
    // start of tile t: wait for this wave's copies, barrier; but at the last
    // tile, refill the ring stages tile t-1 used with K of t+2 and V of t+1
    // and copy the ids of t+3
    // (the ids of tile t+4 go to the slot tile t's ids held, last read a tile earlier; the ids of
    // the next tile's gathers are read into registers here, a tile before their use)
    auto tile_start = [&](int t) __attribute__((always_inline)) {
        wait_vmcnt<0>();
        lds_barrier();
        if (t < ntiles - 1) {
            if (t + 4 < ntiles) copy_ids(t + 4);
            if (t + 2 < ntiles) gather(t + 2, false, kid);
            gather(t + 1, true, vid);
            kid = read_ids(t + 3);
            vid = read_ids(t + 2);
        }
    };
    auto tile = [&](int t, int stage) __attribute__((always_inline)) {
        tile_start(t);
        const int next = stage ^ 1;
        unit(2 * t, stage, next, true, true);
        unit(2 * t + 1, stage, next, true, true);
    };

    lds_barrier();
    if (tw >= 0) {  // scores of units 0 and 1, the first unit's weights against its exact column max
        floatx16_t s0 = scores(0, 0);
        sc = scores(0, 1);
        mask(s0, 0);
        m = column_max(s0);  // key 0 is visible to every column: finite
        weights(s0, m, pb, lt, lr);
    }
    // tiles before this wave's last, its last tile, then the block's remaining tiles
    int t = 0;
    for (; t + 2 <= tw; t += 2) {
        tile(t, 0);
        tile(t + 1, 1);
    }
    if (t < tw) {
        tile(t, 0);
        ++t;
    }
    if (tw >= 0) {  // this wave's last tile (V of it was copied in the tile before)
        tile_start(t);
        // its second half lies past every key of this wave: no softmax and no P.V for it
        const bool half = (wlast & (pf::kKT - 1)) < pf::kKT / 2;
        if (t & 1) {
            unit(2 * t, 1, 0, false, !half);
            if (!half) unit(2 * t + 1, 1, 0, false, false);
        } else {
            unit(2 * t, 0, 1, false, !half);
            if (!half) unit(2 * t + 1, 0, 1, false, false);
        }
        ++t;
    }
    for (; t < ntiles; ++t) tile_start(t);

    // normalised by the sum of the weights P.V applied (V = 1 gives 1 exactly);
    // lse from the sum of the unrounded weights
    if constexpr (LSE) lt = add_with_other_half(lt);
    lr = add_with_other_half(lr);
    if constexpr (SH) {
        if (valid) {
            const float inv = 1.0f / lr;
            const int64_t r = ((int64_t)split * a.total_q + row0 + tl) * a.q_heads + hq;
            float *op = a.part_o + r * pf::kD;
#pragma unroll
            for (int db = 0; db < 4; ++db)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    *reinterpret_cast<float4 *>(op + db * 32 + 8 * i + 4 * jj) =
                        make_float4(acc[db][4 * i] * inv, acc[db][4 * i + 1] * inv, acc[db][4 * i + 2] * inv,
                                    acc[db][4 * i + 3] * inv);
            if (jj == 0) a.part_lse[r] = (m + __log2f(lt)) * kLn2;
        }
        return;
    }
    if (valid) {
        const float inv = 1.0f / lr;
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
        if constexpr (LSE)
            if (a.lse != nullptr && jj == 0) a.lse[(int64_t)(row0 + tl) * a.q_heads + hq] = (m + __log2f(lt)) * kLn2;
    }
}

namespace {

// Query blocks (times the kv heads) of a layout with BQ query tokens per block:
// a bound on the sum over requests of ceil(E_b / BQ) from total_q alone (ids
// past the real count exit at once), so that no caller-given length can
// leave query rows without a block.
int64_t prefill_blocks(const PrefillArgs &a, int BQ) {
    return ((int64_t)a.total_q + (int64_t)a.batch * (BQ - 1)) / BQ * a.kv_heads;
}

// Gathers may address pool rows as 32-bit byte offsets from the pool base
// when every row lies within 4 GiB of it and slot ids fit 24 bits (the
// offset is a 24-bit multiply).
bool prefill_o32(const PrefillArgs &a) {
    const uint64_t row_bytes = (uint64_t)a.kv_heads * pf::kRow;
    return a.num_slots <= ((int64_t)1 << 24) && (uint64_t)a.num_slots * row_bytes <= ((uint64_t)1 << 32);
}

// The single-block layout, with the unrounded weight sums only when an lse is asked for.
template <int GQ, bool PL>
void launch_long(const PrefillArgs &a, int64_t grid, hipStream_t stream) {
    if (a.lse != nullptr)
        hipLaunchKernelGGL((prefill_mfma_long_kernel<GQ, PL, true>), dim3((unsigned)grid), dim3(pfl::kThreads), 0,
                           stream, a);
    else
        hipLaunchKernelGGL((prefill_mfma_long_kernel<GQ, PL, false>), dim3((unsigned)grid), dim3(pfl::kThreads), 0,
                           stream, a);
}

// The two-blocks-per-CU kernel with the gather addressing the pool allows, and
// the unrounded weight sums only when an lse is asked for (the shared-prefix
// mode always writes one).
template <int GQ, bool SH, bool PL>
void launch_small(const PrefillArgs &a, int64_t grid, hipStream_t stream) {
    const dim3 g((unsigned)grid), t(pfc::kThreads);
    const bool o32 = prefill_o32(a);
    if (SH || a.lse != nullptr) {
        if (o32) hipLaunchKernelGGL((prefill_mfma_kernel<GQ, SH, PL, true, true>), g, t, 0, stream, a);
        else hipLaunchKernelGGL((prefill_mfma_kernel<GQ, SH, PL, false, true>), g, t, 0, stream, a);
    } else if constexpr (!SH) {
        if (o32) hipLaunchKernelGGL((prefill_mfma_kernel<GQ, SH, PL, true, false>), g, t, 0, stream, a);
        else hipLaunchKernelGGL((prefill_mfma_kernel<GQ, SH, PL, false, false>), g, t, 0, stream, a);
    }
}

template <int GQ>
hipError_t run_prefill_mfma(const PrefillArgs &a, hipStream_t stream) {
    int BQ = 0;
    const bool long_chunks = prefill_layout(a.batch, a.total_q, GQ, &BQ) == 1;
    const int64_t grid = prefill_blocks(a, BQ);
    if (grid < 1) return hipSuccess;
    if (grid > 0x7fffffff) return hipErrorInvalidValue;
    if (long_chunks)
        launch_long<GQ, false>(a, grid, stream);
    else
        launch_small<GQ, false, false>(a, grid, stream);
    return hipGetLastError();
}

template <int GQ>
hipError_t run_prefill_planned(const PrefillArgs &a, int layout, int entries, hipStream_t stream) {
    const int64_t grid = (int64_t)entries * a.kv_heads;
    if (grid < 1) return hipSuccess;
    if (grid > 0x7fffffff) return hipErrorInvalidValue;
    if (layout == 1)
        launch_long<GQ, true>(a, grid, stream);
    else
        launch_small<GQ, false, true>(a, grid, stream);
    return hipGetLastError();
}

}  // namespace

// Requests of 2048 or more new tokens on average: long, uniform blocks, where
// the single-block layout's deeper ring keeps the matrix cores busier;
// otherwise block starts and the spread of block lengths weigh more, and two
// blocks per CU hide them.
int prefill_layout(int64_t batch, int64_t total_q, int group, int *bq) {
    const bool long_chunks = total_q >= 2048 * batch;
    if (bq != nullptr) *bq = (long_chunks ? pfl::kCols : pfc::kCols) / (group > 0 ? group : 1);
    return long_chunks ? 1 : 0;
}

int prefill_small_bq(int group) { return pfc::kCols / (group > 0 ? group : 1); }

hipError_t launch_prefill_planned(const PrefillArgs &a, int layout, int entries, hipStream_t stream) {
    if (a.plan == nullptr || (layout != 0 && layout != 1) || entries < 0) return hipErrorInvalidValue;
    switch (a.q_heads / a.kv_heads) {
        case 1: return run_prefill_planned<1>(a, layout, entries, stream);
        case 2: return run_prefill_planned<2>(a, layout, entries, stream);
        case 4: return run_prefill_planned<4>(a, layout, entries, stream);
        case 8: return run_prefill_planned<8>(a, layout, entries, stream);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_prefill_shared(const PrefillArgs &a, hipStream_t stream) {
    if (a.batch > pf::kMaxBatch || a.splits < 1) return hipErrorInvalidValue;
    const int g = a.q_heads / a.kv_heads;
    const int BQ = pfc::kCols / g;
    const int64_t grid = prefill_blocks(a, BQ) * a.splits;
    if (grid < 1) return hipSuccess;
    if (grid > 0x7fffffff) return hipErrorInvalidValue;
    switch (g) {
        case 1: launch_small<1, true, false>(a, grid, stream); break;
        case 2: launch_small<2, true, false>(a, grid, stream); break;
        case 4: launch_small<4, true, false>(a, grid, stream); break;
        case 8: launch_small<8, true, false>(a, grid, stream); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_prefill(const PrefillArgs &a, DType dtype, int head_dim, hipStream_t stream) {
    if (dtype == kBF16 && head_dim == pf::kD && a.batch <= pf::kMaxBatch) {
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
