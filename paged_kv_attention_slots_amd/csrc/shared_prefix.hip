// Cascade decode over a shared radix prefix.
//
// The radix prefix cache of the Stage 4 milestone's engine lets requests
// share the KV of a common prefix: their page-table rows hold the same slot
// ids for its first P tokens.  Decode attention over such a group is split in
// two by key range, as the log-sum-exp rule allows for any partition of the
// keys:
//   1. prefix pass: the group's queries against the shared keys 0 .. P-1,
//      read once for the whole group.  This is a matrix product (many query
//      columns against the same keys), so it runs on the prefill MFMA kernel in
//      its shared-prefix mode, split along the keys into `splits` ranges to
//      fill the GPU; each range leaves a normalised float32 partial output and
//      its lse;
//   2. suffix pass: each request against its own keys P .. seq_len-1, on the
//      split-K decode kernel (a per-request key start): float32 output + lse
//      where one block covers the request's own keys, else the pieces'
//      unnormalised states, left for step 3 (no decode merge runs);
//   3. merge: out = sum_i w_i o_i / sum_i w_i with w_i = exp(lse_i - max lse)
//      over the prefix splits and the suffix (or its pieces), lse = max +
//      log(sum_i w_i), rounded once to bf16.
// The result is the ordinary decode attention; only the number of times the
// prefix's K/V rows are read changes (once per group instead of once per
// request).
#include <math.h>

#include "common.h"
#include "launch.h"

namespace msgl {

struct CascadeMergeArgs {
    bf16_t *out;                // [batch, q_heads, D]
    float *lse;                 // nullable [batch, q_heads]
    const float *suffix_o;      // [batch, q_heads, D]
    const float *suffix_lse;    // [batch, q_heads]
    const float *prefix_o;      // [splits, batch, q_heads, D]
    const float *prefix_lse;    // [splits, batch, q_heads]; -inf marks an empty split
    const int32_t *prefix_lens; // [batch]; 0: no shared prefix (the suffix is the whole result)
    int32_t batch;
    int32_t q_heads;
    int32_t splits;             // 0 when the prefix pass did not run
    // the suffix pass's split kernel: a request whose own keys were cut across
    // blocks left its pieces' unnormalised states here instead of an output
    const int64_t *ctrl;        // [2] total work units, units per block
    const int32_t *prefix;      // [batch + 1] work units before each request
    const float *part_o;        // [batch + grid, q_heads, D] unnormalised outputs
    const float *part_ml;       // [batch + grid, q_heads, 2] (max in log2 units, sum)
    int32_t group;              // q heads per kv head
    int32_t wpb;                // kv heads per decode block
};

namespace {

MSGL_DEV float lanes_max(float x) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x = fmaxf(x, __shfl_xor(x, off));
    return x;
}

MSGL_DEV float lanes_sum(float x) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off);
    return x;
}

}  // namespace

// One wave per (request, q head); each lane owns D / 64 elements.  Lane s
// reads split s's lse, so the weights take one round trip; the splits' partial
// outputs are then read with every split's loads in flight at once (the loop
// over kMaxPrefixSplits is unrolled).  An empty split (lse = -inf) was never
// written and is skipped.  The suffix is either the split kernel's normalised
// output and lse, or, for a request whose own keys were cut across decode
// blocks, its pieces' unnormalised states (the decode merge's inputs), which
// enter the same log-sum-exp sum directly: no separate decode merge runs.
template <int D>
__global__ __launch_bounds__(256) void cascade_merge_kernel(CascadeMergeArgs a) {
    constexpr int PER = D / 64;
    static_assert(kMaxPrefixSplits <= 64, "one lane per split");
    const int b = blockIdx.x;
    const int h = blockIdx.y * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (h >= a.q_heads) return;
    const int64_t bh = (int64_t)b * a.q_heads + h;
    const int S = a.prefix_lens[b] > 0 ? min(a.splits, kMaxPrefixSplits) : 0;
    const int64_t sstride = (int64_t)a.batch * a.q_heads;
    // the suffix's pieces: n > 1 when the split kernel cut this request's own keys across blocks
    const int W = a.prefix[b + 1] - a.prefix[b];
    const int L = W - kPieceUnits;
    int n = 1;
    int64_t i0 = 0;
    if (L > 1) {
        const int64_t total = a.ctrl[0], share = a.ctrl[1];
        const int hg = (h / a.group) / a.wpb;
        const int64_t first_tok = (int64_t)hg * total + a.prefix[b] + kPieceUnits;
        const int first = (int)(first_tok / share);
        n = (int)((first_tok + L - 1) / share) - first + 1;
        i0 = ((int64_t)b + first) * a.q_heads + h;  // piece k at (i0 + k q_heads)
    }
    // reference: the largest lse of the splits, the suffix or its pieces (natural log)
    const float x = lane < S ? a.prefix_lse[lane * sstride + bh] : -INFINITY;
    float m = x;
    const float xs = n == 1 ? a.suffix_lse[bh] : -INFINITY;
    for (int k = lane; n > 1 && k < n; k += 64) {
        const float2 v = *reinterpret_cast<const float2 *>(a.part_ml + (i0 + (int64_t)k * a.q_heads) * 2);
        m = fmaxf(m, (v.x + __log2f(v.y)) * kLn2);
    }
    m = fmaxf(lanes_max(m), xs);
    const float wx = x == -INFINITY ? 0.0f : expf(x - m);
    const float ws = n == 1 ? expf(xs - m) : 0.0f;
    const uint64_t live = __ballot(x != -INFINITY);
    float l = wx;
    float acc[PER];
#pragma unroll
    for (int e = 0; e < PER; ++e) acc[e] = n == 1 ? ws * a.suffix_o[bh * D + lane * PER + e] : 0.0f;
#pragma unroll
    for (int s = 0; s < kMaxPrefixSplits; ++s) {
        const float w = __shfl(wx, s);
        if ((live >> s) & 1) {
            const float *po = a.prefix_o + (s * sstride + bh) * D + lane * PER;
#pragma unroll
            for (int e = 0; e < PER; ++e) acc[e] = fmaf(w, po[e], acc[e]);
        }
    }
    // a piece k weighs 2^(m_k - m log2 e) on its unnormalised output and its sum
    const float m2 = m * kLog2e;
    for (int c0 = 0; n > 1 && c0 < n; c0 += 64) {
        const int k = c0 + lane;
        float wk = 0.0f;
        if (k < n) {
            const float2 v = *reinterpret_cast<const float2 *>(a.part_ml + (i0 + (int64_t)k * a.q_heads) * 2);
            wk = fast_exp2(v.x - m2);
            l = fmaf(wk, v.y, l);
        }
        const int cn = min(64, n - c0);
        for (int t = 0; t < cn; ++t) {
            const float w = __shfl(wk, t);
            const float *po = a.part_o + (i0 + (int64_t)(c0 + t) * a.q_heads) * D + lane * PER;
#pragma unroll
            for (int e = 0; e < PER; ++e) acc[e] = fmaf(w, po[e], acc[e]);
        }
    }
    l = lanes_sum(l) + ws;
    const float inv = 1.0f / l;
    bf16_t *op = a.out + bh * D + lane * PER;
    if constexpr (PER == 2) {
        *reinterpret_cast<uint32_t *>(op) = pack_bf16x2(acc[0] * inv, acc[1] * inv);
    } else {
#pragma unroll
        for (int e = 0; e < PER; ++e) op[e] = (bf16_t)f32_to_bf16_bits(acc[e] * inv);
    }
    if (a.lse != nullptr && lane == 0) a.lse[bh] = m + logf(l);
}

size_t shared_prefix_workspace_bytes(int batch, int q_heads, int head_dim, int max_seq_len, int chunk) {
    const size_t rows = (size_t)batch * q_heads;
    const size_t per_split = rows * ((size_t)head_dim + 1) * sizeof(float);
    return align256(decode_workspace_bytes(batch, q_heads, head_dim, max_seq_len, chunk)) +
           align256(per_split) * (1 + kMaxPrefixSplits);
}

int prefix_splits(int num_groups, int max_group_size, int max_prefix_len, int q_heads, int kv_heads, int cus) {
    const int bq = 128 / (q_heads / kv_heads);  // query columns of one prefill block / group size
    const int64_t blocks = (int64_t)num_groups * ((max_group_size + bq - 1) / bq) * kv_heads;
    int64_t s = (2 * (int64_t)cus + blocks - 1) / (blocks > 0 ? blocks : 1);  // about two blocks per CU
    const int64_t by_len = (max_prefix_len + 255) / 256;                       // at least 4 key tiles each
    s = s < by_len ? s : by_len;
    s = s < kMaxPrefixSplits ? s : kMaxPrefixSplits;
    return (int)(s < 1 ? 1 : s);
}

hipError_t launch_decode_shared_prefix(const SharedPrefixArgs &sp, const DecodeArgs &dec_in, int head_dim,
                                       hipStream_t stream, bool prepare_only) {
    if (head_dim != 128) return hipErrorInvalidValue;
    char *ws = static_cast<char *>(sp.workspace);
    const size_t rows = (size_t)dec_in.batch * dec_in.q_heads;
    const size_t per_split = align256(rows * ((size_t)head_dim + 1) * sizeof(float));
    char *extra = ws + align256(decode_workspace_bytes(dec_in.batch, dec_in.q_heads, head_dim, dec_in.max_seq_len,
                                                       dec_in.chunk));
    float *suffix_o = reinterpret_cast<float *>(extra);
    float *suffix_lse = suffix_o + rows * head_dim;
    float *prefix_o = reinterpret_cast<float *>(extra + per_split);
    float *prefix_lse = prefix_o + (size_t)kMaxPrefixSplits * rows * head_dim;

    DecodeArgs dec = dec_in;
    dec.out = suffix_o;
    dec.lse = suffix_lse;
    dec.key_start = sp.prefix_lens;
    dec.out_f32 = 1;
    if (prepare_only) return launch_decode(dec, kBF16, head_dim, stream, true);

    int splits = 0;
    if (sp.num_groups > 0 && sp.max_prefix_len > 0) {
        splits = prefix_splits(sp.num_groups, sp.max_group_size, sp.max_prefix_len, dec.q_heads, dec.kv_heads,
                               sp.cus);
        PrefillArgs p;
        p.out = nullptr;
        p.lse = nullptr;
        p.q = dec.q;
        p.k_pool = dec.k_pool;
        p.v_pool = dec.v_pool;
        p.page_table = dec.page_table;
        p.row_stride = dec.row_stride;
        p.table_idx = dec.table_idx;
        p.seq_lens = dec.seq_lens;
        p.cached_lens = sp.prefix_lens;
        p.cu_q = sp.group_start;
        p.num_slots = dec.num_slots;
        p.batch = sp.num_groups;
        p.total_q = dec.batch;
        p.max_extend = sp.max_group_size;
        p.q_heads = dec.q_heads;
        p.kv_heads = dec.kv_heads;
        p.scale_log2 = dec.scale_log2;
        p.splits = splits;
        p.part_o = prefix_o;
        p.part_lse = prefix_lse;
        p.plan = nullptr;
        hipError_t e = launch_prefill_shared(p, stream);
        if (e != hipSuccess) return e;
    }
    hipError_t e = launch_decode(dec, kBF16, head_dim, stream, false, true);
    if (e != hipSuccess) return e;
    CascadeMergeArgs m;
    m.out = static_cast<bf16_t *>(dec_in.out);
    m.lse = dec_in.lse;
    m.suffix_o = suffix_o;
    m.suffix_lse = suffix_lse;
    m.prefix_o = prefix_o;
    m.prefix_lse = prefix_lse;
    m.prefix_lens = sp.prefix_lens;
    m.batch = dec.batch;
    m.q_heads = dec.q_heads;
    m.splits = splits;
    m.ctrl = dec.ctrl;
    m.prefix = dec.prefix;
    m.part_o = dec.part_o;
    m.part_ml = dec.part_ml;
    m.group = dec.q_heads / dec.kv_heads;
    m.wpb = decode_waves(dec.kv_heads);
    hipLaunchKernelGGL(cascade_merge_kernel<128>, dim3(dec.batch, (dec.q_heads + 3) / 4), dim3(256), 0, stream, m);
    return hipGetLastError();
}

}  // namespace msgl
