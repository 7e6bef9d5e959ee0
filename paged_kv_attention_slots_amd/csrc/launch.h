// Host-side launchers of the msgl kernels (internal; the C ABI is include/msgl.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace msgl {

enum DType { kF32 = 0, kBF16 = 1 };

constexpr float kLog2eHost = 1.4426950408889634f;

// Minimum keys per decode block (the `chunk` argument) when the caller passes 0.
constexpr int kDefaultChunk = 64;
// Bytes of the decode workspace's control block.
constexpr size_t kCtrlBytes = 256;
// Work units a decode request costs beyond its keys (the split's fixed cost per piece).
constexpr int kPieceUnits = 32;
// Upper bound of the decode grid (it sizes the workspace's partial states).
constexpr int kMaxDecodeGrid = 4096;

inline size_t decode_prefix_bytes(int batch) { return ((size_t)(batch + 1) * 4 + 255) / 256 * 256; }
inline size_t align256(size_t n) { return (n + 255) / 256 * 256; }

// Key splits of the shared-prefix pass (upper bound; sizes the workspace).
constexpr int kMaxPrefixSplits = 16;

struct StoreKvArgs {
    void *k_pool;
    void *v_pool;
    const void *k_new;
    const void *v_new;
    const int32_t *out_loc;
    int32_t num_tokens;
    int32_t row_vec16;  // 16-byte vectors per [kv_heads, head_dim] row
    int64_t num_slots;  // rows with an out_loc outside [0, num_slots) are skipped
};

struct RopeStoreKvArgs {
    void *q_out;       // [num_tokens, q_heads, head_dim]; may equal q
    const void *q;
    void *k_pool;
    void *v_pool;
    const void *k_new;
    const void *v_new;
    const int32_t *positions;
    const int32_t *out_loc;
    int64_t num_slots;  // rows with an out_loc outside [0, num_slots) are not written
    int32_t num_tokens;
    int32_t q_heads;
    int32_t kv_heads;
    int32_t head_dim;
    double base;        // rotary base (theta)
};

struct VocabEmbedArgs {
    void *out;            // [num_tokens, row_vec * 16 bytes]
    const void *weight;   // [rows, row_vec * 16 bytes]
    const int32_t *ids;   // [num_tokens]
    int64_t vocab_start;  // vocabulary id of weight's row 0
    int64_t rows;
    int32_t row_vec;      // 16-byte vectors per row
    int32_t num_tokens;
};

struct DecodeArgs {
    void *out;
    float *lse;
    const void *q;
    const void *k_pool;
    const void *v_pool;
    const int32_t *page_table;
    int64_t row_stride;
    const int32_t *table_idx;
    const int32_t *seq_lens;
    int64_t num_slots;  // slot ids outside [0, num_slots) read slot 0 instead
    int32_t batch;
    int32_t q_heads;
    int32_t kv_heads;
    int32_t chunk;        // minimum keys per block
    int32_t wpb;          // waves (kv heads) per decode block
    int32_t max_seq_len;  // lengths are cut at min(max_seq_len, row_stride)
    float scale_log2;     // sm_scale * log2(e)
    int64_t *ctrl;        // [2] total keys, keys per block (written by the split kernel)
    int32_t *prefix;      // [batch + 1] keys before each request (written by the split kernel)
    float *part_o;        // [batch + kMaxDecodeGrid, q_heads, head_dim]
    float *part_ml;       // [batch + kMaxDecodeGrid, q_heads, 2]  (max in log2 units, sum)
    const int32_t *key_start;  // nullable: request b attends keys key_start[b] .. seq_lens[b]-1
    int32_t out_f32;      // nonzero: out is float32 whatever the storage type
    // nonzero: the split kernel also writes request b's new K/V row (k_new[b],
    // v_new[b]) to slot out_loc[b] of k_pool_w / v_pool_w (the same pools as
    // k_pool / v_pool) before it reads that request's last key
    int32_t fuse_store;
    void *k_pool_w;
    void *v_pool_w;
    const void *k_new;
    const void *v_new;
    const int32_t *out_loc;
};

struct PrefillArgs {
    void *out;
    float *lse;
    const void *q;
    const void *k_pool;
    const void *v_pool;
    const int32_t *page_table;
    int64_t row_stride;
    const int32_t *table_idx;
    const int32_t *seq_lens;
    const int32_t *cached_lens;
    const int32_t *cu_q;
    int64_t num_slots;  // slot ids outside [0, num_slots) read an in-pool slot (the last one on the MFMA path)
    int32_t batch;
    int32_t total_q;
    int32_t max_extend;
    int32_t q_heads;
    int32_t kv_heads;
    float scale_log2;
    // shared-prefix mode only (prefill_mfma_kernel<GQ, true>): key splits per
    // query block, and the partial outputs [splits, total_q, q_heads, head_dim]
    // and lse [splits, total_q, q_heads] (float32, natural log)
    int32_t splits;
    float *part_o;
    float *part_lse;
    // planned launches only: the host plan's block list (kPlanEntryInts int32
    // per entry, device memory) and its entry count; null / 0 otherwise
    const int32_t *plan;
    int32_t plan_entries;
};

// Host plan of a prefill launch: a header of kPlanHeaderInts int32, then one
// entry of kPlanEntryInts int32 per query block, in launch order.
constexpr int32_t kPlanMagic = 0x4d504c31;  // "MPL1"
constexpr int kPlanHeaderInts = 8;           // magic, layout, query tokens per block, entries, batch, total_q, q_heads, kv_heads
constexpr int kPlanKeyTile = 64;            // keys per tile of the MFMA kernels (orders the entries)
constexpr int kPlanEntryInts = 8;            // request, query block, new tokens, cached tokens, first q row, table row, key tiles, 0
// Layout of the bf16 MFMA prefill kernels for a batch: 1 = the single-block
// long-chunk layout, 0 = two blocks per CU; *bq receives its query tokens per
// block for q_heads / kv_heads = group.
int prefill_layout(int64_t batch, int64_t total_q, int group, int *bq);
// Query tokens per block of the two-blocks-per-CU layout (the smaller one).
int prefill_small_bq(int group);
hipError_t launch_prefill_planned(const PrefillArgs &a, int layout, int entries, hipStream_t stream);

size_t decode_workspace_bytes(int batch, int q_heads, int head_dim, int max_seq_len, int chunk);

// Cascade decode over shared radix prefixes (bf16, head_dim 128).
struct SharedPrefixArgs {
    const int32_t *group_start;  // [num_groups + 1] batch rows of each group
    const int32_t *prefix_lens;  // [batch] shared prefix length of each request's group
    int32_t num_groups;
    int32_t max_group_size;
    int32_t max_prefix_len;
    int32_t cus;                 // compute units of the device (sizes the key split)
    void *workspace;             // shared_prefix_workspace_bytes(...)
};
size_t shared_prefix_workspace_bytes(int batch, int q_heads, int head_dim, int max_seq_len, int chunk);
int prefix_splits(int num_groups, int max_group_size, int max_prefix_len, int q_heads, int kv_heads, int cus);
// dec: the decode arguments of the whole batch (out = the bf16 output, lse,
// workspace = the start of the shared-prefix workspace); prepare_only as for
// launch_decode.
hipError_t launch_decode_shared_prefix(const SharedPrefixArgs &sp, const DecodeArgs &dec, int head_dim,
                                       hipStream_t stream, bool prepare_only = false);
int device_cu_count();

hipError_t launch_store_kv(const StoreKvArgs &a, hipStream_t stream);
hipError_t launch_rope_store_kv(const RopeStoreKvArgs &a, DType dtype, hipStream_t stream);
hipError_t launch_vocab_embed(const VocabEmbedArgs &a, hipStream_t stream);
// prepare_only resolves the cached device queries and launches nothing (call
// it before capturing the launch into a graph); split_only launches the split
// kernel alone, leaving the pieces of requests cut across blocks in the
// workspace for a merge of the caller's (the cascade's).
hipError_t launch_decode(const DecodeArgs &a, DType dtype, int head_dim, hipStream_t stream,
                         bool prepare_only = false, bool split_only = false);
// Kv heads per decode block.
int decode_waves(int kv_heads);
// bf16 prefill on matrix cores when the shape is supported, else the VALU path.
hipError_t launch_prefill(const PrefillArgs &a, DType dtype, int head_dim, hipStream_t stream);
hipError_t launch_prefill_valu(const PrefillArgs &a, DType dtype, int head_dim, hipStream_t stream);
// Shared-prefix pass of the cascade decode: bf16, head_dim 128 (a.splits,
// a.part_o and a.part_lse set; a.batch = groups, a.cu_q = group offsets).
hipError_t launch_prefill_shared(const PrefillArgs &a, hipStream_t stream);

}  // namespace msgl
