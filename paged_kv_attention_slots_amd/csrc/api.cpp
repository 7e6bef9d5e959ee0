// C ABI of libmsgl (declared in include/msgl.h): argument checks, dispatch to
// the kernel launchers, decode-step graph capture, the host-side batch
// validators and the prefill launch's host plan.  Nothing here allocates
// device memory or synchronises.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "../../include/msgl.h"
#include "launch.h"
#include "check_batch.h"

namespace {

thread_local std::string g_err;

msgl_status fail(msgl_status s, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return s;
}

msgl_status ok() { return MSGL_OK; }

msgl_status from_hip(hipError_t e, const char *what) {
    if (e == hipSuccess) return ok();
    return fail(MSGL_HIP_ERROR, "%s: %s", what, hipGetErrorString(e));
}

int elem_bytes(msgl_dtype d) { return d == MSGL_F32 ? 4 : 2; }

msgl_status check_common(msgl_dtype dtype, int32_t head_dim, int32_t kv_heads, int64_t num_slots) {
    if (dtype != MSGL_F32 && dtype != MSGL_BF16) return fail(MSGL_UNSUPPORTED, "dtype %d not supported", (int)dtype);
    if (head_dim != 64 && head_dim != 128) return fail(MSGL_UNSUPPORTED, "head_dim %d not supported (64 or 128)", head_dim);
    if (kv_heads < 1 || kv_heads > 64) return fail(kv_heads < 1 ? MSGL_INVALID_ARG : MSGL_UNSUPPORTED, "kv_heads %d out of range [1, 64]", kv_heads);
    if (num_slots < 1) return fail(MSGL_INVALID_ARG, "num_slots %lld < 1", (long long)num_slots);
    return ok();
}

msgl_status check_group(int32_t q_heads, int32_t kv_heads) {
    if (q_heads < 1 || q_heads % kv_heads != 0)
        return fail(MSGL_INVALID_ARG, "q_heads %d is not a multiple of kv_heads %d", q_heads, kv_heads);
    const int g = q_heads / kv_heads;
    if (g != 1 && g != 2 && g != 4 && g != 8)
        return fail(MSGL_UNSUPPORTED, "group size q_heads/kv_heads = %d not in {1, 2, 4, 8}", g);
    return ok();
}

constexpr int32_t kMaxDecodeBatch = 8192;

int32_t effective_chunk(int32_t chunk) { return chunk == 0 ? msgl::kDefaultChunk : chunk; }

// Checks of a decode call's scalars and pointers, all but the workspace.
msgl_status check_decode_args(const void *out, const void *q, const void *k_pool, const void *v_pool,
                              int64_t num_slots, const int32_t *page_table, int32_t row_stride,
                              const int32_t *table_idx, const int32_t *seq_lens, int32_t batch,
                              int32_t q_heads, int32_t kv_heads, int32_t head_dim, int32_t page_size,
                              int32_t max_seq_len, int32_t chunk, msgl_dtype dtype) {
    msgl_status s = check_common(dtype, head_dim, kv_heads, num_slots);
    if (s != MSGL_OK) return s;
    if ((s = check_group(q_heads, kv_heads)) != MSGL_OK) return s;
    if (batch < 0 || batch > kMaxDecodeBatch)
        return fail(batch < 0 ? MSGL_INVALID_ARG : MSGL_UNSUPPORTED, "batch %d out of range [0, %d]", batch, kMaxDecodeBatch);
    if (batch > 0 && (!out || !q || !k_pool || !v_pool || !page_table || !table_idx || !seq_lens))
        return fail(MSGL_INVALID_ARG, "NULL pointer argument");
    if (row_stride < 1) return fail(MSGL_INVALID_ARG, "row_stride %d < 1", row_stride);
    if (max_seq_len < 1 || max_seq_len > row_stride)
        return fail(MSGL_INVALID_ARG, "max_seq_len %d not in [1, row_stride=%d]", max_seq_len, row_stride);
    if (page_size < 1) return fail(MSGL_INVALID_ARG, "page_size %d < 1", page_size);
    // the split's running count of work units (keys + 32 per request) is int32
    if ((int64_t)batch * ((int64_t)max_seq_len + 32) >= ((int64_t)1 << 31))
        return fail(MSGL_UNSUPPORTED, "batch %d x (max_seq_len %d + 32) work units reach 2^31", batch, max_seq_len);
    const int32_t c = effective_chunk(chunk);
    if (c < 64 || c % 64 != 0) return fail(MSGL_INVALID_ARG, "chunk %d is not a positive multiple of 64", chunk);
    return ok();
}

msgl_status check_decode(const void *out, const void *q, const void *k_pool, const void *v_pool,
                         int64_t num_slots, const int32_t *page_table, int32_t row_stride,
                         const int32_t *table_idx, const int32_t *seq_lens, int32_t batch,
                         int32_t q_heads, int32_t kv_heads, int32_t head_dim, int32_t page_size,
                         int32_t max_seq_len, int32_t chunk, msgl_dtype dtype, const void *workspace,
                         size_t workspace_bytes) {
    msgl_status s = check_decode_args(out, q, k_pool, v_pool, num_slots, page_table, row_stride, table_idx,
                                      seq_lens, batch, q_heads, kv_heads, head_dim, page_size, max_seq_len,
                                      chunk, dtype);
    if (s != MSGL_OK) return s;
    if (batch > 0 && !workspace) return fail(MSGL_INVALID_ARG, "NULL pointer argument");
    const size_t need = msgl::decode_workspace_bytes(batch, q_heads, head_dim, max_seq_len, effective_chunk(chunk));
    if (workspace_bytes < need)
        return fail(MSGL_WORKSPACE_TOO_SMALL, "workspace %zu bytes < %zu required", workspace_bytes, need);
    return ok();
}

msgl::DecodeArgs decode_args(void *out, float *lse, const void *q, const void *k_pool,
                             const void *v_pool, int64_t num_slots, const int32_t *page_table,
                             int32_t row_stride,
                             const int32_t *table_idx, const int32_t *seq_lens, int32_t batch,
                             int32_t q_heads, int32_t kv_heads, int32_t head_dim,
                             int32_t max_seq_len, int32_t chunk, float sm_scale, void *workspace) {
    msgl::DecodeArgs a;
    const int32_t c = effective_chunk(chunk);
    a.out = out;
    a.lse = lse;
    a.q = q;
    a.k_pool = k_pool;
    a.v_pool = v_pool;
    a.page_table = page_table;
    a.row_stride = row_stride;
    a.table_idx = table_idx;
    a.seq_lens = seq_lens;
    a.num_slots = num_slots;
    a.batch = batch;
    a.q_heads = q_heads;
    a.kv_heads = kv_heads;
    a.chunk = c;
    a.max_seq_len = max_seq_len;
    a.scale_log2 = sm_scale * msgl::kLog2eHost;
    char *ws = static_cast<char *>(workspace);
    a.ctrl = reinterpret_cast<int64_t *>(ws);
    a.prefix = reinterpret_cast<int32_t *>(ws + msgl::kCtrlBytes);
    const size_t pieces = (size_t)batch + msgl::kMaxDecodeGrid;
    a.part_o = reinterpret_cast<float *>(ws + msgl::kCtrlBytes + msgl::decode_prefix_bytes(batch));
    a.part_ml = a.part_o + pieces * q_heads * head_dim;
    a.key_start = nullptr;
    a.out_f32 = 0;
    a.fuse_store = 0;
    a.k_pool_w = nullptr;
    a.v_pool_w = nullptr;
    a.k_new = nullptr;
    a.v_new = nullptr;
    a.out_loc = nullptr;
    return a;
}

msgl_status check_store(void *k_pool, void *v_pool, int64_t num_slots, int32_t kv_heads,
                        int32_t head_dim, msgl_dtype dtype, const void *k_new, const void *v_new,
                        const int32_t *out_loc, int32_t num_tokens) {
    msgl_status s = check_common(dtype, head_dim, kv_heads, num_slots);
    if (s != MSGL_OK) return s;
    if (num_tokens < 0) return fail(MSGL_INVALID_ARG, "num_tokens %d < 0", num_tokens);
    if (num_tokens > 0 && (!k_pool || !v_pool || !k_new || !v_new || !out_loc))
        return fail(MSGL_INVALID_ARG, "NULL pointer argument");
    return ok();
}

msgl::StoreKvArgs store_args(void *k_pool, void *v_pool, int64_t num_slots, int32_t kv_heads,
                             int32_t head_dim,
                             msgl_dtype dtype, const void *k_new, const void *v_new,
                             const int32_t *out_loc, int32_t num_tokens) {
    msgl::StoreKvArgs a;
    a.k_pool = k_pool;
    a.v_pool = v_pool;
    a.k_new = k_new;
    a.v_new = v_new;
    a.out_loc = out_loc;
    a.num_tokens = num_tokens;
    a.row_vec16 = kv_heads * head_dim * elem_bytes(dtype) / 16;
    a.num_slots = num_slots;
    return a;
}

}  // namespace

struct msgl_graph {
    hipGraph_t graph = nullptr;
    hipGraphExec_t exec = nullptr;
};

// ---------------------------------------------------------------------------
// Decode attention without a caller workspace (msgl_decode_attn_noalloc): the
// workspace lives in a fixed device array, `scratch`, one copy per device,
// held for the life of the process.  Host code never passes the array's name
// to a kernel (on the host it only names a stand-in); the device address is
// resolved once per device with hipGetSymbolAddress and kept.

static __device__ __align__(256) unsigned char scratch[MSGL_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_addr[kMaxDevices];  // device address of `scratch`, per device (null until resolved)

// Address of the calling device's scratch array.  The stream must belong to
// the current device (the address is per device).
msgl_status scratch_address(void *stream, void **addr) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return from_hip(e, "hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices) return fail(MSGL_UNSUPPORTED, "device %d beyond the %d served", dev, kMaxDevices);
    if (stream != nullptr) {
        hipDevice_t sdev = -1;
        e = hipStreamGetDevice(static_cast<hipStream_t>(stream), &sdev);
        if (e != hipSuccess) return from_hip(e, "hipStreamGetDevice");
        if (sdev != dev)
            return fail(MSGL_INVALID_ARG, "the stream belongs to device %d, the current device is %d", sdev, dev);
    }
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_addr[dev] == nullptr) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return from_hip(e, "hipGetSymbolAddress(scratch)");
        if (p == nullptr) return fail(MSGL_HIP_ERROR, "hipGetSymbolAddress(scratch) returned NULL");
        g_scratch_addr[dev] = p;
    }
    *addr = g_scratch_addr[dev];
    return ok();
}

}  // namespace

extern "C" {

const char *msgl_last_error(void) { return g_err.c_str(); }

int msgl_version(void) { return 100; }

msgl_status msgl_store_kv(void *k_pool, void *v_pool, int64_t num_slots, int32_t kv_heads,
                          int32_t head_dim, msgl_dtype dtype, const void *k_new,
                          const void *v_new, const int32_t *out_loc, int32_t num_tokens,
                          void *stream) {
    msgl_status s = check_store(k_pool, v_pool, num_slots, kv_heads, head_dim, dtype, k_new, v_new,
                                out_loc, num_tokens);
    if (s != MSGL_OK) return s;
    if (num_tokens == 0) return ok();
    return from_hip(msgl::launch_store_kv(store_args(k_pool, v_pool, num_slots, kv_heads, head_dim, dtype, k_new,
                                                     v_new, out_loc, num_tokens),
                                          static_cast<hipStream_t>(stream)),
                    "store_kv launch");
}

msgl_status msgl_rope_store_kv(void *q_out, const void *q, void *k_pool, void *v_pool,
                               int64_t num_slots, int32_t q_heads, int32_t kv_heads,
                               int32_t head_dim, msgl_dtype dtype, const void *k_new,
                               const void *v_new, const int32_t *positions, const int32_t *out_loc,
                               int32_t num_tokens, double rope_base, void *stream) {
    msgl_status s = check_store(k_pool, v_pool, num_slots, kv_heads, head_dim, dtype, k_new, v_new,
                                out_loc, num_tokens);
    if (s != MSGL_OK) return s;
    if (q_heads < 1 || q_heads > 256) return fail(MSGL_INVALID_ARG, "q_heads %d out of range [1, 256]", q_heads);
    if (!(rope_base > 0.0) || !std::isfinite(rope_base))
        return fail(MSGL_INVALID_ARG, "rope_base %g is not a positive finite number", rope_base);
    if (num_tokens == 0) return ok();
    if (!q_out || !q || !positions) return fail(MSGL_INVALID_ARG, "NULL pointer argument");
    msgl::RopeStoreKvArgs a;
    a.q_out = q_out;
    a.q = q;
    a.k_pool = k_pool;
    a.v_pool = v_pool;
    a.k_new = k_new;
    a.v_new = v_new;
    a.positions = positions;
    a.out_loc = out_loc;
    a.num_slots = num_slots;
    a.num_tokens = num_tokens;
    a.q_heads = q_heads;
    a.kv_heads = kv_heads;
    a.head_dim = head_dim;
    a.base = rope_base;
    return from_hip(msgl::launch_rope_store_kv(a, static_cast<msgl::DType>(dtype), static_cast<hipStream_t>(stream)),
                    "rope_store_kv launch");
}

msgl_status msgl_vocab_embed(void *out, const void *weight, int64_t vocab_start, int64_t vocab_rows,
                             int32_t hidden, msgl_dtype dtype, const int32_t *ids, int32_t num_tokens,
                             void *stream) {
    if (dtype != MSGL_F32 && dtype != MSGL_BF16) return fail(MSGL_UNSUPPORTED, "dtype %d not supported", (int)dtype);
    if (hidden < 1) return fail(MSGL_INVALID_ARG, "hidden %d < 1", hidden);
    const int64_t row_bytes = (int64_t)hidden * elem_bytes(dtype);
    if (row_bytes % 16 != 0)
        return fail(MSGL_UNSUPPORTED, "row of %lld bytes is not a multiple of 16", (long long)row_bytes);
    if (vocab_rows < 1) return fail(MSGL_INVALID_ARG, "vocab_rows %lld < 1", (long long)vocab_rows);
    if (vocab_start < 0) return fail(MSGL_INVALID_ARG, "vocab_start %lld < 0", (long long)vocab_start);
    if (num_tokens < 0) return fail(MSGL_INVALID_ARG, "num_tokens %d < 0", num_tokens);
    if (num_tokens == 0) return ok();
    if (!out || !weight || !ids) return fail(MSGL_INVALID_ARG, "NULL pointer argument");
    msgl::VocabEmbedArgs a;
    a.out = out;
    a.weight = weight;
    a.ids = ids;
    a.vocab_start = vocab_start;
    a.rows = vocab_rows;
    a.row_vec = (int32_t)(row_bytes / 16);
    a.num_tokens = num_tokens;
    return from_hip(msgl::launch_vocab_embed(a, static_cast<hipStream_t>(stream)), "vocab_embed launch");
}

size_t msgl_decode_workspace_bytes(int32_t batch, int32_t q_heads, int32_t head_dim,
                                   int32_t max_seq_len, int32_t chunk) {
    if (batch < 0 || q_heads < 1 || head_dim < 1 || max_seq_len < 1) return 0;
    return msgl::decode_workspace_bytes(batch, q_heads, head_dim, max_seq_len, effective_chunk(chunk));
}

msgl_status msgl_decode_attn(void *out, float *lse, const void *q, const void *k_pool,
                             const void *v_pool, int64_t num_slots, const int32_t *page_table,
                             int32_t row_stride, const int32_t *table_idx,
                             const int32_t *seq_lens, int32_t batch, int32_t q_heads,
                             int32_t kv_heads, int32_t head_dim, int32_t page_size,
                             int32_t max_seq_len, int32_t chunk, float sm_scale,
                             msgl_dtype dtype, void *workspace, size_t workspace_bytes,
                             void *stream) {
    msgl_status s = check_decode(out, q, k_pool, v_pool, num_slots, page_table, row_stride, table_idx,
                                 seq_lens, batch, q_heads, kv_heads, head_dim, page_size, max_seq_len,
                                 chunk, dtype, workspace, workspace_bytes);
    if (s != MSGL_OK) return s;
    if (batch == 0) return ok();
    msgl::DecodeArgs a = decode_args(out, lse, q, k_pool, v_pool, num_slots, page_table, row_stride, table_idx,
                                     seq_lens, batch, q_heads, kv_heads, head_dim, max_seq_len, chunk,
                                     sm_scale, workspace);
    return from_hip(msgl::launch_decode(a, static_cast<msgl::DType>(dtype), head_dim,
                                        static_cast<hipStream_t>(stream)),
                    "decode launch");
}

// Decode attention with the fixed scratch in place of a workspace.
size_t msgl_noalloc_scratch_bytes(void) { return MSGL_NOALLOC_SCRATCH_BYTES; }

msgl_status msgl_decode_attn_noalloc(void *out, float *lse, const void *q, const void *k_pool,
                                     const void *v_pool, int64_t num_slots, const int32_t *page_table,
                                     int32_t row_stride, const int32_t *table_idx,
                                     const int32_t *seq_lens, int32_t batch, int32_t q_heads,
                                     int32_t kv_heads, int32_t head_dim, int32_t page_size,
                                     int32_t max_seq_len, int32_t chunk, float sm_scale,
                                     msgl_dtype dtype, void *stream) {
    msgl_status s = check_decode_args(out, q, k_pool, v_pool, num_slots, page_table, row_stride, table_idx,
                                      seq_lens, batch, q_heads, kv_heads, head_dim, page_size, max_seq_len,
                                      chunk, dtype);
    if (s != MSGL_OK) return s;
    const size_t need = msgl::decode_workspace_bytes(batch, q_heads, head_dim, max_seq_len, effective_chunk(chunk));
    if (need > (size_t)MSGL_NOALLOC_SCRATCH_BYTES)
        return fail(MSGL_WORKSPACE_TOO_SMALL,
                    "batch %d x %d q heads x head_dim %d needs %zu bytes of workspace, beyond the %zu of the "
                    "fixed scratch (msgl_decode_attn with a workspace serves it)",
                    batch, q_heads, head_dim, need, (size_t)MSGL_NOALLOC_SCRATCH_BYTES);
    if (batch == 0) return ok();
    void *ws = nullptr;
    if ((s = scratch_address(stream, &ws)) != MSGL_OK) return s;
    msgl::DecodeArgs a = decode_args(out, lse, q, k_pool, v_pool, num_slots, page_table, row_stride, table_idx,
                                     seq_lens, batch, q_heads, kv_heads, head_dim, max_seq_len, chunk,
                                     sm_scale, ws);
    return from_hip(msgl::launch_decode(a, static_cast<msgl::DType>(dtype), head_dim,
                                        static_cast<hipStream_t>(stream)),
                    "decode launch");
}

size_t msgl_decode_shared_prefix_workspace_bytes(int32_t batch, int32_t q_heads, int32_t head_dim,
                                                 int32_t max_seq_len, int32_t chunk) {
    if (batch < 0 || q_heads < 1 || head_dim < 1 || max_seq_len < 1) return 0;
    return msgl::shared_prefix_workspace_bytes(batch, q_heads, head_dim, max_seq_len, effective_chunk(chunk));
}

msgl_status msgl_decode_attn_shared_prefix(void *out, float *lse, const void *q, const void *k_pool,
                                           const void *v_pool, int64_t num_slots, const int32_t *page_table,
                                           int32_t row_stride, const int32_t *table_idx,
                                           const int32_t *seq_lens, int32_t batch,
                                           const int32_t *group_start, const int32_t *prefix_lens,
                                           int32_t num_groups, int32_t max_group_size, int32_t max_prefix_len,
                                           int32_t q_heads, int32_t kv_heads, int32_t head_dim,
                                           int32_t page_size, int32_t max_seq_len, int32_t chunk,
                                           float sm_scale, msgl_dtype dtype, void *workspace,
                                           size_t workspace_bytes, void *stream) {
    if (dtype != MSGL_BF16 || head_dim != 128)
        return fail(MSGL_UNSUPPORTED, "the shared-prefix decode runs bf16 with head_dim 128 only");
    const size_t need = msgl::shared_prefix_workspace_bytes(batch < 0 ? 0 : batch, q_heads < 1 ? 1 : q_heads,
                                                            head_dim, max_seq_len, effective_chunk(chunk));
    // the decode checks, against the decode part of the workspace
    msgl_status s = check_decode(out, q, k_pool, v_pool, num_slots, page_table, row_stride, table_idx, seq_lens,
                                 batch, q_heads, kv_heads, head_dim, page_size, max_seq_len, chunk, dtype,
                                 workspace, workspace_bytes);
    if (s != MSGL_OK) return s;
    if (workspace_bytes < need)
        return fail(MSGL_WORKSPACE_TOO_SMALL, "workspace %zu bytes < %zu required", workspace_bytes, need);
    if (num_groups < 0 || num_groups > batch)
        return fail(MSGL_INVALID_ARG, "num_groups %d not in [0, batch=%d]", num_groups, batch);
    if (num_groups > 1024) return fail(MSGL_UNSUPPORTED, "num_groups %d > 1024", num_groups);
    if (max_prefix_len < 0 || max_prefix_len >= max_seq_len)
        return fail(MSGL_INVALID_ARG, "max_prefix_len %d not in [0, max_seq_len)", max_prefix_len);
    if (num_groups > 0 && (max_group_size < 1 || max_group_size > batch))
        return fail(MSGL_INVALID_ARG, "max_group_size %d not in [1, batch=%d]", max_group_size, batch);
    if (batch == 0) return ok();
    if (!prefix_lens || (num_groups > 0 && !group_start)) return fail(MSGL_INVALID_ARG, "NULL pointer argument");
    msgl::DecodeArgs d = decode_args(out, lse, q, k_pool, v_pool, num_slots, page_table, row_stride, table_idx,
                                     seq_lens, batch, q_heads, kv_heads, head_dim, max_seq_len, chunk, sm_scale,
                                     workspace);
    msgl::SharedPrefixArgs sp;
    sp.group_start = group_start;
    sp.prefix_lens = prefix_lens;
    sp.num_groups = num_groups;
    sp.max_group_size = max_group_size;
    sp.max_prefix_len = max_prefix_len;
    sp.cus = msgl::device_cu_count();
    sp.workspace = workspace;
    return from_hip(msgl::launch_decode_shared_prefix(sp, d, head_dim, static_cast<hipStream_t>(stream)),
                    "shared-prefix decode launch");
}

msgl_status msgl_prefill_attn(void *out, float *lse, const void *q, const void *k_pool,
                              const void *v_pool, int64_t num_slots, const int32_t *page_table,
                              int32_t row_stride, const int32_t *table_idx,
                              const int32_t *seq_lens, const int32_t *cached_lens,
                              const int32_t *cu_q, int32_t batch, int32_t total_q,
                              int32_t max_extend, int32_t q_heads, int32_t kv_heads,
                              int32_t head_dim, int32_t page_size, float sm_scale,
                              msgl_dtype dtype, void *stream) {
    msgl_status s = check_common(dtype, head_dim, kv_heads, num_slots);
    if (s != MSGL_OK) return s;
    if ((s = check_group(q_heads, kv_heads)) != MSGL_OK) return s;
    if (batch < 0 || total_q < 0) return fail(MSGL_INVALID_ARG, "negative batch or total_q");
    if (batch == 0 || total_q == 0) {
        if (batch == 0 && total_q == 0) return ok();
        return fail(MSGL_INVALID_ARG, "batch %d and total_q %d must both be zero or both positive", batch, total_q);
    }
    if (total_q < batch) return fail(MSGL_INVALID_ARG, "total_q %d < batch %d (each request needs a new token)", total_q, batch);
    if (max_extend < 1 || max_extend > total_q)
        return fail(MSGL_INVALID_ARG, "max_extend %d not in [1, total_q=%d]", max_extend, total_q);
    if (!out || !q || !k_pool || !v_pool || !page_table || !table_idx || !seq_lens || !cached_lens || !cu_q)
        return fail(MSGL_INVALID_ARG, "NULL pointer argument");
    if (row_stride < 1) return fail(MSGL_INVALID_ARG, "row_stride %d < 1", row_stride);
    if (page_size < 1) return fail(MSGL_INVALID_ARG, "page_size %d < 1", page_size);
    msgl::PrefillArgs a;
    a.out = out;
    a.lse = lse;
    a.q = q;
    a.k_pool = k_pool;
    a.v_pool = v_pool;
    a.page_table = page_table;
    a.row_stride = row_stride;
    a.table_idx = table_idx;
    a.seq_lens = seq_lens;
    a.cached_lens = cached_lens;
    a.cu_q = cu_q;
    a.num_slots = num_slots;
    a.batch = batch;
    a.total_q = total_q;
    a.max_extend = max_extend;
    a.q_heads = q_heads;
    a.kv_heads = kv_heads;
    a.scale_log2 = sm_scale * msgl::kLog2eHost;
    a.splits = 1;
    a.part_o = nullptr;
    a.part_lse = nullptr;
    a.plan = nullptr;
    return from_hip(msgl::launch_prefill(a, static_cast<msgl::DType>(dtype), head_dim,
                                         static_cast<hipStream_t>(stream)),
                    "prefill launch");
}

// ---------------------------------------------------------------------------
// Host plan of a prefill launch: the block list that the kernel would otherwise
// derive on the device from the lengths (every (request, query block) pair,
// the most key tiles first, ties in request order), made on the host from the
// host copies of the batch metadata.

size_t msgl_prefill_plan_bytes(int32_t batch, int32_t total_q, int32_t q_heads, int32_t kv_heads) {
    if (batch < 0 || total_q < 0 || kv_heads < 1 || q_heads < kv_heads || q_heads % kv_heads != 0) return 0;
    const int64_t bq = msgl::prefill_small_bq(q_heads / kv_heads);
    const int64_t entries = ((int64_t)total_q + (int64_t)batch * (bq - 1)) / bq;  // >= sum_b ceil(E_b / bq)
    return (size_t)(msgl::kPlanHeaderInts + entries * msgl::kPlanEntryInts) * sizeof(int32_t);
}

msgl_status msgl_prefill_plan(int32_t *plan, size_t plan_bytes, const int32_t *seq_lens,
                              const int32_t *cached_lens, const int32_t *cu_q, const int32_t *table_idx,
                              int32_t batch, int32_t total_q, int32_t rows, int32_t row_stride,
                              int32_t q_heads, int32_t kv_heads, int32_t head_dim, msgl_dtype dtype) {
    if (dtype != MSGL_BF16 || head_dim != 128)
        return fail(MSGL_UNSUPPORTED, "the planned prefill runs the bf16 matrix-core kernels (head_dim 128)");
    msgl_status s = check_common(dtype, head_dim, kv_heads, 1);
    if (s != MSGL_OK) return s;
    if ((s = check_group(q_heads, kv_heads)) != MSGL_OK) return s;
    if (batch < 0 || total_q < 0) return fail(MSGL_INVALID_ARG, "negative batch or total_q");
    if (!plan || (batch > 0 && (!seq_lens || !cached_lens || !cu_q || !table_idx)))
        return fail(MSGL_INVALID_ARG, "NULL pointer argument");
    if (rows < 1 || row_stride < 1) return fail(MSGL_INVALID_ARG, "rows %d or row_stride %d < 1", rows, row_stride);
    if (batch == 0 && total_q != 0) return fail(MSGL_INVALID_ARG, "total_q %d without requests", total_q);
    if (batch > 0 && cu_q[0] != 0) return fail(MSGL_INVALID_ARG, "cu_q[0] = %d, not 0", cu_q[0]);
    if (batch > 0 && cu_q[batch] != total_q)
        return fail(MSGL_INVALID_ARG, "cu_q[batch] = %d differs from total_q %d", cu_q[batch], total_q);
    const int g = q_heads / kv_heads;
    int bq = 0;
    const int layout = msgl::prefill_layout(batch, total_q, g, &bq);
    struct Entry {
        int32_t tiles, b, qb;
    };
    std::vector<Entry> list;
    for (int32_t b = 0; b < batch; ++b) {
        const int64_t e = (int64_t)cu_q[b + 1] - cu_q[b];
        const int64_t c = cached_lens[b];
        if (e < 1 || c < 0 || c + e != seq_lens[b])
            return fail(MSGL_INVALID_ARG, "request %d: cu_q step %lld, cached %lld, seq_len %d (need step >= 1 and "
                        "cached + step == seq_len)", b, (long long)e, (long long)c, seq_lens[b]);
        if (seq_lens[b] > row_stride)
            return fail(MSGL_INVALID_ARG, "request %d: seq_len %d exceeds row_stride %d", b, seq_lens[b], row_stride);
        if (table_idx[b] < 0 || table_idx[b] >= rows)
            return fail(MSGL_INVALID_ARG, "request %d: table row %d not in [0, %d)", b, table_idx[b], rows);
        for (int64_t qb = 0; qb * bq < e; ++qb) {
            const int64_t keys = c + std::min<int64_t>((qb + 1) * bq, e);
            list.push_back({(int32_t)((keys + msgl::kPlanKeyTile - 1) / msgl::kPlanKeyTile), b, (int32_t)qb});
        }
    }
    const size_t need = (msgl::kPlanHeaderInts + list.size() * (size_t)msgl::kPlanEntryInts) * sizeof(int32_t);
    if (plan_bytes < need) return fail(MSGL_WORKSPACE_TOO_SMALL, "plan buffer %zu bytes < %zu required", plan_bytes, need);
    std::stable_sort(list.begin(), list.end(), [](const Entry &x, const Entry &y) { return x.tiles > y.tiles; });
    const int32_t head[msgl::kPlanHeaderInts] = {msgl::kPlanMagic, layout, bq, (int32_t)list.size(),
                                                 batch, total_q, q_heads, kv_heads};
    for (int i = 0; i < msgl::kPlanHeaderInts; ++i) plan[i] = head[i];
    int32_t *e = plan + msgl::kPlanHeaderInts;
    for (const Entry &x : list) {
        const int32_t ent[msgl::kPlanEntryInts] = {x.b, x.qb, cu_q[x.b + 1] - cu_q[x.b], cached_lens[x.b],
                                                   cu_q[x.b], table_idx[x.b], x.tiles, 0};
        for (int i = 0; i < msgl::kPlanEntryInts; ++i) e[i] = ent[i];
        e += msgl::kPlanEntryInts;
    }
    return ok();
}

msgl_status msgl_prefill_attn_planned(void *out, float *lse, const void *q, const void *k_pool,
                                      const void *v_pool, int64_t num_slots, const int32_t *page_table,
                                      int32_t row_stride, int32_t q_heads, int32_t kv_heads, int32_t head_dim,
                                      int32_t page_size, float sm_scale, msgl_dtype dtype,
                                      const int32_t *plan_host, const int32_t *plan_dev, size_t plan_bytes,
                                      void *stream) {
    if (dtype != MSGL_BF16 || head_dim != 128)
        return fail(MSGL_UNSUPPORTED, "the planned prefill runs the bf16 matrix-core kernels (head_dim 128)");
    msgl_status s = check_common(dtype, head_dim, kv_heads, num_slots);
    if (s != MSGL_OK) return s;
    if ((s = check_group(q_heads, kv_heads)) != MSGL_OK) return s;
    if (!plan_host || !plan_dev) return fail(MSGL_INVALID_ARG, "NULL plan");
    if (plan_bytes < msgl::kPlanHeaderInts * sizeof(int32_t) || plan_host[0] != msgl::kPlanMagic)
        return fail(MSGL_INVALID_ARG, "not a prefill plan (bad header)");
    const int32_t layout = plan_host[1], bq = plan_host[2], entries = plan_host[3];
    const int32_t batch = plan_host[4], total_q = plan_host[5];
    int want_bq = 0;
    const int want_layout = msgl::prefill_layout(batch, total_q, q_heads / kv_heads, &want_bq);
    if (plan_host[6] != q_heads || plan_host[7] != kv_heads || layout != want_layout || bq != want_bq ||
        entries < 0 || batch < 0 || total_q < 0)
        return fail(MSGL_INVALID_ARG, "the plan was made for other heads or is malformed (layout %d, %d tokens per "
                    "block, %d entries)", layout, bq, entries);
    if (plan_bytes < (msgl::kPlanHeaderInts + (size_t)entries * msgl::kPlanEntryInts) * sizeof(int32_t))
        return fail(MSGL_INVALID_ARG, "plan_bytes %zu too small for %d entries", plan_bytes, entries);
    if (entries == 0) return ok();
    if (!out || !q || !k_pool || !v_pool || !page_table) return fail(MSGL_INVALID_ARG, "NULL pointer argument");
    if (row_stride < 1) return fail(MSGL_INVALID_ARG, "row_stride %d < 1", row_stride);
    if (page_size < 1) return fail(MSGL_INVALID_ARG, "page_size %d < 1", page_size);
    msgl::PrefillArgs a{};
    a.out = out;
    a.lse = lse;
    a.q = q;
    a.k_pool = k_pool;
    a.v_pool = v_pool;
    a.page_table = page_table;
    a.row_stride = row_stride;
    a.num_slots = num_slots;
    a.batch = batch;
    a.total_q = total_q;
    a.max_extend = 0;
    a.q_heads = q_heads;
    a.kv_heads = kv_heads;
    a.scale_log2 = sm_scale * msgl::kLog2eHost;
    a.splits = 1;
    a.plan = plan_dev + msgl::kPlanHeaderInts;
    return from_hip(msgl::launch_prefill_planned(a, layout, entries, static_cast<hipStream_t>(stream)),
                    "planned prefill launch");
}

msgl_status msgl_decode_graph_create(msgl_graph **graph, void *k_pool, void *v_pool,
                                     int64_t num_slots, const void *k_new, const void *v_new,
                                     const int32_t *out_loc, void *out, float *lse,
                                     const void *q, const int32_t *page_table,
                                     int32_t row_stride, const int32_t *table_idx,
                                     const int32_t *seq_lens, int32_t padded_batch,
                                     int32_t q_heads, int32_t kv_heads, int32_t head_dim,
                                     int32_t page_size, int32_t max_seq_len, int32_t chunk,
                                     float sm_scale, msgl_dtype dtype, void *workspace,
                                     size_t workspace_bytes, void *stream) {
    if (!graph) return fail(MSGL_INVALID_ARG, "NULL graph handle pointer");
    *graph = nullptr;
    if (!stream) return fail(MSGL_INVALID_ARG, "graph capture needs a non-null stream");
    if (padded_batch < 1) return fail(MSGL_INVALID_ARG, "padded_batch %d < 1", padded_batch);
    msgl_status s = check_store(k_pool, v_pool, num_slots, kv_heads, head_dim, dtype, k_new, v_new,
                                out_loc, padded_batch);
    if (s != MSGL_OK) return s;
    s = check_decode(out, q, k_pool, v_pool, num_slots, page_table, row_stride, table_idx, seq_lens,
                     padded_batch, q_heads, kv_heads, head_dim, page_size, max_seq_len, chunk, dtype,
                     workspace, workspace_bytes);
    if (s != MSGL_OK) return s;
    hipStream_t st = static_cast<hipStream_t>(stream);
    msgl::DecodeArgs da = decode_args(out, lse, q, k_pool, v_pool, num_slots, page_table, row_stride, table_idx,
                                      seq_lens, padded_batch, q_heads, kv_heads, head_dim, max_seq_len,
                                      chunk, sm_scale, workspace);
    // the KV write rides in the split kernel: the wave that reads a request's
    // last key writes that key's row first (one kernel fewer per replay)
    da.fuse_store = 1;
    da.k_pool_w = k_pool;
    da.v_pool_w = v_pool;
    da.k_new = k_new;
    da.v_new = v_new;
    da.out_loc = out_loc;
    hipError_t e = msgl::launch_decode(da, static_cast<msgl::DType>(dtype), head_dim, st, true);
    if (e != hipSuccess) return from_hip(e, "decode preparation");
    e = hipStreamBeginCapture(st, hipStreamCaptureModeThreadLocal);
    if (e != hipSuccess) return from_hip(e, "hipStreamBeginCapture");
    hipError_t e1 = hipSuccess;
    hipError_t e2 = msgl::launch_decode(da, static_cast<msgl::DType>(dtype), head_dim, st);
    hipGraph_t g = nullptr;
    e = hipStreamEndCapture(st, &g);
    if (e1 != hipSuccess || e2 != hipSuccess || e != hipSuccess) {
        if (g) (void)hipGraphDestroy(g);
        return from_hip(e1 != hipSuccess ? e1 : (e2 != hipSuccess ? e2 : e), "decode graph capture");
    }
    hipGraphExec_t ex = nullptr;
    e = hipGraphInstantiate(&ex, g, nullptr, nullptr, 0);
    if (e != hipSuccess) {
        (void)hipGraphDestroy(g);
        return from_hip(e, "hipGraphInstantiate");
    }
    msgl_graph *h = new (std::nothrow) msgl_graph;
    if (!h) {
        (void)hipGraphExecDestroy(ex);
        (void)hipGraphDestroy(g);
        return fail(MSGL_INVALID_ARG, "out of host memory");
    }
    h->graph = g;
    h->exec = ex;
    *graph = h;
    return ok();
}

msgl_status msgl_graph_launch(msgl_graph *graph, void *stream) {
    if (!graph || !graph->exec) return fail(MSGL_INVALID_ARG, "NULL graph");
    return from_hip(hipGraphLaunch(graph->exec, static_cast<hipStream_t>(stream)), "hipGraphLaunch");
}

void msgl_graph_destroy(msgl_graph *graph) {
    if (!graph) return;
    if (graph->exec) (void)hipGraphExecDestroy(graph->exec);
    if (graph->graph) (void)hipGraphDestroy(graph->graph);
    delete graph;
}

msgl_status msgl_validate_shared_prefix(const int32_t *page_table, int32_t rows, int32_t row_stride,
                                        const int32_t *table_idx, const int32_t *seq_lens, int32_t batch,
                                        const int32_t *group_start, const int32_t *prefix_lens,
                                        int32_t num_groups, int32_t max_group_size, int32_t max_prefix_len) {
    if (!page_table || !table_idx || !seq_lens || !prefix_lens || (num_groups > 0 && !group_start))
        return fail(MSGL_INVALID_ARG, "NULL pointer argument");
    if (rows < 1 || row_stride < 1 || batch < 0 || num_groups < 0) return fail(MSGL_INVALID_ARG, "bad scalar argument");
    std::vector<char> grouped((size_t)batch, 0);
    if (num_groups > 0 && group_start[0] != 0) return fail(MSGL_INVALID_ARG, "group_start[0] = %d, expected 0", group_start[0]);
    for (int32_t g = 0; g < num_groups; ++g) {
        const int32_t b0 = group_start[g], b1 = group_start[g + 1];
        if (b1 <= b0 || b1 > batch)
            return fail(MSGL_INVALID_ARG, "group %d spans rows [%d, %d) of a batch of %d", g, b0, b1, batch);
        if (b1 - b0 > max_group_size)
            return fail(MSGL_INVALID_ARG, "group %d has %d requests > max_group_size %d", g, b1 - b0, max_group_size);
        const int32_t P = prefix_lens[b0];
        const int32_t *row0 = page_table + (int64_t)table_idx[b0] * row_stride;
        for (int32_t b = b0; b < b1; ++b) {
            grouped[(size_t)b] = 1;
            if (table_idx[b] < 0 || table_idx[b] >= rows)
                return fail(MSGL_INVALID_ARG, "table_idx[%d] = %d outside [0, %d)", b, table_idx[b], rows);
            if (prefix_lens[b] != P)
                return fail(MSGL_INVALID_ARG, "prefix_lens[%d] = %d differs from its group's %d", b, prefix_lens[b], P);
            if (P < 0 || P > max_prefix_len || P >= seq_lens[b] || P > row_stride)
                return fail(MSGL_INVALID_ARG, "prefix_lens[%d] = %d not in [0, min(seq_len - 1, max_prefix_len)]", b, P);
            const int32_t *row = page_table + (int64_t)table_idx[b] * row_stride;
            for (int32_t j = 0; j < P; ++j)
                if (row[j] != row0[j])
                    return fail(MSGL_INVALID_ARG, "request %d's page-table entry %d differs from its group's prefix", b, j);
        }
    }
    for (int32_t b = 0; b < batch; ++b)
        if (!grouped[(size_t)b] && prefix_lens[b] != 0)
            return fail(MSGL_INVALID_ARG, "request %d is in no group but has prefix_lens %d (expected 0)", b, prefix_lens[b]);
    return ok();
}

msgl_status msgl_check_batch(const int32_t *page_table, int32_t rows, int32_t row_stride,
                             const int32_t *table_idx, const int32_t *seq_lens, const int32_t *cached_lens,
                             const int32_t *cu_q, int32_t batch, int32_t max_seq_len, int64_t num_slots,
                             int32_t page_size, const int32_t *out_loc, int32_t num_tokens, int64_t dummy_slot,
                             int32_t *result, uint32_t *seen, void *stream) {
    if (!page_table || !table_idx || !seq_lens || !result) return fail(MSGL_INVALID_ARG, "NULL pointer argument");
    if (rows < 1 || row_stride < 1 || batch < 0 || max_seq_len < 1 || num_slots < 1 || page_size < 1 ||
        num_tokens < 0)
        return fail(MSGL_INVALID_ARG, "bad scalar argument");
    if (out_loc && !cu_q && cached_lens)
        return fail(MSGL_INVALID_ARG, "checking out_loc of a batch with cached_lens needs cu_q");
    if (out_loc && !cu_q && num_tokens != batch)
        return fail(MSGL_INVALID_ARG, "out_loc of a decode batch has %d entries for %d requests", num_tokens, batch);
    if (num_slots > INT32_MAX) return fail(MSGL_UNSUPPORTED, "num_slots %lld above 2^31 - 1", (long long)num_slots);
    msgl::CheckBatchArgs a;
    a.page_table = page_table;
    a.rows = rows;
    a.row_stride = row_stride;
    a.table_idx = table_idx;
    a.seq_lens = seq_lens;
    a.cached_lens = cached_lens;
    a.cu_q = cu_q;
    a.batch = batch;
    a.max_seq_len = max_seq_len;
    a.num_slots = num_slots;
    a.page_size = page_size;
    a.out_loc = out_loc;
    a.num_tokens = num_tokens;
    a.dummy_slot = dummy_slot;
    a.result = result;
    a.seen = out_loc ? seen : nullptr;
    a.seen_words = a.seen ? (num_slots + 31) / 32 : 0;
    return from_hip(msgl::launch_check_batch(a, static_cast<hipStream_t>(stream)), "check_batch launch");
}

msgl_status msgl_validate_batch(const int32_t *page_table, int32_t rows, int32_t row_stride,
                                const int32_t *table_idx, const int32_t *seq_lens,
                                const int32_t *cached_lens, const int32_t *cu_q, int32_t batch,
                                int32_t max_seq_len, int64_t num_slots, int32_t page_size,
                                const int32_t *out_loc, int32_t num_tokens, int64_t dummy_slot) {
    if (!page_table || !table_idx || !seq_lens) return fail(MSGL_INVALID_ARG, "NULL pointer argument");
    if (rows < 1 || row_stride < 1 || batch < 0 || num_slots < 1 || page_size < 1 || num_tokens < 0)
        return fail(MSGL_INVALID_ARG, "bad scalar argument");
    const int32_t lim = max_seq_len < row_stride ? max_seq_len : row_stride;
    if (cu_q && cu_q[0] != 0) return fail(MSGL_INVALID_ARG, "cu_q[0] = %d, expected 0", cu_q[0]);
    for (int32_t b = 0; b < batch; ++b) {
        const int32_t r = table_idx[b];
        if (r < 0 || r >= rows) return fail(MSGL_INVALID_ARG, "table_idx[%d] = %d outside [0, %d)", b, r, rows);
        const int32_t L = seq_lens[b];
        if (L < 1 || L > lim) return fail(MSGL_INVALID_ARG, "seq_lens[%d] = %d outside [1, %d]", b, L, lim);
        const int32_t C = cached_lens ? cached_lens[b] : L - 1;
        if (C < 0 || C >= L) return fail(MSGL_INVALID_ARG, "cached_lens[%d] = %d outside [0, %d)", b, C, L);
        if (cu_q && cu_q[b + 1] - cu_q[b] != L - C)
            return fail(MSGL_INVALID_ARG, "cu_q[%d+1] - cu_q[%d] = %d, expected seq_len - cached_len = %d", b, b,
                        cu_q[b + 1] - cu_q[b], L - C);
        const int32_t *row = page_table + (int64_t)r * row_stride;
        for (int32_t j = 0; j < L; ++j) {
            if (row[j] < 0 || row[j] >= num_slots)
                return fail(MSGL_INVALID_ARG, "page_table[%d, %d] = %d outside [0, %lld)", r, j, row[j],
                            (long long)num_slots);
            if (page_size > 1) {
                const int32_t off = j % page_size;
                if (off == 0 && row[j] % page_size != 0)
                    return fail(MSGL_INVALID_ARG, "page_table[%d, %d] = %d does not start a page", r, j, row[j]);
                if (off != 0 && row[j] != row[j - 1] + 1)
                    return fail(MSGL_INVALID_ARG, "page_table[%d, %d] breaks page contiguity", r, j);
            }
        }
    }
    if (out_loc) {
        // out_loc is page_table[row, cached:len] of each request, in batch order
        // (decode, cached_lens NULL: one token per request, its last key)
        int64_t expected = 0;
        for (int32_t b = 0; b < batch; ++b) expected += seq_lens[b] - (cached_lens ? cached_lens[b] : seq_lens[b] - 1);
        if (expected != num_tokens)
            return fail(MSGL_INVALID_ARG, "out_loc has %d entries, the batch's new tokens are %lld", num_tokens,
                        (long long)expected);
        int64_t t = 0;
        for (int32_t b = 0; b < batch && t < num_tokens; ++b) {
            const int32_t L = seq_lens[b];
            const int32_t C = cached_lens ? cached_lens[b] : L - 1;
            const int32_t *row = page_table + (int64_t)table_idx[b] * row_stride;
            for (int32_t i = C; i < L && t < num_tokens; ++i, ++t)
                if (out_loc[t] != row[i])
                    return fail(MSGL_INVALID_ARG, "out_loc[%lld] = %d, expected page_table[%d, %d] = %d", (long long)t,
                                out_loc[t], table_idx[b], i, row[i]);
        }
        std::vector<unsigned char> seen((size_t)num_slots, 0);
        for (int32_t t = 0; t < num_tokens; ++t) {
            const int32_t s = out_loc[t];
            if (s < 0 || s >= num_slots)
                return fail(MSGL_INVALID_ARG, "out_loc[%d] = %d outside [0, %lld)", t, s, (long long)num_slots);
            if (seen[(size_t)s] && s != dummy_slot)
                return fail(MSGL_INVALID_ARG, "out_loc[%d] = %d repeats a slot", t, s);
            seen[(size_t)s] = 1;
        }
    }
    return ok();
}

}  // extern "C"
