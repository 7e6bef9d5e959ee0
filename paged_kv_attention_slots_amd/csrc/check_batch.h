// Host-side launcher of the device-side batch-metadata check (internal; the
// C ABI is include/msgl.h's msgl_check_batch).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace msgl {

// Device-side metadata check (the codes are those of msgl.h's MSGL_CHECK_*).
constexpr int kCheckTableIdx = 1, kCheckSeqLen = 2, kCheckCachedLen = 4, kCheckCuQ = 8, kCheckSlot = 16,
              kCheckPage = 32, kCheckOutLoc = 64, kCheckRepeat = 128, kCheckTokenCount = 256;
struct CheckBatchArgs {
    const int32_t *page_table;
    int32_t rows;
    int32_t row_stride;
    const int32_t *table_idx;
    const int32_t *seq_lens;
    const int32_t *cached_lens;  // NULL: decode (cached = seq_len - 1)
    const int32_t *cu_q;         // NULL: not checked (decode: token b is request b's)
    int32_t batch;
    int32_t max_seq_len;
    int64_t num_slots;
    int32_t page_size;
    const int32_t *out_loc;      // NULL: not checked
    int32_t num_tokens;
    int64_t dummy_slot;
    int32_t *result;             // [4] device: codes, flagged requests, first request, first token
    uint32_t *seen;              // NULL, or seen_words zeroed-by-the-call bitmap words over the slots
    int64_t seen_words;
};
hipError_t launch_check_batch(const CheckBatchArgs &a, hipStream_t stream);

}  // namespace msgl
