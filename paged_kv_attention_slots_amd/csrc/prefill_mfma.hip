// Prefill / extend attention on matrix cores (bf16 MFMA) - dispatch.
#include "launch.h"

namespace msgl {

hipError_t launch_prefill(const PrefillArgs &a, DType dtype, int head_dim, hipStream_t stream) {
    return launch_prefill_valu(a, dtype, head_dim, stream);
}

}  // namespace msgl
