// Grouped-query paged decode attention on the matrix cores (gfx950 MFMA).
#include <hip/hip_runtime.h>

#include "internal.h"
#include "kernel_common.h"

namespace pa {

bool mfma_supported(int dtype, int head_dim, int block_size, int group) {
    (void)dtype, (void)head_dim, (void)block_size, (void)group;
    return false;
}

int launch_decode_mfma(const DecodeArgs &a) {
    (void)a;
    return fail(PA_ERR_UNSUPPORTED, "MFMA decode not built");
}

}  // namespace pa
