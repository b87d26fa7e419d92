// Host-only entry points and helpers of libpa: the thread's last error, status text,
// the ABI version and the host checks of tables and copy pairs ("PagedAttention" concept
// report (compassingai.com) §13: bounds are checked before work is scheduled).  Nothing
// here touches HIP, so this file and allocator.cpp also build as plain C++ (the
// sanitizer build of the host code).
#include <cstdarg>
#include <cstdio>
#include <cstdlib>

#include "internal.h"

namespace pa {

static thread_local char g_err[512];

int fail(int status, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return status;
}

void clear_error() { g_err[0] = 0; }

}  // namespace pa

using namespace pa;

extern "C" {

const char *pa_status_str(int status) {
    switch (status) {
        case PA_OK: return "ok";
        case PA_ERR_INVALID: return "invalid argument";
        case PA_ERR_BOUNDS: return "index out of bounds";
        case PA_ERR_OOM: return "out of blocks";
        case PA_ERR_UNSUPPORTED: return "unsupported configuration";
        case PA_ERR_HIP: return "HIP runtime error";
        default: return "unknown status";
    }
}

const char *pa_last_error(void) { return g_err; }

int pa_abi_version(void) { return 4; }

int pa_check_tables(const int32_t *block_tables, const int32_t *context_lens, int num_seqs,
                    int max_blocks_per_seq, int block_size, int num_blocks) {
    clear_error();
    if (num_seqs < 0 || max_blocks_per_seq <= 0 || block_size <= 0 || num_blocks <= 0 ||
        (num_seqs && (!block_tables || !context_lens)))
        return fail(PA_ERR_INVALID, "bad argument");
    for (int s = 0; s < num_seqs; ++s) {
        const int n = context_lens[s];
        if (n < 0) return fail(PA_ERR_INVALID, "context_lens[%d] = %d", s, n);
        const int nb = (n + block_size - 1) / block_size;
        if (nb > max_blocks_per_seq)
            return fail(PA_ERR_BOUNDS, "sequence %d needs %d blocks > %d", s, nb, max_blocks_per_seq);
        for (int j = 0; j < nb; ++j) {
            const int32_t b = block_tables[(int64_t)s * max_blocks_per_seq + j];
            if (b < 0 || b >= num_blocks)
                return fail(PA_ERR_BOUNDS, "block_tables[%d][%d] = %d outside [0, %d)", s, j, b, num_blocks);
        }
    }
    return PA_OK;
}

int pa_check_copy_pairs(const int32_t *src, const int32_t *dst, int num_pairs, int num_blocks) {
    clear_error();
    if (num_pairs < 0 || num_blocks <= 0 || (num_pairs && (!src || !dst)))
        return fail(PA_ERR_INVALID, "bad argument");
    // 1 = seen as src, 2 = seen as dst
    char *mark = (char *)calloc((size_t)num_blocks, 1);
    if (!mark) return fail(PA_ERR_OOM, "host allocation failed");
    int rc = PA_OK;
    for (int p = 0; p < num_pairs && rc == PA_OK; ++p) {
        if (src[p] < 0 || src[p] >= num_blocks || dst[p] < 0 || dst[p] >= num_blocks)
            rc = fail(PA_ERR_BOUNDS, "pair %d (%d -> %d) outside [0, %d)", p, src[p], dst[p], num_blocks);
    }
    for (int p = 0; p < num_pairs && rc == PA_OK; ++p) mark[src[p]] |= 1;
    for (int p = 0; p < num_pairs && rc == PA_OK; ++p) {
        if (mark[dst[p]] & 1) rc = fail(PA_ERR_INVALID, "pair %d: dst %d is also a src", p, dst[p]);
        else if (mark[dst[p]] & 2) rc = fail(PA_ERR_INVALID, "pair %d: dst %d repeated", p, dst[p]);
        else mark[dst[p]] |= 2;
    }
    free(mark);
    return rc;
}

}  // extern "C"
