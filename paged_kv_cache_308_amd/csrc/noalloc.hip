// pa_decode_noalloc: pa_decode with its partials in a fixed device array of the library
// instead of a caller-provided workspace, for callers that cannot allocate device memory
// (work under graph capture, serving loops that must not allocate).
//
// The array lives in this file's device code: every GPU the library runs on holds one
// copy of PA_NOALLOC_SCRATCH_BYTES bytes until the process ends.  Host code never passes
// the array's name to a kernel (on the host it is only a stand-in for the symbol): the
// first call on a device, with that device current, looks up the array's device address
// with hipGetSymbolAddress and keeps it per device; launches get that address.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "internal.h"

static __device__ __align__(256) uint8_t scratch[PA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::atomic<void *> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of the current device's copy of `scratch`, looked up once per device.
int scratch_address(void **out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0)
        return pa::fail(PA_ERR_HIP, "no current device");
    if (dev >= kMaxDevices) return pa::fail(PA_ERR_UNSUPPORTED, "device %d (at most %d devices)", dev, kMaxDevices);
    void *p = g_scratch[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> g(g_scratch_mu);
        p = g_scratch[dev].load(std::memory_order_relaxed);
        if (!p) {
            const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (e != hipSuccess || !p)
                return pa::fail(PA_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev,
                                hipGetErrorString(e));
            g_scratch[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return PA_OK;
}

}  // namespace

extern "C" {

int pa_decode_noalloc(void *out, const void *query, const void *key_cache, const void *value_cache,
                      const int32_t *block_tables, int max_blocks_per_seq, const int32_t *context_lens,
                      int num_seqs, int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                      int num_blocks, int max_context_len, float scale, int dtype, int partition_size,
                      int variant, void *stream) {
    pa::clear_error();
    void *ws = nullptr;
    size_t ws_bytes = 0;
    if (partition_size != 0 && num_seqs > 0) {
        const size_t need = pa_decode_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                                      max_context_len, partition_size);
        if (need > (size_t)PA_NOALLOC_SCRATCH_BYTES)
            return pa::fail(PA_ERR_INVALID,
                            "the partials need %zu bytes; the library's fixed scratch holds %zu "
                            "(use pa_decode with a workspace)",
                            need, (size_t)PA_NOALLOC_SCRATCH_BYTES);
        const int rc = scratch_address(&ws);
        if (rc != PA_OK) return rc;
        ws_bytes = (size_t)PA_NOALLOC_SCRATCH_BYTES;
    }
    const int rc = pa_decode(out, query, key_cache, value_cache, block_tables, max_blocks_per_seq, context_lens,
                             num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks,
                             max_context_len, scale, dtype, partition_size, variant, ws, ws_bytes, stream);
    return rc;
}

}  // extern "C"
