// paged_attn_decode_append_noalloc: the one-call decode step with its
// split-K workspace in a static device array instead of a caller buffer, for
// callers that cannot allocate device memory (code under stream capture,
// serving loops and harnesses that forbid hipMalloc).
//
// The array lives in this library's code object; every GPU the library runs
// on holds its own copy until the process ends. Host code never passes the
// array's name to a kernel (on the host it is only a stand-in symbol): the
// device address is looked up once per device with hipGetSymbolAddress, with
// that device current, and that address is what the kernels receive.
#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>
#include <mutex>

#include "pagedkv.h"

namespace {

constexpr size_t kScratchBytes = PKV_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's copy of `scratch` (looked up on the
// first call on that device), or an error status.
int scratch_for_current_device(void** out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return PKV_ERR_HIP;
    if (dev < 0 || dev >= kMaxDevices) return PKV_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return PKV_ERR_HIP;
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return PKV_OK;
}

}  // namespace

extern "C" int paged_attn_decode_append_noalloc(void* out, float* lse, const void* q, void* k_cache, void* v_cache,
                                                const void* k_new, const void* v_new, const int32_t* block_table,
                                                int32_t table_stride, const int32_t* seq_lens, int32_t num_seqs,
                                                int32_t max_seq_len, int32_t num_blocks, int32_t n_q, int32_t n_kv,
                                                int32_t head_dim, int32_t block_size, float scale, int32_t dtype,
                                                void* stream) {
    void* ws = nullptr;
    const int rc0 = scratch_for_current_device(&ws);
    if (rc0 != PKV_OK) return rc0;
    // the same entry point, on the static array; it validates everything
    // (workspace size included) before launching anything
    const int rc = paged_attn_decode_append(out, lse, q, k_cache, v_cache, k_new, v_new, block_table, table_stride,
                                            seq_lens, num_seqs, max_seq_len, num_blocks, n_q, n_kv, head_dim,
                                            block_size, scale, dtype, ws, kScratchBytes, stream);
    return rc == PKV_ERR_WORKSPACE_TOO_SMALL ? PKV_ERR_SCRATCH_LIMIT : rc;
}
