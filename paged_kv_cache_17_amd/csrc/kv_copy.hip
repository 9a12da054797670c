// Whole-block copies inside the K/V pools: the data side of copy-on-write.
//
// Serving tutorial section 4.2: when a block shared by several sequences
// (a common prefix, or the prompt's tail block under beam / parallel
// sampling) is about to be written by one of them, that sequence gets a
// copy of the block and its table entry is remapped; the shared copy is
// never modified in place. kvpool_cow picks the new block ids; this kernel
// copies the contents. A block is contiguous in each pool
// ([num_blocks][n_kv][B][d]: n_kv * B * d elements), so a copy is two plain
// memcpy's of block_bytes; one workgroup per (pair, pool) streams it with
// 16-byte accesses when sizes and addresses allow.
#include "device_common.h"
#include "kernels.h"

namespace pkv {
namespace {

constexpr int kCopyThreads = 256;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// kUnit: bytes per access - 16 when sizes and addresses allow, else 2, else
// 1 (an 8-bit pool whose block is an odd number of bytes).
template <int kUnit>
__global__ __launch_bounds__(kCopyThreads) void copy_blocks_kernel(char* __restrict__ k_cache,
                                                                   char* __restrict__ v_cache,
                                                                   const int32_t* __restrict__ src_ids,
                                                                   const int32_t* __restrict__ dst_ids,
                                                                   int num_blocks, size_t block_bytes) {
    const int pair = blockIdx.x;
    char* pool = blockIdx.y == 0 ? k_cache : v_cache;
    const int src = src_ids[pair];
    const int dst = dst_ids[pair];
    // ids the host could not check: a pair naming a block outside the pool
    // (or a block onto itself) is skipped
    if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks || src == dst) return;
    const char* s = pool + static_cast<size_t>(src) * block_bytes;
    char* d = pool + static_cast<size_t>(dst) * block_bytes;
    if constexpr (kUnit == 16) {
        const size_t n = block_bytes / 16;
        const u32x4* s4 = reinterpret_cast<const u32x4*>(s);
        u32x4* d4 = reinterpret_cast<u32x4*>(d);
        for (size_t i = threadIdx.x; i < n; i += kCopyThreads) d4[i] = __builtin_nontemporal_load(s4 + i);
    } else if constexpr (kUnit == 2) {
        const size_t n = block_bytes / 2;
        const uint16_t* s2 = reinterpret_cast<const uint16_t*>(s);
        uint16_t* d2 = reinterpret_cast<uint16_t*>(d);
        for (size_t i = threadIdx.x; i < n; i += kCopyThreads) d2[i] = s2[i];
    } else {
        for (size_t i = threadIdx.x; i < block_bytes; i += kCopyThreads) d[i] = s[i];
    }
}

}  // namespace

hipError_t launch_copy_blocks(void* k_cache, void* v_cache, const int32_t* src_ids, const int32_t* dst_ids,
                              int n, int num_blocks, size_t block_bytes, hipStream_t stream) {
    const dim3 grid(n, 2);
    const uintptr_t addr = reinterpret_cast<uintptr_t>(k_cache) | reinterpret_cast<uintptr_t>(v_cache);
    char* k = static_cast<char*>(k_cache);
    char* v = static_cast<char*>(v_cache);
    if (block_bytes % 16 == 0 && (addr & 15) == 0)
        hipLaunchKernelGGL(copy_blocks_kernel<16>, grid, dim3(kCopyThreads), 0, stream, k, v, src_ids, dst_ids,
                           num_blocks, block_bytes);
    else if (block_bytes % 2 == 0 && (addr & 1) == 0)
        hipLaunchKernelGGL(copy_blocks_kernel<2>, grid, dim3(kCopyThreads), 0, stream, k, v, src_ids, dst_ids,
                           num_blocks, block_bytes);
    else
        hipLaunchKernelGGL(copy_blocks_kernel<1>, grid, dim3(kCopyThreads), 0, stream, k, v, src_ids, dst_ids,
                           num_blocks, block_bytes);
    return hipGetLastError();
}

}  // namespace pkv
