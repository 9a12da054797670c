// Read-only streaming probes (measurement only, not part of the computation):
// how fast this GPU reads HBM when nothing else is done with the bytes.
//
//  * contiguous: one buffer, grid-stride, 16-byte loads, four per thread in
//    flight;
//  * scattered tiles: the decode split pass's access pattern without its
//    math. Tile t of a seeded order names one 4 KiB tile in each of two
//    pools (the K and the V tile of one (block, kv head)); wave w streams
//    its own run of the order, each lane loading 16 bytes four times from
//    each pool per tile, and issues the next tile's loads before it folds
//    the current ones into a checksum (one tile in flight while one is
//    consumed).
// Every loaded value reaches `sink`, so no load is dead code.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "pagedkv.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kWave = 64;

__device__ __forceinline__ uint32_t fold(u32x4 v) { return v[0] ^ v[1] ^ v[2] ^ v[3]; }

__global__ __launch_bounds__(256) void stream_contig_kernel(const u32x4* __restrict__ p, size_t n16,
                                                            uint32_t* __restrict__ sink) {
    const size_t stride = static_cast<size_t>(gridDim.x) * blockDim.x;
    size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    uint32_t acc = 0;
    for (; i + 3 * stride < n16; i += 4 * stride) {
        const u32x4 a = __builtin_nontemporal_load(p + i);
        const u32x4 b = __builtin_nontemporal_load(p + i + stride);
        const u32x4 c = __builtin_nontemporal_load(p + i + 2 * stride);
        const u32x4 d = __builtin_nontemporal_load(p + i + 3 * stride);
        acc ^= fold(a) ^ fold(b) ^ fold(c) ^ fold(d);
    }
    for (; i < n16; i += stride) acc ^= fold(__builtin_nontemporal_load(p + i));
    sink[static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x] = acc;
}

template <int kTile16>
__global__ __launch_bounds__(kWave) void stream_tiles_kernel(const u32x4* __restrict__ kp,
                                                             const u32x4* __restrict__ vp,
                                                             const int32_t* __restrict__ order, int tiles,
                                                             uint32_t* __restrict__ sink) {
    const int w = blockIdx.x, W = gridDim.x, lane = threadIdx.x;
    const int t0 = static_cast<int>(static_cast<long long>(w) * tiles / W);
    const int t1 = static_cast<int>(static_cast<long long>(w + 1) * tiles / W);
    constexpr int kPer = kTile16 / kWave;   // loads per lane per tile and pool
    uint32_t acc = 0;
    u32x4 buf[2 * kPer];
    auto issue = [&](int t) {
        const size_t base = static_cast<size_t>(order[t]) * kTile16 + lane;
#pragma unroll
        for (int i = 0; i < kPer; ++i) buf[i] = __builtin_nontemporal_load(kp + base + i * kWave);
#pragma unroll
        for (int i = 0; i < kPer; ++i) buf[kPer + i] = __builtin_nontemporal_load(vp + base + i * kWave);
    };
    if (t0 < t1) issue(t0);
    for (int t = t0; t < t1; ++t) {
        u32x4 cur[2 * kPer];
#pragma unroll
        for (int i = 0; i < 2 * kPer; ++i) cur[i] = buf[i];
        if (t + 1 < t1) issue(t + 1);
#pragma unroll
        for (int i = 0; i < 2 * kPer; ++i) acc ^= fold(cur[i]);
    }
    sink[static_cast<size_t>(w) * kWave + lane] = acc;
}

}  // namespace

extern "C" int pkv_stream_read(const void* a, const void* b, size_t bytes, const int32_t* order, int32_t tiles,
                               int32_t tile_bytes, int32_t workgroups, uint32_t* sink, void* stream) {
    if (!a || !sink) return PKV_ERR_NULL_POINTER;
    if (workgroups < 1) return PKV_ERR_INVALID_ARGUMENT;
    if ((reinterpret_cast<uintptr_t>(a) & 15) || (b && (reinterpret_cast<uintptr_t>(b) & 15)))
        return PKV_ERR_INVALID_ARGUMENT;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (!order) {
        if (bytes % 16) return PKV_ERR_INVALID_ARGUMENT;
        hipLaunchKernelGGL(stream_contig_kernel, dim3(workgroups), dim3(256), 0, st,
                           static_cast<const u32x4*>(a), bytes / 16, sink);
    } else {
        if (!b) return PKV_ERR_NULL_POINTER;
        if (tiles < 0) return PKV_ERR_INVALID_ARGUMENT;
        if (tile_bytes == 4096)
            hipLaunchKernelGGL(stream_tiles_kernel<256>, dim3(workgroups), dim3(kWave), 0, st,
                               static_cast<const u32x4*>(a), static_cast<const u32x4*>(b), order, tiles, sink);
        else if (tile_bytes == 2048)
            hipLaunchKernelGGL(stream_tiles_kernel<128>, dim3(workgroups), dim3(kWave), 0, st,
                               static_cast<const u32x4*>(a), static_cast<const u32x4*>(b), order, tiles, sink);
        else
            return PKV_ERR_INVALID_ARGUMENT;
    }
    return hipGetLastError() == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}
