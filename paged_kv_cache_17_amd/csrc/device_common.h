// Device-side helpers shared by the paged-KV kernels (gfx950, wave64).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pkv {

constexpr int kWave = 64;
constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kLog2e = 1.44269504088896340736f;

// bf16 is the upper half of a binary32 value: widening is a shift.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// Round to bf16 (nearest even) with the hardware pack-convert instruction.
__device__ __forceinline__ uint32_t pack2_bf16(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    return static_cast<uint16_t>(pack2_bf16(f, 0.0f) & 0xffffu);
}

template <typename T> struct Elem;
template <> struct Elem<float> {
    __device__ static __forceinline__ float load(const float* p) { return *p; }
    __device__ static __forceinline__ void store(float* p, float v) { *p = v; }
};
template <> struct Elem<uint16_t> {
    __device__ static __forceinline__ float load(const uint16_t* p) {
        return __uint_as_float(static_cast<uint32_t>(*p) << 16);
    }
    __device__ static __forceinline__ void store(uint16_t* p, float v) { *p = f32_to_bf16(v); }
};

// Largest s with start[s] <= row, for a non-decreasing prefix-sum array of
// n+1 entries (result clamped to [0, n-1]).
__device__ __forceinline__ int seq_of_row(const int32_t* __restrict__ start, int n, int row) {
    int lo = 0, hi = n - 1;
    while (lo < hi) {
        int mid = (lo + hi + 1) >> 1;
        if (start[mid] <= row) lo = mid; else hi = mid - 1;
    }
    return lo;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
    return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;
}

// Sum over the 16 lanes of a DPP row (lanes 16r..16r+15): swap neighbours,
// swap pairs, mirror within 8, mirror within 16. Every lane of the row ends
// with the row total.
__device__ __forceinline__ float row16_sum(float v) {
    v += __builtin_amdgcn_update_dpp(0.0f, v, 0xB1, 0xF, 0xF, false);   // quad_perm [1,0,3,2]
    v += __builtin_amdgcn_update_dpp(0.0f, v, 0x4E, 0xF, 0xF, false);   // quad_perm [2,3,0,1]
    v += __builtin_amdgcn_update_dpp(0.0f, v, 0x141, 0xF, 0xF, false);  // row_half_mirror
    v += __builtin_amdgcn_update_dpp(0.0f, v, 0x140, 0xF, 0xF, false);  // row_mirror
    return v;
}

// True when a sequence length can be attended: at least one key, within the
// caller's bound and within what the table row can map.
__device__ __forceinline__ bool seq_len_ok(int L, int need, int max_seq_len, int table_tokens) {
    return L >= 1 && L >= need && L <= max_seq_len && L <= table_tokens;
}

}  // namespace pkv
