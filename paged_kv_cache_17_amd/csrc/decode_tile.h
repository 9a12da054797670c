// Per-tile decode math for bf16 K/V, head_dim 128, block_size 16.
//
// A tile is one (block, kv head) slice: 16 tokens x 128 dims of K (4 KiB,
// contiguous) and the same of V. A wave reads it with four 16-byte loads per
// lane: lane l takes dims 8c..8c+7 (c = l % 16) of token 4i + r
// (r = l / 16) in load i, so each load instruction covers one contiguous
// KiB. Every group of 16 lanes (a DPP row) therefore sees whole tokens and
// keeps its own online-softmax state for the G query heads that share the kv
// head (chapter 5 section 3.1: grouped-query attention; section 4.1: online
// softmax - running max, running sum, rescaled output).
#pragma once

#include "device_common.h"

namespace pkv {

constexpr int kTileD = 128;
constexpr int kTileB = 16;
constexpr int kTileElems = kTileD * kTileB;   // elements of K (or V) per tile

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Each element is copied to a scalar before the bit cast: bit-casting a
// vector element accessor directly (k.y) has been seen to read element 0.
__device__ __forceinline__ float dot2_bf16(uint32_t k, uint32_t q, float acc) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, k), __builtin_bit_cast(bf16x2, q),
                                           acc, false);
}

__device__ __forceinline__ float dot8_bf16(const u32x4 k, const u32x4 q) {
    const uint32_t k0 = k[0], k1 = k[1], k2 = k[2], k3 = k[3];
    const uint32_t q0 = q[0], q1 = q[1], q2 = q[2], q3 = q[3];
    return dot2_bf16(k3, q3, dot2_bf16(k2, q2, dot2_bf16(k1, q1, dot2_bf16(k0, q0, 0.0f))));
}

__device__ __forceinline__ void widen8_bf16(const u32x4 v, float (&f)[8]) {
    const uint32_t v0 = v[0], v1 = v[1], v2 = v[2], v3 = v[3];
    f[0] = bf16_lo(v0); f[1] = bf16_hi(v0);
    f[2] = bf16_lo(v1); f[3] = bf16_hi(v1);
    f[4] = bf16_lo(v2); f[5] = bf16_hi(v2);
    f[6] = bf16_lo(v3); f[7] = bf16_hi(v3);
}

// Quantised tiles (8-bit codes, symmetric absmax, one fp32 scale per token
// and kv head): lane l holds 8 codes (8 bytes) of token 4i + r, dims 8c..8c+7,
// in load i, the same positions as the bf16 layout. A code is a signed
// integer of magnitude <= 127, so it is exact in bf16 and in fp32.
__device__ __forceinline__ float code_at(uint32_t w, int byte) {
    return static_cast<float>(static_cast<int8_t>(static_cast<uint8_t>(w >> (8 * byte))));
}

// Eight codes as four bf16 pairs (exact), for the bf16 dot instruction.
__device__ __forceinline__ u32x4 codes8_to_bf16x8(const u32x2 w) {
    const uint32_t a = w[0], b = w[1];
    u32x4 r;
    r[0] = pack2_bf16(code_at(a, 0), code_at(a, 1));
    r[1] = pack2_bf16(code_at(a, 2), code_at(a, 3));
    r[2] = pack2_bf16(code_at(b, 0), code_at(b, 1));
    r[3] = pack2_bf16(code_at(b, 2), code_at(b, 3));
    return r;
}

__device__ __forceinline__ void widen8_codes(const u32x2 w, float (&f)[8]) {
    const uint32_t a = w[0], b = w[1];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        f[e] = code_at(a, e);
        f[4 + e] = code_at(b, e);
    }
}

// Issue the eight 16-byte loads of one tile (K then V). `k`/`v` point at the
// tile start plus this lane's 8-element offset.
__device__ __forceinline__ void load_tile(const uint16_t* k, const uint16_t* v, u32x4 (&kr)[4], u32x4 (&vr)[4]) {
    const u32x4* kp = reinterpret_cast<const u32x4*>(k);
    const u32x4* vp = reinterpret_cast<const u32x4*>(v);
#pragma unroll
    for (int i = 0; i < 4; ++i) kr[i] = __builtin_nontemporal_load(kp + i * 64);
#pragma unroll
    for (int i = 0; i < 4; ++i) vr[i] = __builtin_nontemporal_load(vp + i * 64);
}

template <int G>
struct DecodeState {
    float m[G];        // running max of scaled scores (log2 units), per head
    float l[G];        // running sum of 2^(s - m)
    float acc[G][8];   // running sum of 2^(s - m) * v for this lane's 8 dims

    __device__ __forceinline__ void reset() {
#pragma unroll
        for (int h = 0; h < G; ++h) {
            m[h] = -INFINITY;
            l[h] = 0.0f;
#pragma unroll
            for (int k = 0; k < 8; ++k) acc[h][k] = 0.0f;
        }
    }

    // Fold one tile into the row state. Tokens 4i + r >= ntok are past the
    // end of the sequence: they get weight 0, and their V (never written,
    // possibly NaN) is replaced by 0 so 0 * NaN cannot reach the sum.
    __device__ __forceinline__ void tile(const u32x4 (&kr)[4], const u32x4 (&vr)[4], const u32x4 (&qv)[G],
                                         int r, int ntok, float sl2) {
        float sc[4][G];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const bool valid = 4 * i + r < ntok;
#pragma unroll
            for (int h = 0; h < G; ++h) {
                const float full = row16_sum(dot8_bf16(kr[i], qv[h]));
                sc[i][h] = valid ? full * sl2 : -INFINITY;
            }
        }
        float vf[4][8];
#pragma unroll
        for (int i = 0; i < 4; ++i) widen8_bf16(vr[i], vf[i]);
        if (ntok < kTileB) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const bool valid = 4 * i + r < ntok;
#pragma unroll
                for (int k = 0; k < 8; ++k) vf[i][k] = valid ? vf[i][k] : 0.0f;
            }
        }
#pragma unroll
        for (int h = 0; h < G; ++h) {
            const float mx = fmaxf(fmaxf(sc[0][h], sc[1][h]), fmaxf(sc[2][h], sc[3][h]));
            const float mn = fmaxf(m[h], mx);
            const float mu = (mn == -INFINITY) ? 0.0f : mn;
            const float alpha = __builtin_amdgcn_exp2f(m[h] - mu);
            float p[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) p[i] = __builtin_amdgcn_exp2f(sc[i][h] - mu);
            l[h] = fmaf(l[h], alpha, (p[0] + p[1]) + (p[2] + p[3]));
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                float x = acc[h][k] * alpha;
#pragma unroll
                for (int i = 0; i < 4; ++i) x = fmaf(p[i], vf[i][k], x);
                acc[h][k] = x;
            }
            m[h] = mn;
        }
    }

    // The same for a quantised tile: scores are code dot products times the
    // token's K scale; V's scale is folded into the weight of each token
    // (the normaliser keeps the unscaled weights). sk[i], sv[i]: scales of
    // token 4i + r. Past the end of the sequence the weight is 0 and the V
    // scale (possibly never written) is not used.
    __device__ __forceinline__ void tile_q8(const u32x2 (&kr)[4], const u32x2 (&vr)[4], const float (&sk)[4],
                                            const float (&sv)[4], const u32x4 (&qv)[G], int r, int ntok,
                                            float sl2) {
        float sc[4][G];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const bool valid = 4 * i + r < ntok;
            const u32x4 kb = codes8_to_bf16x8(kr[i]);
#pragma unroll
            for (int h = 0; h < G; ++h) {
                const float full = row16_sum(dot8_bf16(kb, qv[h]));
                sc[i][h] = valid ? full * sk[i] * sl2 : -INFINITY;
            }
        }
        float vf[4][8];
#pragma unroll
        for (int i = 0; i < 4; ++i) widen8_codes(vr[i], vf[i]);
        float svv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) svv[i] = (4 * i + r < ntok) ? sv[i] : 0.0f;
#pragma unroll
        for (int h = 0; h < G; ++h) {
            const float mx = fmaxf(fmaxf(sc[0][h], sc[1][h]), fmaxf(sc[2][h], sc[3][h]));
            const float mn = fmaxf(m[h], mx);
            const float mu = (mn == -INFINITY) ? 0.0f : mn;
            const float alpha = __builtin_amdgcn_exp2f(m[h] - mu);
            float p[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) p[i] = __builtin_amdgcn_exp2f(sc[i][h] - mu);
            l[h] = fmaf(l[h], alpha, (p[0] + p[1]) + (p[2] + p[3]));
#pragma unroll
            for (int i = 0; i < 4; ++i) p[i] *= svv[i];
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                float x = acc[h][k] * alpha;
#pragma unroll
                for (int i = 0; i < 4; ++i) x = fmaf(p[i], vf[i][k], x);
                acc[h][k] = x;
            }
            m[h] = mn;
        }
    }

    // Combine the four row states (lanes c, c+16, c+32, c+48); afterwards
    // every row holds the wave's merged state.
    __device__ __forceinline__ void merge_rows() {
#pragma unroll
        for (int h = 0; h < G; ++h) {
            float M = fmaxf(m[h], __shfl_xor(m[h], 16, kWave));
            M = fmaxf(M, __shfl_xor(M, 32, kWave));
            const float w = __builtin_amdgcn_exp2f(m[h] - ((M == -INFINITY) ? 0.0f : M));
            float lw = l[h] * w;
            lw += __shfl_xor(lw, 16, kWave);
            lw += __shfl_xor(lw, 32, kWave);
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                float x = acc[h][k] * w;
                x += __shfl_xor(x, 16, kWave);
                x += __shfl_xor(x, 32, kWave);
                acc[h][k] = x;
            }
            m[h] = M;
            l[h] = lw;
        }
    }
};

}  // namespace pkv
