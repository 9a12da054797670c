// Decode tile math on the matrix cores, for four query heads per kv head.
//
// A tile is one (block, kv head) slice: 16 tokens x 128 dims of K and of V.
// With four query heads sharing the kv head (chapter 5 section 3.1), the
// scores of a tile are a 16 x 4 product over 128 dims and the output update
// a 4 x 128 product over 16 tokens: small, but dense contractions. Both run
// as 16 x 16 MFMAs (heads padded to 16), which costs far fewer issue slots
// than the same products on the vector ALU and leaves the ALU to the
// softmax. Lane l has n = l % 16 and q = l / 16:
//
//  * S^T = K Q^T, four v_mfma_f32_16x16x32_bf16 (A[n][8q + e],
//    B[8q + e][n], D[4q + e][n]): A = token n's K at dims 32b + 8q + e,
//    B = head n's query at the same dims (zero for n >= 4), b = 0..3. The
//    sum over dims does not depend on which dims a lane holds as long as A
//    and B agree, and D gives lane (q, n) head n's scores for tokens
//    4q .. 4q + 3;
//  * O += P V, eight v_mfma_f32_16x16x16_bf16 (A[n][4q + e],
//    B[4q + e][n], D[4q + e][n]): A = head n's weights for tokens 4q + e,
//    exactly the S^T layout above; B = V of those tokens at dim 8n + j for
//    block j = 0..7, so D gives lanes q = 0 head e's output at dims
//    8n .. 8n + 7 across the eight blocks (rows 4 .. 15 stay zero).
//
// Online softmax per head (chapter 5 section 4.1): the 16 lanes of a head
// share one reference max, moved only when a score exceeds it by 2^8 (the
// accumulators are then rescaled; exact, rare). Weights go to the MFMA in
// bf16; the normaliser sums the same weights in fp32.
#pragma once

#include "decode_tile.h"
#include "kernels.h"

namespace pkv {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) short i16x4;

__device__ __forceinline__ float xor16_max(float x) { return fmaxf(x, __shfl_xor(x, 16, kWave)); }

// Operand for the P V product from four tokens' 8-element rows (dims 8n ..
// 8n + 7, bf16): element j of each row, tokens in order.
__device__ __forceinline__ i16x4 v_operand_bf16(const u32x4 (&v)[4], int j) {
    const uint32_t sel = (j & 1) ? 0x07060302u : 0x05040100u;
    const int w = j >> 1;
    const uint32_t lo = __builtin_amdgcn_perm(static_cast<uint32_t>(v[1][w]), static_cast<uint32_t>(v[0][w]), sel);
    const uint32_t hi = __builtin_amdgcn_perm(static_cast<uint32_t>(v[3][w]), static_cast<uint32_t>(v[2][w]), sel);
    return __builtin_bit_cast(i16x4, u32x2{lo, hi});
}

// The same from four tokens' 8-code rows (exact in bf16).
__device__ __forceinline__ i16x4 v_operand_codes(const u32x2 (&v)[4], int j) {
    const int w = j >> 2, byte = j & 3;
    const uint32_t lo = pack2_bf16(code_at(static_cast<uint32_t>(v[0][w]), byte),
                                   code_at(static_cast<uint32_t>(v[1][w]), byte));
    const uint32_t hi = pack2_bf16(code_at(static_cast<uint32_t>(v[2][w]), byte),
                                   code_at(static_cast<uint32_t>(v[3][w]), byte));
    return __builtin_bit_cast(i16x4, u32x2{lo, hi});
}

struct MfmaStateG4 {
    static constexpr float kLazy = 8.0f;
    float mref;        // reference max of head n (log2 units), shared by its 16 lanes
    float mref_safe;   // mref, or 0 while it is still -inf
    float l;           // sum of this lane's weights (head n, tokens 4q .. 4q+3)
    f32x4 acc[8];      // block j: O[4q + e][8n + j]; rows 0..3 (lanes q = 0) are the heads

    __device__ __forceinline__ void reset() {
        mref = -INFINITY;
        mref_safe = 0.0f;
        l = 0.0f;
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    }

    // Raw scores s (head n, tokens 4q + e) -> weights -> O += P V. ks / vs:
    // the K and V scales of tokens 4q + e (8-bit tiles; unused for bf16);
    // vb(j): the V operand of block j.
    template <bool kScaled, class VOperand>
    __device__ __forceinline__ void update(const f32x4 s, const float (&ks)[4], const float (&vs)[4],
                                           VOperand&& vb, int lane, int ntok, float sl2) {
        const int n = lane & 15;
        const int q = lane >> 4;
        float x[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float raw = kScaled ? s[e] * ks[e] : s[e];
            x[e] = 4 * q + e < ntok ? raw * sl2 : -INFINITY;
        }
        float mx = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
        mx = xor16_max(mx);
        mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
        const bool need = n < 4 && mx > mref + kLazy;
        if (__builtin_amdgcn_ballot_w64(need)) {
            const float nref = need ? mx : mref;
            const float alpha = (nref == mref) ? 1.0f : __builtin_amdgcn_exp2f(mref - nref);
            l *= alpha;
            // output rows are heads: head e's factor sits in lane e
            float al[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) al[e] = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(alpha), e));
#pragma unroll
            for (int j = 0; j < 8; ++j)
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[j][e] *= al[e];
            mref = nref;
            mref_safe = (nref == -INFINITY) ? 0.0f : nref;
        }
        float p[4], w[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            p[e] = n < 4 ? __builtin_amdgcn_exp2f(x[e] - mref_safe) : 0.0f;
            // past the sequence end the V scale may be unset: weight 0, no product
            w[e] = kScaled ? (4 * q + e < ntok ? p[e] * vs[e] : 0.0f) : p[e];
        }
        l += (p[0] + p[1]) + (p[2] + p[3]);
        const i16x4 pa = __builtin_bit_cast(i16x4, u32x2{pack2_bf16(w[0], w[1]), pack2_bf16(w[2], w[3])});
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[j] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pa, vb(j), acc[j], 0, 0, 0);
    }

    // This wave's partial for the segment: lanes q = 0 hold the four heads'
    // outputs at dims 8n .. 8n+7; head n's (m, l) goes from lane n.
    __device__ __forceinline__ void write_partial(float* ws_o, PartialML* ws_ml, size_t slot, bool bad,
                                                  int lane) const {
        const int n = lane & 15;
        const int q = lane >> 4;
        float lt = l + __shfl_xor(l, 16, kWave);
        lt += __shfl_xor(lt, 32, kWave);
        if (q == 0) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                float4* o = reinterpret_cast<float4*>(ws_o + (slot * 4 + e) * kTileD + 8 * n);
                o[0] = make_float4(acc[0][e], acc[1][e], acc[2][e], acc[3][e]);
                o[1] = make_float4(acc[4][e], acc[5][e], acc[6][e], acc[7][e]);
            }
            if (n < 4) ws_ml[slot * 4 + n] = bad ? PartialML{NAN, NAN} : PartialML{mref_safe, lt};
        }
    }
};

}  // namespace pkv
