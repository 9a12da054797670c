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

// Rows of the products: (query i, head h) pairs of one kv head, row r =
// i * G + h, in NB blocks of 16 (decode: the G heads of one query, NB = 1;
// small chunks: up to 32 rows, NB = 2). Lane (q, n) owns row 16b + n of
// block b for the softmax and rows 16b + 4q + e of the output. `ok` marks
// rows that exist; `back` = C - 1 - i, the number of the chunk's last keys
// row r may not see (0 for decode). With ntok = the sequence's keys from
// the tile's first key to its end (not capped at the tile), row r sees the
// tile's tokens below ntok - back (chapter 5 section 4.1 and the lab's
// causal chunk mask: query i at position L - C + i sees keys up to it).
template <int NB>
struct MfmaState {
    static constexpr float kLazy = 8.0f;
    float mref[NB];       // reference max of row 16b + n (log2 units), shared by its lanes
    float mref_safe[NB];  // mref, or 0 while it is still -inf
    float l[NB];          // sum of this lane's weights (row 16b + n, tokens 4q .. 4q+3)
    f32x4 acc[NB][8];     // block b, dim block j: O[row 16b + 4q + e][8n + j]
    bool ok[NB];          // row 16b + n exists
    int back[NB];         // keys at the end of the chunk row 16b + n may not see

    __device__ __forceinline__ void reset() {
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            mref[b] = -INFINITY;
            mref_safe[b] = 0.0f;
            l[b] = 0.0f;
#pragma unroll
            for (int j = 0; j < 8; ++j) acc[b][j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        }
    }

    // Raw scores s[b] (row 16b + n, tokens 4q + e) -> weights -> O += P V.
    // ks / vs: the K and V scales of tokens 4q + e (8-bit tiles; unused for
    // bf16); vb(j): the V operand of dim block j.
    template <bool kScaled, class VOperand>
    __device__ __forceinline__ void update(const f32x4 (&s)[NB], const float (&ks)[4], const float (&vs)[4],
                                           VOperand&& vb, int lane, int ntok, float sl2) {
        const int q = lane >> 4;
        i16x4 pa[NB];
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            const int lim = ntok - back[b];   // tokens 4q + e < lim are seen by this row
            float x[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float raw = kScaled ? s[b][e] * ks[e] : s[b][e];
                x[e] = 4 * q + e < lim ? raw * sl2 : -INFINITY;
            }
            float mx = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
            mx = xor16_max(mx);
            mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
            const bool need = ok[b] && mx > mref[b] + kLazy;
            if (__builtin_amdgcn_ballot_w64(need)) {
                const float nref = need ? mx : mref[b];
                const float alpha = (nref == mref[b]) ? 1.0f : __builtin_amdgcn_exp2f(mref[b] - nref);
                l[b] *= alpha;
                // output row 4q + e of the block takes the factor of lane 4q + e
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float al = __shfl(alpha, 4 * q + e, kWave);
#pragma unroll
                    for (int j = 0; j < 8; ++j) acc[b][j][e] *= al;
                }
                mref[b] = nref;
                mref_safe[b] = (nref == -INFINITY) ? 0.0f : nref;
            }
            float p[4], w[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                p[e] = ok[b] ? __builtin_amdgcn_exp2f(x[e] - mref_safe[b]) : 0.0f;
                // past the sequence end the V scale may be unset: weight 0, no product
                w[e] = kScaled ? (4 * q + e < lim ? p[e] * vs[e] : 0.0f) : p[e];
            }
            l[b] += (p[0] + p[1]) + (p[2] + p[3]);
            pa[b] = __builtin_bit_cast(i16x4, u32x2{pack2_bf16(w[0], w[1]), pack2_bf16(w[2], w[3])});
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const i16x4 v = vb(j);
#pragma unroll
            for (int b = 0; b < NB; ++b) acc[b][j] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pa[b], v, acc[b][j], 0, 0, 0);
        }
    }

    // This wave's partial for the segment, `rows` rows per slot (rows <
    // `used` exist): lane (q, n) stores rows 16b + 4q + e at dims 8n .. 8n+7,
    // and the (m, l) of row 16b + n (m = -inf for a row that saw no key).
    __device__ __forceinline__ void write_partial(float* ws_o, PartialML* ws_ml, size_t slot, int rows, int used,
                                                  bool bad, int lane) const {
        const int n = lane & 15;
        const int q = lane >> 4;
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            float lt = l[b] + __shfl_xor(l[b], 16, kWave);
            lt += __shfl_xor(lt, 32, kWave);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 16 * b + 4 * q + e;
                if (r < used) {
                    float4* o = reinterpret_cast<float4*>(ws_o + (slot * rows + r) * kTileD + 8 * n);
                    o[0] = make_float4(acc[b][0][e], acc[b][1][e], acc[b][2][e], acc[b][3][e]);
                    o[1] = make_float4(acc[b][4][e], acc[b][5][e], acc[b][6][e], acc[b][7][e]);
                }
            }
            const int r = 16 * b + n;
            if (q == 0 && r < used)
                ws_ml[slot * rows + r] = bad ? PartialML{NAN, NAN}
                                             : PartialML{lt > 0.0f ? mref_safe[b] : -INFINITY, lt};
        }
    }
};

}  // namespace pkv
