// Split pass of decode attention for bf16 K/V, head_dim 128, block_size 16.
//
// This is the bandwidth-bound stage: every cached K/V byte of a sequence
// is read once (chapter 5 section 2.2: decode re-reads the whole cache every
// step; section 3.2: the kernel follows the block table to scattered
// blocks). Layout of the work:
//  * one workgroup per (key range, kv head, sequence); its WAVES waves take
//    the range's blocks in turn (wave w: blocks w, w + WAVES, ...);
//  * the G query heads sharing a kv head (chapter 5 section 3.1) are all
//    held by every wave, so each K/V tile is read from HBM exactly once;
//  * a (block, kv head) tile of K is 16 tokens x 128 dims = 4 KiB
//    contiguous; lane l loads 16 bytes at l*16 + i*1 KiB (i = 0..3), i.e.
//    dims 8c..8c+7 (c = l % 16) of token 4i + r (r = l / 16): each load
//    instruction reads one contiguous KiB;
//  * q.k partial dots use the bf16 dot2 instruction, then a 4-step DPP sum
//    over the 16 lanes of a row gives every lane the full score of its
//    row's 4 tokens for each of the G heads;
//  * every row of 16 lanes keeps its own online-softmax state per head
//    (max, sum, 8 output dims per lane) over the tokens it sees
//    (chapter 5 section 4.1); the 4 row states and then the wave states
//    are merged once at the end of the range.
// The block table slice of the range is staged in LDS once per workgroup
// and validated there.
#include "device_common.h"
#include "kernels.h"

namespace pkv {
namespace {

constexpr int kD = 128;
constexpr int kBS = 16;
constexpr int kMaxSplitBlocks = 128;   // split_tokens <= 2048

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float dot8(const u32x4& k, const u32x4& q) {
    float acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, k.x),
                                                __builtin_bit_cast(bf16x2, q.x), 0.0f, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, k.y),
                                          __builtin_bit_cast(bf16x2, q.y), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, k.z),
                                          __builtin_bit_cast(bf16x2, q.z), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, k.w),
                                          __builtin_bit_cast(bf16x2, q.w), acc, false);
    return acc;
}

__device__ __forceinline__ void widen8(const u32x4& v, float (&f)[8]) {
    f[0] = bf16_lo(v.x); f[1] = bf16_hi(v.x);
    f[2] = bf16_lo(v.y); f[3] = bf16_hi(v.y);
    f[4] = bf16_lo(v.z); f[5] = bf16_hi(v.z);
    f[6] = bf16_lo(v.w); f[7] = bf16_hi(v.w);
}

template <int G, int WAVES>
__global__ __launch_bounds__(kWave * WAVES) void decode_split_kernel(AttnArgs a) {
    __shared__ int s_tbl[kMaxSplitBlocks];
    __shared__ float s_state[WAVES > 1 ? WAVES : 1][G][kD + 2];

    const int split = blockIdx.x;
    const int g = blockIdx.y;
    const int s = blockIdx.z;
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;

    const int L = a.seq_lens[s];
    if (!seq_len_ok(L, 1, a.max_seq_len, a.table_stride * kBS)) return;
    const int tok_lo = split * a.split_tokens;
    if (tok_lo >= L) return;
    const int tok_hi = min(L, tok_lo + a.split_tokens);
    const int blk_lo = tok_lo / kBS;
    const int nblk = (tok_hi - tok_lo + kBS - 1) / kBS;

    // Stage and validate this range's table slice.
    const int32_t* trow = a.table + static_cast<size_t>(s) * a.table_stride + blk_lo;
    int bad = 0;
    for (int j = tid; j < nblk; j += kWave * WAVES) {
        int b = trow[j];
        if (b < 0 || b >= a.num_blocks) { bad = 1; b = 0; }
        s_tbl[j] = b;
    }
    bad = __syncthreads_or(bad);

    const int n_q = a.n_kv * G;
    const size_t part0 = (static_cast<size_t>(s) * n_q + g * G) * a.max_splits + split;
    if (bad) {
        if (tid < G) a.ws_ml[part0 + static_cast<size_t>(tid) * a.max_splits] = PartialML{NAN, NAN};
        return;
    }

    const int c = lane & 15;   // 8-dim chunk
    const int r = lane >> 4;   // token within each group of 4

    u32x4 qv[G];
    const uint16_t* qbase = static_cast<const uint16_t*>(a.q) + (static_cast<size_t>(s) * n_q + g * G) * kD + c * 8;
#pragma unroll
    for (int h = 0; h < G; ++h) qv[h] = *reinterpret_cast<const u32x4*>(qbase + h * kD);

    float m[G], l[G], acc[G][8];
#pragma unroll
    for (int h = 0; h < G; ++h) {
        m[h] = -INFINITY;
        l[h] = 0.0f;
#pragma unroll
        for (int k = 0; k < 8; ++k) acc[h][k] = 0.0f;
    }

    const size_t tile_stride = static_cast<size_t>(a.n_kv) * kBS * kD;   // elements per block
    const uint16_t* kbase = static_cast<const uint16_t*>(a.k_cache) + static_cast<size_t>(g) * kBS * kD + lane * 8;
    const uint16_t* vbase = static_cast<const uint16_t*>(a.v_cache) + static_cast<size_t>(g) * kBS * kD + lane * 8;
    const float sl2 = a.scale_log2;

    for (int jb = wave; jb < nblk; jb += WAVES) {
        const size_t off = static_cast<size_t>(s_tbl[jb]) * tile_stride;
        const u32x4* kp = reinterpret_cast<const u32x4*>(kbase + off);
        const u32x4* vp = reinterpret_cast<const u32x4*>(vbase + off);
        u32x4 kr[4], vr[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) kr[i] = __builtin_nontemporal_load(kp + i * 64);
#pragma unroll
        for (int i = 0; i < 4; ++i) vr[i] = __builtin_nontemporal_load(vp + i * 64);

        const int tok0 = tok_lo + jb * kBS + r;
        float sc[4][G];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const bool valid = tok0 + 4 * i < tok_hi;
#pragma unroll
            for (int h = 0; h < G; ++h) {
                const float full = row16_sum(dot8(kr[i], qv[h]));
                sc[i][h] = valid ? full * sl2 : -INFINITY;
            }
        }
        float vf[4][8];
#pragma unroll
        for (int i = 0; i < 4; ++i) widen8(vr[i], vf[i]);
        if (tok_lo + (jb + 1) * kBS > tok_hi) {
            // Last, partly filled block: slots past the sequence end hold
            // whatever was there before (never written); their weight is 0,
            // and 0 * NaN must not reach the sum.
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const bool valid = tok0 + 4 * i < tok_hi;
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

    // Merge the 4 row states of this wave (lanes c, c+16, c+32, c+48).
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

    if constexpr (WAVES == 1) {
        if (r == 0) {
#pragma unroll
            for (int h = 0; h < G; ++h) {
                const size_t part = part0 + static_cast<size_t>(h) * a.max_splits;
                float4* o = reinterpret_cast<float4*>(a.ws_o + part * kD + c * 8);
                o[0] = make_float4(acc[h][0], acc[h][1], acc[h][2], acc[h][3]);
                o[1] = make_float4(acc[h][4], acc[h][5], acc[h][6], acc[h][7]);
                if (c == 0) a.ws_ml[part] = PartialML{m[h], l[h]};
            }
        }
    } else {
        if (r == 0) {
#pragma unroll
            for (int h = 0; h < G; ++h) {
#pragma unroll
                for (int k = 0; k < 8; ++k) s_state[wave][h][c * 8 + k] = acc[h][k];
                if (c == 0) {
                    s_state[wave][h][kD] = m[h];
                    s_state[wave][h][kD + 1] = l[h];
                }
            }
        }
        __syncthreads();
        // Merge the wave states: thread tid covers (head, dim) pairs.
        for (int e = tid; e < G * kD; e += kWave * WAVES) {
            const int h = e / kD;
            const int k = e % kD;
            float M = -INFINITY;
#pragma unroll
            for (int w = 0; w < WAVES; ++w) M = fmaxf(M, s_state[w][h][kD]);
            const float mu = (M == -INFINITY) ? 0.0f : M;
            float x = 0.0f, lw = 0.0f;
#pragma unroll
            for (int w = 0; w < WAVES; ++w) {
                const float wt = __builtin_amdgcn_exp2f(s_state[w][h][kD] - mu);
                x = fmaf(wt, s_state[w][h][k], x);
                lw = fmaf(wt, s_state[w][h][kD + 1], lw);
            }
            const size_t part = part0 + static_cast<size_t>(h) * a.max_splits;
            a.ws_o[part * kD + k] = x;
            if (k == 0) a.ws_ml[part] = PartialML{M, lw};
        }
    }
}

template <int G>
hipError_t launch_g(const AttnArgs& a, hipStream_t stream) {
    constexpr int kWaves = 4;
    const dim3 grid(a.max_splits, a.n_kv, a.num_seqs);
    hipLaunchKernelGGL((decode_split_kernel<G, kWaves>), grid, dim3(kWave * kWaves), 0, stream, a);
    return hipGetLastError();
}

}  // namespace

bool decode_fast_supported(int n_q, int n_kv, int head_dim, int block_size, int split_tokens) {
    if (head_dim != kD || block_size != kBS || n_kv < 1 || n_q % n_kv) return false;
    if (split_tokens % kBS || split_tokens / kBS > kMaxSplitBlocks) return false;
    const int G = n_q / n_kv;
    return G == 1 || G == 2 || G == 4 || G == 8;
}

hipError_t launch_decode_fast(const AttnArgs& a, hipStream_t stream) {
    switch (a.n_q / a.n_kv) {
        case 1: return launch_g<1>(a, stream);
        case 2: return launch_g<2>(a, stream);
        case 4: return launch_g<4>(a, stream);
        case 8: return launch_g<8>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace pkv
