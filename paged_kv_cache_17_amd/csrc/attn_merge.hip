// Merge pass: combine each query row's per-range softmax states.
//
// Chapter 5 section 4.1 (online softmax): partial results computed over
// separate key tiles combine exactly once each is rescaled by
// exp(m_j - M), M the largest partial max. With per-range max m_j, sum l_j
// and unnormalised output o_j (all in log2 units here):
//   w_j = 2^(m_j - M),  out = sum_j w_j o_j / sum_j w_j l_j,
//   lse = ln 2 * (M + log2(sum_j w_j l_j)).
// Partials are merged in index order, so results do not depend on timing.
//
// Where a row's partials live depends on the first pass:
//  * fixed split: slots (row, head, j) for the ranges j holding keys 0..t;
//  * balanced decode: with T tiles spread over W' = min(W, T) non-empty
//    waves, the waves covering the row's (sequence, kv head) tile segment
//    wrote slots w + segment for w in [wave_of(first tile),
//    wave_of(last tile)], each holding the G heads of the kv head.
#include "device_common.h"
#include "kernels.h"

namespace pkv {
namespace {

// Wave whose tile range [floor(wT/W), floor((w+1)T/W)) contains tile t.
__device__ __forceinline__ long long wave_of(long long t, long long W, long long T) {
    return ((t + 1) * W + T - 1) / T - 1;
}

template <typename T>
__global__ __launch_bounds__(128) void merge_kernel(AttnArgs a, T* __restrict__ out,
                                                    float* __restrict__ lse) {
    const int row = blockIdx.x;
    const int h = blockIdx.y;
    int s = row, C = 1, i = 0;
    if (a.q_start) {
        s = seq_of_row(a.q_start, a.num_seqs, row);
        C = a.q_start[s + 1] - a.q_start[s];
        i = row - a.q_start[s];
    }
    const int L = a.seq_lens[s];
    const int d = a.head_dim;
    T* orow = out + (static_cast<size_t>(row) * a.n_q + h) * d;
    bool ok = C >= 1 && i >= 0 && i < C && seq_len_ok(L, C, a.max_seq_len, a.table_stride * a.block_size);
    size_t first = 0, step = 1;
    int count = 0;
    if (ok && a.waves > 0) {
        const int G = a.n_q / a.n_kv;
        const int g = h / G;
        const long long P = a.prefix[s];
        const long long nb = a.prefix[s + 1] - P;
        const long long Tt = static_cast<long long>(a.n_kv) * a.prefix[a.num_seqs];
        ok = nb == (L + a.block_size - 1) / a.block_size && Tt > 0;
        if (ok) {
            const long long t_first = a.n_kv * P + g * nb;
            const long long Wt = Tt < a.waves ? Tt : a.waves;
            const long long w_lo = wave_of(t_first, Wt, Tt);
            const long long w_hi = wave_of(t_first + nb - 1, Wt, Tt);
            const long long seg = static_cast<long long>(s) * a.n_kv + g;
            first = static_cast<size_t>((w_lo + seg) * G + (h - g * G));
            step = G;
            count = static_cast<int>(w_hi - w_lo + 1);
        }
    } else if (ok) {
        const int t = L - C + i;
        count = (t + a.split_tokens) / a.split_tokens;   // ranges holding keys 0..t
        ok = count <= a.max_splits;
        first = (static_cast<size_t>(row) * a.n_q + h) * a.max_splits;
    }
    float M = -INFINITY;
    bool nan = !ok;
    for (int j = 0; j < count && ok; ++j) {
        const float m = a.ws_ml[first + j * step].m;
        nan |= isnan(m);
        M = fmaxf(M, m);
    }
    if (nan) {
        for (int k = threadIdx.x; k < d; k += blockDim.x) Elem<T>::store(orow + k, NAN);
        if (lse && threadIdx.x == 0) lse[static_cast<size_t>(row) * a.n_q + h] = NAN;
        return;
    }
    float den = 0.0f;
    for (int j = 0; j < count; ++j) {
        const PartialML p = a.ws_ml[first + j * step];
        den = fmaf(exp2f(p.m - M), p.l, den);
    }
    const float inv = 1.0f / den;
    for (int k = threadIdx.x; k < d; k += blockDim.x) {
        float num = 0.0f;
        for (int j = 0; j < count; ++j) {
            const size_t idx = first + j * step;
            num = fmaf(exp2f(a.ws_ml[idx].m - M), a.ws_o[idx * d + k], num);
        }
        Elem<T>::store(orow + k, num * inv);
    }
    if (lse && threadIdx.x == 0) lse[static_cast<size_t>(row) * a.n_q + h] = kLn2 * (M + log2f(den));
}

// Balanced-decode merge: one workgroup per (sequence, kv head) combines the
// G heads' partials. Everything a row needs is fetched in three dependent
// rounds: the sequence's length and prefix entries, the partials' (m, l)
// (their weights staged in LDS), then the partial outputs (one element per
// thread and partial). A segment spread over more than kMergeMaxParts waves
// recomputes the weights on the fly instead of staging them.
constexpr int kMergeMaxParts = 256;

template <int G>
__global__ __launch_bounds__(256) void merge_balanced_kernel(AttnArgs a, uint16_t* __restrict__ out,
                                                             float* __restrict__ lse) {
    constexpr int D = 128;
    __shared__ float s_w[kMergeMaxParts][G];     // weights 2^(m_j - M_h)
    __shared__ float s_M[G];
    __shared__ float s_inv[G];
    __shared__ float s_lse[G];
    __shared__ int s_info[3];                    // count, first slot, ok
    const int s = blockIdx.x;
    const int g = blockIdx.y;
    const int tid = threadIdx.x;
    if (tid == 0) {
        const int L = a.seq_lens[s];
        const long long P = a.prefix[s];
        const long long nb = a.prefix[s + 1] - P;
        const long long Tt = static_cast<long long>(a.n_kv) * a.prefix[a.num_seqs];
        bool ok = seq_len_ok(L, 1, a.max_seq_len, a.table_stride * a.block_size) &&
                  nb == (L + a.block_size - 1) / a.block_size && Tt > 0;
        int count = 0;
        long long first = 0;
        if (ok) {
            const long long t_first = a.n_kv * P + g * nb;
            const long long Wt = Tt < a.waves ? Tt : a.waves;
            const long long w_lo = wave_of(t_first, Wt, Tt);
            const long long w_hi = wave_of(t_first + nb - 1, Wt, Tt);
            first = w_lo + static_cast<long long>(s) * a.n_kv + g;
            count = static_cast<int>(w_hi - w_lo + 1);
        }
        s_info[0] = count;
        s_info[1] = static_cast<int>(first);
        s_info[2] = ok;
    }
    __syncthreads();
    const int count = s_info[0];
    const size_t first = static_cast<size_t>(s_info[1]);
    const bool ok = s_info[2];
    const bool staged = count <= kMergeMaxParts;
    if (ok && tid < G) {
        const int h = tid;
        float M = -INFINITY;
        bool nan = false;
        for (int j = 0; j < count; ++j) {
            const float m = a.ws_ml[(first + j) * G + h].m;
            nan |= isnan(m);
            M = fmaxf(M, m);
        }
        float den = 0.0f;
        for (int j = 0; j < count; ++j) {
            const PartialML p = a.ws_ml[(first + j) * G + h];
            const float w = exp2f(p.m - M);
            if (staged) s_w[j][h] = w;
            den = fmaf(w, p.l, den);
        }
        s_M[h] = M;
        s_inv[h] = nan ? NAN : 1.0f / den;
        s_lse[h] = nan ? NAN : kLn2 * (M + log2f(den));
    }
    __syncthreads();
    uint16_t* obase = out + (static_cast<size_t>(s) * a.n_q + g * G) * D;
    for (int e = tid; e < G * D; e += 256) {
        const int h = e / D;
        const int k = e - h * D;
        float num = 0.0f;
        float inv = NAN;
        if (ok && staged) {
#pragma unroll 4
            for (int j = 0; j < count; ++j) num = fmaf(s_w[j][h], a.ws_o[((first + j) * G + h) * D + k], num);
            inv = s_inv[h];
        } else if (ok) {
            const float M = s_M[h];
            for (int j = 0; j < count; ++j)
                num = fmaf(exp2f(a.ws_ml[(first + j) * G + h].m - M), a.ws_o[((first + j) * G + h) * D + k], num);
            inv = s_inv[h];
        }
        obase[e] = f32_to_bf16(num * inv);
    }
    if (lse && tid < G) lse[static_cast<size_t>(s) * a.n_q + g * G + tid] = ok ? s_lse[tid] : NAN;
}

}  // namespace

hipError_t launch_merge(const AttnArgs& a, void* out, float* lse, bool bf16, hipStream_t stream) {
    if (a.waves > 0 && bf16 && a.head_dim == 128) {
        const dim3 grid(a.num_seqs, a.n_kv);
        auto out16 = static_cast<uint16_t*>(out);
        switch (a.n_q / a.n_kv) {
            case 1: hipLaunchKernelGGL(merge_balanced_kernel<1>, grid, dim3(256), 0, stream, a, out16, lse); break;
            case 2: hipLaunchKernelGGL(merge_balanced_kernel<2>, grid, dim3(256), 0, stream, a, out16, lse); break;
            case 4: hipLaunchKernelGGL(merge_balanced_kernel<4>, grid, dim3(256), 0, stream, a, out16, lse); break;
            case 8: hipLaunchKernelGGL(merge_balanced_kernel<8>, grid, dim3(256), 0, stream, a, out16, lse); break;
            default: return hipErrorInvalidValue;
        }
        return hipGetLastError();
    }
    const dim3 grid(a.num_rows, a.n_q);
    if (bf16)
        hipLaunchKernelGGL(merge_kernel<uint16_t>, grid, dim3(128), 0, stream, a,
                           static_cast<uint16_t*>(out), lse);
    else
        hipLaunchKernelGGL(merge_kernel<float>, grid, dim3(128), 0, stream, a,
                           static_cast<float*>(out), lse);
    return hipGetLastError();
}

}  // namespace pkv
