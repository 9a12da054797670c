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

}  // namespace

hipError_t launch_merge(const AttnArgs& a, void* out, float* lse, bool bf16, hipStream_t stream) {
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
