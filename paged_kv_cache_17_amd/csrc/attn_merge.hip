// Merge pass: combine each query row's per-range softmax states.
//
// Chapter 5 section 4.1 (online softmax): partial results computed over
// separate key tiles combine exactly once each is rescaled by
// exp(m_j - M), M the largest partial max. With per-range max m_j, sum l_j
// and unnormalised output o_j (all in log2 units here):
//   w_j = 2^(m_j - M),  out = sum_j w_j o_j / sum_j w_j l_j,
//   lse = ln 2 * (M + log2(sum_j w_j l_j)).
// Ranges are merged in index order, so results do not depend on timing.
#include "device_common.h"
#include "kernels.h"

namespace pkv {
namespace {

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
    int nsplit = 0;
    if (ok) {
        const int t = L - C + i;
        nsplit = (t + a.split_tokens) / a.split_tokens;   // ranges holding keys 0..t
        ok = nsplit <= a.max_splits;
    }
    const size_t base = (static_cast<size_t>(row) * a.n_q + h) * a.max_splits;
    float M = -INFINITY;
    bool nan = !ok;
    for (int j = 0; j < nsplit && ok; ++j) {
        const float m = a.ws_ml[base + j].m;
        nan |= isnan(m);
        M = fmaxf(M, m);
    }
    if (nan) {
        for (int k = threadIdx.x; k < d; k += blockDim.x) Elem<T>::store(orow + k, NAN);
        if (lse && threadIdx.x == 0) lse[static_cast<size_t>(row) * a.n_q + h] = NAN;
        return;
    }
    float den = 0.0f;
    for (int j = 0; j < nsplit; ++j) {
        const PartialML p = a.ws_ml[base + j];
        den = fmaf(exp2f(p.m - M), p.l, den);
    }
    const float inv = 1.0f / den;
    for (int k = threadIdx.x; k < d; k += blockDim.x) {
        float num = 0.0f;
        for (int j = 0; j < nsplit; ++j)
            num = fmaf(exp2f(a.ws_ml[base + j].m - M), a.ws_o[(base + j) * d + k], num);
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
