// Split pass for any head width, block size, group size and dtype.
//
// One wave handles one (query row, query head, key range). It reads the
// query into LDS, scores every allowed key of its range (one key per lane,
// gathering the key's block through the table), takes the range's max and
// the sum of 2^(score - max), then accumulates the weighted values (one
// output element per lane). The range's state (max, sum, unnormalised
// output) goes to the workspace for the merge pass.
//
// Scores: lab page (Inference Engineering), function forward - q.k scaled,
// causal mask j <= position, max-subtracted softmax, weighted sum of V.
// Split state: chapter 5 section 4.1 (per-tile max, sum and output).
// Scores are kept in log2 units (scale * log2 e folded in) so the
// exponentials are exp2.
#include "device_common.h"
#include "kernels.h"

namespace pkv {
namespace {

template <typename T>
__global__ __launch_bounds__(kWave) void split_generic_kernel(AttnArgs a) {
    extern __shared__ float smem[];
    const int row = blockIdx.x;
    const int h = blockIdx.y;
    const int split = blockIdx.z;
    const int lane = threadIdx.x;

    int s = row, C = 1, i = 0;
    if (a.q_start) {
        s = seq_of_row(a.q_start, a.num_seqs, row);
        C = a.q_start[s + 1] - a.q_start[s];
        i = row - a.q_start[s];
    }
    const int L = a.seq_lens[s];
    if (C < 1 || i < 0 || i >= C || !seq_len_ok(L, C, a.max_seq_len, a.table_stride * a.block_size))
        return;   // the merge pass writes NaN for this row
    const int t = L - C + i;                  // absolute position: keys 0..t are allowed
    const int lo = split * a.split_tokens;
    if (lo > t) return;                       // range holds no allowed key
    const int hi = min(t + 1, lo + a.split_tokens);

    const int d = a.head_dim, bs = a.block_size;
    const int g = h / (a.n_q / a.n_kv);
    float* qs = smem;
    float* sc = smem + d;
    const T* qrow = static_cast<const T*>(a.q) + (static_cast<size_t>(row) * a.n_q + h) * d;
    for (int k = lane; k < d; k += kWave) qs[k] = Elem<T>::load(qrow + k);
    __syncthreads();

    const int32_t* trow = a.table + static_cast<size_t>(s) * a.table_stride;
    const T* kc = static_cast<const T*>(a.k_cache);
    const T* vc = static_cast<const T*>(a.v_cache);
    bool bad = false;
    float mloc = -INFINITY;
    for (int j = lo + lane; j < hi; j += kWave) {
        const int blk = trow[j / bs];
        float v = 0.0f;
        if (blk < 0 || blk >= a.num_blocks) {
            bad = true;
        } else {
            const T* kp = kc + ((static_cast<size_t>(blk) * a.n_kv + g) * bs + j % bs) * d;
            float acc = 0.0f;
            for (int k = 0; k < d; ++k) acc = fmaf(qs[k], Elem<T>::load(kp + k), acc);
            v = acc * a.scale_log2;
        }
        sc[j - lo] = v;
        mloc = fmaxf(mloc, v);
    }
    const size_t part = (static_cast<size_t>(row) * a.n_q + h) * a.max_splits + split;
    if (__any(bad)) {
        if (lane == 0) a.ws_ml[part] = PartialML{NAN, NAN};
        return;
    }
    const float m = wave_max(mloc);
    __syncthreads();
    float lsum = 0.0f;
    for (int j = lo + lane; j < hi; j += kWave) {
        const float p = exp2f(sc[j - lo] - m);
        sc[j - lo] = p;
        lsum += p;
    }
    const float l = wave_sum(lsum);
    __syncthreads();
    float* o = a.ws_o + part * d;
    for (int k = lane; k < d; k += kWave) {
        float acc = 0.0f;
        for (int j = lo; j < hi; ++j) {
            const int blk = trow[j / bs];
            acc = fmaf(sc[j - lo], Elem<T>::load(vc + ((static_cast<size_t>(blk) * a.n_kv + g) * bs + j % bs) * d + k), acc);
        }
        o[k] = acc;
    }
    if (lane == 0) a.ws_ml[part] = PartialML{m, l};
}

}  // namespace

hipError_t launch_split_generic(const AttnArgs& a, bool bf16, hipStream_t stream) {
    const dim3 grid(a.num_rows, a.n_q, a.max_splits);
    const size_t lds = sizeof(float) * (static_cast<size_t>(a.head_dim) + a.split_tokens);
    if (bf16)
        hipLaunchKernelGGL(split_generic_kernel<uint16_t>, grid, dim3(kWave), lds, stream, a);
    else
        hipLaunchKernelGGL(split_generic_kernel<float>, grid, dim3(kWave), lds, stream, a);
    return hipGetLastError();
}

}  // namespace pkv
