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

// Balanced merge: one workgroup of 256 threads per (sequence, kv head)
// combines the rows' partials in three rounds of independent loads: (1) the
// sequence's length, query rows and prefix entries; (2) every partial's
// (m, l) for the rows, one partial per thread, staged in LDS, then per row a
// wave reduces the maximum and the weighted sum; (3) the partial outputs,
// four dims per thread, all partials' loads in flight together. Rows are
// (query i, head h) pairs, r = i * G + h, RS per partial slot: decode has
// one query (RS = G), small chunks C_s <= RS / G queries (RS = 32), written
// to row q_start[s] + i. A workgroup takes RB of the rows (rows RB * z ..,
// z = blockIdx.z), so small chunks spread over several workgroups.
constexpr int kMergeThreads = 256;
constexpr int kMergeMaxParts = 256;   // partials staged at once in LDS

template <int G, int RS, int RB>
__global__ __launch_bounds__(kMergeThreads) void merge_balanced_kernel(AttnArgs a, uint16_t* __restrict__ out,
                                                                       float* __restrict__ lse) {
    constexpr int D = 128;
    __shared__ float s_m[kMergeMaxParts][RB];    // m_j, then the weight 2^(m_j - M)
    __shared__ float s_l[kMergeMaxParts][RB];
    __shared__ float s_M[RB];
    __shared__ float s_den[RB];
    __shared__ int s_info[5];                    // count, first slot, ok, first query row, rows used
    const int s = blockIdx.x;
    const int g = blockIdx.y;
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    if (tid == 0) {
        // every load of this round is unconditional, so they are in flight
        // together (decode has no q_start: prefix stands in, unused)
        const int32_t* qsp = a.q_start ? a.q_start : a.prefix;
        const int L = a.seq_lens[s];
        const int q0 = qsp[s], q1 = qsp[s + 1];
        const int p0 = a.prefix[s], p1 = a.prefix[s + 1], pS = a.prefix[a.num_seqs];
        const int row0 = a.q_start ? q0 : s;
        const int C = a.q_start ? q1 - q0 : 1;
        const long long P = p0;
        const long long nb = p1 - p0;
        const long long Tt = static_cast<long long>(a.n_kv) * pS;
        // (& rather than &&: the length's load then stays with the others)
        bool ok = (C >= 1) & (C * G <= RS) & seq_len_ok(L, C, a.max_seq_len, a.table_stride * a.block_size) &
                  (nb == (L + a.block_size - 1) / a.block_size) & (Tt > 0);
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
        s_info[3] = row0;
        s_info[4] = C >= 1 ? min(C * G, RS) - RB * static_cast<int>(blockIdx.z) : 0;   // rows from here on
    }
    if (tid < RB) {
        s_M[tid] = -INFINITY;
        s_den[tid] = 0.0f;
    }
    __syncthreads();
    const int count = s_info[0];
    const size_t first = static_cast<size_t>(s_info[1]);
    const bool ok = s_info[2];
    const int row0 = s_info[3];
    const int used = min(s_info[4], RB);      // rows of this workgroup: rb .. rb + used - 1
    const int rb = RB * static_cast<int>(blockIdx.z);
    if (used <= 0) return;

    // Output task of this thread: row r_o, dims k_o .. k_o + 3 (one task per
    // thread at most). Its first kPre partials' outputs are requested now,
    // so that their round trip overlaps the (m, l) round below.
    static_assert(RB * (D / 4) <= kMergeThreads, "one output task per thread");
    constexpr int kPre = 8;
    const bool has_out = tid < used * (D / 4);
    const int r_o = tid / (D / 4);
    const int k_o = 4 * (tid - r_o * (D / 4));
    const float* ob = a.ws_o + (first * RS + rb + r_o) * D + k_o;
    // Unconditional loads (partials past `count` re-read the last one, and
    // slot 0 stands in when there is none), so that all are issued together.
    float4 pre[kPre];
    if (has_out) {
#pragma unroll
        for (int u = 0; u < kPre; ++u)
            pre[u] = *reinterpret_cast<const float4*>(ob + static_cast<size_t>(max(min(u, count - 1), 0)) * RS * D);
    }

    // Per-row maximum over all partials; a NaN partial makes it NaN.
    for (int j0 = 0; j0 < count; j0 += kMergeMaxParts) {
        const int n = min(count - j0, kMergeMaxParts);
        if (tid < n) {
            // all RB rows' loads in flight at once (rows past `used` re-read
            // the last used row and are not stored)
            PartialML p[RB];
#pragma unroll
            for (int r = 0; r < RB; ++r) p[r] = a.ws_ml[(first + j0 + tid) * RS + rb + min(r, used - 1)];
#pragma unroll
            for (int r = 0; r < RB; ++r)
                if (r < used) {
                    s_m[tid][r] = p[r].m;
                    s_l[tid][r] = p[r].l;
                }
        }
        __syncthreads();
        for (int r = wave; r < used; r += kMergeThreads / kWave) {
            float M = -INFINITY;
            bool bad = false;
            for (int j = lane; j < n; j += kWave) {
                bad |= isnan(s_m[j][r]);
                M = fmaxf(M, s_m[j][r]);
            }
            M = wave_max(M);
            bad = __builtin_amdgcn_ballot_w64(bad) != 0;
            if (lane == 0) s_M[r] = (bad || isnan(s_M[r])) ? NAN : fmaxf(s_M[r], M);
        }
        __syncthreads();
    }
    // Weights and their sum (the staged block is still in LDS when
    // count <= kMergeMaxParts; otherwise they are recomputed below). A
    // partial with m = -inf (a row that saw none of its range's keys) has
    // weight 0.
    const bool staged = count <= kMergeMaxParts;
    for (int r = wave; r < used; r += kMergeThreads / kWave) {
        const float M = s_M[r];
        float den = 0.0f;
        for (int j = lane; j < count; j += kWave) {
            float m, l;
            if (staged) {
                m = s_m[j][r];
                l = s_l[j][r];
            } else {
                const PartialML p = a.ws_ml[(first + j) * RS + rb + r];
                m = p.m;
                l = p.l;
            }
            const float w = exp2f(m - M);
            if (staged) s_m[j][r] = w;
            den = fmaf(w, l, den);
        }
        den = wave_sum(den);
        if (lane == 0) s_den[r] = den;
    }
    __syncthreads();

    // Outputs: the first kPre partials from the registers, the rest in
    // groups of 8 loads.
    if (has_out) {
        const int r = r_o;
        const int k = k_o;
        const int qi = (rb + r) / G;
        const int h = rb + r - qi * G;
        const float M = s_M[r];
        float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
#pragma unroll
        for (int u = 0; u < kPre; ++u) {
            if (u < count) {
                const float wj = staged ? s_m[u][r] : exp2f(a.ws_ml[(first + u) * RS + rb + r].m - M);
                acc.x = fmaf(wj, pre[u].x, acc.x);
                acc.y = fmaf(wj, pre[u].y, acc.y);
                acc.z = fmaf(wj, pre[u].z, acc.z);
                acc.w = fmaf(wj, pre[u].w, acc.w);
            }
        }
        int j = kPre;
        for (; j + 8 <= count; j += 8) {
            float4 v[8];
            float wv[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) v[u] = *reinterpret_cast<const float4*>(ob + static_cast<size_t>(j + u) * RS * D);
#pragma unroll
            for (int u = 0; u < 8; ++u)
                wv[u] = staged ? s_m[j + u][r] : exp2f(a.ws_ml[(first + j + u) * RS + rb + r].m - M);
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                acc.x = fmaf(wv[u], v[u].x, acc.x);
                acc.y = fmaf(wv[u], v[u].y, acc.y);
                acc.z = fmaf(wv[u], v[u].z, acc.z);
                acc.w = fmaf(wv[u], v[u].w, acc.w);
            }
        }
        for (; j < count; ++j) {
            const float4 v = *reinterpret_cast<const float4*>(ob + static_cast<size_t>(j) * RS * D);
            const float wj = staged ? s_m[j][r] : exp2f(a.ws_ml[(first + j) * RS + rb + r].m - M);
            acc.x = fmaf(wj, v.x, acc.x);
            acc.y = fmaf(wj, v.y, acc.y);
            acc.z = fmaf(wj, v.z, acc.z);
            acc.w = fmaf(wj, v.w, acc.w);
        }
        const float inv = (ok && !isnan(M)) ? 1.0f / s_den[r] : NAN;
        uint2 w2;
        w2.x = pack2_bf16(acc.x * inv, acc.y * inv);
        w2.y = pack2_bf16(acc.z * inv, acc.w * inv);
        *reinterpret_cast<uint2*>(out + ((static_cast<size_t>(row0) + qi) * a.n_q + g * G + h) * D + k) = w2;
    }
    if (lse && tid < used) {
        const int qi = (rb + tid) / G;
        const float M = s_M[tid];
        lse[(static_cast<size_t>(row0) + qi) * a.n_q + g * G + (rb + tid - qi * G)] =
            (ok && !isnan(M)) ? kLn2 * (M + log2f(s_den[tid])) : NAN;
    }
}

constexpr int kChunkMergeRows = 8;   // rows per merge workgroup for small chunks

template <int G>
void launch_merge_balanced(const AttnArgs& a, dim3 grid, uint16_t* out, float* lse, bool chunk, hipStream_t stream) {
    if (chunk) {
        grid.z = (min(a.max_q_len * G, kChunkSlotRows) + kChunkMergeRows - 1) / kChunkMergeRows;
        hipLaunchKernelGGL((merge_balanced_kernel<G, kChunkSlotRows, kChunkMergeRows>), grid, dim3(kMergeThreads), 0,
                           stream, a, out, lse);
    } else {
        hipLaunchKernelGGL((merge_balanced_kernel<G, G, G>), grid, dim3(kMergeThreads), 0, stream, a, out, lse);
    }
}

}  // namespace

hipError_t launch_merge(const AttnArgs& a, void* out, float* lse, bool bf16, hipStream_t stream) {
    if (a.waves > 0 && bf16 && a.head_dim == 128) {
        const dim3 grid(a.num_seqs, a.n_kv);
        auto out16 = static_cast<uint16_t*>(out);
        const bool chunk = a.q_start != nullptr;   // small chunks: kChunkSlotRows rows per slot
        switch (a.n_q / a.n_kv) {
            case 1: launch_merge_balanced<1>(a, grid, out16, lse, chunk, stream); break;
            case 2: launch_merge_balanced<2>(a, grid, out16, lse, chunk, stream); break;
            case 4: launch_merge_balanced<4>(a, grid, out16, lse, chunk, stream); break;
            case 8: launch_merge_balanced<8>(a, grid, out16, lse, chunk, stream); break;
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
