// Token sampling after the LM head: temperature, top-k, top-p, draw.
//
// Lab page (Inference Engineering), function sample; chapter 5's
// filter-and-sample listing; serving tutorial demos D01/D02. Per row of
// logits, in this order:
//  * temperature T = 0: greedy, the lowest index among tied maxima;
//  * z = logit / T (fp32, correctly rounded), ordered by decreasing z with
//    ties going to the lower index;
//  * top-k (k > 0): keep the first k of that order;
//  * masses p = exp(z - max z);
//  * top-p (p < 1): keep the shortest prefix of the order whose cumulative
//    mass reaches p times the kept total - the boundary token and the
//    largest are always kept;
//  * draw: the first index, in vocabulary order, whose cumulative kept mass
//    exceeds u times the kept total (u in [0, 1) is an input: the only
//    random number the step uses).
//
// One 512-thread workgroup per row; the row is read once per pass (it stays
// in L2). Selections avoid sorting: the k-th largest z is found by a radix
// descent over order-preserving 32-bit keys (four 8-bit digits, counts per
// digit in LDS), the top-p boundary by the same descent over masses (fp64
// sums per digit); ties at a boundary are resolved in index order with
// wave ballots over contiguous per-wave segments of the row. Sums are fp64.
#include "device_common.h"
#include "kernels.h"

namespace pkv {
namespace {

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / kWave;

__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;
}
__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;
}

// Larger float -> larger key (NaN excluded).
__device__ __forceinline__ uint32_t order_key(float x) {
    const uint32_t b = __float_as_uint(x);
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

struct Row {
    const float* x;
    int V;
    float T;
    __device__ __forceinline__ float z(int j) const { return x[j] / T; }
};

// Wave-0 search over 256 digit bins from the top: the first bin b (from 255
// down) at which `before + sum of bins >= b` reaches `need`. Returns b
// (or -1 if never reached) and, in *above, the total of the bins above b.
template <typename C>
__device__ __forceinline__ int find_bin_from_top(const C* bins, C need, C* above, int lane) {
    // lane l holds bins 255-4l .. 252-4l (descending)
    C v[4];
    C local = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        v[i] = bins[255 - 4 * lane - i];
        local += v[i];
    }
    C incl = local;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        const C y = __shfl_up(incl, o, kWave);
        if (lane >= o) incl += y;
    }
    const C excl = incl - local;
    const bool hit = incl >= need;
    const unsigned long long m = __builtin_amdgcn_ballot_w64(hit);
    if (!m) return -1;
    const int first = __builtin_ctzll(m);
    int bin = -1;
    C ab = 0;
    if (lane == first) {
        C run = excl;
        for (int i = 0; i < 4; ++i) {
            if (run + v[i] >= need) {
                bin = 255 - 4 * lane - i;
                break;
            }
            run += v[i];
        }
        ab = run;
    }
    bin = __shfl(bin, first, kWave);
    *above = __shfl(ab, first, kWave);
    return bin;
}

__global__ __launch_bounds__(kThreads) void sample_kernel(SampleArgs a) {
    const int row = blockIdx.x;
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const Row r{a.logits + static_cast<size_t>(row) * a.ld, a.vocab, a.temperature[row]};
    const int V = r.V;

    __shared__ uint32_t s_cnt[256];
    __shared__ double s_mass[256];
    __shared__ float s_f[kWaves];
    __shared__ int s_i[kWaves];
    __shared__ double s_d[kWaves];
    __shared__ uint32_t s_u[kWaves];
    __shared__ int s_bin;
    __shared__ double s_above;

    auto write = [&](int token, int kk, int kp) {
        if (tid == 0) {
            a.token[row] = token;
            if (a.kept) {
                a.kept[2 * row] = kk;
                a.kept[2 * row + 1] = kp;
            }
        }
    };
    if (!(r.T >= 0.0f)) {   // negative or NaN temperature: no token
        write(-1, 0, 0);
        return;
    }

    // ---- greedy: argmax, lowest index among ties ----------------------------
    if (r.T == 0.0f) {
        float best = -INFINITY;
        int bi = V;
        for (int j = tid; j < V; j += kThreads) {
            const float v = r.x[j];
            if (v > best) {
                best = v;
                bi = j;
            }
        }
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) {
            const float ov = __shfl_xor(best, o, kWave);
            const int oi = __shfl_xor(bi, o, kWave);
            if (ov > best || (ov == best && oi < bi)) {
                best = ov;
                bi = oi;
            }
        }
        if (lane == 0) {
            s_f[wave] = best;
            s_i[wave] = bi;
        }
        __syncthreads();
        if (tid == 0) {
            for (int w = 1; w < kWaves; ++w)
                if (s_f[w] > best || (s_f[w] == best && s_i[w] < bi)) {
                    best = s_f[w];
                    bi = s_i[w];
                }
        }
        write(bi < V ? bi : -1, 1, 1);
        return;
    }

    // ---- max of z -------------------------------------------------------------
    float mz = -INFINITY;
    for (int j = tid; j < V; j += kThreads) mz = fmaxf(mz, r.z(j));
    mz = wave_max(mz);
    if (lane == 0) s_f[wave] = mz;
    __syncthreads();
    mz = s_f[0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) mz = fmaxf(mz, s_f[w]);
    __syncthreads();

    // Contiguous segment of the row owned by this wave (index order).
    const int seg_lo = static_cast<int>(static_cast<long long>(wave) * V / kWaves);
    const int seg_hi = static_cast<int>(static_cast<long long>(wave + 1) * V / kWaves);

    // The `rank`-th (1-based) index, in index order, among elements with
    // pred(j) true; every thread gets it.
    auto nth_index = [&](auto pred, uint32_t rank) -> int {
        uint32_t c = 0;
        for (int j0 = seg_lo; j0 < seg_hi; j0 += kWave) {
            const int j = j0 + lane;
            const bool p = j < seg_hi && pred(j);
            c += __builtin_popcountll(__builtin_amdgcn_ballot_w64(p));
        }
        if (lane == 0) s_u[wave] = c;
        __syncthreads();
        uint32_t before = 0;
        int w_hit = -1;
        for (int w = 0; w < kWaves; ++w) {
            if (w_hit < 0 && before + s_u[w] >= rank) w_hit = w;
            else if (w_hit < 0) before += s_u[w];
        }
        if (wave == w_hit) {
            uint32_t acc = before;
            int found = -1;
            for (int j0 = seg_lo; j0 < seg_hi && found < 0; j0 += kWave) {
                const int j = j0 + lane;
                const bool p = j < seg_hi && pred(j);
                const unsigned long long m = __builtin_amdgcn_ballot_w64(p);
                const uint32_t n = __builtin_popcountll(m);
                if (acc + n >= rank) {
                    unsigned long long mm = m;
                    for (uint32_t q = acc + 1; q < rank; ++q) mm &= mm - 1;   // drop earlier set bits
                    found = j0 + __builtin_ctzll(mm);
                }
                acc += n;
            }
            if (lane == 0) s_i[0] = found;
        }
        __syncthreads();
        const int idx = s_i[0];
        __syncthreads();
        return idx;
    };

    // ---- top-k: the k-th largest key, ties by index ---------------------------
    const int k = a.top_k[row];
    uint32_t kkey = 0;        // kept: key > kkey, or key == kkey and j <= kidx
    int kidx = V;
    int kept_k = V;
    if (k > 0 && k < V) {
        uint32_t prefix = 0, mask = 0, rem = static_cast<uint32_t>(k);
        for (int shift = 24; shift >= 0; shift -= 8) {
            for (int i = tid; i < 256; i += kThreads) s_cnt[i] = 0;
            __syncthreads();
            for (int j = tid; j < V; j += kThreads) {
                const uint32_t key = order_key(r.z(j));
                if ((key & mask) == prefix) atomicAdd(&s_cnt[(key >> shift) & 255u], 1u);
            }
            __syncthreads();
            if (wave == 0) {
                uint32_t above = 0;
                int b = find_bin_from_top(s_cnt, rem, &above, lane);
                if (b < 0) {    // only with non-finite logits: keep the bucket's lowest bin
                    b = 0;
                    above = 0;
                }
                if (lane == 0) {
                    s_bin = b;
                    s_u[0] = above;
                }
            }
            __syncthreads();
            prefix |= static_cast<uint32_t>(s_bin) << shift;
            mask |= 255u << shift;
            rem -= s_u[0];
            __syncthreads();
        }
        kkey = prefix;
        const uint32_t ties = s_cnt[kkey & 255u];
        if (rem < ties) kidx = nth_index([&](int j) { return order_key(r.z(j)) == kkey; }, rem);
        kept_k = k;
    }
    auto in_k = [&](int j, uint32_t key) { return key > kkey || (key == kkey && j <= kidx); };

    // ---- top-p: boundary of the descending-mass prefix --------------------------
    const float tp = a.top_p[row];
    uint32_t pkey = 0;        // kept: in_k and (key > pkey, or key == pkey and j <= pidx)
    int pidx = V;
    if (tp < 1.0f) {
        double tot = 0.0;
        for (int j = tid; j < V; j += kThreads) {
            const float zj = r.z(j);
            if (in_k(j, order_key(zj))) tot += static_cast<double>(expf(zj - mz));
        }
        tot = wave_sum_f64(tot);
        if (lane == 0) s_d[wave] = tot;
        __syncthreads();
        tot = 0.0;
        for (int w = 0; w < kWaves; ++w) tot += s_d[w];
        __syncthreads();
        const double need = static_cast<double>(tp) * tot;
        uint32_t prefix = 0, mask = 0;
        double above = 0.0;
        for (int shift = 24; shift >= 0; shift -= 8) {
            for (int i = tid; i < 256; i += kThreads) {
                s_mass[i] = 0.0;
                s_cnt[i] = 0;
            }
            __syncthreads();
            for (int j = tid; j < V; j += kThreads) {
                const float zj = r.z(j);
                const uint32_t key = order_key(zj);
                if ((key & mask) == prefix && in_k(j, key)) {
                    atomicAdd(&s_mass[(key >> shift) & 255u], static_cast<double>(expf(zj - mz)));
                    atomicAdd(&s_cnt[(key >> shift) & 255u], 1u);
                }
            }
            __syncthreads();
            if (wave == 0) {
                double ab = 0.0;
                int b = find_bin_from_top(s_mass, need - above, &ab, lane);
                if (b < 0) {
                    // rounding kept the mass just short of `need`: the
                    // boundary is the lowest non-empty bin
                    b = 0;
                    for (int i = 0; i < 256; ++i)
                        if (s_cnt[i]) {
                            b = i;
                            break;
                        }
                    ab = 0.0;
                    for (int i = 255; i > b; --i) ab += s_mass[i];
                }
                if (lane == 0) {
                    s_bin = b;
                    s_above = ab;
                }
            }
            __syncthreads();
            prefix |= static_cast<uint32_t>(s_bin) << shift;
            mask |= 255u << shift;
            above += s_above;
            __syncthreads();
        }
        pkey = prefix;
        const uint32_t ties = s_cnt[pkey & 255u];
        // every tie has the same mass; keep the first t of them in index order
        const float zb = (pkey & 0x80000000u) ? __uint_as_float(pkey & 0x7fffffffu) : __uint_as_float(~pkey);
        const double pb = static_cast<double>(expf(zb - mz));
        double t = (need - above) / pb;
        uint32_t keep = t <= 1.0 ? 1u : static_cast<uint32_t>(fmin(ceil(t), static_cast<double>(ties)));
        if (keep < 1u) keep = 1u;
        if (keep < ties)
            pidx = nth_index([&](int j) {
                const uint32_t key = order_key(r.z(j));
                return key == pkey && in_k(j, key);
            }, keep);
    }
    auto kept = [&](int j, uint32_t key) { return in_k(j, key) && (key > pkey || (key == pkey && j <= pidx)); };

    // ---- draw: inverse CDF in index order --------------------------------------
    double wsum = 0.0;
    uint32_t wcnt = 0;
    for (int j0 = seg_lo; j0 < seg_hi; j0 += kWave) {
        const int j = j0 + lane;
        if (j < seg_hi) {
            const float zj = r.z(j);
            if (kept(j, order_key(zj))) {
                wsum += static_cast<double>(expf(zj - mz));
                ++wcnt;
            }
        }
    }
    wsum = wave_sum_f64(wsum);
    wcnt = wave_sum_u32(wcnt);
    if (lane == 0) {
        s_d[wave] = wsum;
        s_u[wave] = wcnt;
    }
    __syncthreads();
    double total = 0.0;
    uint32_t kept_p = 0;
    for (int w = 0; w < kWaves; ++w) {
        total += s_d[w];
        kept_p += s_u[w];
    }
    const double target = static_cast<double>(a.u[row]) * total;
    double before = 0.0;
    int w_hit = -1, w_last = -1;
    for (int w = 0; w < kWaves; ++w) {
        if (s_u[w]) w_last = w;
        if (w_hit < 0 && s_u[w] && before + s_d[w] > target) w_hit = w;
        else if (w_hit < 0) before += s_d[w];
    }
    if (w_hit < 0) w_hit = w_last;   // rounding put the target at the total
    if (wave == w_hit) {
        double run = before;
        int found = -1, last = -1;
        for (int j0 = seg_lo; j0 < seg_hi && found < 0; j0 += kWave) {
            const int j = j0 + lane;
            double p = 0.0;
            bool in = false;
            if (j < seg_hi) {
                const float zj = r.z(j);
                in = kept(j, order_key(zj));
                if (in) p = static_cast<double>(expf(zj - mz));
            }
            double incl = p;
#pragma unroll
            for (int o = 1; o < kWave; o <<= 1) {
                const double y = __shfl_up(incl, o, kWave);
                if (lane >= o) incl += y;
            }
            const unsigned long long cross = __builtin_amdgcn_ballot_w64(in && run + incl > target);
            const unsigned long long any = __builtin_amdgcn_ballot_w64(in);
            if (any) last = j0 + 63 - __builtin_clzll(any);
            if (cross) found = j0 + __builtin_ctzll(cross);
            run += __shfl(incl, kWave - 1, kWave);
        }
        if (lane == 0) s_i[0] = found >= 0 ? found : last;
    }
    __syncthreads();
    write(s_i[0], kept_k, static_cast<int>(kept_p));
}

}  // namespace

hipError_t launch_sample(const SampleArgs& a, int rows, hipStream_t stream) {
    hipLaunchKernelGGL(sample_kernel, dim3(rows), dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace pkv
