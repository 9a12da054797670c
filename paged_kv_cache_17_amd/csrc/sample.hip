// Token sampling after the LM head: temperature, top-k, top-p, draw.
//
// Lab page (Inference Engineering), function sample; chapter 5's
// filter-and-sample listing; serving tutorial demos D01/D02. Per row of
// logits, in this order:
//  * temperature T = 0: greedy, the lowest index among tied maxima;
//  * z = logit / T (fp32, correctly rounded), ordered by decreasing z with
//    ties going to the lower index;
//  * top-k (k > 0): keep the first k of that order;
//  * masses p = exp(z - max z), evaluated in fp64;
//  * top-p (p < 1): keep the shortest prefix of the order whose cumulative
//    mass reaches p times the kept total - the boundary token and the
//    largest are always kept;
//  * draw: the first index, in vocabulary order, whose cumulative kept mass
//    exceeds u times the kept total (u in [0, 1) is an input: the only
//    random number the step uses).
//
// Three paths, chosen per row on the device:
//  * candidate path (greedy rows, and top-k sets of at most kSampleMaxK
//    tokens): the row is cut into chunks of at most kSampleChunk logits,
//    one 256-thread workgroup each, which reads its chunk once into
//    registers and keeps its own top-k by a radix descent over
//    order-preserving 32-bit keys (11-, 11- and 10-bit digits; any token of
//    the row's top-k is in its chunk's top-k), recording its k-th key. One
//    workgroup per row then keeps the candidates at or above the largest of
//    those k-th keys (no other token can reach the row's top-k), orders
//    them by counting (bitonic sort in LDS when many are tied), and runs
//    top-p and the draw on the first k.
//  * histogram path (top-k off, rows of at most kSampleHistChunks chunks):
//    each chunk workgroup records its largest z and, with top-p on, the
//    fp64 masses exp(z - chunk max) summed per bin of the key's top 11
//    bits. One workgroup per row rescales and adds the chunks' histograms,
//    finds the bin holding the top-p boundary, gathers that bin's tokens
//    into LDS in one pass over the row and finishes the boundary there
//    (two more key digits, then index digits among tied keys). The draw
//    picks the chunk from per-chunk kept masses and walks that chunk only.
//  * whole-row path (top-k between kSampleMaxK and the vocabulary, rows
//    wider than kSampleHistChunks chunks, or a boundary bin of more than
//    kBucketCap tokens): one 1024-thread workgroup per row finds the k-th
//    largest key and the top-p boundary by radix descents over the row
//    (counts, and fp64 mass sums, per 8-bit digit in LDS); ties at a
//    boundary are resolved in index order with wave ballots.
// The second kernel runs the finishing step: each workgroup takes its row's
// path.
#include "device_common.h"
#include "kernels.h"

namespace pkv {
namespace {

constexpr int kChunkThreads = 256;
constexpr int kPerThread = kSampleChunk / kChunkThreads;
constexpr int kChunkWaves = kChunkThreads / kWave;
constexpr int kChunkKeep = 512;              // keys at or above a chunk's bound kept in LDS
constexpr int kThreads = 1024;               // second kernel: one row per workgroup
constexpr int kWaves = kThreads / kWave;
static_assert(kPerThread * kChunkThreads == kSampleChunk, "chunk split");
static_assert(kSampleMaxK <= 4 * kWave, "one wave scans the top-k (4 per lane)");
static_assert(kSampleMaxCand % kThreads == 0, "candidates per thread");
static_assert(kChunkKeep + 2048 / 2 <= kSampleHistBins, "chunk pool: keep list and 2048 u32 digit bins");

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
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = max(v, static_cast<uint32_t>(__shfl_xor(v, o, kWave)));
    return v;
}
template <typename C>
__device__ __forceinline__ C wave_incl_scan(C v, int lane) {
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        const C y = __shfl_up(v, o, kWave);
        if (lane >= o) v += y;
    }
    return v;
}

// Larger float -> larger key (NaN excluded), and back.
__device__ __forceinline__ uint32_t order_key(float x) {
    const uint32_t b = __float_as_uint(x);
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ __forceinline__ float key_value(uint32_t k) {
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}
// (key, index) as one 64-bit value whose descending order is decreasing z
// with ties to the lower index; 0 is below every real candidate.
__device__ __forceinline__ uint64_t composite(uint32_t key, uint32_t idx) {
    return (static_cast<uint64_t>(key) << 32) | static_cast<uint32_t>(~idx);
}
__device__ __forceinline__ uint32_t comp_key(uint64_t c) { return static_cast<uint32_t>(c >> 32); }
__device__ __forceinline__ int comp_index(uint64_t c) { return static_cast<int>(~static_cast<uint32_t>(c)); }

// Tokens kept by top-k: the whole vocabulary when it is off.
__device__ __forceinline__ int kept_by_k(int k, int V) { return (k <= 0 || k >= V) ? V : k; }

// Rows the candidate path finishes: greedy rows and top-k sets small
// enough for one finishing workgroup. Every other row with T > 0 takes the
// whole-row path.
__device__ __forceinline__ bool on_candidate_path(float T, int k_eff, int chunks) {
    return T == 0.0f || (k_eff <= kSampleMaxK && chunks * k_eff <= kSampleMaxCand);
}

// Rows with top-k off (T > 0) and at most kSampleHistChunks chunks; the
// candidate path keeps precedence (a vocabulary of at most kSampleMaxK).
__device__ __forceinline__ bool on_hist_path(float T, int k_eff, int V, int chunks) {
    return T > 0.0f && k_eff >= V && chunks <= kSampleHistChunks;
}

// Workspace of (row, chunk): candidates, or the chunk's mass histogram; and
// the chunk's header (histogram rows only).
__device__ __forceinline__ unsigned char* chunk_region(const SampleArgs& a, int row, int s) {
    return a.ws + (static_cast<size_t>(row) * a.chunks + s) * a.region;
}
__device__ __forceinline__ uint2* chunk_cands(const SampleArgs& a, int row, int s) {
    return reinterpret_cast<uint2*>(chunk_region(a, row, s));
}
__device__ __forceinline__ double* chunk_hist(const SampleArgs& a, int row, int s) {
    return reinterpret_cast<double*>(chunk_region(a, row, s));
}
__device__ __forceinline__ SampleChunkHead* chunk_head(const SampleArgs& a, int row, int s) {
    return reinterpret_cast<SampleChunkHead*>(a.ws + static_cast<size_t>(a.rows) * a.chunks * a.region) +
           static_cast<size_t>(row) * a.chunks + s;
}

// Histogram rows: the boundary bin's tokens gathered by the row's
// workgroups (workgroup g writes the g-th quarter), and counters: [0]
// workgroups done, [2 + 2g] and [3 + 2g] workgroup g's tokens (0xFFFFFFFF:
// more than its quarter) and tokens above the bin; after the chunk headers.
__device__ __forceinline__ unsigned char* row_extra(const SampleArgs& a, int row) {
    return a.ws + static_cast<size_t>(a.rows) * a.chunks * (a.region + sizeof(SampleChunkHead)) +
           static_cast<size_t>(row) * (static_cast<size_t>(kSampleBucketCap) * 8u + 64u);
}
__device__ __forceinline__ uint64_t* row_list(const SampleArgs& a, int row) {
    return reinterpret_cast<uint64_t*>(row_extra(a, row));
}
__device__ __forceinline__ uint32_t* row_counters(const SampleArgs& a, int row) {
    return reinterpret_cast<uint32_t*>(row_extra(a, row) + static_cast<size_t>(kSampleBucketCap) * 8u);
}

__device__ __forceinline__ void write_result(const SampleArgs& a, int row, int token, int kk, int kp) {
    a.token[row] = token;
    if (a.kept) {
        a.kept[2 * row] = kk;
        a.kept[2 * row + 1] = kp;
    }
}

// Wave-level search over NB digit bins from the top: the first bin b (from
// NB-1 down) at which the running total of the bins from the top reaches
// `need`. Returns b (or -1 if never reached) and, in *above, the total of
// the bins above b. Lane l owns bins NB-1-B*l down to NB-B*(l+1), B = NB/64;
// the sums read them in a rotated order so that lanes hit different banks.
template <int NB, typename C>
__device__ __forceinline__ int find_bin_from_top(const C* bins, C need, C* above, int lane) {
    constexpr int B = NB / kWave;
    static_assert(B * kWave == NB && (B & (B - 1)) == 0, "bins per lane");
    const int top = NB - 1 - B * lane;
    C local = 0;
#pragma unroll
    for (int i = 0; i < B; ++i) local += bins[top - ((i + lane) & (B - 1))];
    const C incl = wave_incl_scan(local, lane);
    const unsigned long long m = __builtin_amdgcn_ballot_w64(incl >= need);
    if (!m) return -1;
    const int first = __builtin_ctzll(m);
    int bin = -1;
    C ab = 0;
    if (lane == first) {
        C run = incl - local;
        for (int i = 0; i < B; ++i) {
            const C v = bins[top - i];
            if (run + v >= need) {
                bin = top - i;
                break;
            }
            run += v;
        }
        ab = run;
    }
    bin = __shfl(bin, first, kWave);
    *above = __shfl(ab, first, kWave);
    return bin;
}

// ---- candidate path, pass 1: each chunk's own top-k --------------------------

// One digit of the chunk's radix descent: histogram of the digit at `shift`
// (NB bins) over the keys that match `prefix` under `mask`, then the bin
// that holds the rem-th largest of them.
template <int NB>
__device__ __forceinline__ void chunk_digit(const uint32_t (&key)[kPerThread], int shift,
                                            uint32_t* s_hist, int* s_bin, uint32_t* s_above, uint32_t& prefix,
                                            uint32_t& mask, uint32_t& rem) {
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    for (int b = tid; b < NB; b += kChunkThreads) s_hist[b] = 0u;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kPerThread; ++i)
        if ((key[i] & mask) == prefix) atomicAdd(&s_hist[(key[i] >> shift) & (NB - 1)], 1u);
    __syncthreads();
    if (tid < kWave) {
        uint32_t above = 0;
        const int b = find_bin_from_top<NB>(s_hist, rem, &above, lane);
        if (lane == 0) {
            *s_bin = b < 0 ? 0 : b;    // b >= 0: rem never exceeds the matching keys
            *s_above = above;
        }
    }
    __syncthreads();
    prefix |= static_cast<uint32_t>(*s_bin) << shift;
    mask |= static_cast<uint32_t>(NB - 1) << shift;
    rem -= *s_above;
}

// Histogram path, pass 1: the chunk's largest z, its total mass and, with
// top-p on, its fp64 masses exp(z - chunk max) per bin of the key's top 11
// bits, stored as inclusive suffix sums (I[b] = mass of the bins b and
// above; the bins of every chunk line up, so the row adds them after
// rescaling). Keys of 0 lie past the chunk's end.
__device__ __forceinline__ void chunk_masses(const SampleArgs& a, int row, int s,
                                             const uint32_t (&key)[kPerThread], double* s_hm, uint32_t* s_tw) {
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const bool hist = a.top_p[row] < 1.0f;
    __shared__ double s_wt[kChunkWaves];
    uint32_t mk = 0;
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) mk = max(mk, key[i]);
    mk = wave_max_u32(mk);
    if (lane == 0) s_tw[wave] = mk;
    if (hist)
        for (int b = tid; b < kSampleHistBins; b += kChunkThreads) s_hm[b] = 0.0;
    __syncthreads();
    mk = s_tw[0];
#pragma unroll
    for (int w = 1; w < kChunkWaves; ++w) mk = max(mk, s_tw[w]);
    const float mc = key_value(mk);
    const double mcd = static_cast<double>(mc);
    double tot = 0.0;
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) {
        if (!key[i]) continue;
        const double m = exp(static_cast<double>(key_value(key[i])) - mcd);
        if (hist) atomicAdd(&s_hm[key[i] >> 21], m);
        else tot += m;
    }
    SampleChunkHead* h = chunk_head(a, row, s);
    if (hist) {
        __syncthreads();
        // suffix sums: thread t owns bins 8t .. 8t + 7; then the threads
        // above it (a suffix scan over lanes, then over waves)
        constexpr int kPer = kSampleHistBins / kChunkThreads;
        double l[kPer];
        double run = 0.0;
#pragma unroll
        for (int i = kPer - 1; i >= 0; --i) {
            run += s_hm[kPer * tid + i];
            l[i] = run;
        }
        double suf = run;   // inclusive over lanes lane .. 63 of this wave
#pragma unroll
        for (int o = 1; o < kWave; o <<= 1) {
            const double y = __shfl_down(suf, o, kWave);
            if (lane + o < kWave) suf += y;
        }
        if (lane == 0) s_wt[wave] = suf;
        __syncthreads();
        double above = __shfl_down(suf, 1, kWave);   // lanes above this one
        if (lane == kWave - 1) above = 0.0;
        for (int w = kChunkWaves - 1; w > wave; --w) above += s_wt[w];
        double* out = chunk_hist(a, row, s);
#pragma unroll
        for (int i = 0; i < kPer; ++i) out[kPer * tid + i] = l[i] + above;
        if (tid == 0) {
            h->mc = mc;
            h->total = l[0] + above;
        }
    } else {
        tot = wave_sum_f64(tot);
        if (lane == 0) s_wt[wave] = tot;
        __syncthreads();
        if (tid == 0) {
            double t = 0.0;
#pragma unroll
            for (int w = 0; w < kChunkWaves; ++w) t += s_wt[w];
            h->mc = mc;
            h->total = t;
        }
    }
}

// One workgroup per (row, chunk), blockIdx.x = row * chunks + chunk.
// Candidate rows: writes the chunk's min(k, chunk length) best (key, index)
// pairs to its candidate slots, best first (decreasing key, ties by lower
// index). Histogram rows: chunk_masses.
__global__ __launch_bounds__(kChunkThreads) __attribute__((amdgpu_waves_per_eu(4)))
void sample_chunk_kernel(SampleArgs a) {
    const int S = a.chunks;
    const int row = blockIdx.x / S;
    const int s = blockIdx.x - row * S;
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const int V = a.vocab;
    const float T = a.temperature[row];
    if (!(T >= 0.0f)) return;
    const int k_eff = T > 0.0f ? kept_by_k(a.top_k[row], V) : 1;
    const bool cand = on_candidate_path(T, k_eff, S);
    if (!cand && !on_hist_path(T, k_eff, V, S)) return;
    const int C = (V + S - 1) / S;
    const int lo = s * C;
    const int hi = min(V, lo + C);
    if (lo >= hi) return;
    const uint32_t want = static_cast<uint32_t>(min(k_eff, hi - lo));
    const float* x = a.logits + static_cast<size_t>(row) * a.ld;

    // element i of this thread: index lo + i * kChunkThreads + tid. Past the
    // chunk's end the key is 0, which no finite z has (it is a negative NaN's
    // key): such slots land in the lowest bin and are never taken.
    // The loads are unconditional (clamped to the last element) so that all
    // of them are in flight together.
    const int jb = lo + tid;
    uint32_t key[kPerThread];
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) key[i] = __float_as_uint(x[min(jb + i * kChunkThreads, hi - 1)]);
    if (T > 0.0f) {
#pragma unroll
        for (int i = 0; i < kPerThread; ++i) key[i] = __float_as_uint(__uint_as_float(key[i]) / T);
    }
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) key[i] = jb + i * kChunkThreads < hi ? order_key(__uint_as_float(key[i])) : 0u;

    __shared__ uint32_t s_tw[kChunkWaves];
    __shared__ uint64_t s_pool[kSampleHistBins];   // histogram rows: fp64 bins; candidate rows: keep list + digit bins
    __shared__ uint32_t s_tc[kPerThread * kChunkWaves];
    if (!cand) {
        if (s == 0 && tid == 0) row_counters(a, row)[0] = 0u;   // counted up by the finishing kernel
        chunk_masses(a, row, s, key, reinterpret_cast<double*>(s_pool), s_tw);
        return;
    }
    uint64_t* s_keep = s_pool;
    uint32_t* s_hist = reinterpret_cast<uint32_t*>(s_pool + kChunkKeep);
    __shared__ int s_bin;
    __shared__ uint32_t s_above, s_n;
    const unsigned long long below = (1ull << lane) - 1ull;

    // Bound: each wave finds the q-th largest of its lanes' maxima, q =
    // ceil(want / 4), by bisection over the key bits with ballots; every
    // wave then has q keys at or above the smallest of the four, so the
    // chunk has at least want: its want-th largest key is not below it and
    // keys under it are never taken.
    uint32_t mx = 0;
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) mx = max(mx, key[i]);
    const uint32_t q = (want + kChunkWaves - 1) / kChunkWaves;
    uint32_t tw = 0;
    for (int bit = 31; bit >= 0; --bit) {
        const uint32_t cand = tw | (1u << bit);
        if (static_cast<uint32_t>(__builtin_popcountll(__builtin_amdgcn_ballot_w64(mx >= cand))) >= q) tw = cand;
    }
    if (lane == 0) s_tw[wave] = tw;
    if (tid == 0) s_n = 0u;
    __syncthreads();
    uint32_t thr = s_tw[0];
#pragma unroll
    for (int w = 1; w < kChunkWaves; ++w) thr = min(thr, s_tw[w]);
    thr = max(thr, 1u);

    // the keys at or above the bound, as (key, index) composites
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) {
        const bool keep = key[i] >= thr;
        const unsigned long long km = __builtin_amdgcn_ballot_w64(keep);
        if (km) {
            uint32_t base = 0;
            if (lane == 0) base = atomicAdd(&s_n, static_cast<uint32_t>(__builtin_popcountll(km)));
            base = __shfl(base, 0, kWave);
            const uint32_t slot = base + __builtin_popcountll(km & below);
            if (keep && slot < kChunkKeep) s_keep[slot] = composite(key[i], static_cast<uint32_t>(jb + i * kChunkThreads));
        }
    }
    __syncthreads();
    uint32_t kept = s_n;

    if (kept > kChunkKeep) {
        // Many keys share the bound (ties or a flat chunk): radix descent to
        // the want-th largest key; keys above it are taken, and the first
        // `rem` of the keys equal to it in index order.
        uint32_t prefix = 0, mask = 0, rem = want;
        chunk_digit<2048>(key, 21, s_hist, &s_bin, &s_above, prefix, mask, rem);
        chunk_digit<2048>(key, 10, s_hist, &s_bin, &s_above, prefix, mask, rem);
        chunk_digit<1024>(key, 0, s_hist, &s_bin, &s_above, prefix, mask, rem);
        const uint32_t kth = prefix;
        const bool all_ties = rem >= s_hist[kth & 1023u];
        if (!all_ties) {
#pragma unroll
            for (int i = 0; i < kPerThread; ++i) {
                const unsigned long long m = __builtin_amdgcn_ballot_w64(key[i] == kth);
                if (lane == 0) s_tc[i * kChunkWaves + wave] = __builtin_popcountll(m);
            }
            __syncthreads();
            if (wave == 0) {   // exclusive scan in (i, wave) order = index order
                const uint32_t e0 = s_tc[2 * lane], e1 = s_tc[2 * lane + 1];
                const uint32_t incl = wave_incl_scan(e0 + e1, lane);
                s_tc[2 * lane] = incl - e0 - e1;
                s_tc[2 * lane + 1] = incl - e1;
            }
        }
        if (tid == 0) s_n = 0u;
        __syncthreads();
#pragma unroll
        for (int i = 0; i < kPerThread; ++i) {
            bool take = key[i] > kth;
            const bool tie = key[i] == kth;
            if (all_ties) {
                take = take || tie;
            } else {
                const unsigned long long tb = __builtin_amdgcn_ballot_w64(tie);
                if (tie) take = s_tc[i * kChunkWaves + wave] + __builtin_popcountll(tb & below) < rem;
            }
            const unsigned long long tm = __builtin_amdgcn_ballot_w64(take);
            if (tm) {
                uint32_t base = 0;
                if (lane == 0) base = atomicAdd(&s_n, static_cast<uint32_t>(__builtin_popcountll(tm)));
                base = __shfl(base, 0, kWave);
                const uint32_t slot = base + __builtin_popcountll(tm & below);
                if (take && slot < want)
                    s_keep[slot] = composite(key[i], static_cast<uint32_t>(jb + i * kChunkThreads));
            }
        }
        __syncthreads();
        kept = want;
    }

    // best first: the rank of each kept composite is its slot
    uint2* out = chunk_cands(a, row, s);
    for (uint32_t e = tid; e < kept; e += kChunkThreads) {
        const uint64_t me = s_keep[e];
        uint32_t r = 0;
#pragma unroll 8
        for (uint32_t f = 0; f < kept; ++f) r += s_keep[f] > me;
        if (r < want) out[r] = make_uint2(comp_key(me), static_cast<uint32_t>(comp_index(me)));
    }
}

// ---- candidate path, pass 2: merge, top-k, top-p, draw ----------------------
constexpr int kCandPerThread = kSampleMaxCand / kThreads;
constexpr int kMergeChunks = 32;   // up to this many sorted lists are merged by rank
constexpr int kSearchLanes = 8;    // binary searches one thread runs together

// One digit of the finishing radix descent over 64-bit composites (the
// digit's NB bins at `shift`). Returns true when the bucket chosen holds
// exactly the rem still wanted, so that every composite matching the new
// prefix is taken and the descent can stop.
template <int NB>
__device__ __forceinline__ bool cand_digit(const uint64_t (&c)[kCandPerThread], int shift, uint32_t* s_hist,
                                           int* s_dig, uint64_t& prefix, uint64_t& mask, uint32_t& rem) {
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    for (int b = tid; b < NB; b += kThreads) s_hist[b] = 0u;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kCandPerThread; ++i)
        if (c[i] && (c[i] & mask) == prefix) atomicAdd(&s_hist[(c[i] >> shift) & (NB - 1)], 1u);
    __syncthreads();
    if (tid < kWave) {
        uint32_t above = 0;
        int b = find_bin_from_top<NB>(s_hist, rem, &above, lane);
        b = b < 0 ? 0 : b;    // b >= 0: rem never exceeds the matching candidates
        if (lane == 0) {
            s_dig[0] = b;
            s_dig[1] = static_cast<int>(above);
            s_dig[2] = s_hist[b] == rem - above;
        }
    }
    __syncthreads();
    prefix |= static_cast<uint64_t>(s_dig[0]) << shift;
    mask |= static_cast<uint64_t>(NB - 1) << shift;
    rem -= static_cast<uint32_t>(s_dig[1]);
    return s_dig[2] != 0;
}

// pool: kernel-wide LDS of at least kMergeChunks * kSampleMaxK + 2 * kThreads words.
__device__ __forceinline__ void finish_from_candidates(const SampleArgs& a, int row, float T, int k_eff,
                                                       uint64_t* pool) {
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const int V = a.vocab;
    const int S = a.chunks;
    const int C = (V + S - 1) / S;

    uint32_t* s_hist = reinterpret_cast<uint32_t*>(pool + kMergeChunks * kSampleMaxK + kThreads);   // [2048]
    __shared__ int s_dig[3];                  // digit step: bin, count above it, bucket == rest
    __shared__ uint32_t s_cnt;
    __shared__ uint64_t s_sel[kSampleMaxK];   // the row's top-k, any order
    __shared__ uint64_t s_top[kSampleMaxK];   // the row's top-k, best first
    __shared__ double s_m[kSampleMaxK];       // masses, best first
    __shared__ double s_dm[kSampleMaxK];      // kept masses, vocabulary order
    __shared__ int s_di[kSampleMaxK];
    __shared__ int s_t;

    // the chunks' candidates as composites; 0 = empty (below every real one)
    const int n = S * k_eff;
    auto load = [&](int e) -> uint64_t {
        const int s = e / k_eff;
        const int t = e - s * k_eff;
        if (t >= min(V, s * C + C) - s * C) return 0;
        const uint2 p = chunk_cands(a, row, s)[t];
        return composite(p.x, p.y);
    };

    if (S <= kMergeChunks) {
        uint64_t* s_c = pool;                                  // [kMergeChunks * kSampleMaxK]
        uint64_t* s_sv = pool + kMergeChunks * kSampleMaxK;    // [kThreads]
        __shared__ uint64_t s_tau;
        for (int e = tid; e < n; e += kThreads) s_c[e] = load(e);
        if (tid == 0) s_cnt = 0u;
        __syncthreads();
        // Each chunk's list is sorted, best first, and all but possibly the
        // last hold k entries. Each of those `full` lists has q = ceil(k /
        // full) entries at or above its q-th, so the row's k-th largest is
        // at least the smallest of those q-th entries: only candidates at or
        // above it can be in the top k, and their rank among themselves is
        // their rank in the row.
        const int full = S - (V - (S - 1) * C < k_eff ? 1 : 0);
        if (wave == 0) {
            uint64_t t = ~0ull;
            if (full > 0 && lane < full) t = s_c[lane * k_eff + (k_eff + full - 1) / full - 1];
#pragma unroll
            for (int o = 32; o > 0; o >>= 1) {
                const uint64_t y = __shfl_xor(t, o, kWave);
                t = y < t ? y : t;
            }
            if (lane == 0) s_tau = full > 0 ? t : 1ull;
        }
        __syncthreads();
        const uint64_t tau = s_tau;
        const unsigned long long below = (1ull << lane) - 1ull;
        for (int e0 = 0; e0 < n; e0 += kThreads) {
            const int e = e0 + tid;
            const uint64_t me = e < n ? s_c[e] : 0ull;
            const bool keep = me >= tau && me != 0ull;
            const unsigned long long km = __builtin_amdgcn_ballot_w64(keep);
            if (km) {
                uint32_t base = 0;
                if (lane == 0) base = atomicAdd(&s_cnt, static_cast<uint32_t>(__builtin_popcountll(km)));
                base = __shfl(base, 0, kWave);
                const uint32_t slot = base + __builtin_popcountll(km & below);
                if (keep && slot < static_cast<uint32_t>(kThreads)) s_sv[slot] = me;
            }
        }
        __syncthreads();
        const int m = static_cast<int>(s_cnt);
        if (m <= kThreads) {
            if (tid < m) {
                const uint64_t me = s_sv[tid];
                int r = 0;
#pragma unroll 8
                for (int j = 0; j < m; ++j) r += s_sv[j] > me;
                if (r < k_eff) s_top[r] = me;
            }
        } else {
            // many candidates share the bound: a candidate's rank is its
            // position in its own list plus, for every other list, the
            // number of entries above it (binary searches)
            int step0 = 1;
            while (2 * step0 <= k_eff) step0 <<= 1;
            for (int e = tid; e < n; e += kThreads) {
                const uint64_t me = s_c[e];
                if (!me) continue;
                const int own = e / k_eff;
                int r = e - own * k_eff;
                for (int g = 0; g < S; g += kSearchLanes) {   // independent searches side by side
                    int pos[kSearchLanes];
#pragma unroll
                    for (int u = 0; u < kSearchLanes; ++u) pos[u] = 0;
                    for (int st = step0; st > 0; st >>= 1) {
#pragma unroll
                        for (int u = 0; u < kSearchLanes; ++u) {
                            const int s2 = min(g + u, S - 1);
                            if (pos[u] + st <= k_eff && s_c[s2 * k_eff + pos[u] + st - 1] > me) pos[u] += st;
                        }
                    }
#pragma unroll
                    for (int u = 0; u < kSearchLanes; ++u)
                        if (g + u < S && g + u != own) r += pos[u];
                }
                if (r < k_eff) s_top[r] = me;
            }
        }
        __syncthreads();
    } else {
        uint64_t c[kCandPerThread];
#pragma unroll
        for (int i = 0; i < kCandPerThread; ++i) {
            const int e = i * kThreads + tid;
            c[i] = e < n ? load(e) : 0;
        }
        if (tid == 0) s_cnt = 0u;

        // the k-th largest composite: key digits first, then index digits
        // (composites are distinct, so exactly k are at or above it)
        uint64_t prefix = 0, mask = 0;
        uint32_t rem = static_cast<uint32_t>(k_eff);
        bool done = cand_digit<2048>(c, 53, s_hist, s_dig, prefix, mask, rem);
        if (!done) done = cand_digit<2048>(c, 42, s_hist, s_dig, prefix, mask, rem);
        if (!done) done = cand_digit<1024>(c, 32, s_hist, s_dig, prefix, mask, rem);
        if (!done) done = cand_digit<2048>(c, 21, s_hist, s_dig, prefix, mask, rem);
        if (!done) done = cand_digit<2048>(c, 10, s_hist, s_dig, prefix, mask, rem);
        if (!done) cand_digit<1024>(c, 0, s_hist, s_dig, prefix, mask, rem);
        // taken: above the prefix, or matching it (the last bucket is taken whole)
        const unsigned long long below = (1ull << lane) - 1ull;
#pragma unroll
        for (int i = 0; i < kCandPerThread; ++i) {
            const bool take = c[i] && (c[i] & mask) >= prefix;
            const unsigned long long tm = __builtin_amdgcn_ballot_w64(take);
            if (tm) {
                uint32_t base = 0;
                if (lane == 0) base = atomicAdd(&s_cnt, static_cast<uint32_t>(__builtin_popcountll(tm)));
                base = __shfl(base, 0, kWave);
                const uint32_t slot = base + __builtin_popcountll(tm & below);
                if (take && slot < static_cast<uint32_t>(k_eff)) s_sel[slot] = c[i];
            }
        }
        __syncthreads();
        // best first, by counting
        if (tid < k_eff) {
            const uint64_t me = s_sel[tid];
            int r = 0;
#pragma unroll 8
            for (int j = 0; j < k_eff; ++j) r += s_sel[j] > me;
            s_top[r] = me;
        }
        __syncthreads();
    }
    if (T == 0.0f) {   // greedy: keys were the raw logits
        if (tid == 0) write_result(a, row, comp_index(s_top[0]), 1, 1);
        return;
    }

    const double zmax = static_cast<double>(key_value(comp_key(s_top[0])));
    if (tid < k_eff) s_m[tid] = exp(static_cast<double>(key_value(comp_key(s_top[tid]))) - zmax);
    __syncthreads();

    // top-p over the masses, best first (lane l holds entries 4l .. 4l+3)
    if (wave == 0) {
        double mm[4], loc = 0.0;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int i = 4 * lane + r;
            mm[r] = i < k_eff ? s_m[i] : 0.0;
            loc += mm[r];
        }
        const double incl = wave_incl_scan(loc, lane);
        const double total = __shfl(incl, kWave - 1, kWave);
        int t = k_eff;
        const float tp = a.top_p[row];
        if (tp < 1.0f) {
            const double need = static_cast<double>(tp) * total;
            double before = incl - loc;
            uint32_t cnt = 0;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = 4 * lane + r;
                if (i < k_eff && (i == 0 || before < need)) ++cnt;
                before += mm[r];
            }
            t = static_cast<int>(wave_sum_u32(cnt));
        }
        if (lane == 0) s_t = t;
    }
    __syncthreads();
    const int t = s_t;
    // kept tokens into vocabulary order (indices are distinct)
    if (tid < t) {
        const int me = comp_index(s_top[tid]);
        int pos = 0;
        for (int i = 0; i < t; ++i) pos += comp_index(s_top[i]) < me;
        s_di[pos] = me;
        s_dm[pos] = s_m[tid];
    }
    __syncthreads();
    // draw: first kept index whose cumulative mass exceeds u * total
    if (wave == 0) {
        double mm[4], loc = 0.0;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int i = 4 * lane + r;
            mm[r] = i < t ? s_dm[i] : 0.0;
            loc += mm[r];
        }
        const double incl = wave_incl_scan(loc, lane);
        const double target = static_cast<double>(a.u[row]) * __shfl(incl, kWave - 1, kWave);
        double run = incl - loc;
        int found = -1;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int i = 4 * lane + r;
            run += mm[r];
            if (found < 0 && i < t && run > target) found = i;
        }
        const unsigned long long hit = __builtin_amdgcn_ballot_w64(found >= 0);
        const int pos = hit ? __shfl(found, __builtin_ctzll(hit), kWave) : t - 1;  // rounding put u at the total
        if (lane == 0) write_result(a, row, s_di[pos], k_eff, t);
    }
}

// ---- whole-row path ------------------------------------------------------------
constexpr int kBatch = 8;   // loads issued together by the row loops

struct Row {
    const float* x;
    int V;
    float T;
    __device__ __forceinline__ float z(int j) const { return x[j] / T; }
};

// f(j, z_j) for j = tid, tid + kThreads, ... below V.
template <class F>
__device__ __forceinline__ void each_z(const Row& r, F&& f) {
    int j = threadIdx.x;
    for (; j + (kBatch - 1) * kThreads < r.V; j += kBatch * kThreads) {
        float v[kBatch];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) v[u] = r.x[j + u * kThreads];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) f(j + u * kThreads, v[u] / r.T);
    }
    for (; j < r.V; j += kThreads) f(j, r.z(j));
}

// f(j0, in, z) over the wave's segment [lo, hi) in index order, 64 indices
// j0 + lane at a time (in: j0 + lane < hi; z = 0 where not in). Wave-uniform.
template <class F>
__device__ __forceinline__ void each_seg(const Row& r, int lo, int hi, int lane, F&& f) {
    int j0 = lo;
    for (; j0 + kBatch * kWave <= hi; j0 += kBatch * kWave) {
        float v[kBatch];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) v[u] = r.x[j0 + u * kWave + lane];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) f(j0 + u * kWave, true, v[u] / r.T);
    }
    for (; j0 < hi; j0 += kWave) {
        const bool in = j0 + lane < hi;
        f(j0, in, in ? r.z(j0 + lane) : 0.0f);
    }
}

__device__ __forceinline__ void sample_whole_row(const SampleArgs& a, int row, float T, int kept_k) {
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const Row r{a.logits + static_cast<size_t>(row) * a.ld, a.vocab, T};
    const int V = r.V;
    const int k = a.top_k[row];
    __shared__ uint32_t s_cnt[256];
    __shared__ double s_mass[256];
    __shared__ float s_f[kWaves];
    __shared__ int s_i[kWaves];
    __shared__ double s_d[kWaves];
    __shared__ uint32_t s_u[kWaves];
    __shared__ int s_bin;
    __shared__ double s_above;

    // ---- max of z -------------------------------------------------------------
    float mz = -INFINITY;
    each_z(r, [&](int, float zj) { mz = fmaxf(mz, zj); });
    mz = wave_max(mz);
    if (lane == 0) s_f[wave] = mz;
    __syncthreads();
    mz = s_f[0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) mz = fmaxf(mz, s_f[w]);
    __syncthreads();
    const double zmax = static_cast<double>(mz);
    auto mass = [&](float zj) { return exp(static_cast<double>(zj) - zmax); };

    // Contiguous segment of the row owned by this wave (index order).
    const int seg_lo = static_cast<int>(static_cast<long long>(wave) * V / kWaves);
    const int seg_hi = static_cast<int>(static_cast<long long>(wave + 1) * V / kWaves);
    const unsigned long long lanes_below = (1ull << lane) - 1ull;

    // The `rank`-th (1-based) index, in index order, among elements with
    // pred(j, z_j) true; every thread gets it.
    auto nth_index = [&](auto pred, uint32_t rank) -> int {
        uint32_t c = 0;
        each_seg(r, seg_lo, seg_hi, lane, [&](int j0, bool in, float zj) {
            c += __builtin_popcountll(__builtin_amdgcn_ballot_w64(in && pred(j0 + lane, zj)));
        });
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
            each_seg(r, seg_lo, seg_hi, lane, [&](int j0, bool in, float zj) {
                const unsigned long long m = __builtin_amdgcn_ballot_w64(in && pred(j0 + lane, zj));
                const uint32_t n = __builtin_popcountll(m);
                if (found < 0 && acc + n >= rank) {
                    // the (rank - acc)-th set lane of m
                    const bool mine = ((m >> lane) & 1ull) && acc + __builtin_popcountll(m & lanes_below) + 1 == rank;
                    const unsigned long long hit = __builtin_amdgcn_ballot_w64(mine);
                    found = j0 + __builtin_ctzll(hit);
                }
                acc += n;
            });
            if (lane == 0) s_i[0] = found;
        }
        __syncthreads();
        const int idx = s_i[0];
        __syncthreads();
        return idx;
    };

    // ---- top-k: the k-th largest key, ties by index ---------------------------
    uint32_t kkey = 0;        // kept: key > kkey, or key == kkey and j <= kidx
    int kidx = V;
    if (kept_k < V) {
        uint32_t prefix = 0, mask = 0, rem = static_cast<uint32_t>(k);
        for (int shift = 24; shift >= 0; shift -= 8) {
            for (int i = tid; i < 256; i += kThreads) s_cnt[i] = 0;
            __syncthreads();
            each_z(r, [&](int, float zj) {
                const uint32_t key = order_key(zj);
                if ((key & mask) == prefix) atomicAdd(&s_cnt[(key >> shift) & 255u], 1u);
            });
            __syncthreads();
            if (wave == 0) {
                uint32_t above = 0;
                int b = find_bin_from_top<256>(s_cnt, rem, &above, lane);
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
        if (rem < ties) kidx = nth_index([&](int, float zj) { return order_key(zj) == kkey; }, rem);
    }
    auto in_k = [&](int j, uint32_t key) { return key > kkey || (key == kkey && j <= kidx); };

    // ---- top-p: boundary of the descending-mass prefix --------------------------
    const float tp = a.top_p[row];
    uint32_t pkey = 0;        // kept: in_k and (key > pkey, or key == pkey and j <= pidx)
    int pidx = V;
    if (tp < 1.0f) {
        double tot = 0.0;
        each_z(r, [&](int j, float zj) {
            if (in_k(j, order_key(zj))) tot += mass(zj);
        });
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
            each_z(r, [&](int j, float zj) {
                const uint32_t key = order_key(zj);
                if ((key & mask) == prefix && in_k(j, key)) {
                    atomicAdd(&s_mass[(key >> shift) & 255u], mass(zj));
                    atomicAdd(&s_cnt[(key >> shift) & 255u], 1u);
                }
            });
            __syncthreads();
            if (wave == 0) {
                double ab = 0.0;
                int b = find_bin_from_top<256>(s_mass, need - above, &ab, lane);
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
        const double pb = mass(key_value(pkey));
        const double t = (need - above) / pb;
        uint32_t keep = t <= 1.0 ? 1u : static_cast<uint32_t>(fmin(ceil(t), static_cast<double>(ties)));
        if (keep < 1u) keep = 1u;
        if (keep < ties)
            pidx = nth_index([&](int j, float zj) {
                const uint32_t key = order_key(zj);
                return key == pkey && in_k(j, key);
            }, keep);
    }
    auto kept = [&](int j, uint32_t key) { return in_k(j, key) && (key > pkey || (key == pkey && j <= pidx)); };

    // ---- draw: inverse CDF in index order --------------------------------------
    double wsum = 0.0;
    uint32_t wcnt = 0;
    each_seg(r, seg_lo, seg_hi, lane, [&](int j0, bool in, float zj) {
        if (in && kept(j0 + lane, order_key(zj))) {
            wsum += mass(zj);
            ++wcnt;
        }
    });
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
        each_seg(r, seg_lo, seg_hi, lane, [&](int j0, bool in, float zj) {
            if (found >= 0) return;
            const bool k_in = in && kept(j0 + lane, order_key(zj));
            const double incl = wave_incl_scan(k_in ? mass(zj) : 0.0, lane);
            const unsigned long long cross = __builtin_amdgcn_ballot_w64(k_in && run + incl > target);
            const unsigned long long any = __builtin_amdgcn_ballot_w64(k_in);
            if (any) last = j0 + 63 - __builtin_clzll(any);
            if (cross) found = j0 + __builtin_ctzll(cross);
            run += __shfl(incl, kWave - 1, kWave);
        });
        if (lane == 0) s_i[0] = found >= 0 ? found : last;
    }
    __syncthreads();
    if (tid == 0) write_result(a, row, s_i[0], kept_k, static_cast<int>(kept_p));
}

// ---- histogram path, pass 2 ----------------------------------------------------------
constexpr int kBucketCap = kSampleBucketCap;   // tokens of the top-p boundary bin held in LDS
constexpr int kPoolWords = 3 * kSampleHistBins / 2 + kBucketCap;   // fp64 bins, u32 counts, the bin's tokens
static_assert(kSampleHistBins == 2 * kThreads, "two merged bins per thread");
static_assert(kSampleHistChunks <= kWave, "one lane per chunk in the draw");
static_assert(kSampleChunk == kWaves * 8 * kWave, "the walk covers a chunk with 8 loads per lane");
static_assert(kSampleHistChunks * kSampleChunk <= (1 << 19), "indices fit the 19 bits of the tie digits");
static_assert(kPoolWords >= kMergeChunks * kSampleMaxK + 2 * kThreads, "the pool holds the candidate finish");
static_assert(kBucketCap % (kWaves * kWave) == 0, "whole rows of the per-wave regions");

// One digit of the boundary search inside the gathered bin: fp64 masses and
// counts of the tokens matching `prefix` under `pmask`, per NB bins of the
// key bits at `shift`; then the bin, from the top, at which the mass
// reaches `rest`. `above` grows by the mass of the bins above it. When
// rounding leaves the gathered mass just short of `rest`, the boundary is
// the lowest token: the lowest non-empty bin is taken.
template <int NB>
__device__ __forceinline__ void bucket_digit(const uint64_t* s_bk, uint32_t n1, int shift, double zmax, double rest,
                                             double* s_bin, uint32_t* s_cnt, int* s_ri, double* s_rd,
                                             uint32_t& prefix, uint32_t& pmask, double& above) {
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    for (int b = tid; b < NB; b += kThreads) {
        s_bin[b] = 0.0;
        s_cnt[b] = 0u;
    }
    __syncthreads();
    for (uint32_t e = tid; e < n1; e += kThreads) {
        const uint32_t key = comp_key(s_bk[e]);
        if ((key & pmask) == prefix) {
            const uint32_t b = (key >> shift) & (NB - 1);
            atomicAdd(&s_bin[b], exp(static_cast<double>(key_value(key)) - zmax));
            atomicAdd(&s_cnt[b], 1u);
        }
    }
    __syncthreads();
    if (tid < kWave) {
        double ab = 0.0;
        int b = find_bin_from_top<NB>(s_bin, rest, &ab, lane);
        if (lane == 0) {
            if (b < 0) {
                b = 0;
                while (b < NB - 1 && s_cnt[b] == 0u) ++b;
                ab = 0.0;
                for (int i = NB - 1; i > b; --i) ab += s_bin[i];
            }
            s_ri[0] = b;
            s_rd[0] = ab;
        }
    }
    __syncthreads();
    prefix |= static_cast<uint32_t>(s_ri[0]) << shift;
    pmask |= static_cast<uint32_t>(NB - 1) << shift;
    above += s_rd[0];
}

// One digit of the search for the rem-th smallest index among the gathered
// tokens whose key is `key` (index bits at `shift`, NB bins, counted from
// the top as NB - 1 - digit).
template <int NB>
__device__ __forceinline__ void tie_digit(const uint64_t* s_bk, uint32_t n1, uint32_t key, int shift,
                                          uint32_t* s_cnt, int* s_ri, uint32_t& ip, uint32_t& imask, uint32_t& rem) {
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    for (int b = tid; b < NB; b += kThreads) s_cnt[b] = 0u;
    __syncthreads();
    for (uint32_t e = tid; e < n1; e += kThreads) {
        const uint64_t c = s_bk[e];
        const uint32_t idx = static_cast<uint32_t>(comp_index(c));
        if (comp_key(c) == key && (idx & imask) == ip) atomicAdd(&s_cnt[NB - 1 - ((idx >> shift) & (NB - 1))], 1u);
    }
    __syncthreads();
    if (tid < kWave) {
        uint32_t ab = 0;
        const int b = find_bin_from_top<NB>(s_cnt, rem, &ab, lane);   // rem never exceeds the tied tokens
        if (lane == 0) {
            s_ri[0] = b < 0 ? NB - 1 : b;
            s_ri[1] = static_cast<int>(ab);
        }
    }
    __syncthreads();
    ip |= static_cast<uint32_t>(NB - 1 - s_ri[0]) << shift;
    imask |= static_cast<uint32_t>(NB - 1) << shift;
    rem -= static_cast<uint32_t>(s_ri[1]);
}

// The least order key kx of a logit x with key(fl(x / T)) >= target, or
// 0xFFFFFFFF when no finite logit reaches it; called by a whole wave.
// Correctly rounded division by T > 0 is monotone in x, and so is the key of
// its result: a test of the scaled logit's key against `target` is a test of
// kx against this value. Each step tests 64 evenly spaced keys of the range
// left (those of -inf .. +inf at first; finite logits lie strictly inside).
__device__ __forceinline__ uint32_t wave_key_threshold(uint32_t target, float T, int lane) {
    auto reaches = [&](uint32_t kx) { return order_key(key_value(kx) / T) >= target; };
    uint32_t lo = 0x007FFFFFu, hi = 0xFF800000u;   // reaches(hi); every key below lo fails
    if (!reaches(hi)) return 0xFFFFFFFFu;
    while (lo < hi) {
        const uint32_t step = (hi - lo + kWave - 1) / kWave;
        const uint32_t c = min(hi, lo + static_cast<uint32_t>(lane) * step);
        const unsigned long long ok = __builtin_amdgcn_ballot_w64(reaches(c));
        if (!ok) {
            lo = __shfl(c, kWave - 1, kWave) + 1;
        } else {
            const int f = __builtin_ctzll(ok);
            hi = __shfl(c, f, kWave);
            if (f > 0) lo = __shfl(c, f - 1, kWave) + 1;
            else lo = hi;
        }
    }
    return lo;
}

constexpr int kGatherBatch = 8;                    // float4 loads per lane in flight in the gathering pass
constexpr int kWaveCap = kBucketCap / kWaves;      // tokens of the bin one wave's slice may hold

// The gathering pass's test of one element per lane (every lane of the wave
// together): whether x lies in the bin (appended to the wave's region, at
// most kWaveCap) and whether it lies above it (counted). kByKey compares
// order keys (needed when a threshold is +0, which a float compare does not
// tell from -0), else floats; kAll: every lane holds an element.
template <bool kByKey, bool kAll>
struct BinTest {
    uint32_t k_lo, k_hi;
    float f_lo, f_hi;
    uint2* s_reg;
    __device__ __forceinline__ void operator()(float xj, int j, bool in, uint32_t& n_w, uint32_t& above_w) const {
        bool mem, abv;
        if constexpr (kByKey) {
            const uint32_t kx = order_key(xj);
            mem = kx >= k_lo && kx < k_hi;
            abv = kx >= k_hi;
        } else {
            mem = xj >= f_lo && xj < f_hi;
            abv = xj >= f_hi;
        }
        if constexpr (!kAll) {
            mem = mem && in;
            abv = abv && in;
        }
        above_w += static_cast<uint32_t>(__builtin_popcountll(__builtin_amdgcn_ballot_w64(abv)));
        const unsigned long long m = __builtin_amdgcn_ballot_w64(mem);
        if (m) {
            const uint32_t slot =
                n_w + __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(m >> 32),
                                                 __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(m), 0u));
            if (mem && slot < static_cast<uint32_t>(kWaveCap)) s_reg[slot] = make_uint2(__float_as_uint(xj), static_cast<uint32_t>(j));
            n_w += static_cast<uint32_t>(__builtin_popcountll(m));
        }
    }
};

// One wave's float4 units [ubeg, uend) of the row (x4 = the row from its
// first 16-byte boundary, element h0): kGatherBatch loads per lane at a time.
template <bool kByKey>
__device__ __forceinline__ void gather_units(const float4* x4, int h0, int ubeg, int uend, int lane,
                                             const BinTest<kByKey, true>& full, const BinTest<kByKey, false>& part,
                                             uint32_t& n_w, uint32_t& above_w) {
    int u0 = ubeg;
    for (; u0 + kGatherBatch * kWave <= uend; u0 += kGatherBatch * kWave) {
        float4 v[kGatherBatch];
#pragma unroll
        for (int i = 0; i < kGatherBatch; ++i) v[i] = x4[u0 + i * kWave + lane];
#pragma unroll
        for (int i = 0; i < kGatherBatch; ++i) {
            const int j = h0 + 4 * (u0 + i * kWave + lane);
            full(v[i].x, j, true, n_w, above_w);
            full(v[i].y, j + 1, true, n_w, above_w);
            full(v[i].z, j + 2, true, n_w, above_w);
            full(v[i].w, j + 3, true, n_w, above_w);
        }
    }
    for (; u0 < uend; u0 += kWave) {
        const int uu = u0 + lane;
        const bool in = uu < uend;
        const float4 v = x4[in ? uu : uend - 1];
        const int j = h0 + 4 * uu;
        part(v.x, j, in, n_w, above_w);
        part(v.y, j + 1, in, n_w, above_w);
        part(v.z, j + 2, in, n_w, above_w);
        part(v.w, j + 3, in, n_w, above_w);
    }
}

// Rows with top-k off, from the chunks' maxima and histograms. Returns
// false, the same in every thread, when the top-p boundary's bin holds more
// than kBucketCap tokens; the caller then takes the whole-row path.
__device__ __forceinline__ bool finish_from_histograms(const SampleArgs& a, int row, int g, float T, uint64_t* pool) {
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const int V = a.vocab;
    const int S = a.chunks;
    const int C = (V + S - 1) / S;
    const Row r{a.logits + static_cast<size_t>(row) * a.ld, V, T};
    double* s_bin = reinterpret_cast<double*>(pool);                          // [kSampleHistBins]
    uint32_t* s_cnt = reinterpret_cast<uint32_t*>(pool + kSampleHistBins);    // [kSampleHistBins]
    uint64_t* s_bk = pool + 3 * kSampleHistBins / 2;                          // [kBucketCap]
    __shared__ double s_scale[kSampleHistChunks];   // exp(chunk max - row max)
    __shared__ double s_kc[kSampleHistChunks];      // kept mass per chunk
    __shared__ double s_wd[kWaves];
    __shared__ uint32_t s_wu[kWaves];
    __shared__ int s_ri[2];
    __shared__ double s_rd[2];
    __shared__ uint32_t s_n;
    __shared__ uint32_t s_thr[2];
    __shared__ uint32_t s_wn[kWaves];
    __shared__ uint64_t s_small[kWave];
    __shared__ double s_kcw[kWaves][kSampleHistChunks];   // per wave: kept mass of gathered tokens per chunk
    __shared__ uint32_t s_base;

    const float tp = a.top_p[row];
    if (g != 0 && !(tp < 1.0f)) return true;   // only the gathering pass is shared out

    // ---- max z from the chunks' maxima ----------------------------------------------
    if (tid < S) s_scale[tid] = static_cast<double>(chunk_head(a, row, tid)->mc);
    __syncthreads();
    double zmax = s_scale[0];
    for (int c = 1; c < S; ++c) zmax = fmax(zmax, s_scale[c]);
    __syncthreads();
    if (tid < S) {
        s_scale[tid] = exp(s_scale[tid] - zmax);
        s_kc[tid] = 0.0;
    }
    if (tid == 0) s_n = 0u;
    __syncthreads();

    uint32_t pkey = 0;   // kept: key > pkey, or key == pkey and index <= pidx
    int pidx = V;
    uint32_t kept_p = static_cast<uint32_t>(V);
    if (tp < 1.0f) {
        // ---- the bin holding the boundary: the largest b with I[b] >= need, where
        // I[b] = sum over chunks of scale x suffix mass (two levels: the 64
        // group starts 32k, then the 33 bins from the group's start) --------
        if (wave == 0) {
            const double t = lane < S ? s_scale[lane] * chunk_head(a, row, lane)->total : 0.0;
            const double tot = wave_sum_f64(t);
            if (lane == 0) s_rd[0] = tot;
        }
        __syncthreads();
        const double need = static_cast<double>(tp) * s_rd[0];
        // I at bin b by the 16 lanes of a group (chunks cs, cs + 16, ...), the
        // same order wherever it is evaluated
        auto suffix_at = [&](int b) -> double {
            double v = 0.0;
            if (b < kSampleHistBins)
                for (int c = tid & 15; c < S; c += 16) v += s_scale[c] * chunk_hist(a, row, c)[b];
#pragma unroll
            for (int o = 1; o < 16; o <<= 1) v += __shfl_xor(v, o, kWave);
            return v;
        };
        {
            const double v = suffix_at(32 * (tid >> 4));
            if ((tid & 15) == 0) s_bin[tid >> 4] = v;
        }
        __syncthreads();
        if (wave == 0) {
            const unsigned long long ok = __builtin_amdgcn_ballot_w64(s_bin[lane] >= need);
            if (lane == 0) s_ri[0] = ok ? 63 - __builtin_clzll(ok) : 0;
        }
        __syncthreads();
        const int kA = s_ri[0];
        if (tid < 33 * 16) {
            const double v = suffix_at(32 * kA + (tid >> 4));
            if ((tid & 15) == 0) s_bin[64 + (tid >> 4)] = v;
        }
        __syncthreads();
        if (wave == 0) {
            const unsigned long long ok = __builtin_amdgcn_ballot_w64(lane < 32 && s_bin[64 + lane] >= need);
            const int i = ok ? 63 - __builtin_clzll(ok) : 0;
            if (lane == 0) {
                s_ri[0] = 32 * kA + i;
                s_rd[0] = s_bin[64 + i + 1];   // I[b1 + 1]: the mass above the bin
            }
        }
        __syncthreads();
        const uint32_t b1 = static_cast<uint32_t>(s_ri[0]);
        double above = s_rd[0];

        // ---- gather the boundary bin's tokens; count the tokens above it ----------
        // The bin test is a test of x itself against two thresholds: as
        // floats, or as order keys when one of them is +0 (which a float
        // compare does not tell from -0). Each wave appends to its own region
        // of the list (no atomics); the regions are compacted afterwards.
        if (wave < 2) {
            const uint32_t hb = b1 + static_cast<uint32_t>(wave);
            const uint32_t k = hb >= static_cast<uint32_t>(kSampleHistBins) ? 0xFFFFFFFFu
                                                                             : wave_key_threshold(hb << 21, T, lane);
            if (lane == 0) s_thr[wave] = k;
        }
        if (tid == 0) s_n = 0u;   // set when a wave's share overflows its region
        __syncthreads();
        const uint32_t k_lo = s_thr[0], k_hi = s_thr[1];
        const float f_lo = key_value(k_lo);                              // NaN when nothing reaches the bin
        const float f_hi = k_hi == 0xFFFFFFFFu ? INFINITY : key_value(k_hi);
        const bool by_key = k_lo == 0x80000000u || k_hi == 0x80000000u;
        uint32_t n_w = 0;       // tokens of the bin in this wave's slice
        uint32_t above_w = 0;   // tokens above the bin in this wave's slice
        uint2* s_reg = reinterpret_cast<uint2*>(s_bk) + wave * kWaveCap;
        // elements before the first 16-byte boundary and after the last: wave 0
        const float* x = r.x;
        const int h0 = min(V, static_cast<int>((4u - ((reinterpret_cast<uintptr_t>(x) >> 2) & 3u)) & 3u));
        const int n4 = (V - h0) / 4;
        const int t0 = h0 + 4 * n4;
        const float4* x4 = reinterpret_cast<const float4*>(x + h0);
        // this workgroup's share of the units, then this wave's
        const int gbeg = static_cast<int>(static_cast<long long>(g) * n4 / kSampleRowSplit);
        const int gend = static_cast<int>(static_cast<long long>(g + 1) * n4 / kSampleRowSplit);
        const int ubeg = gbeg + static_cast<int>(static_cast<long long>(wave) * (gend - gbeg) / kWaves);
        const int uend = gbeg + static_cast<int>(static_cast<long long>(wave + 1) * (gend - gbeg) / kWaves);
        if (by_key) {
            const BinTest<true, true> full{k_lo, k_hi, f_lo, f_hi, s_reg};
            const BinTest<true, false> part{k_lo, k_hi, f_lo, f_hi, s_reg};
            if (wave == 0 && g == 0) {
                const bool in = lane < h0 + (V - t0);
                const int j = lane < h0 ? lane : t0 + (lane - h0);
                part(x[in ? j : 0], j, in, n_w, above_w);
            }
            gather_units<true>(x4, h0, ubeg, uend, lane, full, part, n_w, above_w);
        } else {
            const BinTest<false, true> full{k_lo, k_hi, f_lo, f_hi, s_reg};
            const BinTest<false, false> part{k_lo, k_hi, f_lo, f_hi, s_reg};
            if (wave == 0 && g == 0) {
                const bool in = lane < h0 + (V - t0);
                const int j = lane < h0 ? lane : t0 + (lane - h0);
                part(x[in ? j : 0], j, in, n_w, above_w);
            }
            gather_units<false>(x4, h0, ubeg, uend, lane, full, part, n_w, above_w);
        }
        if (lane == 0) {
            s_wn[wave] = n_w;
            s_wu[wave] = above_w;
            if (n_w > static_cast<uint32_t>(kWaveCap)) s_n = 1u;
        }
        __syncthreads();
        constexpr uint32_t kShare = kBucketCap / kSampleRowSplit;   // list entries per workgroup
        uint32_t n_g = 0, pre = 0, above_g = 0;
        for (int w = 0; w < kWaves; ++w) {
            if (w == wave) pre = n_g;
            n_g += s_wn[w];
            above_g += s_wu[w];
        }
        const bool wg_over = s_n != 0u || n_g > kShare;
        if (!wg_over) {   // compact the waves' regions, logit keys becoming keys of z = x / T
            uint2 mine[kWaveCap / kWave];
#pragma unroll
            for (int i = 0; i < kWaveCap / kWave; ++i) {
                const uint32_t e = static_cast<uint32_t>(i * kWave + lane);
                mine[i] = e < n_w ? s_reg[e] : make_uint2(0u, 0u);
            }
            __syncthreads();
#pragma unroll
            for (int i = 0; i < kWaveCap / kWave; ++i) {
                const uint32_t e = static_cast<uint32_t>(i * kWave + lane);
                if (e < n_w) s_bk[pre + e] = composite(order_key(__uint_as_float(mine[i].x) / T), mine[i].y);
            }
            __syncthreads();
        }

        // ---- the row's workgroups pool their shares; the last one to finish goes on
        uint32_t* rc = row_counters(a, row);
        uint64_t* rl = row_list(a, row);
        if (!wg_over)
            for (uint32_t e = tid; e < n_g; e += kThreads) rl[g * kShare + e] = s_bk[e];
        if (tid == 0) {
            rc[2 + 2 * g] = wg_over ? 0xFFFFFFFFu : n_g;
            rc[3 + 2 * g] = above_g;
        }
        __syncthreads();
        if (tid == 0) {
            // release: the workgroup's entries (complete in L2 after the
            // barrier) are written back before it reports; the last to
            // report acquires them (one fence each way, not one per wave)
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
            const uint32_t t = atomicAdd(&rc[0], 1u);
            const bool last = t == static_cast<uint32_t>(kSampleRowSplit - 1);
            if (last) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
            s_n = last ? 1u : 0u;
        }
        __syncthreads();
        if (!s_n) return true;
        // every other workgroup of the row has published its share: append
        // theirs after this one's own (already in LDS)
        uint32_t cnt[kSampleRowSplit], start[kSampleRowSplit];
        uint32_t n1 = n_g, n_above = 0;
        bool over = wg_over;
#pragma unroll
        for (int h = 0; h < kSampleRowSplit; ++h) {
            cnt[h] = h == g ? n_g : rc[2 + 2 * h];
            over = over || cnt[h] == 0xFFFFFFFFu;
            n_above += h == g ? above_g : rc[3 + 2 * h];
        }
        if (over) return false;
#pragma unroll
        for (int h = 0; h < kSampleRowSplit; ++h) {   // the other shares, in order, after this one's
            start[h] = n1;
            if (h != g) n1 += cnt[h];
        }
        for (uint32_t e = n_g + tid; e < n1; e += kThreads) {
            int hh = 0;
#pragma unroll
            for (int h = 0; h < kSampleRowSplit; ++h)
                if (h != g && e >= start[h]) hh = h;   // the last share starting at or below e
            s_bk[e] = rl[hh * kShare + (e - start[hh])];
        }
        __syncthreads();

        // ---- the boundary key: more digits over the gathered tokens ----------------
        uint32_t prefix = b1 << 21, pmask = 0xFFE00000u;
        bucket_digit<2048>(s_bk, n1, 10, zmax, need - above, s_bin, s_cnt, s_ri, s_rd, prefix, pmask, above);
        const uint32_t m2 = s_cnt[(prefix >> 10) & 2047u];   // tokens sharing the 21-bit prefix
        if (tid == 0) s_n = 0u;
        __syncthreads();
        if (m2 <= static_cast<uint32_t>(kWave)) {
            // Few: one wave orders them (distinct composites: ranks by
            // comparison) and scans their masses in that order.
            for (uint32_t e = tid; e < n1; e += kThreads) {
                const uint64_t c = s_bk[e];
                if ((comp_key(c) & pmask) == prefix) s_small[atomicAdd(&s_n, 1u)] = c;
            }
            __syncthreads();
            if (wave == 0) {
                const uint64_t me = lane < static_cast<int>(m2) ? s_small[lane] : 0ull;
                int rk = 0;
                for (int i = 0; i < static_cast<int>(m2); ++i) rk += __shfl(me, i, kWave) > me ? 1 : 0;
                // element of rank `lane`, best first
                const uint32_t lo32 = static_cast<uint32_t>(__builtin_amdgcn_ds_permute(4 * rk, static_cast<int>(me)));
                const uint32_t hi32 = static_cast<uint32_t>(__builtin_amdgcn_ds_permute(4 * rk, static_cast<int>(me >> 32)));
                const uint64_t srt = (static_cast<uint64_t>(hi32) << 32) | lo32;
                const bool real = lane < static_cast<int>(m2);
                const double m = real ? exp(static_cast<double>(key_value(comp_key(srt))) - zmax) : 0.0;
                const double incl = wave_incl_scan(m, lane);
                const unsigned long long reach = __builtin_amdgcn_ballot_w64(real && above + incl >= need);
                const int t = reach ? __builtin_ctzll(reach) : static_cast<int>(m2) - 1;   // rounding: the last
                const uint64_t bnd = __shfl(srt, t, kWave);
                if (lane == 0) {
                    s_ri[0] = static_cast<int>(comp_key(bnd));
                    s_ri[1] = comp_index(bnd);
                }
            }
            __syncthreads();
            pkey = static_cast<uint32_t>(s_ri[0]);
            pidx = s_ri[1];
        } else {
            bucket_digit<1024>(s_bk, n1, 0, zmax, need - above, s_bin, s_cnt, s_ri, s_rd, prefix, pmask, above);
            pkey = prefix;
            const uint32_t ties = s_cnt[pkey & 1023u];
            __syncthreads();   // the tie count is read before the counts are reused
            // every tie has the same mass; keep the first `keep` of them in index order
            const double pb = exp(static_cast<double>(key_value(pkey)) - zmax);
            const double t = (need - above) / pb;
            const uint32_t keep = t <= 1.0 ? 1u : static_cast<uint32_t>(fmin(ceil(t), static_cast<double>(ties)));
            if (keep < ties) {
                uint32_t ip = 0, imask = 0, rem = keep;
                tie_digit<1024>(s_bk, n1, pkey, 9, s_cnt, s_ri, ip, imask, rem);
                tie_digit<512>(s_bk, n1, pkey, 0, s_cnt, s_ri, ip, imask, rem);
                pidx = static_cast<int>(ip);
            }
        }

        // ---- kept mass per chunk: the bins above b1, plus the gathered tokens kept --
        // Gathered tokens: each mass once; consecutive list entries mostly
        // share a chunk, so a wave adds the entries of one chunk at a time
        // into its own row of s_kcw.
        for (int i = tid; i < kWaves * kSampleHistChunks; i += kThreads) (&s_kcw[0][0])[i] = 0.0;
        __syncthreads();
        uint32_t nk = 0;
        for (uint32_t e0 = static_cast<uint32_t>(wave) * kWave; e0 < n1; e0 += kThreads) {   // wave-uniform
            const uint32_t e = e0 + lane;
            int ch = -1;
            double m = 0.0;
            if (e < n1) {
                const uint64_t cc = s_bk[e];
                const uint32_t key = comp_key(cc);
                const int j = comp_index(cc);
                if (key > pkey || (key == pkey && j <= pidx)) {
                    ch = j / C;
                    m = exp(static_cast<double>(key_value(key)) - zmax);
                    ++nk;
                }
            }
            unsigned long long todo = __builtin_amdgcn_ballot_w64(ch >= 0);
            while (todo) {
                const int c0 = __shfl(ch, __builtin_ctzll(todo), kWave);
                const bool mine = ch == c0;
                const double sum = wave_sum_f64(mine ? m : 0.0);
                if (lane == 0) s_kcw[wave][c0] += sum;
                todo &= ~__builtin_amdgcn_ballot_w64(mine);
            }
        }
        nk = wave_sum_u32(nk);
        if (lane == 0) s_wu[wave] = nk;
        __syncthreads();
        kept_p = n_above;
        for (int w = 0; w < kWaves; ++w) kept_p += s_wu[w];
        if (tid < S) {
            const double acc = b1 + 1 < static_cast<uint32_t>(kSampleHistBins) ? chunk_hist(a, row, tid)[b1 + 1] : 0.0;
            double bsum = 0.0;
            for (int w = 0; w < kWaves; ++w) bsum += s_kcw[w][tid];
            s_kc[tid] = s_scale[tid] * acc + bsum;
        }
        __syncthreads();
    } else {
        if (tid < S) s_kc[tid] = s_scale[tid] * chunk_head(a, row, tid)->total;
        __syncthreads();
    }

    // ---- draw: the chunk, then the token, in vocabulary order ----------------------
    if (wave == 0) {
        const double kc = lane < S ? s_kc[lane] : 0.0;
        const double incl = wave_incl_scan(kc, lane);
        const double target = static_cast<double>(a.u[row]) * __shfl(incl, kWave - 1, kWave);
        const unsigned long long hit = __builtin_amdgcn_ballot_w64(kc > 0.0 && incl > target);
        const unsigned long long any = __builtin_amdgcn_ballot_w64(kc > 0.0);
        // rounding may put the target at the total: the last chunk with kept mass
        const int c = hit ? __builtin_ctzll(hit) : (any ? 63 - __builtin_clzll(any) : 0);
        const double before = __shfl(incl - kc, c, kWave);
        if (lane == 0) {
            s_ri[0] = c;
            s_rd[0] = target;
            s_rd[1] = before;
        }
    }
    __syncthreads();
    const double target = s_rd[0];
    const int lo = s_ri[0] * C;
    const int hi = min(V, lo + C);
    const int base = lo + wave * (8 * kWave);   // this wave's 512 indices of the chunk
    double mm[8];
    uint32_t kbits = 0;
    double wsum = 0.0;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
        const int j = base + u * kWave + lane;
        const float zj = r.x[min(j, hi - 1)] / T;
        const uint32_t key = order_key(zj);
        const bool kp = j < hi && (key > pkey || (key == pkey && j <= pidx));
        mm[u] = kp ? exp(static_cast<double>(zj) - zmax) : 0.0;
        kbits |= static_cast<uint32_t>(kp) << u;
        wsum += mm[u];
    }
    wsum = wave_sum_f64(wsum);
    const bool wany = __builtin_amdgcn_ballot_w64(kbits != 0u) != 0ull;
    if (lane == 0) {
        s_wd[wave] = wsum;
        s_wu[wave] = wany;
    }
    __syncthreads();
    double pre = s_rd[1], pre_last = pre;
    int wh = -1, wl = 0;
    for (int w = 0; w < kWaves; ++w) {
        if (!s_wu[w]) continue;
        if (pre + s_wd[w] > target) {
            wh = w;
            break;
        }
        wl = w;
        pre_last = pre;
        pre += s_wd[w];
    }
    if (wh < 0) {   // rounding put the target at the chunk's total: its last kept token
        wh = wl;
        pre = pre_last;
    }
    if (wave == wh) {
        double run = pre;
        int found = -1, last = -1;
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const bool kp = (kbits >> u) & 1u;
            const double incl = wave_incl_scan(mm[u], lane);
            const unsigned long long cross = __builtin_amdgcn_ballot_w64(kp && run + incl > target);
            const unsigned long long any = __builtin_amdgcn_ballot_w64(kp);
            const int j0 = base + u * kWave;
            if (any) last = j0 + 63 - __builtin_clzll(any);
            if (found < 0 && cross) found = j0 + __builtin_ctzll(cross);
            run += __shfl(incl, kWave - 1, kWave);
        }
        if (lane == 0) write_result(a, row, found >= 0 ? found : last, V, static_cast<int>(kept_p));
    }
    return true;
}

// ---- the finishing kernel: one workgroup per row, on the row's path ---------------
// blockIdx.x = row * kSampleRowSplit + g: histogram rows share the gathering
// pass among their g workgroups; every other row is finished by g = 0 alone.
__global__ __launch_bounds__(kThreads) void sample_row_kernel(SampleArgs a) {
    __shared__ uint64_t s_pool[kPoolWords];
    const int row = blockIdx.x / kSampleRowSplit;
    const int g = blockIdx.x - row * kSampleRowSplit;
    const float T = a.temperature[row];
    if (!(T >= 0.0f)) {   // negative or NaN temperature: no token
        if (g == 0 && threadIdx.x == 0) write_result(a, row, -1, 0, 0);
        return;
    }
    const int k_eff = T > 0.0f ? kept_by_k(a.top_k[row], a.vocab) : 1;
    if (on_hist_path(T, k_eff, a.vocab, a.chunks) && !on_candidate_path(T, k_eff, a.chunks)) {
        if (!finish_from_histograms(a, row, g, T, s_pool)) sample_whole_row(a, row, T, k_eff);
        return;
    }
    if (g != 0) return;
    if (on_candidate_path(T, k_eff, a.chunks)) finish_from_candidates(a, row, T, k_eff, s_pool);
    else sample_whole_row(a, row, T, k_eff);
}

}  // namespace

hipError_t launch_sample(const SampleArgs& a, int rows, hipStream_t stream) {
    hipLaunchKernelGGL(sample_chunk_kernel, dim3(rows * a.chunks), dim3(kChunkThreads), 0, stream, a);
    hipLaunchKernelGGL(sample_row_kernel, dim3(rows * kSampleRowSplit), dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace pkv
