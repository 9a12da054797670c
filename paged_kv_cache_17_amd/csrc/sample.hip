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
// Two paths, chosen per row on the device:
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
//  * whole-row path (top-k off or large): one 1024-thread workgroup per row
//    finds the k-th largest key and the top-p boundary by radix descents
//    over the row (counts, and fp64 mass sums, per 8-bit digit in LDS);
//    ties at a boundary are resolved in index order with wave ballots.
// The second kernel runs both: each workgroup takes its row's path.
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

// One workgroup per (row, chunk), blockIdx.x = row * chunks + chunk. Writes
// the chunk's min(k, chunk length) best (key, index) pairs to its candidate
// slots, best first (decreasing key, ties by lower index).
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
    if (!on_candidate_path(T, k_eff, S)) return;
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
    __shared__ uint64_t s_keep[kChunkKeep];
    __shared__ uint32_t s_hist[2048];
    __shared__ uint32_t s_tc[kPerThread * kChunkWaves];
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
    uint2* out = a.cand + (static_cast<size_t>(row) * S + s) * kSampleMaxK;
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

__device__ __forceinline__ void finish_from_candidates(const SampleArgs& a, int row, float T, int k_eff) {
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const int V = a.vocab;
    const int S = a.chunks;
    const int C = (V + S - 1) / S;

    __shared__ uint32_t s_hist[2048];
    __shared__ int s_dig[3];                  // digit step: bin, count above it, bucket == rest
    __shared__ uint32_t s_cnt;
    __shared__ uint64_t s_sel[kSampleMaxK];   // the row's top-k, any order
    __shared__ uint64_t s_top[kSampleMaxK];   // the row's top-k, best first
    __shared__ double s_m[kSampleMaxK];       // masses, best first
    __shared__ double s_dm[kSampleMaxK];      // kept masses, vocabulary order
    __shared__ int s_di[kSampleMaxK];
    __shared__ int s_t;

    // the chunks' candidates as composites; 0 = empty (below every real one)
    const uint2* cand = a.cand + static_cast<size_t>(row) * S * kSampleMaxK;
    const int n = S * k_eff;
    auto load = [&](int e) -> uint64_t {
        const int s = e / k_eff;
        const int t = e - s * k_eff;
        if (t >= min(V, s * C + C) - s * C) return 0;
        const uint2 p = cand[static_cast<size_t>(s) * kSampleMaxK + t];
        return composite(p.x, p.y);
    };

    if (S <= kMergeChunks) {
        __shared__ uint64_t s_c[kMergeChunks * kSampleMaxK];
        __shared__ uint64_t s_sv[kThreads];
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

// ---- pass 2 of the candidate path, and the whole-row path -------------------------
__global__ __launch_bounds__(kThreads) void sample_row_kernel(SampleArgs a) {
    const int row = blockIdx.x;
    const float T = a.temperature[row];
    if (!(T >= 0.0f)) {   // negative or NaN temperature: no token
        if (threadIdx.x == 0) write_result(a, row, -1, 0, 0);
        return;
    }
    const int k_eff = T > 0.0f ? kept_by_k(a.top_k[row], a.vocab) : 1;
    if (on_candidate_path(T, k_eff, a.chunks)) finish_from_candidates(a, row, T, k_eff);
    else sample_whole_row(a, row, T, k_eff);
}

}  // namespace

hipError_t launch_sample(const SampleArgs& a, int rows, hipStream_t stream) {
    hipLaunchKernelGGL(sample_chunk_kernel, dim3(rows * a.chunks), dim3(kChunkThreads), 0, stream, a);
    hipLaunchKernelGGL(sample_row_kernel, dim3(rows), dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace pkv
