// Token sampling after the LM head: temperature, top-k, top-p, draw.
//
// Lab page (Inference Engineering), function sample; chapter 5's
// filter-and-sample listing; serving tutorial demos D01/D02. Per row of
// logits, in this order:
//  * temperature T = 0: greedy, the lowest index among tied maxima;
//  * z = logit / T (fp32, correctly rounded), ordered by decreasing z with
//    ties going to the lower index;
//  * top-k (k > 0): keep the first k of that order;
//  * masses p = exp(z - max z), evaluated in fp64 (exp_f64.h; the z of
//    each logit by an fp64 product that rounds as the division would);
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
//    bits (as suffix sums), and lists its tokens in a few bins around its
//    own top-p boundary with a count per bin. One workgroup per row
//    rescales and adds the chunks' sums to find the bin holding the row's
//    boundary, takes that bin's tokens from the chunks' lists (a chunk
//    whose window misses the bin is scanned again, unless its largest z
//    lies below it) and finishes the boundary there (two more key digits,
//    then index digits among tied keys). The draw picks the chunk from
//    per-chunk kept masses and walks that chunk only (prefetched while
//    the boundary is found, on a guess from the bin's masses).
//  * whole-row path (top-k between kSampleMaxK and the vocabulary, rows
//    wider than kSampleHistChunks chunks, or a boundary bin of more than
//    kBucketCap tokens): one 1024-thread workgroup per row finds the k-th
//    largest key and the top-p boundary by radix descents over the row
//    (counts, and fp64 mass sums, per 8-bit digit in LDS); ties at a
//    boundary are resolved in index order with wave ballots.
// The second kernel runs the finishing step: each workgroup takes its row's
// path.
#include "device_common.h"
#include "exp_f64.h"
#include "kernels.h"

namespace pkv {
namespace {

constexpr int kChunkThreads = 256;
constexpr int kPerThread = kSampleChunk / kChunkThreads;
constexpr int kChunkWaves = kChunkThreads / kWave;
constexpr int kChunkKeep = 512;              // keys at or above a chunk's bound kept in LDS
constexpr int kThreads = 1024;               // finishing kernel: one row per workgroup
constexpr int kWaves = kThreads / kWave;
static_assert(kPerThread * kChunkThreads == kSampleChunk, "chunk split");
static_assert(kSampleMaxK <= 4 * kWave, "one wave scans the top-k (4 per lane)");
static_assert(kSampleMaxCand % kThreads == 0, "candidates per thread");
static_assert(kChunkKeep + 2048 / 2 <= kSampleHistBins, "chunk pool: keep list and 2048 u32 digit bins");

// 2^(j/32) for exp_tab, copied into LDS by each kernel that evaluates
// masses (32 threads, before its first barrier). The entries are selected
// from literals, not loaded: a load here would have to wait for every load
// the thread has in flight.
__shared__ double s_exp2[32];
__device__ __forceinline__ void put_exp2_table() {
    const int j = threadIdx.x & 31;
    double t = kExp2Frac[0];
#pragma unroll
    for (int i = 1; i < 32; ++i) t = j == i ? kExp2Frac[i] : t;
    if (threadIdx.x < 32) s_exp2[threadIdx.x] = t;
}
__device__ __forceinline__ double mass_exp(double x) { return exp_nonpos(x, s_exp2); }
// The polynomial's addends held in registers (opaque to the compiler, which
// would otherwise rebuild each of them for every exponential of a loop).
__device__ __forceinline__ ExpCoef held_coef() {
    ExpCoef k = kExpCoef;
    asm volatile("" : "+v"(k.c5), "+v"(k.c4), "+v"(k.c3));
    return k;
}
__device__ __forceinline__ double mass_exp(double x, const ExpCoef& k) { return exp_nonpos(x, s_exp2, k); }

// Wave-wide inclusive scans by DPP moves (row_shr 1, 2, 4, 8 inside each row
// of 16 lanes, then row_bcast 15 into rows 1 and 3 and row_bcast 31 into
// rows 2 and 3), a few cycles a step instead of an LDS permute's latency;
// totals are lane 63's. Lanes reading past their row take the identity.
template <int kCtrl, int kRowMask = 0xF>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v, uint32_t identity) {
    return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(static_cast<int>(identity), static_cast<int>(v), kCtrl,
                                                             kRowMask, 0xF, false));
}
template <int kCtrl, int kRowMask = 0xF>
__device__ __forceinline__ double dpp_f64(double v, double identity) {
    const uint64_t b = static_cast<uint64_t>(__double_as_longlong(v));
    const uint64_t id = static_cast<uint64_t>(__double_as_longlong(identity));
    const uint32_t lo = dpp_u32<kCtrl, kRowMask>(static_cast<uint32_t>(b), static_cast<uint32_t>(id));
    const uint32_t hi = dpp_u32<kCtrl, kRowMask>(static_cast<uint32_t>(b >> 32), static_cast<uint32_t>(id >> 32));
    return __longlong_as_double(static_cast<long long>((static_cast<uint64_t>(hi) << 32) | lo));
}
template <typename C, class Op>
__device__ __forceinline__ C dpp_scan(C v, C identity, Op op) {
    auto mv = [&](auto ctrl_tag, auto mask_tag, C x) -> C {
        constexpr int kC = decltype(ctrl_tag)::value, kM = decltype(mask_tag)::value;
        if constexpr (sizeof(C) == 8) return dpp_f64<kC, kM>(x, identity);
        else return dpp_u32<kC, kM>(x, identity);
    };
    using I = std::integral_constant<int, 0xF>;
    v = op(v, mv(std::integral_constant<int, 0x111>{}, I{}, v));   // row_shr:1
    v = op(v, mv(std::integral_constant<int, 0x112>{}, I{}, v));   // row_shr:2
    v = op(v, mv(std::integral_constant<int, 0x114>{}, I{}, v));   // row_shr:4
    v = op(v, mv(std::integral_constant<int, 0x118>{}, I{}, v));   // row_shr:8
    v = op(v, mv(std::integral_constant<int, 0x142>{}, std::integral_constant<int, 0xA>{}, v));   // row_bcast:15
    v = op(v, mv(std::integral_constant<int, 0x143>{}, std::integral_constant<int, 0xC>{}, v));   // row_bcast:31
    return v;
}
__device__ __forceinline__ double lane63_f64(double v) {
    const long long b = __double_as_longlong(v);
    const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(b), kWave - 1));
    const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(b >> 32), kWave - 1));
    return __longlong_as_double(static_cast<long long>((static_cast<uint64_t>(hi) << 32) | lo));
}
__device__ __forceinline__ double wave_sum_f64(double v) {
    return lane63_f64(dpp_scan(v, 0.0, [](double x, double y) { return x + y; }));
}
__device__ __forceinline__ double wave_max_f64(double v) {
    return lane63_f64(dpp_scan(v, -__builtin_inf(), [](double x, double y) { return fmax(x, y); }));
}
__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t v) {
    const uint32_t t = dpp_scan(v, 0u, [](uint32_t x, uint32_t y) { return x + y; });
    return static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(t), kWave - 1));
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    const uint32_t t = dpp_scan(v, 0u, [](uint32_t x, uint32_t y) { return max(x, y); });
    return static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(t), kWave - 1));
}
template <typename C>
__device__ __forceinline__ C wave_incl_scan(C v, int) {
    return dpp_scan(v, C(0), [](C x, C y) { return x + y; });
}

// Larger float -> larger key (NaN excluded), and back.
__device__ __forceinline__ uint32_t order_key(float x) {
    const uint32_t b = __float_as_uint(x);
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ __forceinline__ float key_value(uint32_t k) {
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// base[i] through a 32-bit byte offset from a wave-uniform base (indices
// within a row stay below 2^26), so that each load needs one address
// register rather than two.
__device__ __forceinline__ float load_at(const float* base, int i) {
    return *reinterpret_cast<const float*>(reinterpret_cast<const char*>(base) + static_cast<uint32_t>(i) * 4u);
}

// x[i] <- x[i] / T rounded to fp32 (T > 0 finite, inv = 1 / T rounded to
// fp64), as the division itself would give it. The fp64 product x * inv is within
// a relative 2^-52 of x / T. A quotient of two fp32 values never equals the
// midpoint between two adjacent normal fp32 values (with x = X 2^a, T = M
// 2^c and the midpoint m = N 2^b, X, M, N odd, N of 25 bits, x = m T would
// need the odd integer N M of 25 or more bits to equal X), and the numerator
// of x / T - m is a nonzero multiple of 2^min(a, b + c), which puts x / T
// more than 2^-49 (relative) away from every such midpoint. So rounding the
// product to fp32 gives the correctly rounded quotient whenever the result
// lies above the smallest normal value; at or below it (the subnormals,
// where exact midpoints do occur), and for NaN, the division is done: only
// in a wave that has such a value (rare), so that the common path does not
// compute the divisions.
template <int N>
__device__ __forceinline__ void div_by_t(float (&x)[N], float T, double inv) {
    float q[N];
    bool slow = false;
#pragma unroll
    for (int i = 0; i < N; ++i) {
        q[i] = static_cast<float>(static_cast<double>(x[i]) * inv);
        slow |= !(fabsf(q[i]) > 0x1p-126f);
    }
    if (__builtin_amdgcn_ballot_w64(slow)) {
#pragma unroll
        for (int i = 0; i < N; ++i)
            if (!(fabsf(q[i]) > 0x1p-126f)) q[i] = x[i] / T;
    }
#pragma unroll
    for (int i = 0; i < N; ++i) x[i] = q[i];
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

// Histogram rows, after the chunk headers: per (row, chunk) the suffix sums
// of every 32nd bin (I[32 g], g < 64, contiguous), then per (row, chunk)
// the list of the chunk's tokens near its own top-p boundary (one region of
// kWinWaveCap per wave), then per (row, chunk) its tally.
constexpr int kGroups = kSampleHistBins / 32;
__device__ __forceinline__ size_t hist_base(const SampleArgs& a) {
    return static_cast<size_t>(a.rows) * a.chunks * (a.region + sizeof(SampleChunkHead));
}
__device__ __forceinline__ double* chunk_coarse(const SampleArgs& a, int row, int s) {
    return reinterpret_cast<double*>(a.ws + hist_base(a)) + (static_cast<size_t>(row) * a.chunks + s) * kGroups;
}
__device__ __forceinline__ uint64_t* chunk_list(const SampleArgs& a, int row, int s) {
    return reinterpret_cast<uint64_t*>(a.ws + hist_base(a) + static_cast<size_t>(a.rows) * a.chunks * kGroups * 8u) +
           (static_cast<size_t>(row) * a.chunks + s) * kSampleListCap;
}
__device__ __forceinline__ SampleChunkTally* chunk_tally(const SampleArgs& a, int row, int s) {
    return reinterpret_cast<SampleChunkTally*>(a.ws + hist_base(a) +
                                               static_cast<size_t>(a.rows) * a.chunks * (kGroups + kSampleListCap) * 8u) +
           static_cast<size_t>(row) * a.chunks + s;
}
constexpr int kWinWaveCap = kSampleListCap / kChunkWaves;   // one chunk-pass wave's share of the list

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
    static_assert(B * kWave == NB && (B & (B - 1)) == 0 && B <= kWave, "bins per lane");
    const int top = NB - 1 - B * lane;
    C local = 0;
#pragma unroll
    for (int i = 0; i < B; ++i) local += bins[top - ((i + lane) & (B - 1))];
    const C incl = wave_incl_scan(local, lane);
    const unsigned long long m = __builtin_amdgcn_ballot_w64(incl >= need);
    if (!m) return -1;
    // inside the first group that reaches `need`: its B bins from the top, one
    // per lane, scanned after the mass of the groups above it
    const int first = __builtin_ctzll(m);
    const int gtop = NB - 1 - B * first;
    const C before = __shfl(incl - local, first, kWave);
    const C v = lane < B ? bins[gtop - lane] : C(0);
    const C run = before + wave_incl_scan(v, lane);
    const unsigned long long hit = __builtin_amdgcn_ballot_w64(lane < B && run >= need);
    if (!hit) return -1;   // rounding left the group's bins just short
    const int i = __builtin_ctzll(hit);
    *above = __shfl(run - v, i, kWave);
    return gtop - i;
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
// rescaling), and the list of its tokens in a window of bins around its own
// top-p boundary b_c (the largest b with I[b] >= top-p x I[0]): the
// kSampleWinBins bins from b_c - 2, as (key, index) composites. The row's boundary bin, found
// by the finishing pass from all chunks, usually lies in every chunk's
// window; a chunk whose window misses it is scanned again there. Keys of 0
// lie past the chunk's end; element i of this thread has index jb + i *
// kChunkThreads.
__device__ __forceinline__ void chunk_masses(const SampleArgs& a, int row, int s, int jb, float top_p,
                                             const uint32_t (&key)[kPerThread], double* s_hm, uint32_t* s_tw) {
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const bool hist = top_p < 1.0f;
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
    // Branch-free over the elements: a slot past the chunk's end (key 0)
    // gets mass 0 (added to bin 0, which changes nothing).
    const ExpCoef kc = held_coef();
    double tot = 0.0;
    if (hist) {
#pragma unroll
        for (int i = 0; i < kPerThread; ++i) {
            const bool real = key[i] != 0u;
            const double m = mass_exp((real ? static_cast<double>(key_value(key[i])) : mcd) - mcd, kc);
            atomicAdd(&s_hm[key[i] >> 21], real ? m : 0.0);
        }
    } else {
#pragma unroll
        for (int i = 0; i < kPerThread; ++i) {
            const bool real = key[i] != 0u;
            const double m = mass_exp((real ? static_cast<double>(key_value(key[i])) : mcd) - mcd, kc);
            tot += real ? m : 0.0;
        }
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
        static_assert(32 % kPer == 0, "group starts fall on a thread's first bin");
        if ((kPer * tid) % 32 == 0) chunk_coarse(a, row, s)[kPer * tid / 32] = l[0] + above;
        if (tid == 0) {
            h->mc = mc;
            h->total = l[0] + above;
        }
        // the window: b_c from the suffix sums (non-increasing in b, so the bins
        // reaching the need are those up to b_c)
        double tot = 0.0;
#pragma unroll
        for (int w = 0; w < kChunkWaves; ++w) tot += s_wt[w];
        const double need = static_cast<double>(top_p) * tot;
        uint32_t lb = 0;   // 1 + the largest bin of this thread reaching the need
#pragma unroll
        for (int i = 0; i < kPer; ++i)
            if (l[i] + above >= need) lb = max(lb, static_cast<uint32_t>(kPer * tid + i + 1));
        lb = wave_max_u32(lb);
        __shared__ uint32_t s_lb[kChunkWaves];
        if (lane == 0) s_lb[wave] = lb;
        __syncthreads();
        lb = s_lb[0];
#pragma unroll
        for (int w = 1; w < kChunkWaves; ++w) lb = max(lb, s_lb[w]);
        const uint32_t bc = lb > 0u ? lb - 1u : 0u;   // I[0] reaches any need below the total
        const uint32_t wlo = bc >= 2u ? bc - 2u : 0u;
        const uint32_t whi = min(wlo + static_cast<uint32_t>(kSampleWinBins - 1), static_cast<uint32_t>(kSampleHistBins - 1));
        // each wave lists its tokens in its share of the list; per-lane counts per
        // window bin in the bytes of `per` (at most kPerThread each)
        static_assert(kPerThread < 256 && kSampleWinBins <= 8, "byte counters");
        uint64_t* list = chunk_list(a, row, s) + wave * kWinWaveCap;
        uint32_t n = 0, up = 0;
        uint64_t per = 0;
#pragma unroll
        for (int i = 0; i < kPerThread; ++i) {
            const uint32_t bn = key[i] >> 21;
            const bool inw = key[i] != 0u && bn >= wlo && bn <= whi;
            up += key[i] != 0u && bn > whi ? 1u : 0u;
            per += inw ? 1ull << (8u * (bn - wlo)) : 0ull;
            const unsigned long long m = __builtin_amdgcn_ballot_w64(inw);
            if (m) {
                const uint32_t slot =
                    n + __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(m >> 32),
                                                   __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(m), 0u));
                if (inw && slot < static_cast<uint32_t>(kWinWaveCap))
                    list[slot] = composite(key[i], static_cast<uint32_t>(jb + i * kChunkThreads));
                n += static_cast<uint32_t>(__builtin_popcountll(m));
            }
        }
        up = wave_sum_u32(up);
        uint32_t nb[kSampleWinBins];
#pragma unroll
        for (int q = 0; q < kSampleWinBins; ++q) nb[q] = wave_sum_u32(static_cast<uint32_t>(per >> (8 * q)) & 255u);
        SampleChunkTally* tl = chunk_tally(a, row, s);
        if (lane == 0) {
            tl->listed[wave] = n > static_cast<uint32_t>(kWinWaveCap) ? 0xFFFFFFFFu : n;
            tl->up[wave] = up;
#pragma unroll
            for (int q = 0; q < kSampleWinBins; ++q) tl->inbin[wave][q] = nb[q];
        }
        if (tid == 0) {
            tl->wlo = wlo;
            tl->whi = whi;
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

// One (row, chunk) item of the chunk kernel: the row's parameters and the
// chunk's bounds; live when the row takes the candidate or the histogram
// path.
struct ChunkItem {
    int row, s, lo, hi, k_eff;
    float T, top_p;
    bool cand, live;
};

// The row's T, k and top-p, requested through vector loads (a lane offset
// of 0 the compiler cannot see through) ahead of the logits: as scalar
// loads their wait also held back the logits' loads.
struct RowParams {
    float T;
    int32_t k;
    float top_p;
};
__device__ __forceinline__ RowParams row_params(const SampleArgs& a, int it) {
    int zero;
    asm volatile("v_mov_b32 %0, 0" : "=v"(zero));
    const int row = it / a.chunks + zero;
    return RowParams{a.temperature[row], a.top_k[row], a.top_p[row]};
}

__device__ __forceinline__ ChunkItem chunk_item(const SampleArgs& a, int it, RowParams p) {
    ChunkItem c{};
    c.live = false;
    if (it >= a.rows * a.chunks) return c;
    const int S = a.chunks;
    c.row = it / S;
    c.s = it - c.row * S;
    c.T = p.T;
    c.top_p = p.top_p;
    if (!(c.T >= 0.0f)) return c;
    c.k_eff = c.T > 0.0f ? kept_by_k(p.k, a.vocab) : 1;
    c.cand = on_candidate_path(c.T, c.k_eff, S);
    if (!c.cand && !on_hist_path(c.T, c.k_eff, a.vocab, S)) return c;
    const int C = (a.vocab + S - 1) / S;
    c.lo = c.s * C;
    c.hi = min(a.vocab, c.lo + C);
    c.live = c.lo < c.hi;
    return c;
}

// Element i of this thread: index lo + i * kChunkThreads + tid of chunk s
// of row `row` (bounds from the item index alone, so these loads need not
// wait for the row's parameters). The loads are unconditional (clamped to
// the chunk's last element, or to the row's last one for a chunk past the
// vocabulary) so that all of them are in flight together.
__device__ __forceinline__ void load_item(const SampleArgs& a, int it, uint32_t (&key)[kPerThread]) {
    const int S = a.chunks;
    const int row = it / S;
    const int C = (a.vocab + S - 1) / S;
    const int lo = (it - row * S) * C;
    const int hi = min(a.vocab, lo + C);
    const float* x = a.logits + static_cast<size_t>(row) * a.ld;
    const int jb = lo + static_cast<int>(threadIdx.x);
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) key[i] = __float_as_uint(load_at(x, min(jb + i * kChunkThreads, hi - 1)));
}

// Candidate items: writes the chunk's min(k, chunk length) best (key,
// index) pairs to its candidate slots, best first (decreasing key, ties by
// lower index). Histogram items: chunk_masses. `key` holds the loaded
// logits and becomes their order keys; past the chunk's end the key is 0,
// which no finite z has (it is a negative NaN's key): such slots land in
// the lowest bin and are never taken.
__device__ __forceinline__ void chunk_item_work(const SampleArgs& a, const ChunkItem& c, uint32_t (&key)[kPerThread]) {
    const int row = c.row, s = c.s, lo = c.lo, hi = c.hi, k_eff = c.k_eff;
    const float T = c.T;
    const bool cand = c.cand;
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const uint32_t want = static_cast<uint32_t>(min(k_eff, hi - lo));
    const int jb = lo + tid;
    if (T > 0.0f) {
        const double inv = 1.0 / static_cast<double>(T);
        float z[kPerThread];
#pragma unroll
        for (int i = 0; i < kPerThread; ++i) z[i] = __uint_as_float(key[i]);
        div_by_t(z, T, inv);
#pragma unroll
        for (int i = 0; i < kPerThread; ++i) key[i] = __float_as_uint(z[i]);
    }
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) key[i] = jb + i * kChunkThreads < hi ? order_key(__uint_as_float(key[i])) : 0u;

    __shared__ uint32_t s_tw[kChunkWaves];
    __shared__ uint64_t s_pool[kSampleHistBins];   // histogram rows: fp64 bins; candidate rows: keep list + digit bins
    __shared__ uint32_t s_tc[kPerThread * kChunkWaves];
    if (!cand) {
        chunk_masses(a, row, s, jb, c.top_p, key, reinterpret_cast<double*>(s_pool), s_tw);
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

    // the keys at or above the bound, as (key, index) composites: each wave
    // counts its keys first and claims all their slots with one atomic
    {
        uint32_t wn = 0;
#pragma unroll
        for (int i = 0; i < kPerThread; ++i) wn += __builtin_popcountll(__builtin_amdgcn_ballot_w64(key[i] >= thr));
        uint32_t base = 0;
        if (lane == 0 && wn) base = atomicAdd(&s_n, wn);
        base = __builtin_amdgcn_readlane(base, 0);
#pragma unroll
        for (int i = 0; i < kPerThread; ++i) {
            const bool keep = key[i] >= thr;
            const unsigned long long km = __builtin_amdgcn_ballot_w64(keep);
            const uint32_t slot = base + __builtin_popcountll(km & below);
            if (keep && slot < kChunkKeep) s_keep[slot] = composite(key[i], static_cast<uint32_t>(jb + i * kChunkThreads));
            base += __builtin_popcountll(km);
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

// One workgroup per (row, chunk) item, blockIdx.x = row * chunks + chunk.
__global__ __launch_bounds__(kChunkThreads) __attribute__((amdgpu_waves_per_eu(4)))
void sample_chunk_kernel(SampleArgs a) {
    const int it = static_cast<int>(blockIdx.x);
    if (it >= a.rows * a.chunks) return;
    const RowParams p = row_params(a, it);
    uint32_t key[kPerThread];
    load_item(a, it, key);   // needs no parameter of the row
    put_exp2_table();        // read after the barrier
    // The barrier keeps the logits' loads ahead of the row's checks below
    // (otherwise the compiler moves the exits first, and the loads wait for
    // T and k).
    __syncthreads();
    const ChunkItem c = chunk_item(a, it, p);
    if (!c.live) return;
    chunk_item_work(a, c, key);
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

// ---- histogram path, passes 2 and 3 ---------------------------------------------------
constexpr int kBucketCap = kSampleBucketCap;   // tokens of the top-p boundary bin held in LDS
constexpr int kPoolWords = 3 * kSampleHistBins / 2 + kBucketCap;   // fp64 bins, u32 counts, the bin's tokens
static_assert(kSampleHistBins == 2 * kThreads, "two merged bins per thread");
static_assert(kSampleHistChunks <= kWave, "one lane per chunk in the draw");
static_assert(kSampleChunk == kWaves * 8 * kWave, "the walk covers a chunk with 8 loads per lane");
static_assert(kSampleHistChunks * kSampleChunk <= (1 << 19), "indices fit the 19 bits of the tie digits");
static_assert(kPoolWords >= kMergeChunks * kSampleMaxK + 2 * kThreads, "the pool holds the candidate finish");

// One digit of the boundary search inside the gathered bin: fp64 masses and
// counts of the tokens matching `prefix` under `pmask`, per NB bins of the
// key bits at `shift`; then the bin, from the top, at which the mass
// reaches `rest`. `above` grows by the mass of the bins above it. When
// rounding leaves the gathered mass just short of `rest`, the boundary is
// the lowest token: the lowest non-empty bin is taken. kZeroed: the caller
// has cleared the bins (before a barrier).
template <int NB, bool kZeroed = false>
__device__ __forceinline__ void bucket_digit(const uint64_t* s_bk, uint32_t n1, int shift, double zmax, double rest,
                                             double* s_bin, uint32_t* s_cnt, int* s_ri, double* s_rd,
                                             uint32_t& prefix, uint32_t& pmask, double& above) {
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    if constexpr (!kZeroed) {
        for (int b = tid; b < NB; b += kThreads) {
            s_bin[b] = 0.0;
            s_cnt[b] = 0u;
        }
        __syncthreads();
    }
    for (uint32_t e = tid; e < n1; e += kThreads) {
        const uint32_t key = comp_key(s_bk[e]);
        if ((key & pmask) == prefix) {
            const uint32_t b = (key >> shift) & (NB - 1);
            atomicAdd(&s_bin[b], mass_exp(static_cast<double>(key_value(key)) - zmax));
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

// ---- histogram rows, pass 2 (the finishing kernel) --------------------------------
// The row's boundary bin is found from the chunks' histograms by one wave,
// which loads first the chunks' headers and group sums.
constexpr int kSumBatch = 16;   // chunk sums loaded together per lane

// The boundary search's first loads: the headers of chunks lane and the
// group sums at group `lane` of chunks 0 .. kSumBatch - 1.
// Unconditional (chunk indices clamped, the extra values ignored), so that
// they are issued together.
struct SearchLoads {
    float mc;
    double total;
    double h[kSumBatch];
};
__device__ __forceinline__ SearchLoads search_loads(const SampleArgs& a, int row, int lane) {
    const int S = a.chunks;
    SearchLoads L;
    const SampleChunkHead* hd = chunk_head(a, row, min(lane, S - 1));
    L.mc = hd->mc;
    L.total = hd->total;
#pragma unroll
    for (int u = 0; u < kSumBatch; ++u) L.h[u] = chunk_coarse(a, row, min(u, S - 1))[lane];
    return L;
}

// v + the sum over chunks c0 .. S - 1, in chunk order, of s_scale[c] *
// *src(c) (nothing where !on; src must give a valid address for every
// chunk either way), kSumBatch loads in flight at a time.
template <class Src>
__device__ __forceinline__ double scaled_sum(int c0, int S, const double* s_scale, bool on, Src&& src, double v) {
    for (; c0 < S; c0 += kSumBatch) {
        double h[kSumBatch];
#pragma unroll
        for (int u = 0; u < kSumBatch; ++u) h[u] = *src(min(c0 + u, S - 1));   // all issued, then summed
#pragma unroll
        for (int u = 0; u < kSumBatch; ++u)
            if (on && c0 + u < S) v += s_scale[c0 + u] * h[u];
    }
    return v;
}

// The row's top-p boundary: the bin, the mass of the bins above it, need =
// top-p x the row's mass, and max z; all scaled to exp(z - max z).
struct RowBoundary {
    uint32_t bin;
    double above, need, zmax;
};

// The bin holding the top-p boundary, by one wave: max z and the chunks'
// scales exp(chunk max - max z) (written to s_scale), need = top-p x the
// scaled total, then the largest b with I[b] >= need, I[b] = the sum over
// chunks of scale x the chunk's suffix mass at b, in two levels (the 64
// group starts 32 g from the contiguous group sums, then the 33 bins from
// the chosen group's start).
__device__ __forceinline__ RowBoundary boundary_bin(const SampleArgs& a, int row, float tp, int lane,
                                                    const SearchLoads& L, double* s_scale) {
    const int S = a.chunks;
    const double mc = lane < S ? static_cast<double>(L.mc) : -INFINITY;
    const double zmax = wave_max_f64(mc);
    const double sc = lane < S ? mass_exp(mc - zmax) : 0.0;
    if (lane < S) s_scale[lane] = sc;
    const double need = static_cast<double>(tp) * wave_sum_f64(lane < S ? sc * L.total : 0.0);
    double g = 0.0;
#pragma unroll
    for (int u = 0; u < kSumBatch; ++u)
        if (u < S) g += s_scale[u] * L.h[u];
    g = scaled_sum(kSumBatch, S, s_scale, true, [&](int c) { return chunk_coarse(a, row, c) + lane; }, g);
    const unsigned long long ok = __builtin_amdgcn_ballot_w64(g >= need);
    const int kA = ok ? 63 - __builtin_clzll(ok) : 0;
    const int b = 32 * kA + lane;   // lanes 0 .. 32: the group's bins and the next group's start
    const double v = scaled_sum(0, S, s_scale, lane <= 32 && b < kSampleHistBins,
                                [&](int c) { return chunk_hist(a, row, c) + min(b, kSampleHistBins - 1); }, 0.0);
    const unsigned long long ok2 = __builtin_amdgcn_ballot_w64(lane < 32 && v >= need);
    const int i = ok2 ? 63 - __builtin_clzll(ok2) : 0;
    RowBoundary rb;
    rb.bin = static_cast<uint32_t>(32 * kA + i);
    rb.above = __shfl(v, i + 1, kWave);
    rb.need = need;
    rb.zmax = zmax;
    return rb;
}

// Rows with top-k off, pass 2: from the chunks' maxima and histograms and,
// with top-p on, their lists and tallies. Returns false, the same in every
// thread, when the boundary bin's tokens do not fit (more than kBucketCap
// over the row, or a scanned chunk holding more than its bound); the caller
// then takes the whole-row path.
constexpr int kListBatch = 8;   // list entries per lane loaded together
static_assert(kListBatch * kWave <= kWinWaveCap, "a batch stays inside a wave's region");
static_assert(kThreads * 8 >= kSampleChunk, "a chunk scan covers the chunk in 8 loads per thread");
__device__ __forceinline__ bool finish_from_histograms(const SampleArgs& a, int row, float T, float tp, uint64_t* pool) {
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const int V = a.vocab;
    const int S = a.chunks;
    const int C = (V + S - 1) / S;
    const Row r{a.logits + static_cast<size_t>(row) * a.ld, V, T};
    const double inv = 1.0 / static_cast<double>(T);
    const float ur = a.u[row];
    double* s_bin = reinterpret_cast<double*>(pool);                          // [kSampleHistBins]
    uint32_t* s_cnt = reinterpret_cast<uint32_t*>(pool + kSampleHistBins);    // [kSampleHistBins]
    uint64_t* s_bk = pool + 3 * kSampleHistBins / 2;                          // [kBucketCap]
    __shared__ double s_scale[kSampleHistChunks];   // exp(chunk max - row max)
    __shared__ double s_kc[kSampleHistChunks];      // kept mass per chunk
    __shared__ double s_acc[kSampleHistChunks];     // the chunk's suffix mass above the boundary bin
    __shared__ double s_from[kSampleHistChunks];    // ... from the boundary bin up
    __shared__ double s_wd[kWaves];
    __shared__ uint32_t s_wu[kWaves];
    __shared__ int s_ri[2];
    __shared__ double s_rd[4];
    __shared__ uint32_t s_n;
    __shared__ uint64_t s_small[kWave];
    __shared__ uint32_t s_wlo[kSampleHistChunks], s_whi[kSampleHistChunks], s_lst[kSampleHistChunks][kChunkWaves];
    __shared__ uint32_t s_inb[kSampleHistChunks][kSampleWinBins];   // the chunk's tokens per window bin
    __shared__ double s_mc[kSampleHistChunks];                       // the chunk's max z
    __shared__ uint32_t s_start[kSampleHistChunks], s_cap[kSampleHistChunks], s_mem[kSampleHistChunks];
    __shared__ uint32_t s_up[kSampleHistChunks];
    __shared__ uint32_t s_tot[4];

    uint32_t pkey = 0;   // kept: key > pkey, or key == pkey and index <= pidx
    int pidx = V;
    uint32_t kept_p = static_cast<uint32_t>(V);
    double zmax;
    int pred = -1;   // the chunk whose logits the draw prefetched into xpre[]
    float xpre[8];
    if (tp < 1.0f) {
        // ---- the boundary bin (wave 0) and the chunks' tallies (wave 1) ------------------
        if (wave == 0) {
            const SearchLoads L = search_loads(a, row, lane);
            put_exp2_table();
            if (lane < S) s_mc[lane] = static_cast<double>(L.mc);
            const RowBoundary rb = boundary_bin(a, row, tp, lane, L, s_scale);
            if (lane < S) {
                const double* hc = chunk_hist(a, row, lane);
                s_acc[lane] = rb.bin + 1u < static_cast<uint32_t>(kSampleHistBins) ? hc[rb.bin + 1] : 0.0;
                s_from[lane] = hc[rb.bin];
                s_kc[lane] = 0.0;
            }
            if (lane == 0) {
                s_tot[3] = rb.bin;
                s_rd[0] = rb.need;
                s_rd[1] = rb.above;
                s_rd[2] = rb.zmax;
            }
        } else if (wave == 1 && lane < S) {
            const SampleChunkTally* tl = chunk_tally(a, row, lane);
            s_wlo[lane] = tl->wlo;
            s_whi[lane] = tl->whi;
            uint32_t up = 0;
            uint32_t nb[kSampleWinBins] = {};
#pragma unroll
            for (int w = 0; w < kChunkWaves; ++w) {
                s_lst[lane][w] = tl->listed[w];
                up += tl->up[w];
#pragma unroll
                for (int q = 0; q < kSampleWinBins; ++q) nb[q] += tl->inbin[w][q];
            }
            s_up[lane] = up;
#pragma unroll
            for (int q = 0; q < kSampleWinBins; ++q) s_inb[lane][q] = nb[q];
        }
        for (int b = tid; b < kSampleHistBins; b += kThreads) {   // the first digit's bins
            s_bin[b] = 0.0;
            s_cnt[b] = 0u;
        }
        __syncthreads();
        const uint32_t b1 = s_tot[3];
        const double need = s_rd[0];
        double above = s_rd[1];
        zmax = s_rd[2];
        // ---- each chunk's range of s_bk: its listed tokens when its window holds b1
        // (and no wave's share overflowed), else room for a scan of the chunk; and the
        // draw's likely chunk (the kept mass of chunk c lies between sc x I_c[b1 + 1],
        // none of the bin kept, and sc x I_c[b1], all of it: take the midpoints) -------
        if (wave == 0) {
            bool cover = lane < S && b1 >= s_wlo[lane] && b1 <= s_whi[lane];
            uint32_t nm = 0, na = 0;   // the chunk's tokens in b1, and in the window above it
            if (lane < S) {
#pragma unroll
                for (int w = 0; w < kChunkWaves; ++w) cover = cover && s_lst[lane][w] != 0xFFFFFFFFu;
#pragma unroll
                for (int q = 0; q < kSampleWinBins; ++q) {
                    const uint32_t bq = s_wlo[lane] + static_cast<uint32_t>(q);
                    if (bq == b1) nm = s_inb[lane][q];
                    if (bq > b1 && bq <= s_whi[lane]) na += s_inb[lane][q];
                }
            }
            // Room for a chunk that is scanned: none when its largest z lies below the
            // bin (nothing of it reaches b1: not scanned either); else its mass in the
            // bin, I_c[b1] - I_c[b1 + 1], over the least mass a token of the bin can
            // have, exp(z_lo - chunk max), with slack for the rounding of the sums,
            // and at most the chunk's length.
            const float zlo = key_value(b1 << 21);
            const bool below = lane < S && !cover && static_cast<double>(zlo) > s_mc[lane];
            uint32_t room = 0;
            if (lane < S && !cover && !below) {
                const double mmin = mass_exp(static_cast<double>(zlo) - s_mc[lane]);
                const double mb = s_from[lane] - s_acc[lane] + 1e-15 * s_from[lane];
                const double bound = mmin > 0.0 ? mb / (mmin * (1.0 - 1e-15)) + 1.0 : static_cast<double>(C);
                room = static_cast<uint32_t>(fmin(bound, static_cast<double>(C)));
            }
            if (below) {   // nothing to scan, nothing listed to take
                cover = true;
                nm = 0u;
            }
            const uint32_t cap = cover ? nm : room;
            const uint32_t incl = wave_incl_scan(cap, lane);
            const unsigned long long scan = __builtin_amdgcn_ballot_w64(lane < S && !cover);
            const double sc = lane < S ? s_scale[lane] : 0.0;
            const double mid = lane < S ? 0.5 * sc * (s_acc[lane] + s_from[lane]) : 0.0;
            const double cm = wave_incl_scan(mid, lane);
            const double tgt = static_cast<double>(ur) * __shfl(cm, kWave - 1, kWave);
            const unsigned long long hit = __builtin_amdgcn_ballot_w64(mid > 0.0 && cm > tgt);
            if (lane < S) {
                s_start[lane] = incl - cap;
                s_cap[lane] = cap;
                s_mem[lane] = 0u;
                s_up[lane] = below ? 0u : (cover ? s_up[lane] + na : 0u);   // else counted by the scan
            }
            const uint32_t n1 = __shfl(incl, kWave - 1, kWave);
            if (lane == 0) {
                s_tot[0] = n1 > static_cast<uint32_t>(kBucketCap) ? 0xFFFFFFFFu : n1;
                s_tot[1] = static_cast<uint32_t>(scan);
                s_tot[2] = static_cast<uint32_t>(scan >> 32);
                s_ri[0] = hit ? __builtin_ctzll(hit) : 0;
            }
        }
        __syncthreads();
        if (s_tot[0] == 0xFFFFFFFFu) return false;
        const uint32_t n1 = s_tot[0];
        unsigned long long scan = (static_cast<unsigned long long>(s_tot[2]) << 32) | s_tot[1];
        {   // prefetch the likely chunk for the draw; it arrives during the digits
            pred = s_ri[0];
            const int lo = pred * C;
            const int hi = min(V, lo + C);
            const int base = lo + wave * (8 * kWave);
#pragma unroll
            for (int u = 0; u < 8; ++u) xpre[u] = load_at(r.x, min(base + u * kWave + lane, hi - 1));
        }
        const unsigned long long below = (1ull << lane) - 1ull;
        // ---- the listed tokens of the covered chunks: the bin's tokens to the chunk's
        // range (one wave per chunk; the counts came with the tallies) ----------------
        for (int c = wave; c < S; c += kWaves) {   // wave-uniform
            if (((scan >> c) & 1ull) || s_cap[c] == 0u) continue;   // scanned below, or nothing to take
            const uint32_t st = s_start[c], cap = s_cap[c];
            uint32_t m = 0;
            // the bin's tokens of a batch of list entries to the chunk's range
            auto take = [&](const uint64_t (&t)[kListBatch], uint32_t e0, uint32_t n) {
#pragma unroll
                for (int u = 0; u < kListBatch; ++u) {
                    const uint32_t e = e0 + u * kWave + lane;
                    const bool mem = e < n && (comp_key(t[u]) >> 21) == b1;
                    const unsigned long long mm = __builtin_amdgcn_ballot_w64(mem);
                    const uint32_t slot = m + static_cast<uint32_t>(__builtin_popcountll(mm & below));
                    if (mem && slot < cap) s_bk[st + slot] = t[u];
                    m += static_cast<uint32_t>(__builtin_popcountll(mm));
                }
            };
            // the four waves' lists in pairs, the first batch of both loaded together
            // (inside the regions whatever their lengths), then any further batches
            for (int w = 0; w < kChunkWaves; w += 2) {
                const uint64_t* l0 = chunk_list(a, row, c) + w * kWinWaveCap;
                const uint64_t* l1 = l0 + kWinWaveCap;
                const uint32_t n0 = min(s_lst[c][w], static_cast<uint32_t>(kWinWaveCap));   // listed in full (covered)
                const uint32_t n1w = min(s_lst[c][w + 1], static_cast<uint32_t>(kWinWaveCap));
                uint64_t t0[kListBatch], t1[kListBatch];
#pragma unroll
                for (int u = 0; u < kListBatch; ++u) {
                    t0[u] = l0[u * kWave + lane];
                    t1[u] = l1[u * kWave + lane];
                }
                take(t0, 0u, n0);
                take(t1, 0u, n1w);
                for (int h = 0; h < 2; ++h) {
                    const uint64_t* l = h ? l1 : l0;
                    const uint32_t n = h ? n1w : n0;
                    for (uint32_t e0 = kListBatch * kWave; e0 < n; e0 += kListBatch * kWave) {
                        uint64_t t[kListBatch];
#pragma unroll
                        for (int u = 0; u < kListBatch; ++u) t[u] = l[e0 + u * kWave + lane];
                        take(t, e0, n);
                    }
                }
            }
            if (lane == 0) s_mem[c] = m;
        }
        // ---- the chunks whose window misses b1: scanned by the whole workgroup, each
        // into its room ----------------------------------------------------------------
        while (scan) {   // workgroup-uniform
            const int c = __builtin_ctzll(scan);
            scan &= scan - 1ull;
            const int lo = c * C;
            const int hi = min(V, lo + C);
            const uint32_t st = s_start[c], cap = s_cap[c];
            uint32_t up = 0;
            float zs[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) zs[u] = load_at(r.x, min(lo + u * kThreads + tid, hi - 1));
            div_by_t(zs, T, inv);
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int j = lo + u * kThreads + tid;
                const bool in = j < hi;
                const uint32_t key = order_key(zs[u]);
                const uint32_t bn = key >> 21;
                const bool mem = in && bn == b1;
                up += in && bn > b1 ? 1u : 0u;
                const unsigned long long mm = __builtin_amdgcn_ballot_w64(mem);
                if (mm) {
                    uint32_t base = 0;
                    if (lane == 0) base = atomicAdd(&s_mem[c], static_cast<uint32_t>(__builtin_popcountll(mm)));
                    base = __shfl(base, 0, kWave);
                    const uint32_t slot = base + static_cast<uint32_t>(__builtin_popcountll(mm & below));
                    if (mem && slot < cap) s_bk[st + slot] = composite(key, static_cast<uint32_t>(j));
                }
            }
            up = wave_sum_u32(up);
            if (lane == 0) atomicAdd(&s_up[c], up);
        }
        __syncthreads();
        bool over = false;   // a scanned chunk with more of the bin's tokens than its room (rounding)
        for (int c = 0; c < S; ++c) over = over || s_mem[c] > s_cap[c];
        if (over) return false;
        // the rest of each range: a composite of another bin, which no digit takes
        const uint64_t other = composite(((b1 + 1u) & (kSampleHistBins - 1u)) << 21, 0u);
        for (int c = wave; c < S; c += kWaves)
            for (uint32_t e = s_mem[c] + lane; e < s_cap[c]; e += kWave) s_bk[s_start[c] + e] = other;
        uint32_t n_above = 0;
        for (int c = 0; c < S; ++c) n_above += s_up[c];
        __syncthreads();

        // ---- the boundary key: more digits over the gathered tokens ----------------
        uint32_t prefix = b1 << 21, pmask = 0xFFE00000u;
        bucket_digit<2048, true>(s_bk, n1, 10, zmax, need - above, s_bin, s_cnt, s_ri, s_rd, prefix, pmask, above);
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
                const double m = real ? mass_exp(static_cast<double>(key_value(comp_key(srt))) - zmax) : 0.0;
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
            const double pb = mass_exp(static_cast<double>(key_value(pkey)) - zmax);
            const double t = (need - above) / pb;
            const uint32_t keep = t <= 1.0 ? 1u : static_cast<uint32_t>(fmin(ceil(t), static_cast<double>(ties)));
            if (keep < ties) {
                uint32_t ip = 0, imask = 0, rem = keep;
                tie_digit<1024>(s_bk, n1, pkey, 9, s_cnt, s_ri, ip, imask, rem);
                tie_digit<512>(s_bk, n1, pkey, 0, s_cnt, s_ri, ip, imask, rem);
                pidx = static_cast<int>(ip);
            }
        }

        // ---- kept mass per chunk: the bins above b1, plus the bin's tokens kept --------
        uint32_t nk = 0;
        for (int c = wave; c < S; c += kWaves) {   // wave-uniform
            const uint32_t n = s_mem[c], st = s_start[c];
            double m = 0.0;
            for (uint32_t e = lane; e < n; e += kWave) {
                const uint64_t cc = s_bk[st + e];
                const uint32_t key = comp_key(cc);
                const int j = comp_index(cc);
                if (key > pkey || (key == pkey && j <= pidx)) {
                    m += mass_exp(static_cast<double>(key_value(key)) - zmax);
                    ++nk;
                }
            }
            m = wave_sum_f64(m);
            if (lane == 0) s_kc[c] = s_scale[c] * s_acc[c] + m;
        }
        nk = wave_sum_u32(nk);
        if (lane == 0) s_wu[wave] = nk;
        __syncthreads();
        kept_p = n_above;
        for (int w = 0; w < kWaves; ++w) kept_p += s_wu[w];
    } else {
        // top-p off: every token is kept; the chunks' totals, rescaled
        if (wave == 0) {
            put_exp2_table();
            const double mc = lane < S ? static_cast<double>(chunk_head(a, row, lane)->mc) : -INFINITY;
            const double ct = lane < S ? chunk_head(a, row, lane)->total : 0.0;
            const double zm = wave_max_f64(mc);
            if (lane < S) s_kc[lane] = mass_exp(mc - zm) * ct;
            if (lane == 0) s_rd[0] = zm;
        }
        __syncthreads();
        zmax = s_rd[0];
        __syncthreads();   // s_rd is reused below
    }

    // ---- draw: the chunk, then the token, in vocabulary order ----------------------
    if (wave == 0) {
        const double kc = lane < S ? s_kc[lane] : 0.0;
        const double incl = wave_incl_scan(kc, lane);
        const double target = static_cast<double>(ur) * __shfl(incl, kWave - 1, kWave);
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
    float xv[8];
    if (s_ri[0] == pred) {   // workgroup-uniform
#pragma unroll
        for (int u = 0; u < 8; ++u) xv[u] = xpre[u];
    } else {
#pragma unroll
        for (int u = 0; u < 8; ++u) xv[u] = load_at(r.x, min(base + u * kWave + lane, hi - 1));
    }
    double mm[8];
    uint32_t kbits = 0;
    double wsum = 0.0;
    div_by_t(xv, T, inv);
#pragma unroll
    for (int u = 0; u < 8; ++u) {
        const int j = base + u * kWave + lane;
        const float zj = xv[u];
        const uint32_t key = order_key(zj);
        const bool kp = j < hi && (key > pkey || (key == pkey && j <= pidx));
        mm[u] = kp ? mass_exp(static_cast<double>(zj) - zmax) : 0.0;
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
    // the wave holding the target (every wave finds it): a scan over the waves' sums
    const bool wu = lane < kWaves && s_wu[lane] != 0u;
    const double wd = wu ? s_wd[lane] : 0.0;
    const double cw = s_rd[1] + wave_incl_scan(wd, lane);
    const unsigned long long hitw = __builtin_amdgcn_ballot_w64(wu && cw > target);
    const unsigned long long anyw = __builtin_amdgcn_ballot_w64(wu);
    // rounding may put the target at the chunk's total: its last wave with kept tokens
    const int wh = hitw ? __builtin_ctzll(hitw) : (anyw ? 63 - __builtin_clzll(anyw) : 0);
    const double pre = __shfl(cw - wd, wh, kWave);
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
__global__ __launch_bounds__(kThreads) void sample_row_kernel(SampleArgs a) {
    __shared__ uint64_t s_pool[kPoolWords];
    const int row = blockIdx.x;
    const float T = a.temperature[row];
    const int32_t tk = a.top_k[row];   // loaded together with T and top-p
    const float tp = a.top_p[row];
    if (!(T >= 0.0f)) {   // negative or NaN temperature: no token
        if (threadIdx.x == 0) write_result(a, row, -1, 0, 0);
        return;
    }
    const int k_eff = T > 0.0f ? kept_by_k(tk, a.vocab) : 1;
    if (on_hist_path(T, k_eff, a.vocab, a.chunks) && !on_candidate_path(T, k_eff, a.chunks)) {
        if (!finish_from_histograms(a, row, T, tp, s_pool)) sample_whole_row(a, row, T, k_eff);
        return;
    }
    if (on_candidate_path(T, k_eff, a.chunks)) finish_from_candidates(a, row, T, k_eff, s_pool);
    else sample_whole_row(a, row, T, k_eff);
}

}  // namespace

hipError_t launch_sample(const SampleArgs& a, int rows, hipStream_t stream) {
    const int items = rows * a.chunks;
    hipLaunchKernelGGL(sample_chunk_kernel, dim3(items), dim3(kChunkThreads), 0, stream, a);
    hipLaunchKernelGGL(sample_row_kernel, dim3(rows), dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace pkv
