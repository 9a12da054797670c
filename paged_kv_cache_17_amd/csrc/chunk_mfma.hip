// Chunk attention on the matrix cores: bf16 K/V/q, head_dim 128,
// block_size 16, fp32 accumulation.
//
// A chunk of C queries of one sequence attends causally over its cache
// (lab page, function forward on a prompt chunk at offset start: key j is
// allowed for the query at position start + i iff j <= start + i; chapter 5
// section 4.1: tile K and V, keep a running max / sum / output per query so
// the L x L score matrix is never stored). With several queries per
// sequence the scores are a real dense contraction, so both products run
// on MFMA (v_mfma_f32_32x32x16_bf16, lane layouts: A[l%32][8(l/32)+e],
// B[8(l/32)+e][l%32], C[8(r/4)+4(l/32)+r%4][l%32]).
//
// Work: one workgroup of 4 waves per (query tile, kv head, sequence). Its
// 128 rows are (query head of the group, query) pairs, 32 per wave, so all
// G heads sharing the kv head reuse each staged K/V tile (chapter 5 section
// 3.1). Query tiles are dispatched longest-first.
//
// Per 64-key tile (4 cache blocks gathered through the table):
//  * each wave copies one cache block of K and of V straight from global
//    memory into LDS (global_load_lds, 16 bytes per lane, no registers);
//    the copy of tile kt + 1 runs while tile kt is computed, into the other
//    of two buffers. LDS rows are 256 bytes, unpadded; the 16-byte granule
//    c of row r is stored at position c ^ sw(r), which makes both read
//    patterns below free of bank conflicts;
//  * S^T = K Q^T: A = K rows, B = the wave's queries (kept in registers).
//    LDS row n of a 32-key subtile holds key pi(n) = n with bits 2 and 3
//    swapped; then the accumulator registers of S^T already hold, for each
//    16-key step, the 8 consecutive keys the next product needs in its B
//    operand. All 16 K operand reads are issued at once and each pair of
//    products waits only for its own two (LDS reads complete in order, the
//    global-to-LDS copies count in vmcnt, not lgkmcnt, and the tile loop
//    issues no scalar memory load, whose out-of-order return would share
//    lgkmcnt: checked in the generated code for G = 1, 2, 4, 8);
//  * each lane owns whole query rows (one column of S^T), so the online
//    softmax is lane-local plus one exchange with the other half-wave; the
//    reference max moves only when a score exceeds it by 2^8 (exact, rare
//    rescaling of the accumulators). Only tiles that reach past a row's
//    position evaluate the causal mask;
//  * O^T += V^T P^T: A = V^T read from the row-major V tile with the
//    transposing LDS load ds_read_b64_tr_b16 (in each 16-lane group, lane j
//    element e comes from lane 4e + j/4, element j%4), B = P^T packed to
//    bf16 from registers.
// Keys past the last one a tile needs are loaded as copies of that key
// (finite cache data) and get weight 0.
//
// Chunk step with the append fused in (a.k_new set): each workgroup first
// writes its own query tile's tokens (K and V rows of its kv head) from the
// new rows into their pool slots, and every tile reads the chunk's own keys
// from the new rows rather than from the pool (blocks past the cached keys
// whole, the block where the chunk starts split by row). No workgroup then
// reads a slot that another writes, and the pool ends as after a separate
// append.
#include <type_traits>

#include "device_common.h"
#include "kernels.h"

namespace pkv {
namespace {

constexpr int kD = 128;
constexpr int kBS = 16;
constexpr int kKeys = 64;                 // keys per staged tile
constexpr int kRows = 128;                // (head, query) rows per workgroup
constexpr int kThreads = 256;
constexpr int kRowBytes = kD * 2;         // one K or V row in LDS (unpadded)
constexpr float kLazy = 8.0f;
constexpr int kXcds = 8;                  // dispatch round-robin width
constexpr int kTblCache = 2048;           // table entries held in LDS (32768 keys)

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) short i16x4;
typedef __attribute__((ext_vector_type(8))) short i16x8;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) char lds_char;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// Where one wave copies a tile's cache block from: K and V base of the
// block (this kv head) and the largest row it may read.
struct TileSrc {
    const char* kb;
    const char* vb;
    int cap;
    // chunk step with the append fused in: rows 0 .. fr - 1 of the block are
    // cached keys (read from the pool at kb / vb), rows fr .. are the chunk's
    // own keys, read from its new rows at kn / vn (row fr there, n_kv rows
    // apart); fr = 16: the whole block is cached.
    int fr;
    const char* kn;
    const char* vn;
};

// Transposing LDS read, issued as inline assembly so the compiler does not
// order it after the asynchronous global-to-LDS copies in flight (it cannot
// prove they touch other buffers). The compiler therefore does not track its
// completion either: callers wait with lds_wait_all() before using the data.
template <int OFF>
__device__ __forceinline__ i16x4 lds_read_tr16(uint32_t addr) {
    i16x4 r;
    asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF));
    return r;
}

// Waits for every outstanding LDS read of this wave; the eight values pass
// through the statement, so their uses cannot be scheduled before the wait.
__device__ __forceinline__ void lds_wait_all(i16x4& a, i16x4& b, i16x4& c, i16x4& d,
                                             i16x4& e, i16x4& f, i16x4& g, i16x4& h) {
    asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(a), "+v"(b), "+v"(c), "+v"(d), "+v"(e), "+v"(f), "+v"(g), "+v"(h));
}
__device__ __forceinline__ void lds_pin(i16x4& a, i16x4& b, i16x4& c, i16x4& d,
                                        i16x4& e, i16x4& f, i16x4& g, i16x4& h) {
    asm volatile("" : "+v"(a), "+v"(b), "+v"(c), "+v"(d), "+v"(e), "+v"(f), "+v"(g), "+v"(h));
}

// K operand reads of 16-dim step T for both 32-key subtiles: LDS byte
// offsets koff[T] (base included) + BOFF and + BOFF + 32 rows. Inline
// assembly like lds_read_tr16, so that kwait can wait for them one step at
// a time (the compiler waits for every LDS read at once while copies are in
// flight).
template <int BOFF, int T>
__device__ __forceinline__ void kread(u32x4 (&kop)[2][8], const int (&koff)[8]) {
    asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(kop[0][T]) : "v"(koff[T]), "i"(BOFF));
    asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(kop[1][T]) : "v"(koff[T]), "i"(BOFF + 32 * kRowBytes));
}
// Waits until at most N of this wave's LDS reads are outstanding; the two
// operands pass through the statement so their products stay after it.
template <int N>
__device__ __forceinline__ void kwait(u32x4& a, u32x4& b) {
    asm volatile("s_waitcnt lgkmcnt(%2)" : "+v"(a), "+v"(b) : "i"(N));
}

// Maximum of a value over lanes l and l ^ 32.
__device__ __forceinline__ float max_halves(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_halves(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Granule swizzle of LDS row r (granule = 16 bytes = 8 elements). Bits of
// the result: r2, r0, r1, r0^r1^r3. Reads of 8 or 16 consecutive rows at one
// granule, and of 4 consecutive rows at 2 or 4 adjacent granules, then hit
// distinct banks whether a read phase covers 128 or 256 bytes.
__device__ __forceinline__ int swz(int r) {
    const int r0 = r & 1, r1 = (r >> 1) & 1, r2 = (r >> 2) & 1, r3 = (r >> 3) & 1;
    return r2 | (r0 << 1) | (r1 << 2) | ((r0 ^ r1 ^ r3) << 3);
}

// Offset (within a 32-key subtile, before adding 8h) of the key held by
// accumulator register r of S^T.
__device__ __forceinline__ constexpr int key_of_reg(int r) {
    return 16 * ((r >> 2) >> 1) + 4 * ((r >> 2) & 1) + (r & 3);
}

template <int G, bool FUSED>
__global__ __launch_bounds__(kThreads, 2) void chunk_mfma_kernel(AttnArgs a, uint16_t* __restrict__ out,
                                                                 float* __restrict__ lse) {
    constexpr int QT = kRows / G;                 // queries per workgroup
    // K buffers 0 and 1, then V buffers 0 and 1, at fixed offsets so that
    // every operand read addresses its buffer by an immediate.
    __shared__ __align__(16) uint16_t s_buf[4 * kKeys * kD];
    uint16_t* const s_k0 = s_buf;
    uint16_t* const s_k1 = s_buf + kKeys * kD;
    uint16_t* const s_v0 = s_buf + 2 * kKeys * kD;
    uint16_t* const s_v1 = s_buf + 3 * kKeys * kD;
    const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_char*)s_buf));
    __shared__ int s_bad;
    __shared__ int s_tbl[kTblCache];

    const int n_kv = a.n_kv;
    // Workgroup id -> (sequence, kv head, query tile). The dispatcher deals
    // consecutive ids round-robin to the 8 XCDs; pair p = s * n_kv + g is
    // given to XCD p % 8 and its query tiles get consecutive slots there
    // (longest first), so the tiles reading the same K/V run together and
    // share that XCD's L2.
    const int n_pairs = a.num_seqs * n_kv;
    const int nq_max = (a.max_q_len + QT - 1) / QT;   // query tiles per pair (upper bound)
    const int xcd = blockIdx.x % kXcds;
    const int k_on_xcd = blockIdx.x / kXcds;
    const int pair = (k_on_xcd / nq_max) * kXcds + xcd;
    if (pair >= n_pairs) return;
    const int g = pair % n_kv;
    const int s = pair / n_kv;
    const int tile_rev = k_on_xcd % nq_max;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n = lane & 31;                      // column of S^T / O^T = this lane's row
    const int h = lane >> 5;                      // half-wave

    const int qs = a.q_start[s];
    const int C = a.q_start[s + 1] - qs;
    const int ntiles_q = (C + QT - 1) / QT;
    const int qtile = ntiles_q - 1 - tile_rev;    // longest tiles first
    if (qtile < 0) return;
    const int q0 = qtile * QT;
    const int L = a.seq_lens[s];
    const int P = L - C;                          // cached keys before the chunk

    const int row = wave * 32 + n;                // (head, query) row of this lane
    const int head_l = row / QT;
    const int qi = q0 + row % QT;
    const bool active = qi < C;
    const int pos = P + qi;                       // absolute position: keys 0..pos
    const size_t orow = (static_cast<size_t>(qs) + qi) * a.n_q + g * G + head_l;

    const bool ok = C >= 1 && seq_len_ok(L, C, a.max_seq_len, a.table_stride * kBS);
    const int q_last = min(q0 + QT, C) - 1;
    const int kmax = P + q_last;                  // largest key any row of this tile sees
    const int nblk = kmax / kBS + 1;
    const int32_t* trow = a.table + static_cast<size_t>(s) * a.table_stride;
    // The lane's query row, requested before the table is staged so that the
    // two round trips overlap. Rows past the chunk read its last row (the
    // loads are unconditional, hence issued together) and are zeroed below.
    u32x4 qraw[8];
    {
        const size_t crow = (static_cast<size_t>(qs) + (active ? qi : max(C - 1, 0))) * a.n_q + g * G + head_l;
        const u32x4* qp = reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(a.q) + crow * kD + 8 * h);
        if (C >= 1) {
#pragma unroll
            for (int t = 0; t < 8; ++t) qraw[t] = qp[2 * t];
        }
    }
    if (tid == 0) s_bad = 0;
    __syncthreads();
    if (ok && nblk <= kTblCache)
        for (int b = tid; b < nblk; b += kThreads) {
            const int id = trow[b];
            if (id < 0 || id >= a.num_blocks) s_bad = 1;
            s_tbl[b] = id;
        }
    __syncthreads();
    const size_t blk_bytes = static_cast<size_t>(n_kv) * kBS * kRowBytes;
    const size_t head_bytes = static_cast<size_t>(g) * kBS * kRowBytes;
    // The append of this workgroup's own query tile (chunk step with the
    // append fused in): tokens P + q0 .. P + q_last of kv head g go from the
    // new rows to their pool slots (each token whose table entry lies in the
    // pool, as the separate append writes). The attention reads the chunk's
    // keys from the new rows, so no workgroup reads a slot that another
    // writes. (Issued with the first tile's copies, which measured faster
    // than at the end of the workgroup.)
    auto append_tile = [&]() {
        if constexpr (FUSED) {
            if (!ok || nblk > kTblCache) return;
            const int items = (q_last - q0 + 1) * 2 * (kRowBytes / 16);   // 16-byte granules of K and V rows
            const char* kn = static_cast<const char*>(a.k_new);
            const char* vn = static_cast<const char*>(a.v_new);
            char* kw = static_cast<char*>(a.k_app);
            char* vw = static_cast<char*>(a.v_app);
            for (int b0 = tid; b0 < items; b0 += 4 * kThreads) {
                // four granules per thread, loads first (past the end: the
                // last granule again, the same bytes stored twice)
                u32x4 val[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int it = min(b0 + j * kThreads, items - 1);
                    const int tok = it >> 5, isv = (it >> 4) & 1, gr = it & 15;
                    const char* src = (isv ? vn : kn) +
                                      (static_cast<size_t>(qs + q0 + tok) * n_kv + g) * kRowBytes + gr * 16;
                    val[j] = *reinterpret_cast<const u32x4*>(src);
                }
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int it = min(b0 + j * kThreads, items - 1);
                    const int tok = it >> 5, isv = (it >> 4) & 1, gr = it & 15;
                    const int p = P + q0 + tok;
                    const int id = s_tbl[p / kBS];
                    if (id >= 0 && id < a.num_blocks)
                        *reinterpret_cast<u32x4*>((isv ? vw : kw) + static_cast<size_t>(id) * blk_bytes + head_bytes +
                                                  (p % kBS) * kRowBytes + gr * 16) = val[j];
                }
            }
        }
    };
    if (!ok || nblk > kTblCache || s_bad) {
        append_tile();
        if (active) {
            for (int e = h; e < kD; e += 2) Elem<uint16_t>::store(out + orow * kD + e, NAN);
            if (lse && h == 0) lse[orow] = NAN;
        }
        return;
    }

    // This lane's query in the B-operand layout: dims 16t + 8h + e, t = 0..7.
    // The kernel needs a scale factor >= 0 (it takes the maximum of the raw
    // scores and masks with -inf before scaling): a negative scale is
    // applied as a query with flipped sign bits (exact) times |scale|, and
    // scale 0 as a zero query times 1 (every allowed key then weighs the same).
    const float sl2_in = a.scale_log2;
    const uint32_t q_and = sl2_in == 0.0f ? 0u : 0xFFFFFFFFu;
    const uint32_t q_xor = sl2_in < 0.0f ? 0x80008000u : 0u;
    u32x4 qv[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) qv[t] = active ? (qraw[t] & q_and) ^ q_xor : u32x4{0, 0, 0, 0};

    // Copy of one tile: wave w fetches cache block 4kt + w (keys 16w..16w+15
    // of the tile) into LDS rows 16w..16w+15, four rows per instruction.
    // Lane l writes granule l%16 of row 16w + 4i + l/16.
    const char* kc = static_cast<const char*>(a.k_cache);
    const char* vc = static_cast<const char*>(a.v_cache);
    const int lr = lane >> 4;
    const int lc = lane & 15;
    const int last_blk = kmax / kBS;
    // Source of the copies for tile kt: per-wave block base (K, V) and the
    // row bound. Rows past key kmax are replaced by a row <= kmax of block
    // min(bi, last_blk), whose table entry tbl_of(kt) reads (a tile ahead of
    // its use, so the LDS round trip is off the tile's path).
    auto tbl_of = [&](int kt) { return s_tbl[min(4 * kt + wave, last_blk)]; };
    const size_t new_stride = static_cast<size_t>(n_kv) * kRowBytes;   // between new rows of one kv head
    auto tile_src = [&](int kt, int idv) {
        const int bi = 4 * kt + wave;
        const int cap = bi > last_blk ? (kmax & (kBS - 1)) : min(kmax - kBS * bi, kBS - 1);
        const int id = __builtin_amdgcn_readfirstlane(idv);
        const size_t off = static_cast<size_t>(id) * blk_bytes + head_bytes;
        TileSrc src{kc + off, vc + off, cap, kBS, nullptr, nullptr};
        if constexpr (FUSED) {
            const int b0 = kBS * min(bi, last_blk);                       // first key of the block read
            src.fr = min(max(P - b0, 0), kBS);
            if (src.fr < kBS) {   // new row of key b0 + fr (>= P)
                const size_t noff = (static_cast<size_t>(qs) + (b0 + src.fr - P)) * new_stride +
                                    static_cast<size_t>(g) * kRowBytes;
                src.kn = static_cast<const char*>(a.k_new) + noff;
                src.vn = static_cast<const char*>(a.v_new) + noff;
            }
        }
        return src;
    };
    auto issue_k = [&](const TileSrc& src, uint16_t* sk) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int gran = lc ^ swz(4 * i + lr);                 // logical granule of this lane's slot
            const int rk = min(lr | ((i & 1) << 3) | ((i >> 1) << 2), src.cap);  // key pi(4i + lr)
            __builtin_amdgcn_global_load_lds(src.kb + static_cast<uint32_t>(rk * kRowBytes + gran * 16),
                                             (lds_void*)(sk + (16 * wave + 4 * i) * kD), 16, 0, 0);
        }
    };
    auto issue_v = [&](const TileSrc& src, uint16_t* sv) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int gran = lc ^ swz(4 * i + lr);
            const int rv = min(4 * i + lr, src.cap);
            __builtin_amdgcn_global_load_lds(src.vb + static_cast<uint32_t>(rv * kRowBytes + gran * 16),
                                             (lds_void*)(sv + (16 * wave + 4 * i) * kD), 16, 0, 0);
        }
    };
    // Fused append: a block holding some of the chunk's own keys. Rows fr ..
    // come from the new rows (n_kv rows apart there), rows below fr from the
    // pool; fr = 0 (the whole block new) keeps one source for the wave, and
    // only the block where the chunk starts splits lanes between the two.
    auto issue_fresh = [&](const TileSrc& src, uint16_t* sk, uint16_t* sv) {
        const int ns = static_cast<int>(new_stride);
        if (src.fr == 0) {        // the whole block new: one source, as the cached blocks
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int gran = lc ^ swz(4 * i + lr);
                const int rk = min(lr | ((i & 1) << 3) | ((i >> 1) << 2), src.cap);
                __builtin_amdgcn_global_load_lds(src.kn + static_cast<uint32_t>(__mul24(rk, ns) + gran * 16),
                                                 (lds_void*)(sk + (16 * wave + 4 * i) * kD), 16, 0, 0);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int gran = lc ^ swz(4 * i + lr);
                const int rv = min(4 * i + lr, src.cap);
                __builtin_amdgcn_global_load_lds(src.vn + static_cast<uint32_t>(__mul24(rv, ns) + gran * 16),
                                                 (lds_void*)(sv + (16 * wave + 4 * i) * kD), 16, 0, 0);
            }
            asm volatile("; new block");
        } else {                  // the block where the chunk starts: rows below fr cached
            auto row = [&](const char* pool, const char* fresh, int r, int gran, uint16_t* dst) {
                const uint32_t po = static_cast<uint32_t>(r * kRowBytes + gran * 16);
                const uint32_t no = static_cast<uint32_t>((r - src.fr) * ns + gran * 16);
                __builtin_amdgcn_global_load_lds(r < src.fr ? pool + po : fresh + no, (lds_void*)dst, 16, 0, 0);
            };
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int gran = lc ^ swz(4 * i + lr);
                const int rk = min(lr | ((i & 1) << 3) | ((i >> 1) << 2), src.cap);
                row(src.kb, src.kn, rk, gran, sk + (16 * wave + 4 * i) * kD);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int gran = lc ^ swz(4 * i + lr);
                const int rv = min(4 * i + lr, src.cap);
                row(src.vb, src.vn, rv, gran, sv + (16 * wave + 4 * i) * kD);
            }
            asm volatile("; block split between cached and new keys");
        }
    };
    // The copies of one tile into (k, v). (The empty statements, each
    // different, keep the compiler from merging the two sides into one with
    // per-lane addresses.)
    auto issue = [&](const TileSrc& src, uint16_t* sk, uint16_t* sv) {
        if (!FUSED || src.fr >= kBS) {
            issue_k(src, sk);
            issue_v(src, sv);
            if constexpr (FUSED) asm volatile("; cached block");
        } else {
            issue_fresh(src, sk, sv);
            asm volatile("; block with new keys");
        }
    };

    // K read addresses (LDS bytes, K buffer 0, first subtile): row n,
    // logical granule 2t + h.
    int koff[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) koff[t] = lds0 + n * kRowBytes + (((2 * t + h) ^ swz(n)) * 16);
    // V^T read addresses (LDS bytes from the start of s_buf, within a 16-key step): lane (group gq = lane/16,
    // j = lane%16) reads row 8(gq/2) + 4a + j/4, elements 4(j%4)..+3 of the
    // 16 dims 32dt + 16(gq%2)...
    int voff[4][2];
    {
        const int gq = lane >> 4, j = lane & 15;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
            for (int aa = 0; aa < 2; ++aa) {
                const int r = 8 * (gq >> 1) + 4 * aa + (j >> 2);
                const int gran = 4 * dt + 2 * (gq & 1) + ((j >> 1) & 1);
                voff[dt][aa] = lds0 + r * kRowBytes + ((gran ^ swz(r)) * 16) + (j & 1) * 8;
            }
    }

    f32x16 o[4];                                  // O^T tiles: dims 32dt + C-layout rows
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) o[dt] = f32x16{};
    float mref = -INFINITY, mref_safe = 0.0f, lsum = 0.0f;
    const float sl2 = sl2_in == 0.0f ? 1.0f : fabsf(sl2_in);
    const int ntiles = kmax / kKeys + 1;
    const int pmin = P + q0;                      // smallest position in the tile
    const int kt_diag = (pmin + 1) / kKeys;       // tiles before this one need no mask
    const bf16x2 ones = {static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f)};

    issue(tile_src(0, tbl_of(0)), s_k0, s_v0);
    append_tile();                // its loads wait behind the first tile's copies, not before them
    int nid = tbl_of(1);          // table entry of the tile after the current one
    __syncthreads();
    // One tile: compute from buffers BUF while the next tile is copied into
    // (nk, nv), the other buffers. Called with fixed buffers on even and odd
    // tiles so every LDS address is a per-lane register plus an immediate.
    auto tile = [&](int kt, auto buf, uint16_t* nk, uint16_t* nv) {
        constexpr int BUF = decltype(buf)::value;
        // copies of the next tile: in flight during the whole tile
        if (kt + 1 < ntiles) issue(tile_src(kt + 1, nid), nk, nv);
        nid = tbl_of(kt + 2);

        // S^T for the two 32-key subtiles: all K operands are requested at
        // once (the LDS latency is paid once), and each 16-dim step's pair of
        // products starts as soon as its two operands have arrived.
        constexpr int KB = BUF * kKeys * kRowBytes;
        u32x4 kop[2][8];
        kread<KB, 0>(kop, koff);
        kread<KB, 1>(kop, koff);
        kread<KB, 2>(kop, koff);
        kread<KB, 3>(kop, koff);
        kread<KB, 4>(kop, koff);
        kread<KB, 5>(kop, koff);
        kread<KB, 6>(kop, koff);
        kread<KB, 7>(kop, koff);
        f32x16 sacc[2] = {f32x16{}, f32x16{}};
        auto spair = [&](auto tc) {
            constexpr int T = decltype(tc)::value;
            kwait<14 - 2 * T>(kop[0][T], kop[1][T]);
#pragma unroll
            for (int u = 0; u < 2; ++u)
                sacc[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kop[u][T]), as_bf16x8(qv[T]), sacc[u], 0, 0, 0);
            // keeps each wait next to its own pair of products (the
            // scheduler would otherwise gather the waits at the top)
            __builtin_amdgcn_sched_barrier(0);
        };
        spair(std::integral_constant<int, 0>{});
        spair(std::integral_constant<int, 1>{});
        spair(std::integral_constant<int, 2>{});
        spair(std::integral_constant<int, 3>{});
        spair(std::integral_constant<int, 4>{});
        spair(std::integral_constant<int, 5>{});
        spair(std::integral_constant<int, 6>{});
        spair(std::integral_constant<int, 7>{});
        // V^T operands for the second product, requested while the weights
        // are computed.
        i16x4 vop[4][4][2];
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
            for (int aa = 0; aa < 2; ++aa) {
                constexpr int VB = (2 + BUF) * kKeys * kRowBytes;   // V buffer BUF
                const uint32_t va = voff[dt][aa];
                vop[0][dt][aa] = lds_read_tr16<VB + 0 * 16 * kRowBytes>(va);
                vop[1][dt][aa] = lds_read_tr16<VB + 1 * 16 * kRowBytes>(va);
                vop[2][dt][aa] = lds_read_tr16<VB + 2 * 16 * kRowBytes>(va);
                vop[3][dt][aa] = lds_read_tr16<VB + 3 * 16 * kRowBytes>(va);
            }

        // Causal mask (diagonal tiles only), max, lazy rescale, weights.
        float sv2[2][16];
        float mx = -INFINITY;
        const int lim = pos - kt * kKeys - 8 * h;   // key offsets <= lim are allowed
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                sv2[u][r] = sacc[u][r];
            }
        if (kt >= kt_diag) {
            // tile reaches past some row's position
#pragma unroll
            for (int u = 0; u < 2; ++u)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    sv2[u][r] = (32 * u + key_of_reg(r) <= lim) ? sv2[u][r] : -INFINITY;
        }
        {
            // two independent chains, one per subtile
            float m0 = -INFINITY, m1 = -INFINITY;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                m0 = fmaxf(m0, sv2[0][r]);
                m1 = fmaxf(m1, sv2[1][r]);
            }
            mx = fmaxf(m0, m1);
        }
        mx = max_halves(mx) * sl2;
        const bool need = mx > mref + kLazy;
        if (__builtin_amdgcn_ballot_w64(need)) {
            const float nref = need ? mx : mref;
            const float alpha = (nref == mref) ? 1.0f : __builtin_amdgcn_exp2f(mref - nref);
            lsum *= alpha;
#pragma unroll
            for (int dt = 0; dt < 4; ++dt)
#pragma unroll
                for (int r = 0; r < 16; ++r) o[dt][r] *= alpha;
            mref = nref;
            mref_safe = (nref == -INFINITY) ? 0.0f : nref;
        }
        u32x4 pb[4];                              // P^T operands for the four 16-key steps
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                uint32_t w[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = 8 * half + 2 * e;
                    w[e] = pack2_bf16(__builtin_amdgcn_exp2f(fmaf(sv2[u][r], sl2, -mref_safe)),
                                      __builtin_amdgcn_exp2f(fmaf(sv2[u][r + 1], sl2, -mref_safe)));
                    // the normaliser sums the same rounded weights the product uses
                    lsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w[e]), ones, lsum, false);
                }
                pb[2 * u + half] = u32x4{w[0], w[1], w[2], w[3]};
            }

        // O^T += V^T P^T over the tile's four 16-key steps.
        lds_wait_all(vop[0][0][0], vop[0][0][1], vop[0][1][0], vop[0][1][1],
                     vop[0][2][0], vop[0][2][1], vop[0][3][0], vop[0][3][1]);
#pragma unroll
        for (int t = 1; t < 4; ++t)
            lds_pin(vop[t][0][0], vop[t][0][1], vop[t][1][0], vop[t][1][1],
                    vop[t][2][0], vop[t][2][1], vop[t][3][0], vop[t][3][1]);
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int dt = 0; dt < 4; ++dt) {
                const i16x8 av = __builtin_shufflevector(vop[t][dt][0], vop[t][dt][1], 0, 1, 2, 3, 4, 5, 6, 7);
                o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av),
                                                                as_bf16x8(pb[t]), o[dt], 0, 0, 0);
            }
        // the next tile's copies have landed and every wave is done reading
        // this tile's buffers
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
    };
    for (int kt = 0; kt < ntiles; kt += 2) {
        tile(kt, std::integral_constant<int, 0>{}, s_k1, s_v1);
        if (kt + 1 < ntiles) tile(kt + 1, std::integral_constant<int, 1>{}, s_k0, s_v0);
    }

    // Epilogue: combine the half-waves' sums, normalise, store.
    const float ltot = sum_halves(lsum);
    if (!active) return;
    const float inv = 1.0f / ltot;
    uint16_t* op = out + orow * kD;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int d0 = 32 * dt + 8 * i + 4 * h;
            uint2 w;
            w.x = pack2_bf16(o[dt][4 * i + 0] * inv, o[dt][4 * i + 1] * inv);
            w.y = pack2_bf16(o[dt][4 * i + 2] * inv, o[dt][4 * i + 3] * inv);
            *reinterpret_cast<uint2*>(op + d0) = w;
        }
    if (lse && h == 0) lse[orow] = kLn2 * (mref + log2f(ltot));
}

template <int G, bool FUSED>
hipError_t launch_gf(const AttnArgs& a, void* out, float* lse, hipStream_t stream, KernelEvents ev) {
    constexpr int QT = kRows / G;
    const int nq = (a.max_q_len + QT - 1) / QT;
    const int pairs = a.num_seqs * a.n_kv;
    const int per_xcd = (pairs + kXcds - 1) / kXcds;
    const dim3 grid(per_xcd * nq * kXcds);
    uint16_t* o = static_cast<uint16_t*>(out);
    if (ev.on())
        hipExtLaunchKernelGGL((chunk_mfma_kernel<G, FUSED>), grid, dim3(kThreads), 0, stream, ev.start, ev.stop, 0, a,
                              o, lse);
    else
        hipLaunchKernelGGL((chunk_mfma_kernel<G, FUSED>), grid, dim3(kThreads), 0, stream, a, o, lse);
    return hipGetLastError();
}
template <int G>
hipError_t launch_g(const AttnArgs& a, void* out, float* lse, hipStream_t stream, KernelEvents ev) {
    return a.k_new ? launch_gf<G, true>(a, out, lse, stream, ev) : launch_gf<G, false>(a, out, lse, stream, ev);
}

}  // namespace

bool chunk_mfma_supported(int n_q, int n_kv, int head_dim, int block_size, int max_seq_len) {
    if (head_dim != kD || block_size != kBS || n_kv < 1 || n_q % n_kv) return false;
    if (max_seq_len > kTblCache * kBS) return false;
    const int G = n_q / n_kv;
    return G == 1 || G == 2 || G == 4 || G == 8;
}

hipError_t launch_chunk_mfma(const AttnArgs& a, void* out, float* lse, hipStream_t stream, KernelEvents ev) {
    switch (a.n_q / a.n_kv) {
        case 1: return launch_g<1>(a, out, lse, stream, ev);
        case 2: return launch_g<2>(a, out, lse, stream, ev);
        case 4: return launch_g<4>(a, out, lse, stream, ev);
        case 8: return launch_g<8>(a, out, lse, stream, ev);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace pkv
