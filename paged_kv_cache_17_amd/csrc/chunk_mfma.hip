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
//  * K is staged row-major in LDS, V transposed (an 8 x 8 bf16 transpose in
//    registers per thread), both padded against bank conflicts and double
//    buffered; the next tile's global loads are in flight while the current
//    tile is computed;
//  * S^T = K Q^T: A = K rows read in a permuted order pi, B = the wave's
//    queries (kept in registers). With pi(8i+4h+j) = 16(i/2)+8h+4(i%2)+j the
//    accumulator registers of S^T already hold, for each 16-key step, the
//    8 consecutive keys the next product needs in its B operand;
//  * each lane owns whole query rows (one column of S^T), so the online
//    softmax is lane-local plus one exchange with the other half-wave; the
//    reference max moves only when a score exceeds it by 2^8 (exact, rare
//    rescaling of the accumulators);
//  * O^T += V^T P^T: A = V^T from LDS, B = P^T packed to bf16 from registers.
// Keys past the sequence end get weight 0 and their V is zeroed in LDS.
#include "device_common.h"
#include "kernels.h"

namespace pkv {
namespace {

constexpr int kD = 128;
constexpr int kBS = 16;
constexpr int kKeys = 64;                 // keys per staged tile
constexpr int kRows = 128;                // (head, query) rows per workgroup
constexpr int kThreads = 256;
constexpr int kKPitch = kD + 8;           // bf16 elements per K row in LDS
constexpr int kVPitch = kKeys + 8;        // bf16 elements per V^T row in LDS
constexpr float kLazy = 8.0f;
constexpr int kXcds = 8;                  // dispatch round-robin width
constexpr int kTblCache = 2048;           // table entries cached in LDS (32768 keys)

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) { return pack2_bf16(lo, hi); }

// Row of S^T (key index within a 32-key subtile) held by accumulator
// register r of a lane in half h, given the permuted K-row order.
__device__ __forceinline__ int key_of_reg(int r, int h) {
    const int i = r >> 2, j = r & 3;
    return 16 * (i >> 1) + 8 * h + 4 * (i & 1) + j;
}

template <int G>
__global__ __launch_bounds__(kThreads, 2) void chunk_mfma_kernel(AttnArgs a, uint16_t* __restrict__ out,
                                                                 float* __restrict__ lse) {
    constexpr int QT = kRows / G;                 // queries per workgroup
    __shared__ __align__(16) uint16_t s_kbuf[2][kKeys * kKPitch];
    __shared__ __align__(16) uint16_t s_vbuf[2][kD * kVPitch];
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
    const int wave = tid >> 6;
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
    if (tid == 0) s_bad = 0;
    __syncthreads();
    if (ok)
        for (int b = tid; b < nblk; b += kThreads) {
            const int id = trow[b];
            if (id < 0 || id >= a.num_blocks) s_bad = 1;
            if (b < kTblCache) s_tbl[b] = id;
        }
    __syncthreads();
    if (!ok || s_bad) {
        if (active) {
            for (int e = h; e < kD; e += 2) Elem<uint16_t>::store(out + orow * kD + e, NAN);
            if (lse && h == 0) lse[orow] = NAN;
        }
        return;
    }

    // This lane's query in the B-operand layout: dims 16t + 8h + e, t = 0..7.
    u32x4 qv[8];
    {
        const u32x4* qp = reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(a.q) + orow * kD + 8 * h);
#pragma unroll
        for (int t = 0; t < 8; ++t) qv[t] = active ? qp[2 * t] : u32x4{0, 0, 0, 0};
    }

    // Staging roles: threads 0..127 copy K rows, 128..255 transpose V blocks.
    const bool stage_k = tid < 128;
    const int st = tid & 127;
    const uint16_t* kc = static_cast<const uint16_t*>(a.k_cache);
    const uint16_t* vc = static_cast<const uint16_t*>(a.v_cache);
    const size_t gstride = static_cast<size_t>(g) * kBS * kD;
    u32x4 stage[8];

    // K threads: key rows st/16 + 8m (m = 0..7), dims 8*(st%16)..+7 (a
    // wave's load covers whole 256-byte key rows).
    // V threads: keys 8*(st%8) + m (m = 0..7), dims 8*(st/8)..+7, so the 8
    // lanes that write LDS together hold different key groups of one row
    // of V^T (different banks).
    const int k_row0 = st >> 4, k_dim = 8 * (st & 15);
    const int v_key0 = 8 * (st & 7), v_dim = 8 * (st >> 3);
    const size_t blk_elems = static_cast<size_t>(n_kv) * kBS * kD;
    auto block_ptr = [&](int bi) {
        const int blk = bi < kTblCache ? s_tbl[bi] : trow[bi];
        return (stage_k ? kc : vc) + static_cast<size_t>(blk) * blk_elems + gstride;
    };
    auto load_tile = [&](int kt) {
        const int kbase = kt * kKeys;
        if (stage_k) {
            // rows k_row0 + 8m: m = 0,1 in block 0 of the tile, 2,3 in block 1, ...
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                const int key0 = kbase + 16 * b + k_row0;
                const uint16_t* base = key0 <= kmax ? block_ptr(key0 / kBS) + k_dim : nullptr;
#pragma unroll
                for (int m2 = 0; m2 < 2; ++m2) {
                    const int key = key0 + 8 * m2;
                    stage[2 * b + m2] = key <= kmax
                        ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(base + (key % kBS) * kD))
                        : u32x4{0, 0, 0, 0};
                }
            }
        } else {
            // keys v_key0 .. v_key0 + 7 lie in one block
            const int key0 = kbase + v_key0;
            const uint16_t* base = key0 <= kmax ? block_ptr(key0 / kBS) + v_dim : nullptr;
#pragma unroll
            for (int m = 0; m < 8; ++m) {
                const int key = key0 + m;
                u32x4 v = {0, 0, 0, 0};
                if (key <= kmax && key < L)
                    v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(base + (key % kBS) * kD));
                stage[m] = v;
            }
        }
    };
    auto store_tile = [&](int buf) {
        uint16_t* s_k = s_kbuf[buf];
        uint16_t* s_vt = s_vbuf[buf];
        if (stage_k) {
            // key k goes to row k with bits 2 and 3 swapped: the product reads
            // key pi(n) for lane n, so lane n then reads row n (no bank conflicts)
#pragma unroll
            for (int m = 0; m < 8; ++m) {
                const int k = (st >> 4) + 8 * m;
                const int row = (k & ~12) | ((k & 4) << 1) | ((k & 8) >> 1);
                *reinterpret_cast<u32x4*>(s_k + row * kKPitch + 8 * (st & 15)) = stage[m];
            }
        } else {
            // 8 x 8 transpose: column e (dim v_dim + e) over keys v_key0 + m.
            const int kb = v_key0;
            const int db = v_dim;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int w = e >> 1;
                const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
                u32x4 col;
#pragma unroll
                for (int d2 = 0; d2 < 4; ++d2) {
                    const uint32_t lo = stage[2 * d2][w];
                    const uint32_t hi = stage[2 * d2 + 1][w];
                    col[d2] = __builtin_amdgcn_perm(hi, lo, sel);
                }
                *reinterpret_cast<u32x4*>(s_vt + (db + e) * kVPitch + kb) = col;
            }
        }
    };

    f32x16 o[4];                                  // O^T tiles: dims 32dt + C-layout rows
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) o[dt] = f32x16{};
    float mref = -INFINITY, mref_safe = 0.0f, lsum = 0.0f;
    const float sl2 = a.scale_log2;
    const int ntiles = kmax / kKeys + 1;
    const int pmin = P + q0;                      // smallest position in the tile

    // Double-buffered tiles: tile kt is computed from buffer kt % 2 while
    // the loads of tile kt + 1 are in flight; those are written to the
    // other buffer after the compute, and one barrier per tile separates a
    // buffer's readers from its next writers.
    load_tile(0);
    store_tile(0);
    __syncthreads();
    for (int kt = 0; kt < ntiles; ++kt) {
        const uint16_t* s_k = s_kbuf[kt & 1];
        const uint16_t* s_vt = s_vbuf[kt & 1];
        if (kt + 1 < ntiles) load_tile(kt + 1);

        // S^T for the two 32-key subtiles.
        f32x16 sacc[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            sacc[u] = f32x16{};
            // A row m = n is key pi(n), stored at LDS row n of the subtile
            const uint16_t* kp = s_k + (32 * u + n) * kKPitch + 8 * h;
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                const u32x4 av = *reinterpret_cast<const u32x4*>(kp + 16 * t);
                sacc[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(av), as_bf16x8(qv[t]), sacc[u], 0, 0, 0);
            }
        }

        // Mask, max, lazy rescale, weights.
        const int kbase = kt * kKeys;
        const bool need_mask = kbase + kKeys - 1 > pmin || !active;
        float sv[2][16];
        float mx = -INFINITY;
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float x = sacc[u][r];
                if (need_mask) {
                    const int key = kbase + 32 * u + key_of_reg(r, h);
                    x = (active && key <= pos) ? x : -INFINITY;
                }
                sv[u][r] = x;
                mx = fmaxf(mx, x);
            }
        mx = fmaxf(mx, __shfl_xor(mx, 32, kWave)) * sl2;
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
                float p[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int r = 8 * half + e;   // registers 8*half .. 8*half+7: i = 2*half, 2*half+1
                    p[e] = __builtin_amdgcn_exp2f(fmaf(sv[u][r], sl2, -mref_safe));
                    lsum += p[e];
                }
                pb[2 * u + half] = u32x4{pack_bf16(p[0], p[1]), pack_bf16(p[2], p[3]),
                                         pack_bf16(p[4], p[5]), pack_bf16(p[6], p[7])};
            }

        // O^T += V^T P^T over the tile's four 16-key steps.
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int dt = 0; dt < 4; ++dt) {
                const u32x4 av = *reinterpret_cast<const u32x4*>(s_vt + (32 * dt + n) * kVPitch + 16 * t + 8 * h);
                o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(av), as_bf16x8(pb[t]), o[dt], 0, 0, 0);
            }
        if (kt + 1 < ntiles) store_tile((kt + 1) & 1);
        __syncthreads();
    }

    // Epilogue: combine the half-waves' sums, normalise, store.
    const float ltot = lsum + __shfl_xor(lsum, 32, kWave);
    if (!active) return;
    const float inv = 1.0f / ltot;
    uint16_t* op = out + orow * kD;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int d0 = 32 * dt + 8 * i + 4 * h;
            uint2 w;
            w.x = pack_bf16(o[dt][4 * i + 0] * inv, o[dt][4 * i + 1] * inv);
            w.y = pack_bf16(o[dt][4 * i + 2] * inv, o[dt][4 * i + 3] * inv);
            *reinterpret_cast<uint2*>(op + d0) = w;
        }
    if (lse && h == 0) lse[orow] = kLn2 * (mref + log2f(ltot));
}

template <int G>
hipError_t launch_g(const AttnArgs& a, void* out, float* lse, hipStream_t stream) {
    constexpr int QT = kRows / G;
    const int nq = (a.max_q_len + QT - 1) / QT;
    const int pairs = a.num_seqs * a.n_kv;
    const int per_xcd = (pairs + kXcds - 1) / kXcds;
    const dim3 grid(per_xcd * nq * kXcds);
    hipLaunchKernelGGL(chunk_mfma_kernel<G>, grid, dim3(kThreads), 0, stream, a, static_cast<uint16_t*>(out), lse);
    return hipGetLastError();
}

}  // namespace

bool chunk_mfma_supported(int n_q, int n_kv, int head_dim, int block_size) {
    if (head_dim != kD || block_size != kBS || n_kv < 1 || n_q % n_kv) return false;
    const int G = n_q / n_kv;
    return G == 1 || G == 2 || G == 4 || G == 8;
}

hipError_t launch_chunk_mfma(const AttnArgs& a, void* out, float* lse, hipStream_t stream) {
    switch (a.n_q / a.n_kv) {
        case 1: return launch_g<1>(a, out, lse, stream);
        case 2: return launch_g<2>(a, out, lse, stream);
        case 4: return launch_g<4>(a, out, lse, stream);
        case 8: return launch_g<8>(a, out, lse, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace pkv
