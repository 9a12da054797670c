// Balanced decode pass for bf16 K/V, head_dim 128, block_size 16.
//
// Decode reads every cached K/V byte once per step (chapter 5 section 2.2),
// so the kernel is a gathered stream (section 3.2: blocks found through the
// block table) and its speed is set by how evenly and how continuously the
// chip's waves keep HBM busy. This pass therefore ignores sequence
// boundaries when it hands out work:
//
//  * all (sequence s, kv head g, block b) tiles of the batch are numbered in
//    one sequence: s-major, then g, then b (a "segment" is the run of tiles
//    of one (s, g));
//  * the grid is W single-wave workgroups, W = the CUs times the waves per
//    CU the tile math's policy asks for (at most what fits at once);
//    with W' = min(W, T), wave w < W' streams tiles
//    [floor(w T / W'), floor((w+1) T / W')) of the T tiles - every wave
//    reads the same number of bytes to within one tile and none is empty
//    (waves w >= W' have nothing to do);
//  * a wave keeps the running softmax state of decode_tile.h for the segment
//    it is in; when it leaves a segment it writes that state as one partial.
//    The partial of wave w for segment sigma goes to slot w + sigma: both
//    grow along the tile order, so slots never collide, a segment's partials
//    fill a contiguous run of slots (no wave between two that touch a
//    segment can skip it, since no wave is empty), and W + S * n_kv slots
//    always suffice;
//  * the next tile's loads are issued before the current tile is computed,
//    so every wave always has a tile in flight;
//  * with four query heads per kv head both per-tile products run on the
//    matrix cores (decode_mfma.h); other group sizes use the vector-ALU
//    tile math of decode_tile.h;
//  * the K/V format is a template parameter: bf16 tiles, or 8-bit codes
//    with one fp32 scale per (token, kv head) (half the bytes; the scales
//    are folded into the scores and the weights).
//
// Per-sequence block counts (ceil(L / 16), 0 for an invalid length) and
// their prefix sums are built by every wave in LDS from seq_lens; wave 0
// also stores the prefix for the merge pass. A tile whose table entry is
// outside the pool is not used and its segment's partial is NaN.
#include "decode_mfma.h"
#include "decode_tile.h"
#include "kernels.h"

namespace pkv {
namespace {

// Dynamic LDS of one workgroup: prefix [S+1], then lengths [S].
__host__ __device__ inline size_t balanced_lds_ints(int num_seqs) {
    return 2 * static_cast<size_t>(num_seqs) + 1;
}
__host__ inline size_t balanced_lds_bytes(int num_seqs) {
    return sizeof(int) * balanced_lds_ints(num_seqs);
}


// Query load and partial write of the vector-ALU tile math (decode_tile.h
// layout: lane (r, c) works on dims 8c .. 8c+7; rows r = 0 hold the state
// after the merge).
template <int G>
struct ValuRows {
    using State = DecodeState<G>;
    static constexpr int kQ = G;
    static constexpr int kSlotRows = G;              // partial rows per slot
    static constexpr int kWaves = G == 8 ? 1 : 2;   // waves per SIMD the registers allow
    static constexpr int kWavesPerCU = 0;           // waves per CU launched (0: all that fit)
    static constexpr bool kCodes = false;           // pool of 8-bit codes + scales
    // One query per sequence: the G heads of kv head g.
    __device__ __forceinline__ static void fetch_q(u32x4 (&qv)[kQ], const AttnArgs& a, int s, int g, int lane) {
        const uint16_t* q_sg = static_cast<const uint16_t*>(a.q) + (static_cast<size_t>(s) * a.n_q + g * G) * kTileD;
#pragma unroll
        for (int h = 0; h < G; ++h) qv[h] = *reinterpret_cast<const u32x4*>(q_sg + h * kTileD + (lane & 15) * 8);
    }
    // The segment's row bookkeeping; returns the rows used.
    __device__ __forceinline__ static int begin(State&, const AttnArgs&, int /*s*/, int /*lane*/) { return G; }
    __device__ __forceinline__ static void flush(State& st, const AttnArgs& a, size_t p, int /*used*/, bool bad,
                                                 int lane) {
        const int c = lane & 15;
        st.merge_rows();
        if ((lane >> 4) == 0) {
#pragma unroll
            for (int h = 0; h < G; ++h) {
                float4* o = reinterpret_cast<float4*>(a.ws_o + (p * G + h) * kTileD + c * 8);
                o[0] = make_float4(st.acc[h][0], st.acc[h][1], st.acc[h][2], st.acc[h][3]);
                o[1] = make_float4(st.acc[h][4], st.acc[h][5], st.acc[h][6], st.acc[h][7]);
                if (c == 0) a.ws_ml[p * G + h] = bad ? PartialML{NAN, NAN} : PartialML{st.m[h], st.l[h]};
            }
        }
    }
};

// Query load and partial write of the matrix-core tile math (decode_mfma.h):
// rows r = i * G + h of (query i, head h) in NB blocks of 16; lane (q, n)
// holds row 16b + n's query at dims 32c + 8q .. +7 (c = 0..3), zero for rows
// past the C * G the sequence has. Decode: one query (q_start null), NB = 1,
// G rows per partial slot; small chunks: C <= 32 / G queries, NB = 2, 32.
template <int G, int NB>
struct MfmaRows {
    using State = MfmaState<NB>;
    static constexpr int kQ = 4 * NB;
    static constexpr int kSlotRows = NB == 1 ? G : 16 * NB;
    static constexpr int kWaves = 2;
    static constexpr int kWavesPerCU = 0;
    static constexpr bool kCodes = false;
    // Segment (s, g)'s first query row and number of queries.
    __device__ __forceinline__ static int queries(const AttnArgs& a, int s, int& row0) {
        row0 = s;
        if (!a.q_start) return 1;
        row0 = a.q_start[s];
        return a.q_start[s + 1] - row0;
    }
    __device__ __forceinline__ static void fetch_q(u32x4 (&qv)[kQ], const AttnArgs& a, int s, int g, int lane) {
        const int n = lane & 15;
        const int q = lane >> 4;
        int row0;
        const int used = queries(a, s, row0) * G;
        const uint16_t* qb = static_cast<const uint16_t*>(a.q);
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            const int r = 16 * b + n;
            const int i = r / G;
            const uint16_t* qr = qb + ((static_cast<size_t>(row0) + i) * a.n_q + g * G + (r - i * G)) * kTileD + 8 * q;
#pragma unroll
            for (int c = 0; c < 4; ++c)
                qv[4 * b + c] = r < used ? *reinterpret_cast<const u32x4*>(qr + 32 * c) : u32x4{0, 0, 0, 0};
        }
    }
    // Which rows exist and how many keys at the chunk's end each may not
    // see; returns the rows used.
    __device__ __forceinline__ static int begin(State& st, const AttnArgs& a, int s, int lane) {
        int row0;
        const int C = queries(a, s, row0);
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            const int r = 16 * b + (lane & 15);
            st.ok[b] = r < C * G;
            st.back[b] = C - 1 - r / G;
        }
        return C * G;
    }
    __device__ __forceinline__ static void flush(State& st, const AttnArgs& a, size_t p, int used, bool bad,
                                                 int lane) {
        st.write_partial(a.ws_o, a.ws_ml, p, kSlotRows, used, bad, lane);
    }
};

// bf16 K/V: per tile, eight 16-byte loads per lane (decode_tile.h layout).
template <int G>
struct Bf16Kv : ValuRows<G> {
    static constexpr int kDepth = 2;   // tiles in flight + 1
    struct Regs {
        u32x4 k[4], v[4];
    };
    const uint16_t* kc;
    const uint16_t* vc;
    __device__ __forceinline__ Bf16Kv(const AttnArgs& a, int lane)
        : kc(static_cast<const uint16_t*>(a.k_cache) + lane * 8), vc(static_cast<const uint16_t*>(a.v_cache) + lane * 8) {}
    __device__ __forceinline__ void load(Regs& t, int tile, int /*lane*/) const {
        const size_t off = static_cast<size_t>(tile) * kTileElems;
        load_tile(kc + off, vc + off, t.k, t.v);
    }
    __device__ __forceinline__ void compute(DecodeState<G>& st, const Regs& t, const u32x4 (&qv)[G],
                                            int lane, int ntok, float sl2) const {
        st.tile(t.k, t.v, qv, lane >> 4, ntok, sl2);
    }
};

// 8-bit codes + fp32 scales: per tile, eight 8-byte code loads and the
// scales this lane's scores and weights need.
template <int G>
struct Int8Kv : ValuRows<G> {
    // a tile is half the bytes of a bf16 one: keep two in flight (one with
    // one or two query heads per kv head, whose registers would otherwise
    // spill)
    static constexpr int kDepth = G <= 2 ? 2 : 3;
    static constexpr bool kCodes = true;
    struct Regs {
        u32x2 k[4], v[4];
        float sk[4], sv[4];   // tokens 4i + r
    };
    const int8_t* kc;
    const int8_t* vc;
    const float* ks;
    const float* vs;
    __device__ __forceinline__ Int8Kv(const AttnArgs& a, int lane)
        : kc(static_cast<const int8_t*>(a.k_cache) + lane * 8), vc(static_cast<const int8_t*>(a.v_cache) + lane * 8),
          ks(a.k_scale), vs(a.v_scale) {}
    __device__ __forceinline__ void load(Regs& t, int tile, int lane) const {
        const size_t off = static_cast<size_t>(tile) * kTileElems;   // one byte per element
        const u32x2* kp = reinterpret_cast<const u32x2*>(kc + off);
        const u32x2* vp = reinterpret_cast<const u32x2*>(vc + off);
#pragma unroll
        for (int i = 0; i < 4; ++i) t.k[i] = __builtin_nontemporal_load(kp + i * 64);
#pragma unroll
        for (int i = 0; i < 4; ++i) t.v[i] = __builtin_nontemporal_load(vp + i * 64);
        const size_t so = static_cast<size_t>(tile) * kTileB;
        const int r = lane >> 4;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            t.sk[i] = ks[so + 4 * i + r];
            t.sv[i] = vs[so + 4 * i + r];
        }
    }
    __device__ __forceinline__ void compute(DecodeState<G>& st, const Regs& t, const u32x4 (&qv)[G],
                                            int lane, int ntok, float sl2) const {
        st.tile_q8(t.k, t.v, t.sk, t.sv, qv, lane >> 4, ntok, sl2);
    }
};

// Four query heads per kv head: both products on the matrix cores
// (decode_mfma.h). Lane (q, n) loads token n's K at dims 32b + 8q .. +7
// (b = 0..3) and tokens 4q .. 4q+3's V at dims 8n .. 8n+7: the same bytes per
// tile as the vector-ALU layout, in the operand layouts of the two products.
//
// How many tile loads the chip holds in flight matters more here than
// hiding each wave's own latency: scattered tile reads get slower overall
// when waves keep more of them outstanding. Measured per pass (64-sequence
// batch / 256-sequence batch / 8 x 32k keys; verification chunks):
//  * decode: six waves per CU, each waiting for all its loads (the next
//    tile's included) before a tile's products, 101.2 / 327.7 / 161.2 us,
//    against 101.3 / 336.8 / 164.9 with the next tile's loads left in flight
//    at four waves per CU and 103.3 / 331.9 / 166.6 at eight;
//  * chunks: four waves per CU with the next tile in flight, 114.6 us,
//    against 115.6 waiting at six and 118.1 at eight.
template <int G, int NB>
struct Bf16Mfma : MfmaRows<G, NB> {
    using typename MfmaRows<G, NB>::State;
    using MfmaRows<G, NB>::kQ;
    static constexpr int kDepth = 2;
    static constexpr bool kDrain = NB == 1;
    static constexpr int kWavesPerCU = kDrain ? 6 : 4;
    struct Regs {
        u32x4 k[4], v[4];
    };
    const uint16_t* kc;
    const uint16_t* vc;
    __device__ __forceinline__ Bf16Mfma(const AttnArgs& a, int lane)
        : kc(static_cast<const uint16_t*>(a.k_cache) + (lane & 15) * kTileD + 8 * (lane >> 4)),
          vc(static_cast<const uint16_t*>(a.v_cache) + 4 * (lane >> 4) * kTileD + 8 * (lane & 15)) {}
    __device__ __forceinline__ void load(Regs& t, int tile, int /*lane*/) const {
        const size_t off = static_cast<size_t>(tile) * kTileElems;
        const u32x4* kp = reinterpret_cast<const u32x4*>(kc + off);
        const u32x4* vp = reinterpret_cast<const u32x4*>(vc + off);
#pragma unroll
        for (int b = 0; b < 4; ++b) t.k[b] = __builtin_nontemporal_load(kp + 4 * b);
#pragma unroll
        for (int e = 0; e < 4; ++e) t.v[e] = __builtin_nontemporal_load(vp + e * (kTileD / 8));
    }
    __device__ __forceinline__ void compute(State& st, const Regs& t, const u32x4 (&qv)[kQ], int lane, int ntok,
                                            float sl2) const {
        if constexpr (kDrain) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        f32x4 s[NB];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            s[nb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int b = 0; b < 4; ++b)
                s[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, t.k[b]),
                                                                __builtin_bit_cast(bf16x8, qv[4 * nb + b]), s[nb], 0, 0, 0);
        }
        // rows past the sequence end may hold anything (NaN): zero them
        u32x4 v[4];
        const int q = lane >> 4;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = 4 * q + e < ntok ? t.v[e] : u32x4{0, 0, 0, 0};
        const float none[4] = {1.0f, 1.0f, 1.0f, 1.0f};
        st.template update<false>(s, none, none, [&](int j) { return v_operand_bf16(v, j); }, lane, ntok, sl2);
    }
};

// Decode with 2, 4 or 8 query heads per kv head: one block of 16 rows on
// the matrix cores, G of them used. On the 64-sequence batch (lengths
// 512..4096, 8 kv heads) against the vector-ALU tile math, us per call:
// G = 2 107.8 against 113.1, G = 8 115.7 against 202.5 (there the vector
// ALU's 8 x 16 dot products per token are the bound); G = 1 106.7 against
// 108.1, left on the vector ALU with its 8-bit counterpart.
template <>
struct Bf16Kv<2> : Bf16Mfma<2, 1> {
    using Bf16Mfma<2, 1>::Bf16Mfma;
};
template <>
struct Bf16Kv<4> : Bf16Mfma<4, 1> {
    using Bf16Mfma<4, 1>::Bf16Mfma;
};
template <>
struct Bf16Kv<8> : Bf16Mfma<8, 1> {
    using Bf16Mfma<8, 1>::Bf16Mfma;
};
// 8-bit K/V with G = 2, 4 or 8 query heads per kv head on the matrix cores,
// tiles in registers, the next tile's loads in flight while one is
// computed (us per call on the batch above: G = 2 67.5 against the vector
// ALU's 81.7, G = 8 77.1 against 215.0; G = 1 stays on the vector ALU, 65.5
// against 68.1). Lane (q, n) loads:
//  * token n's codes at bytes 16q .. 16q + 15 and 64 + 16q .. 64 + 16q + 15
//    (two 16-byte loads, each instruction reading one contiguous half of
//    every token's row) for the score product. Which dims a lane holds in
//    that contraction is free as long as its query operand holds the same
//    ones: product b takes dims 64(b / 2) + 16q + 8(b % 2) .. + 7 (fetch_q
//    below loads the query that way);
//  * tokens 4q .. 4q + 3's codes at dims 8n .. 8n + 7 (four 8-byte loads,
//    each instruction reading four whole 128-byte rows) for the output
//    product, in the layout of v_operand_codes;
//  * the K and V scales of tokens 4q .. 4q + 3 (one 16-byte load each).
// 24 registers per tile. The pool of codes and the scale arrays must be
// 16-byte aligned.
template <int G>
struct Int8Regs : MfmaRows<G, 1> {
    using typename MfmaRows<G, 1>::State;
    using MfmaRows<G, 1>::kQ;
    static constexpr int kDepth = 2;
    static constexpr int kWavesPerCU = 8;
    static constexpr bool kCodes = true;
    struct Regs {
        u32x4 k[2];
        u32x2 v[4];
        u32x4 sk, sv;
    };
    const int8_t* kc;
    const int8_t* vc;
    const float* ks;
    const float* vs;
    __device__ __forceinline__ Int8Regs(const AttnArgs& a, int lane)
        : kc(static_cast<const int8_t*>(a.k_cache) + (lane & 15) * kTileD + 16 * (lane >> 4)),
          vc(static_cast<const int8_t*>(a.v_cache) + 4 * (lane >> 4) * kTileD + 8 * (lane & 15)),
          ks(a.k_scale + 4 * (lane >> 4)),
          vs(a.v_scale + 4 * (lane >> 4)) {}
    // The G heads' query (decode: one row per sequence), lane (q, n) head n's
    // dims 64(b / 2) + 16q + 8(b % 2) .. + 7 for product b, zero for n >= G.
    __device__ __forceinline__ static void fetch_q(u32x4 (&qv)[kQ], const AttnArgs& a, int s, int g, int lane) {
        const int n = lane & 15, q = lane >> 4;
        const uint16_t* qr = static_cast<const uint16_t*>(a.q) +
                             (static_cast<size_t>(s) * a.n_q + g * G + min(n, G - 1)) * kTileD + 16 * q;
#pragma unroll
        for (int b = 0; b < 4; ++b)
            qv[b] = n < G ? *reinterpret_cast<const u32x4*>(qr + 64 * (b >> 1) + 8 * (b & 1)) : u32x4{0, 0, 0, 0};
    }
    __device__ __forceinline__ void load(Regs& t, int tile, int /*lane*/) const {
        const size_t off = static_cast<size_t>(tile) * kTileElems;   // one byte per element
        const u32x4* kp = reinterpret_cast<const u32x4*>(kc + off);
        t.k[0] = __builtin_nontemporal_load(kp);
        t.k[1] = __builtin_nontemporal_load(kp + 4);
        const u32x2* vp = reinterpret_cast<const u32x2*>(vc + off);
#pragma unroll
        for (int e = 0; e < 4; ++e) t.v[e] = __builtin_nontemporal_load(vp + e * (kTileD / 8));
        const size_t so = static_cast<size_t>(tile) * kTileB;
        t.sk = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(ks + so));
        t.sv = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vs + so));
    }
    __device__ __forceinline__ void compute(State& st, const Regs& t0, const u32x4 (&qv)[kQ], int lane, int ntok,
                                            float sl2) const {
        // The tile's registers pass through an empty statement here, after
        // the next tile's loads were issued: without it the compiler unpacks
        // a tile's codes at the end of the step before, where the loads of
        // the tile after it are not issued yet, and every step then waits
        // for the tile just requested.
        Regs t = t0;
        asm volatile("" : "+v"(t.k[0]), "+v"(t.k[1]), "+v"(t.v[0]), "+v"(t.v[1]), "+v"(t.v[2]), "+v"(t.v[3]),
                     "+v"(t.sk), "+v"(t.sv));
        f32x4 s[1] = {f32x4{0.0f, 0.0f, 0.0f, 0.0f}};
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const u32x4 w = t.k[b >> 1];
            const u32x2 kb = (b & 1) ? u32x2{w[2], w[3]} : u32x2{w[0], w[1]};
            s[0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, codes8_to_bf16x8(kb)),
                                                           __builtin_bit_cast(bf16x8, qv[b]), s[0], 0, 0, 0);
        }
        // codes are finite whatever a slot past the end holds; its weight is 0
        const float sk[4] = {__uint_as_float(t.sk[0]), __uint_as_float(t.sk[1]), __uint_as_float(t.sk[2]),
                             __uint_as_float(t.sk[3])};
        const float sv[4] = {__uint_as_float(t.sv[0]), __uint_as_float(t.sv[1]), __uint_as_float(t.sv[2]),
                             __uint_as_float(t.sv[3])};
        st.template update<true>(s, sk, sv, [&](int j) { return v_operand_codes(t.v, j); }, lane, ntok, sl2);
    }
};
template <>
struct Int8Kv<2> : Int8Regs<2> {
    using Int8Regs<2>::Int8Regs;
};
template <>
struct Int8Kv<4> : Int8Regs<4> {
    using Int8Regs<4>::Int8Regs;
};
template <>
struct Int8Kv<8> : Int8Regs<8> {
    using Int8Regs<8>::Int8Regs;
};

// Small chunks: up to 32 (query, head) rows per kv head in two blocks.
template <int G>
using ChunkKv = Bf16Mfma<G, 2>;
static_assert(ChunkKv<4>::kSlotRows == kChunkSlotRows, "chunk partial slots");

// Small chunks over an 8-bit pool (verification passes over a quantised
// cache): the rows of ChunkKv, tiles in registers with Bf16Mfma's operand
// layouts. Lane (q, n) loads token n's codes at dims 32b + 8q .. + 7 (four
// 8-byte loads), tokens 4q .. 4q + 3's codes at dims 8n .. 8n + 7 (four
// 8-byte loads, whole rows per instruction) and those tokens' K and V scales
// (one 16-byte load each); codes become bf16 exactly, the K scale multiplies
// the scores and the V scale the weights (as Int8Regs).
template <int G>
struct Int8ChunkKv : MfmaRows<G, 2> {
    using typename MfmaRows<G, 2>::State;
    using MfmaRows<G, 2>::kQ;
    static constexpr int kDepth = 2;
    static constexpr int kWavesPerCU = 4;
    static constexpr bool kCodes = true;
    struct Regs {
        u32x2 k[4];
        u32x2 v[4];
        u32x4 sk, sv;
    };
    const int8_t* kc;
    const int8_t* vc;
    const float* ks;
    const float* vs;
    __device__ __forceinline__ Int8ChunkKv(const AttnArgs& a, int lane)
        : kc(static_cast<const int8_t*>(a.k_cache) + (lane & 15) * kTileD + 8 * (lane >> 4)),
          vc(static_cast<const int8_t*>(a.v_cache) + 4 * (lane >> 4) * kTileD + 8 * (lane & 15)),
          ks(a.k_scale + 4 * (lane >> 4)),
          vs(a.v_scale + 4 * (lane >> 4)) {}
    __device__ __forceinline__ void load(Regs& t, int tile, int /*lane*/) const {
        const size_t off = static_cast<size_t>(tile) * kTileElems;   // one byte per element
        const u32x2* kp = reinterpret_cast<const u32x2*>(kc + off);
        const u32x2* vp = reinterpret_cast<const u32x2*>(vc + off);
#pragma unroll
        for (int b = 0; b < 4; ++b) t.k[b] = __builtin_nontemporal_load(kp + 4 * b);
#pragma unroll
        for (int e = 0; e < 4; ++e) t.v[e] = __builtin_nontemporal_load(vp + e * (kTileD / 8));
        const size_t so = static_cast<size_t>(tile) * kTileB;
        t.sk = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(ks + so));
        t.sv = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vs + so));
    }
    __device__ __forceinline__ void compute(State& st, const Regs& t0, const u32x4 (&qv)[kQ], int lane, int ntok,
                                            float sl2) const {
        Regs t = t0;   // pinned here, after the next tile's loads (see Int8Regs)
        asm volatile("" : "+v"(t.k[0]), "+v"(t.k[1]), "+v"(t.k[2]), "+v"(t.k[3]), "+v"(t.v[0]), "+v"(t.v[1]),
                     "+v"(t.v[2]), "+v"(t.v[3]), "+v"(t.sk), "+v"(t.sv));
        f32x4 s[2];
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
            s[nb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int b = 0; b < 4; ++b)
                s[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, codes8_to_bf16x8(t.k[b])),
                                                                __builtin_bit_cast(bf16x8, qv[4 * nb + b]), s[nb], 0,
                                                                0, 0);
        }
        const float sk[4] = {__uint_as_float(t.sk[0]), __uint_as_float(t.sk[1]), __uint_as_float(t.sk[2]),
                             __uint_as_float(t.sk[3])};
        const float sv[4] = {__uint_as_float(t.sv[0]), __uint_as_float(t.sv[1]), __uint_as_float(t.sv[2]),
                             __uint_as_float(t.sv[3])};
        st.template update<true>(s, sk, sv, [&](int j) { return v_operand_codes(t.v, j); }, lane, ntok, sl2);
    }
};
static_assert(Int8ChunkKv<4>::kSlotRows == kChunkSlotRows, "chunk partial slots");

// Register budget: kWaves waves per SIMD (two: at most 256 registers per
// lane; eight query heads per kv head need more than that for state, query
// and two tiles, so one). How many waves per CU the grid holds is chosen
// apart from this (kWavesPerCU, else all that fit).
template <int G, class Kv, bool kAppend = false>
__global__ __launch_bounds__(kWave) __attribute__((amdgpu_waves_per_eu(Kv::kWaves)))
void decode_balanced_kernel(AttnArgs a) {
    extern __shared__ int s_mem[];
    const int S = a.num_seqs;
    int* P = s_mem;              // [S + 1] prefix sums of per-sequence block counts
    int* Ls = s_mem + S + 1;     // [S] lengths (0 when invalid)
    const int lane = threadIdx.x;
    const int w = blockIdx.x;
    const int table_tokens = a.table_stride * kTileB;

    int carry = 0;
    for (int base = 0; base < S; base += kWave) {
        const int s = base + lane;
        int nb = 0;
        if (s < S) {
            int L = a.seq_lens[s];
            if (seq_len_ok(L, 1, a.max_seq_len, table_tokens)) nb = (L + kTileB - 1) / kTileB;
            else L = 0;
            Ls[s] = L;
        }
        int x = nb;
#pragma unroll
        for (int o = 1; o < kWave; o <<= 1) {
            const int y = __shfl_up(x, o, kWave);
            if (lane >= o) x += y;
        }
        if (s < S) P[s + 1] = carry + x;
        carry += __shfl(x, kWave - 1, kWave);
    }
    if (lane == 0) P[0] = 0;
    __syncthreads();
    if (w == 0)
        for (int s = lane; s <= S; s += kWave) a.prefix[s] = P[s];

    const int n_kv = a.n_kv;
    const long long T = static_cast<long long>(n_kv) * P[S];
    const long long W = T < gridDim.x ? T : static_cast<long long>(gridDim.x);
    if (w >= W) return;
    const int t0 = static_cast<int>(static_cast<long long>(w) * T / W);
    const int t1 = static_cast<int>(static_cast<long long>(w + 1) * T / W);
    if (t0 >= t1) return;
    const int n = t1 - t0;

    // Per-lane description of tile c0 + lane: segment, tile index
    // (block * n_kv + g) and the sequence's keys from the tile's first one
    // to its end (tokens below it are valid; more than 16 for all but the
    // last block, which the chunk rows' masks rely on; -1: bad table entry).
    int i_seg = -1, i_tile = 0, i_ntok = 0;
    auto describe = [&](int c0) {
        const int t = c0 + lane;
        i_seg = -1;
        i_tile = 0;
        i_ntok = 0;
        if (t < t1) {
            int lo = 0, hi = S - 1;
            while (lo < hi) {
                const int mid = (lo + hi + 1) >> 1;
                if (n_kv * P[mid] <= t) lo = mid; else hi = mid - 1;
            }
            const int nb = P[lo + 1] - P[lo];
            const int rr = t - n_kv * P[lo];
            const int g = rr / nb;
            const int bi = rr - g * nb;
            int blk = a.table[static_cast<size_t>(lo) * a.table_stride + bi];
            if (blk < 0 || blk >= a.num_blocks) {
                blk = 0;
                i_ntok = -1;
            } else {
                i_ntok = Ls[lo] - bi * kTileB;
            }
            i_seg = lo * n_kv + g;
            i_tile = blk * n_kv + g;
        }
    };

    const Kv kv(a, lane);
    const float sl2 = a.scale_log2;

    typename Kv::State st;
    st.reset();
    u32x4 qv[Kv::kQ];
    int cur_seg = -1;
    bool cur_bad = false;

    int cur_used = 0;
    auto flush = [&]() __attribute__((always_inline)) {
        kv.flush(st, a, static_cast<size_t>(w) + cur_seg, cur_used, cur_bad, lane);
    };

    // Tiles stream through Kv::kDepth buffers: tile j is issued kDepth - 1
    // tiles before it is computed. Each buffer keeps its tile's segment and
    // valid-token count, so the descriptor window may move ahead of the
    // tile being computed.
    constexpr int D = Kv::kDepth;
    struct Buf {
        typename Kv::Regs t;
        int seg, ntok;
    };
    Buf b[D];
    static_assert(D >= 2, "the next tile is issued before the current one is computed");
    describe(t0);
    // Folded append (decode step stage 1): the new token of segment seg
    // (sequence seg / n_kv, kv head seg % n_kv) sits at row `slot` of the
    // segment's last tile, which only this wave reads. Lanes 0..15 write
    // its K row, 16..31 its V row (dims 8c .. 8c + 7, c = lane % 16), just
    // before the tile's loads are issued: one wave's accesses to one
    // address are performed in order, so those loads return the new row
    // without waiting for the stores to complete. An 8-bit pool takes the
    // row quantised as kv_append_q8 does (chapter 5 section 4: absmax over
    // the row, s = max(absmax, 1e-8) / 127, code = clamp(rint(x / s),
    // -127, 127), fp32, correctly rounded division).
    auto append_row = [&](int tile, int seg, int slot) {
        if (lane < 32) {
            const bool isv = lane >= 16;
            const int c = lane & 15;
            const uint16_t* src = static_cast<const uint16_t*>(isv ? a.v_new : a.k_new);
            const u32x4 x = *reinterpret_cast<const u32x4*>(src + static_cast<size_t>(seg) * kTileD + 8 * c);
            const size_t row = static_cast<size_t>(tile) * kTileB + slot;
            if constexpr (Kv::kCodes) {
                float f[8];
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    f[2 * w] = __uint_as_float(static_cast<uint32_t>(x[w]) << 16);
                    f[2 * w + 1] = __uint_as_float(static_cast<uint32_t>(x[w]) & 0xffff0000u);
                }
                float amax = 0.0f;
#pragma unroll
                for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(f[e]));
#pragma unroll
                for (int o = 1; o < 16; o <<= 1) amax = fmaxf(amax, __shfl_xor(amax, o, kWave));
                const float sc = fmaxf(amax, 1e-8f) / 127.0f;
                uint32_t packed[2] = {0u, 0u};
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float q = fminf(fmaxf(rintf(f[e] / sc), -127.0f), 127.0f);
                    packed[e >> 2] |= (static_cast<uint32_t>(static_cast<int>(q)) & 0xffu) << (8 * (e & 3));
                }
                int8_t* dst = static_cast<int8_t*>(isv ? a.v_app : a.k_app);
                *reinterpret_cast<u32x2*>(dst + row * kTileD + 8 * c) = u32x2{packed[0], packed[1]};
                if (c == 0) (isv ? a.vs_app : a.ks_app)[row] = sc;
            } else {
                uint16_t* dst = static_cast<uint16_t*>(isv ? a.v_app : a.k_app);
                *reinterpret_cast<u32x4*>(dst + row * kTileD + 8 * c) = x;
            }
        }
    };
    auto issue = [&](int j, Buf& bj) {
        const int lj = j & (kWave - 1);
        if (lj == 0 && j > 0) describe(t0 + j);
        bj.seg = __builtin_amdgcn_readlane(i_seg, lj);
        bj.ntok = __builtin_amdgcn_readlane(i_ntok, lj);
        const int tile = __builtin_amdgcn_readlane(i_tile, lj);
        if constexpr (kAppend) {
            // the last tile of a segment holds 1..16 of its keys
            if (bj.ntok > 0 && bj.ntok <= kTileB) append_row(tile, bj.seg, bj.ntok - 1);
        }
        kv.load(bj.t, tile, lane);
    };

    // One step: issue tile i + D - 1 into fut (unless `tail` says it may be
    // past the end), then compute tile i (in cur).
    //
    // The compiler places its waits for loads without regard to branch
    // conditions: a load that some path leaves in flight where paths join
    // counts as in flight on all of them, and the product that reads it
    // then waits for every load issued since, the tiles in flight
    // included. So the paths through a step of the main loop below leave
    // the same loads outstanding: a new segment's query is waited for
    // inside its branch (the empty asm reads the registers), before the
    // issue, and the last D - 1 steps, which issue nothing, run in a loop
    // of their own.
    auto step = [&](int i, const Buf& cur, Buf& fut, bool tail) {
        const int seg = cur.seg;
        const int ntok = cur.ntok;
        if (seg != cur_seg) {
            if (cur_seg >= 0) flush();
            const int s = seg / n_kv;
            const int g = seg - s * n_kv;
            st.reset();
            kv.fetch_q(qv, a, s, g, lane);
            cur_used = kv.begin(st, a, s, lane);
#pragma unroll
            for (int h = 0; h < Kv::kQ; ++h) asm volatile("" : "+v"(qv[h]));
            cur_seg = seg;
            cur_bad = false;
        }
        if (!tail || i + D - 1 < n) issue(i + D - 1, fut);
        if (ntok < 0) {
            cur_bad = true;
        } else {
            kv.compute(st, cur.t, qv, lane, ntok, sl2);
        }
    };

#pragma unroll
    for (int j = 0; j < D - 1; ++j)
        if (j < n) issue(j, b[j]);
    // tile j sits in b[j % D]; every step of an iteration here issues
    int i = 0;
    for (; i + 2 * D - 2 < n; i += D) {
#pragma unroll
        for (int u = 0; u < D; ++u) step(i + u, b[u], b[(u + D - 1) % D], false);
    }
    for (; i < n; i += D) {   // at most two iterations
#pragma unroll
        for (int u = 0; u < D; ++u)
            if (i + u < n) step(i + u, b[u], b[(u + D - 1) % D], true);
    }
    flush();
}

template <int G, class Kv, bool kAppend = false>
hipError_t launch_g(const AttnArgs& a, hipStream_t stream, KernelEvents ev) {
    const size_t lds = balanced_lds_bytes(a.num_seqs);
    if (ev.on())
        hipExtLaunchKernelGGL((decode_balanced_kernel<G, Kv, kAppend>), dim3(a.waves), dim3(kWave), lds, stream,
                              ev.start, ev.stop, 0, a);
    else
        hipLaunchKernelGGL((decode_balanced_kernel<G, Kv, kAppend>), dim3(a.waves), dim3(kWave), lds, stream, a);
    return hipGetLastError();
}

template <int G, class Kv>
int occupancy(size_t lds) {
    int blocks = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, decode_balanced_kernel<G, Kv>, kWave, lds) !=
        hipSuccess)
        return 0;
    return blocks;
}

// Waves per CU the grid holds: the policy's choice, at most what fits.
template <int G, class Kv>
int waves_per_cu(size_t lds) {
    const int fit = occupancy<G, Kv>(lds);
    return Kv::kWavesPerCU > 0 && fit > Kv::kWavesPerCU ? Kv::kWavesPerCU : fit;
}

template <template <int> class Kv>
int waves_for(int n_q, int n_kv, int num_seqs) {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    const size_t lds = balanced_lds_bytes(num_seqs);
    int per_cu = 0;
    switch (n_q / n_kv) {
        case 1: per_cu = waves_per_cu<1, Kv<1>>(lds); break;
        case 2: per_cu = waves_per_cu<2, Kv<2>>(lds); break;
        case 4: per_cu = waves_per_cu<4, Kv<4>>(lds); break;
        case 8: per_cu = waves_per_cu<8, Kv<8>>(lds); break;
        default: return 0;
    }
    if (per_cu < 1) per_cu = 1;
    return cus * per_cu;
}

template <template <int> class Kv>
hipError_t launch_kv(const AttnArgs& a, hipStream_t stream, KernelEvents ev) {
    switch (a.n_q / a.n_kv) {
        case 1: return launch_g<1, Kv<1>>(a, stream, ev);
        case 2: return launch_g<2, Kv<2>>(a, stream, ev);
        case 4: return launch_g<4, Kv<4>>(a, stream, ev);
        case 8: return launch_g<8, Kv<8>>(a, stream, ev);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

// Largest batch the balanced pass takes: its per-wave LDS holds two ints per
// sequence.
constexpr int kBalancedMaxSeqs = 8192;

bool decode_balanced_supported(int n_q, int n_kv, int head_dim, int block_size, int num_seqs) {
    if (head_dim != kTileD || block_size != kTileB || n_kv < 1 || n_q % n_kv) return false;
    if (num_seqs < 1 || num_seqs > kBalancedMaxSeqs) return false;
    const int G = n_q / n_kv;
    return G == 1 || G == 2 || G == 4 || G == 8;
}

int decode_balanced_waves(int n_q, int n_kv, int num_seqs, bool int8_kv) {
    return int8_kv ? waves_for<Int8Kv>(n_q, n_kv, num_seqs) : waves_for<Bf16Kv>(n_q, n_kv, num_seqs);
}

hipError_t launch_decode_balanced(const AttnArgs& a, hipStream_t stream, KernelEvents ev) {
    if (a.k_new && a.k_scale) {   // 8-bit pool with the append folded in
        if (!a.v_new || !a.k_app || !a.v_app || !a.ks_app || !a.vs_app) return hipErrorInvalidValue;
        switch (a.n_q / a.n_kv) {
            case 1: return launch_g<1, Int8Kv<1>, true>(a, stream, ev);
            case 2: return launch_g<2, Int8Kv<2>, true>(a, stream, ev);
            case 4: return launch_g<4, Int8Kv<4>, true>(a, stream, ev);
            case 8: return launch_g<8, Int8Kv<8>, true>(a, stream, ev);
            default: return hipErrorInvalidValue;
        }
    }
    if (a.k_new) {   // bf16 with the append folded in
        if (!a.v_new || !a.k_app || !a.v_app) return hipErrorInvalidValue;
        switch (a.n_q / a.n_kv) {
            case 1: return launch_g<1, Bf16Kv<1>, true>(a, stream, ev);
            case 2: return launch_g<2, Bf16Kv<2>, true>(a, stream, ev);
            case 4: return launch_g<4, Bf16Kv<4>, true>(a, stream, ev);
            case 8: return launch_g<8, Bf16Kv<8>, true>(a, stream, ev);
            default: return hipErrorInvalidValue;
        }
    }
    return a.k_scale ? launch_kv<Int8Kv>(a, stream, ev) : launch_kv<Bf16Kv>(a, stream, ev);
}

bool chunk_balanced_supported(int n_q, int n_kv, int head_dim, int block_size, int num_seqs, int max_q_len) {
    return decode_balanced_supported(n_q, n_kv, head_dim, block_size, num_seqs) && max_q_len >= 1 &&
           max_q_len * (n_q / n_kv) <= kChunkSlotRows;
}

int chunk_balanced_waves(int n_q, int n_kv, int num_seqs, bool int8_kv) {
    return int8_kv ? waves_for<Int8ChunkKv>(n_q, n_kv, num_seqs) : waves_for<ChunkKv>(n_q, n_kv, num_seqs);
}

hipError_t launch_chunk_balanced(const AttnArgs& a, hipStream_t stream, KernelEvents ev) {
    if (a.k_new) return hipErrorInvalidValue;   // chunk appends are launched on their own
    return a.k_scale ? launch_kv<Int8ChunkKv>(a, stream, ev) : launch_kv<ChunkKv>(a, stream, ev);
}

}  // namespace pkv
