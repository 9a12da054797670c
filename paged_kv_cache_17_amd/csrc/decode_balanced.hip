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
//  * the grid is W single-wave workgroups, W = what the chip holds at once;
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
//  * with four query heads per kv head the per-tile math is the
//    reduce-scatter / one-exponential-per-lane form (DecodeStateG4);
//  * the K/V format is a template parameter: bf16 tiles, or 8-bit codes
//    with one fp32 scale per (token, kv head) (half the bytes; the scales
//    are folded into the scores and the weights, see decode_tile.h).
//
// Per-sequence block counts (ceil(L / 16), 0 for an invalid length) and
// their prefix sums are built by every wave in LDS from seq_lens; wave 0
// also stores the prefix for the merge pass. A tile whose table entry is
// outside the pool is not used and its segment's partial is NaN.
#include "decode_tile.h"
#include "kernels.h"

namespace pkv {
namespace {

// Dynamic LDS of one workgroup: prefix [S+1], lengths [S], then a 64-float
// slot (16-byte aligned) for handing weights between lanes.
__host__ __device__ inline size_t balanced_lds_ints(int num_seqs) {
    return (2 * static_cast<size_t>(num_seqs) + 1 + 3) / 4 * 4;
}
__host__ inline size_t balanced_lds_bytes(int num_seqs) {
    return sizeof(int) * (balanced_lds_ints(num_seqs) + kWave);
}

template <int G>
struct BalancedState { using T = DecodeState<G>; };
template <>
struct BalancedState<4> { using T = DecodeStateG4; };

// bf16 K/V: per tile, eight 16-byte loads per lane (decode_tile.h layout).
template <int G>
struct Bf16Kv {
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
    __device__ __forceinline__ void compute(typename BalancedState<G>::T& st, const Regs& t, const u32x4 (&qv)[G],
                                            int lane, int ntok, float sl2, float* s_p) const {
        if constexpr (G == 4) st.tile(t.k, t.v, qv, lane, ntok, sl2, s_p);
        else st.tile(t.k, t.v, qv, lane >> 4, ntok, sl2);
    }
};

// 8-bit codes + fp32 scales: per tile, eight 8-byte code loads and the
// scales this lane's scores and weights need.
template <int G>
struct Int8Kv {
    // a tile is half the bytes of a bf16 one: keep two in flight (one with
    // two query heads per kv head, whose registers would otherwise spill)
    static constexpr int kDepth = G == 2 ? 2 : 3;
    static constexpr int kScales = G == 4 ? 1 : 4;
    struct Regs {
        u32x2 k[4], v[4];
        float sk[kScales], sv[kScales];
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
        if constexpr (G == 4) {
            const int tok = 4 * (lane & 3) + r;        // token of this lane's score
            t.sk[0] = ks[so + tok];
            t.sv[0] = vs[so + tok];
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                t.sk[i] = ks[so + 4 * i + r];
                t.sv[i] = vs[so + 4 * i + r];
            }
        }
    }
    __device__ __forceinline__ void compute(typename BalancedState<G>::T& st, const Regs& t, const u32x4 (&qv)[G],
                                            int lane, int ntok, float sl2, float* s_p) const {
        if constexpr (G == 4) st.tile_q8(t.k, t.v, t.sk[0], t.sv[0], qv, lane, ntok, sl2, s_p);
        else st.tile_q8(t.k, t.v, t.sk, t.sv, qv, lane >> 4, ntok, sl2);
    }
};

// At least two waves per SIMD (at most 256 registers per lane): fewer
// waves would halve the bytes the chip keeps in flight. Eight query heads
// per kv head need more registers than that (state, query and two tiles):
// one wave per SIMD, with the grid sized to match.
template <int G, class Kv>
__global__ __launch_bounds__(kWave) __attribute__((amdgpu_waves_per_eu(G == 8 ? 1 : 2)))
void decode_balanced_kernel(AttnArgs a) {
    extern __shared__ int s_mem[];
    const int S = a.num_seqs;
    int* P = s_mem;              // [S + 1] prefix sums of per-sequence block counts
    int* Ls = s_mem + S + 1;     // [S] lengths (0 when invalid)
    float* s_p = reinterpret_cast<float*>(s_mem + balanced_lds_ints(S));
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
    // (block * n_kv + g) and valid tokens (-1: bad table entry).
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
                i_ntok = min(kTileB, Ls[lo] - bi * kTileB);
            }
            i_seg = lo * n_kv + g;
            i_tile = blk * n_kv + g;
        }
    };

    const int c = lane & 15;
    const int r = lane >> 4;
    const Kv kv(a, lane);
    const uint16_t* qc = static_cast<const uint16_t*>(a.q) + c * 8;
    const float sl2 = a.scale_log2;

    typename BalancedState<G>::T st;
    st.reset();
    u32x4 qv[G];
    int cur_seg = -1;
    bool cur_bad = false;

    auto flush = [&]() __attribute__((always_inline)) {
        float fm[G], fl[G];
        if constexpr (G == 4) {
            st.finish(lane, fm, fl);
        } else {
            st.merge_rows();
#pragma unroll
            for (int h = 0; h < G; ++h) {
                fm[h] = st.m[h];
                fl[h] = st.l[h];
            }
        }
        const size_t p = static_cast<size_t>(w) + cur_seg;
        if (r == 0) {
#pragma unroll
            for (int h = 0; h < G; ++h) {
                float4* o = reinterpret_cast<float4*>(a.ws_o + (p * G + h) * kTileD + c * 8);
                o[0] = make_float4(st.acc[h][0], st.acc[h][1], st.acc[h][2], st.acc[h][3]);
                o[1] = make_float4(st.acc[h][4], st.acc[h][5], st.acc[h][6], st.acc[h][7]);
                if (c == 0) a.ws_ml[p * G + h] = cur_bad ? PartialML{NAN, NAN} : PartialML{fm[h], fl[h]};
            }
        }
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
    describe(t0);
    auto issue = [&](int j, Buf& b) {
        const int lj = j & (kWave - 1);
        if (lj == 0 && j > 0) describe(t0 + j);
        b.seg = __builtin_amdgcn_readlane(i_seg, lj);
        b.ntok = __builtin_amdgcn_readlane(i_ntok, lj);
        kv.load(b.t, __builtin_amdgcn_readlane(i_tile, lj), lane);
    };

    // One step: issue tile i + D - 1 into fut, then compute tile i (in cur).
    auto step = [&](int i, const Buf& cur, Buf& fut) {
        if (i + D - 1 < n) issue(i + D - 1, fut);
        const int seg = cur.seg;
        const int ntok = cur.ntok;
        if (seg != cur_seg) {
            if (cur_seg >= 0) flush();
            const int s = seg / n_kv;
            const int g = seg - s * n_kv;
            const uint16_t* qs = qc + (static_cast<size_t>(s) * n_kv * G + g * G) * kTileD;
#pragma unroll
            for (int h = 0; h < G; ++h) qv[h] = *reinterpret_cast<const u32x4*>(qs + h * kTileD);
            st.reset();
            cur_seg = seg;
            cur_bad = false;
        }
        if (ntok < 0) {
            cur_bad = true;
        } else {
            kv.compute(st, cur.t, qv, lane, ntok, sl2, s_p);
        }
    };

    Buf b0, b1;
    issue(0, b0);
    if constexpr (D == 2) {
        for (int i = 0; i < n; i += 2) {
            step(i, b0, b1);
            if (i + 1 < n) step(i + 1, b1, b0);
        }
    } else {
        static_assert(D == 3, "pipeline depth 2 or 3");
        Buf b2;
        if (n > 1) issue(1, b1);
        for (int i = 0; i < n; i += 3) {
            step(i, b0, b2);
            if (i + 1 < n) step(i + 1, b1, b0);
            if (i + 2 < n) step(i + 2, b2, b1);
        }
    }
    flush();
}

template <int G, class Kv>
hipError_t launch_g(const AttnArgs& a, hipStream_t stream, KernelEvents ev) {
    const size_t lds = balanced_lds_bytes(a.num_seqs);
    if (ev.on())
        hipExtLaunchKernelGGL(decode_balanced_kernel<G, Kv>, dim3(a.waves), dim3(kWave), lds, stream, ev.start,
                              ev.stop, 0, a);
    else
        hipLaunchKernelGGL((decode_balanced_kernel<G, Kv>), dim3(a.waves), dim3(kWave), lds, stream, a);
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

template <template <int> class Kv>
int waves_for(int n_q, int n_kv, int num_seqs) {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    const size_t lds = balanced_lds_bytes(num_seqs);
    int per_cu = 0;
    switch (n_q / n_kv) {
        case 1: per_cu = occupancy<1, Kv<1>>(lds); break;
        case 2: per_cu = occupancy<2, Kv<2>>(lds); break;
        case 4: per_cu = occupancy<4, Kv<4>>(lds); break;
        case 8: per_cu = occupancy<8, Kv<8>>(lds); break;
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
    return a.k_scale ? launch_kv<Int8Kv>(a, stream, ev) : launch_kv<Bf16Kv>(a, stream, ev);
}

}  // namespace pkv
