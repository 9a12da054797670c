// Fixed-split decode pass for bf16 K/V, head_dim 128, block_size 16.
//
// Used when the caller asks for a split size. One workgroup per (key
// range of split_tokens keys, kv head, sequence); its WAVES waves take the
// range's blocks in turn (wave w: blocks w, w + WAVES, ...), each keeping the
// per-row state of decode_tile.h for all G query heads of the kv head, so
// every K/V byte is read from HBM once (chapter 5 section 2.2: decode reads
// the whole cache; section 3.2: the kernel follows the block table). The
// range's table slice is staged in LDS and validated there; the row states
// and then the wave states are merged once at the end of the range
// (chapter 5 section 4.1).
#include "decode_tile.h"
#include "kernels.h"

namespace pkv {
namespace {

constexpr int kMaxSplitBlocks = 128;   // split_tokens <= 2048

template <int G, int WAVES>
__global__ __launch_bounds__(kWave * WAVES) void decode_split_kernel(AttnArgs a) {
    __shared__ int s_tbl[kMaxSplitBlocks];
    __shared__ float s_state[WAVES][G][kTileD + 2];

    const int split = blockIdx.x;
    const int g = blockIdx.y;
    const int s = blockIdx.z;
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;

    const int L = a.seq_lens[s];
    if (!seq_len_ok(L, 1, a.max_seq_len, a.table_stride * kTileB)) return;
    const int tok_lo = split * a.split_tokens;
    if (tok_lo >= L) return;
    const int tok_hi = min(L, tok_lo + a.split_tokens);
    const int blk_lo = tok_lo / kTileB;
    const int nblk = (tok_hi - tok_lo + kTileB - 1) / kTileB;

    const int32_t* trow = a.table + static_cast<size_t>(s) * a.table_stride + blk_lo;
    int bad = 0;
    for (int j = tid; j < nblk; j += kWave * WAVES) {
        int b = trow[j];
        if (b < 0 || b >= a.num_blocks) { bad = 1; b = 0; }
        s_tbl[j] = b;
    }
    bad = __syncthreads_or(bad);

    const int n_q = a.n_kv * G;
    const size_t part0 = (static_cast<size_t>(s) * n_q + g * G) * a.max_splits + split;
    if (bad) {
        if (tid < G) a.ws_ml[part0 + static_cast<size_t>(tid) * a.max_splits] = PartialML{NAN, NAN};
        return;
    }

    const int c = lane & 15;
    const int r = lane >> 4;
    u32x4 qv[G];
    const uint16_t* qbase = static_cast<const uint16_t*>(a.q) + (static_cast<size_t>(s) * n_q + g * G) * kTileD + c * 8;
#pragma unroll
    for (int h = 0; h < G; ++h) qv[h] = *reinterpret_cast<const u32x4*>(qbase + h * kTileD);

    DecodeState<G> st;
    st.reset();
    const size_t tile_stride = static_cast<size_t>(a.n_kv) * kTileElems;
    const uint16_t* kbase = static_cast<const uint16_t*>(a.k_cache) + static_cast<size_t>(g) * kTileElems + lane * 8;
    const uint16_t* vbase = static_cast<const uint16_t*>(a.v_cache) + static_cast<size_t>(g) * kTileElems + lane * 8;
    for (int jb = wave; jb < nblk; jb += WAVES) {
        const size_t off = static_cast<size_t>(s_tbl[jb]) * tile_stride;
        u32x4 kr[4], vr[4];
        load_tile(kbase + off, vbase + off, kr, vr);
        st.tile(kr, vr, qv, r, tok_hi - (tok_lo + jb * kTileB), a.scale_log2);
    }
    st.merge_rows();

    if (r == 0) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
#pragma unroll
            for (int k = 0; k < 8; ++k) s_state[wave][h][c * 8 + k] = st.acc[h][k];
            if (c == 0) {
                s_state[wave][h][kTileD] = st.m[h];
                s_state[wave][h][kTileD + 1] = st.l[h];
            }
        }
    }
    __syncthreads();
    for (int e = tid; e < G * kTileD; e += kWave * WAVES) {
        const int h = e / kTileD;
        const int k = e % kTileD;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < WAVES; ++w) M = fmaxf(M, s_state[w][h][kTileD]);
        const float mu = (M == -INFINITY) ? 0.0f : M;
        float x = 0.0f, lw = 0.0f;
#pragma unroll
        for (int w = 0; w < WAVES; ++w) {
            const float wt = __builtin_amdgcn_exp2f(s_state[w][h][kTileD] - mu);
            x = fmaf(wt, s_state[w][h][k], x);
            lw = fmaf(wt, s_state[w][h][kTileD + 1], lw);
        }
        const size_t part = part0 + static_cast<size_t>(h) * a.max_splits;
        a.ws_o[part * kTileD + k] = x;
        if (k == 0) a.ws_ml[part] = PartialML{M, lw};
    }
}

template <int G>
hipError_t launch_g(const AttnArgs& a, hipStream_t stream, KernelEvents ev) {
    constexpr int kWaves = 4;
    const dim3 grid(a.max_splits, a.n_kv, a.num_seqs);
    if (ev.on())
        hipExtLaunchKernelGGL((decode_split_kernel<G, kWaves>), grid, dim3(kWave * kWaves), 0, stream, ev.start,
                              ev.stop, 0, a);
    else
        hipLaunchKernelGGL((decode_split_kernel<G, kWaves>), grid, dim3(kWave * kWaves), 0, stream, a);
    return hipGetLastError();
}

}  // namespace

bool decode_fast_supported(int n_q, int n_kv, int head_dim, int block_size, int split_tokens) {
    if (head_dim != kTileD || block_size != kTileB || n_kv < 1 || n_q % n_kv) return false;
    if (split_tokens % kTileB || split_tokens / kTileB > kMaxSplitBlocks) return false;
    const int G = n_q / n_kv;
    return G == 1 || G == 2 || G == 4 || G == 8;
}

hipError_t launch_decode_fast(const AttnArgs& a, hipStream_t stream, KernelEvents ev) {
    switch (a.n_q / a.n_kv) {
        case 1: return launch_g<1>(a, stream, ev);
        case 2: return launch_g<2>(a, stream, ev);
        case 4: return launch_g<4>(a, stream, ev);
        case 8: return launch_g<8>(a, stream, ev);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace pkv
