// Whole-block copies inside the K/V pools: the data side of copy-on-write.
//
// Serving tutorial section 4.2: when a block shared by several sequences
// (a common prefix, or the prompt's tail block under beam / parallel
// sampling) is about to be written by one of them, that sequence gets a
// copy of the block and its table entry is remapped; the shared copy is
// never modified in place. kvpool_cow picks the new block ids; this kernel
// copies the contents. A block is contiguous in each pool
// ([num_blocks][n_kv][B][d]: n_kv * B * d elements), so a copy is two plain
// memcpy's of block_bytes; one workgroup per (pair, pool) streams it with
// 16-byte accesses when sizes and addresses allow.
#include "device_common.h"
#include "kernels.h"

namespace pkv {
namespace {

constexpr int kCopyThreads = 256;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// kUnit: bytes per access - 16 when sizes and addresses allow, else 2, else
// 1 (an 8-bit pool whose block is an odd number of bytes).
template <int kUnit>
__global__ __launch_bounds__(kCopyThreads) void copy_blocks_kernel(char* __restrict__ k_cache,
                                                                   char* __restrict__ v_cache,
                                                                   const int32_t* __restrict__ src_ids,
                                                                   const int32_t* __restrict__ dst_ids,
                                                                   int num_blocks, size_t block_bytes) {
    const int pair = blockIdx.x;
    char* pool = blockIdx.y == 0 ? k_cache : v_cache;
    const int src = src_ids[pair];
    const int dst = dst_ids[pair];
    // ids the host could not check: a pair naming a block outside the pool
    // (or a block onto itself) is skipped
    if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks || src == dst) return;
    const char* s = pool + static_cast<size_t>(src) * block_bytes;
    char* d = pool + static_cast<size_t>(dst) * block_bytes;
    if constexpr (kUnit == 16) {
        const size_t n = block_bytes / 16;
        const u32x4* s4 = reinterpret_cast<const u32x4*>(s);
        u32x4* d4 = reinterpret_cast<u32x4*>(d);
        for (size_t i = threadIdx.x; i < n; i += kCopyThreads) d4[i] = __builtin_nontemporal_load(s4 + i);
    } else if constexpr (kUnit == 2) {
        const size_t n = block_bytes / 2;
        const uint16_t* s2 = reinterpret_cast<const uint16_t*>(s);
        uint16_t* d2 = reinterpret_cast<uint16_t*>(d);
        for (size_t i = threadIdx.x; i < n; i += kCopyThreads) d2[i] = s2[i];
    } else {
        for (size_t i = threadIdx.x; i < block_bytes; i += kCopyThreads) d[i] = s[i];
    }
}

// Large chunks over an 8-bit pool (dequant_blocks below): one workgroup per
// (logical block i, sequence s). The block's n_kv * B rows of head_dim
// codes (head_dim 128: 8 threads per row, 16 codes each) become bf16 values
// scale x code (the row's scale, fp32 product rounded to bf16) at staging
// block s * maxb + i, which the compact table names; -1 where the sequence
// has no block i (past its length, or a length out of range) or its table
// entry lies outside the pool.
//
// With the chunk's append fused in (FUSED, a.k_new set: the chunk step), the
// rows of the chunk's own tokens (positions seq_lens[s] - C_s ..) are not
// read from the pool: their bf16 values come from the new rows, are
// quantised exactly as kv_append_q8 does (the row's absmax over 8 threads,
// s = max(absmax, 1e-8) / 127, code = clamp(rint(x / s), -127, 127)), and
// the codes and s go to the pool while bf16(s x code) goes to the staging
// block - the values the separate append followed by this expansion gives.
// Rows past the sequence's end are not staged (the chunk kernel never reads
// them). A sequence the chunk pass rejects gets no append (its rows are NaN).
template <bool FUSED>
__global__ __launch_bounds__(kCopyThreads) void dequant_blocks_kernel(AttnArgs a, uint16_t* __restrict__ ko,
                                                                      uint16_t* __restrict__ vo,
                                                                      int32_t* __restrict__ to, int maxb) {
    constexpr int kD = 128;
    const int i = blockIdx.x;
    const int s = blockIdx.y;
    const int B = a.block_size;
    const int L = a.seq_lens[s];
    const int nb = seq_len_ok(L, 1, a.max_seq_len, a.table_stride * B) ? (L + B - 1) / B : 0;
    const size_t cb = static_cast<size_t>(s) * maxb + i;
    int id = -1;
    if (i < nb) {
        id = a.table[static_cast<size_t>(s) * a.table_stride + i];
        if (id < 0 || id >= a.num_blocks) id = -1;
    }
    if (threadIdx.x == 0) to[cb] = id < 0 ? -1 : static_cast<int32_t>(cb);
    if (id < 0) return;
    const int rows = a.n_kv * B;
    const int c = threadIdx.x & 7;
    if constexpr (FUSED) {
        const int qs = a.q_start[s];
        const int C = a.q_start[s + 1] - qs;
        const int P = L - C;                      // first new position
        if (seq_len_ok(L, C, a.max_seq_len, a.table_stride * B) && B * i + B > P) {
            // a block holding some of the chunk's tokens: slots below tp are
            // cached keys, tp .. tl - 1 new ones (past tl: past the sequence,
            // never read), eight threads (16 values each) per row
            const int tp = min(max(P - B * i, 0), B);
            const int tl = min(L - B * i, B);
            auto row_of = [&](int k, int base, int cnt) { return (k / cnt) * B + base + k % cnt; };
            constexpr int kStride = kCopyThreads / 8;
            constexpr int kUnroll = 4;
            const int n_c = a.n_kv * tp;
            for (int k0 = threadIdx.x >> 3; k0 < n_c; k0 += kUnroll * kStride) {
                u32x4 kc[kUnroll], vc[kUnroll];
                float ks[kUnroll], vs[kUnroll];
#pragma unroll
                for (int j = 0; j < kUnroll; ++j) {
                    const size_t src = static_cast<size_t>(id) * rows + row_of(min(k0 + j * kStride, n_c - 1), 0, tp);
                    kc[j] = *reinterpret_cast<const u32x4*>(static_cast<const int8_t*>(a.k_cache) + src * kD + 16 * c);
                    vc[j] = *reinterpret_cast<const u32x4*>(static_cast<const int8_t*>(a.v_cache) + src * kD + 16 * c);
                    ks[j] = a.k_scale[src];
                    vs[j] = a.v_scale[src];
                }
#pragma unroll
                for (int j = 0; j < kUnroll; ++j) {
                    const size_t dst = cb * rows + row_of(min(k0 + j * kStride, n_c - 1), 0, tp);
                    u32x4 kb[2], vb[2];
#pragma unroll
                    for (int w = 0; w < 4; ++w)
#pragma unroll
                        for (int e = 0; e < 2; ++e) {
                            const int sh = 16 * e;
                            kb[w >> 1][2 * (w & 1) + e] =
                                pack2_bf16(ks[j] * static_cast<float>(static_cast<int8_t>(kc[j][w] >> sh)),
                                           ks[j] * static_cast<float>(static_cast<int8_t>(kc[j][w] >> (sh + 8))));
                            vb[w >> 1][2 * (w & 1) + e] =
                                pack2_bf16(vs[j] * static_cast<float>(static_cast<int8_t>(vc[j][w] >> sh)),
                                           vs[j] * static_cast<float>(static_cast<int8_t>(vc[j][w] >> (sh + 8))));
                        }
                    u32x4* kd = reinterpret_cast<u32x4*>(ko + dst * kD + 16 * c);
                    u32x4* vd = reinterpret_cast<u32x4*>(vo + dst * kD + 16 * c);
                    kd[0] = kb[0];
                    kd[1] = kb[1];
                    vd[0] = vb[0];
                    vd[1] = vb[1];
                }
            }
            const int n_n = a.n_kv * (tl - tp);
            for (int k0 = threadIdx.x >> 3; k0 < n_n; k0 += kUnroll * kStride) {
                // every new row's values first (past the end: the last row
                // again, the same bytes stored twice)
                u32x4 x[kUnroll][2][2];
#pragma unroll
                for (int j = 0; j < kUnroll; ++j) {
                    const int k = min(k0 + j * kStride, n_n - 1);
                    const int h = k / (tl - tp);
                    const int key = B * i + tp + k % (tl - tp);
                    const size_t nr = (static_cast<size_t>(qs) + (key - P)) * a.n_kv + h;   // its new row
                    const u32x4* kn = reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(a.k_new) + nr * kD +
                                                                     16 * c);
                    const u32x4* vn = reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(a.v_new) + nr * kD +
                                                                     16 * c);
                    x[j][0][0] = kn[0];
                    x[j][0][1] = kn[1];
                    x[j][1][0] = vn[0];
                    x[j][1][1] = vn[1];
                }
#pragma unroll
                for (int j = 0; j < kUnroll; ++j) {
                    const int r = row_of(min(k0 + j * kStride, n_n - 1), tp, tl - tp);
                    const size_t src = static_cast<size_t>(id) * rows + r;
                    const size_t dst = cb * rows + r;
#pragma unroll
                    for (int kv = 0; kv < 2; ++kv) {
                        float f[16];
#pragma unroll
                        for (int e = 0; e < 8; ++e) {
                            const uint32_t w = x[j][kv][e >> 2][e & 3];
                            f[2 * e] = __uint_as_float(w << 16);
                            f[2 * e + 1] = __uint_as_float(w & 0xffff0000u);
                        }
                        float amax = 0.0f;
#pragma unroll
                        for (int e = 0; e < 16; ++e) amax = fmaxf(amax, fabsf(f[e]));
#pragma unroll
                        for (int o = 1; o < 8; o <<= 1) amax = fmaxf(amax, __shfl_xor(amax, o, kWave));
                        const float sc = fmaxf(amax, 1e-8f) / 127.0f;
                        u32x4 codes = {0u, 0u, 0u, 0u};
                        u32x4 st[2];
#pragma unroll
                        for (int e = 0; e < 16; ++e) {
                            f[e] = fminf(fmaxf(rintf(f[e] / sc), -127.0f), 127.0f);
                            codes[e >> 2] |= (static_cast<uint32_t>(static_cast<int>(f[e])) & 0xffu) << (8 * (e & 3));
                        }
#pragma unroll
                        for (int e = 0; e < 8; ++e) st[e >> 2][e & 3] = pack2_bf16(sc * f[2 * e], sc * f[2 * e + 1]);
                        int8_t* pc = static_cast<int8_t*>(kv ? a.v_app : a.k_app);
                        *reinterpret_cast<u32x4*>(pc + src * kD + 16 * c) = codes;
                        if (c == 0) (kv ? a.vs_app : a.ks_app)[src] = sc;
                        u32x4* sd = reinterpret_cast<u32x4*>((kv ? vo : ko) + dst * kD + 16 * c);
                        sd[0] = st[0];
                        sd[1] = st[1];
                    }
                }
            }
            return;
        }
    }
    constexpr int kStride = kCopyThreads / 8;    // rows per pass of the workgroup
    constexpr int kUnroll = 4;                   // passes whose loads are in flight together
    for (int r0 = threadIdx.x >> 3; r0 < rows; r0 += kUnroll * kStride) {
        // every load first; rows past the end re-read the last row and store
        // it again, identical bytes (no branch, so the loads stay together)
        u32x4 kc[kUnroll], vc[kUnroll];
        float ks[kUnroll], vs[kUnroll];
#pragma unroll
        for (int j = 0; j < kUnroll; ++j) {
            const size_t src = static_cast<size_t>(id) * rows + min(r0 + j * kStride, rows - 1);
            kc[j] = *reinterpret_cast<const u32x4*>(static_cast<const int8_t*>(a.k_cache) + src * kD + 16 * c);
            vc[j] = *reinterpret_cast<const u32x4*>(static_cast<const int8_t*>(a.v_cache) + src * kD + 16 * c);
            ks[j] = a.k_scale[src];
            vs[j] = a.v_scale[src];
        }
#pragma unroll
        for (int j = 0; j < kUnroll; ++j) {
            const size_t dst = cb * rows + min(r0 + j * kStride, rows - 1);
            u32x4 kb[2], vb[2];
#pragma unroll
            for (int w = 0; w < 4; ++w)
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    const int sh = 16 * e;
                    const float k0 = static_cast<float>(static_cast<int8_t>(kc[j][w] >> sh));
                    const float k1 = static_cast<float>(static_cast<int8_t>(kc[j][w] >> (sh + 8)));
                    const float v0 = static_cast<float>(static_cast<int8_t>(vc[j][w] >> sh));
                    const float v1 = static_cast<float>(static_cast<int8_t>(vc[j][w] >> (sh + 8)));
                    kb[w >> 1][2 * (w & 1) + e] = pack2_bf16(ks[j] * k0, ks[j] * k1);
                    vb[w >> 1][2 * (w & 1) + e] = pack2_bf16(vs[j] * v0, vs[j] * v1);
                }
            u32x4* kd = reinterpret_cast<u32x4*>(ko + dst * kD + 16 * c);
            u32x4* vd = reinterpret_cast<u32x4*>(vo + dst * kD + 16 * c);
            kd[0] = kb[0];
            kd[1] = kb[1];
            vd[0] = vb[0];
            vd[1] = vb[1];
        }
    }
}

}  // namespace

hipError_t launch_copy_blocks(void* k_cache, void* v_cache, const int32_t* src_ids, const int32_t* dst_ids,
                              int n, int num_blocks, size_t block_bytes, hipStream_t stream) {
    const dim3 grid(n, 2);
    const uintptr_t addr = reinterpret_cast<uintptr_t>(k_cache) | reinterpret_cast<uintptr_t>(v_cache);
    char* k = static_cast<char*>(k_cache);
    char* v = static_cast<char*>(v_cache);
    if (block_bytes % 16 == 0 && (addr & 15) == 0)
        hipLaunchKernelGGL(copy_blocks_kernel<16>, grid, dim3(kCopyThreads), 0, stream, k, v, src_ids, dst_ids,
                           num_blocks, block_bytes);
    else if (block_bytes % 2 == 0 && (addr & 1) == 0)
        hipLaunchKernelGGL(copy_blocks_kernel<2>, grid, dim3(kCopyThreads), 0, stream, k, v, src_ids, dst_ids,
                           num_blocks, block_bytes);
    else
        hipLaunchKernelGGL(copy_blocks_kernel<1>, grid, dim3(kCopyThreads), 0, stream, k, v, src_ids, dst_ids,
                           num_blocks, block_bytes);
    return hipGetLastError();
}

hipError_t launch_dequant_blocks(const AttnArgs& a, uint16_t* k_out, uint16_t* v_out, int32_t* table_out, int maxb,
                                 hipStream_t stream) {
    if (a.k_new)
        hipLaunchKernelGGL(dequant_blocks_kernel<true>, dim3(maxb, a.num_seqs), dim3(kCopyThreads), 0, stream, a,
                           k_out, v_out, table_out, maxb);
    else
        hipLaunchKernelGGL(dequant_blocks_kernel<false>, dim3(maxb, a.num_seqs), dim3(kCopyThreads), 0, stream, a,
                           k_out, v_out, table_out, maxb);
    return hipGetLastError();
}

}  // namespace pkv
