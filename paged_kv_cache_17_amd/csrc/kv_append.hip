// kv_append: scatter new tokens' K/V into the block pool through the table.
//
// Lab page (Inference Engineering), KVPool.write: the token at position p
// of a sequence is stored in slot p % B of block table[p / B], for every kv
// head. One thread moves one UNIT-byte piece of one (token, kv head) row,
// so consecutive threads write consecutive bytes of a pool slot.
#include "device_common.h"
#include "kernels.h"

namespace pkv {
namespace {

typedef uint32_t piece_u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t piece_u32x2 __attribute__((ext_vector_type(2)));
template <int UNIT> struct Piece;
template <> struct Piece<16> { using T = piece_u32x4; };
template <> struct Piece<8> { using T = piece_u32x2; };
template <> struct Piece<4> { using T = uint32_t; };
template <> struct Piece<2> { using T = uint16_t; };

// Sequences whose prefix array fits this many entries have it staged in LDS
// once per workgroup, so the per-thread search for a token's sequence does
// not chain global loads. The staging array is dynamic LDS of exactly
// num_seqs + 1 entries, so a small batch does not cap the workgroups a CU
// holds (a fixed 16 KiB array allowed ten).
constexpr int kStagedSeqs = 4096;
__host__ __device__ constexpr size_t staged_bytes(int num_seqs) {
    return num_seqs <= kStagedSeqs ? static_cast<size_t>(num_seqs + 1) * sizeof(int) : 0;
}

// Position of sequence s's first new token: start_pos[s], or (chunk step,
// start_pos null) the last C_s of its seq_lens[s] keys; -1 for a sequence
// whose length the chunk pass rejects (it gets no append).
__device__ __forceinline__ int first_new_pos(const int32_t* start_pos, const int32_t* starts, int s,
                                             const int32_t* seq_lens, int max_seq_len, int capacity) {
    if (start_pos) return start_pos[s];
    const int C = starts[s + 1] - starts[s];
    const int L = seq_lens[s];
    return seq_len_ok(L, C, max_seq_len, capacity) ? L - C : -1;
}

template <int UNIT>
__global__ __launch_bounds__(256) void kv_append_kernel(
    char* __restrict__ kc, char* __restrict__ vc,
    const char* __restrict__ kn, const char* __restrict__ vn,
    const int32_t* __restrict__ table, int table_stride,
    const int32_t* __restrict__ start_pos, const int32_t* __restrict__ new_start,
    int num_seqs, int total_new, int num_blocks, int n_kv, int row_bytes, int bs,
    const int32_t* __restrict__ seq_lens, int max_seq_len) {
    using P = typename Piece<UNIT>::T;
    extern __shared__ int s_start[];
    // The piece this thread moves is requested first: its address depends on
    // the thread's index alone, so its round trip overlaps the staging and
    // the sequence's lookups (a thread past the end reads the last piece).
    const int units = row_bytes / UNIT;
    const long long total = static_cast<long long>(total_new) * n_kv * units;
    const long long idx = static_cast<long long>(blockIdx.x) * blockDim.x + threadIdx.x;
    const long long ic = idx < total ? idx : total - 1;
    const int u = static_cast<int>(ic % units);
    const long long th = ic / units;
    const int h = static_cast<int>(th % n_kv);
    const int t = static_cast<int>(th / n_kv);
    const size_t src = (static_cast<size_t>(t) * n_kv + h) * row_bytes + static_cast<size_t>(u) * UNIT;
    const P kp = *reinterpret_cast<const P*>(kn + src);
    const P vp = *reinterpret_cast<const P*>(vn + src);
    const bool staged = num_seqs <= kStagedSeqs;
    if (staged)
        for (int i = threadIdx.x; i <= num_seqs; i += blockDim.x) s_start[i] = new_start[i];
    __syncthreads();
    if (idx >= total) return;
    const int32_t* starts = staged ? s_start : new_start;
    const int s = seq_of_row(starts, num_seqs, t);
    const int first = first_new_pos(start_pos, starts, s, seq_lens, max_seq_len, table_stride * bs);
    if (first < 0) return;
    const int pos = first + (t - starts[s]);
    if (pos < 0 || pos / bs >= table_stride) return;
    const int blk = table[static_cast<size_t>(s) * table_stride + pos / bs];
    if (blk < 0 || blk >= num_blocks) return;   // unmapped slot: nothing is written
    const size_t dst = ((static_cast<size_t>(blk) * n_kv + h) * bs + pos % bs) * row_bytes +
                       static_cast<size_t>(u) * UNIT;
    *reinterpret_cast<P*>(kc + dst) = kp;
    *reinterpret_cast<P*>(vc + dst) = vp;
}

template <int UNIT>
hipError_t launch_unit(void* kc, void* vc, const void* kn, const void* vn, const int32_t* table,
                       int table_stride, const int32_t* start_pos, const int32_t* new_start,
                       int num_seqs, int total_new, int num_blocks, int n_kv, int row_bytes, int bs,
                       hipStream_t stream, const int32_t* seq_lens = nullptr, int max_seq_len = 0) {
    const long long work = static_cast<long long>(total_new) * n_kv * (row_bytes / UNIT);
    const unsigned grid = static_cast<unsigned>((work + 255) / 256);
    hipLaunchKernelGGL(kv_append_kernel<UNIT>, dim3(grid), dim3(256), staged_bytes(num_seqs), stream,
                       static_cast<char*>(kc), static_cast<char*>(vc),
                       static_cast<const char*>(kn), static_cast<const char*>(vn), table,
                       table_stride, start_pos, new_start, num_seqs, total_new, num_blocks, n_kv,
                       row_bytes, bs, seq_lens, max_seq_len);
    return hipGetLastError();
}

// Quantising append: one wave per (new token, kv head) row of K and of V.
// Symmetric absmax quantisation (chapter 5 section 4, group-wise: one scale
// per group of consecutive elements, here the head_dim values of one token
// and kv head): s = max(max_i |x_i|, 1e-8) / 127, code_i =
// clamp(rint(x_i / s), -127, 127) (ties to even), all in fp32 with
// correctly rounded division; the pool keeps the 8-bit codes and s.
template <typename TIn>
__global__ __launch_bounds__(256) void kv_append_q8_kernel(
    int8_t* __restrict__ kc, int8_t* __restrict__ vc, float* __restrict__ ks, float* __restrict__ vs,
    const TIn* __restrict__ kn, const TIn* __restrict__ vn, const int32_t* __restrict__ table, int table_stride,
    const int32_t* __restrict__ start_pos, const int32_t* __restrict__ new_start, int num_seqs, int total_new,
    int num_blocks, int n_kv, int d, int bs, const int32_t* __restrict__ seq_lens, int max_seq_len) {
    extern __shared__ int s_start[];
    const bool staged = num_seqs <= kStagedSeqs;
    if (staged)
        for (int i = threadIdx.x; i <= num_seqs; i += blockDim.x) s_start[i] = new_start[i];
    __syncthreads();
    const int lane = threadIdx.x & (kWave - 1);
    const long long row = static_cast<long long>(blockIdx.x) * (blockDim.x / kWave) + threadIdx.x / kWave;
    if (row >= 2LL * total_new * n_kv) return;                // whole wave exits together
    const bool is_v = row & 1;
    const long long th = row >> 1;
    const int h = static_cast<int>(th % n_kv);
    const int t = static_cast<int>(th / n_kv);
    const int32_t* starts = staged ? s_start : new_start;
    const int s = seq_of_row(starts, num_seqs, t);
    const int first = first_new_pos(start_pos, starts, s, seq_lens, max_seq_len, table_stride * bs);
    if (first < 0) return;
    const int pos = first + (t - starts[s]);
    if (pos < 0 || pos / bs >= table_stride) return;
    const int blk = table[static_cast<size_t>(s) * table_stride + pos / bs];
    if (blk < 0 || blk >= num_blocks) return;                 // unmapped slot: nothing is written
    const TIn* src = (is_v ? vn : kn) + (static_cast<size_t>(t) * n_kv + h) * d;
    float amax = 0.0f;
    for (int e = lane; e < d; e += kWave) amax = fmaxf(amax, fabsf(Elem<TIn>::load(src + e)));
    amax = wave_max(amax);
    const float scale = fmaxf(amax, 1e-8f) / 127.0f;
    const size_t slot = (static_cast<size_t>(blk) * n_kv + h) * bs + pos % bs;
    int8_t* dst = (is_v ? vc : kc) + slot * d;
    for (int e = lane; e < d; e += kWave) {
        const float c = fminf(fmaxf(rintf(Elem<TIn>::load(src + e) / scale), -127.0f), 127.0f);
        dst[e] = static_cast<int8_t>(c);
    }
    if (lane == 0) (is_v ? vs : ks)[slot] = scale;
}

// The same quantising append for bf16 rows of 128 values: 16 lanes per
// (new token, kv head), each holding 8 values of its K row and 8 of its V
// row in registers, so the row is read once, the max is a 16-lane
// reduction and the codes leave as one 8-byte store per lane. The row's
// values are requested before the staging and the lookups (a lane past the
// end reads the last row); the arithmetic is kv_append_q8_kernel's.
__global__ __launch_bounds__(256) void kv_append_q8_d128_kernel(
    int8_t* __restrict__ kc, int8_t* __restrict__ vc, float* __restrict__ ks, float* __restrict__ vs,
    const uint16_t* __restrict__ kn, const uint16_t* __restrict__ vn, const int32_t* __restrict__ table,
    int table_stride, const int32_t* __restrict__ start_pos, const int32_t* __restrict__ new_start, int num_seqs,
    int total_new, int num_blocks, int n_kv, int bs, const int32_t* __restrict__ seq_lens, int max_seq_len) {
    constexpr int kD = 128, kLanes = 16;
    extern __shared__ int s_start[];
    const int c = threadIdx.x & (kLanes - 1);
    const long long total = static_cast<long long>(total_new) * n_kv;
    const long long th = static_cast<long long>(blockIdx.x) * (blockDim.x / kLanes) + threadIdx.x / kLanes;
    const long long tc = th < total ? th : total - 1;
    const size_t src = static_cast<size_t>(tc) * kD + 8 * c;
    const piece_u32x4 kx = *reinterpret_cast<const piece_u32x4*>(kn + src);
    const piece_u32x4 vx = *reinterpret_cast<const piece_u32x4*>(vn + src);
    const bool staged = num_seqs <= kStagedSeqs;
    if (staged)
        for (int i = threadIdx.x; i <= num_seqs; i += blockDim.x) s_start[i] = new_start[i];
    __syncthreads();
    if (th >= total) return;                                   // the 16 lanes of a row exit together
    const int h = static_cast<int>(tc % n_kv);
    const int t = static_cast<int>(tc / n_kv);
    const int32_t* starts = staged ? s_start : new_start;
    const int s = seq_of_row(starts, num_seqs, t);
    const int first = first_new_pos(start_pos, starts, s, seq_lens, max_seq_len, table_stride * bs);
    if (first < 0) return;
    const int pos = first + (t - starts[s]);
    if (pos < 0 || pos / bs >= table_stride) return;
    const int blk = table[static_cast<size_t>(s) * table_stride + pos / bs];
    if (blk < 0 || blk >= num_blocks) return;                 // unmapped slot: nothing is written
    const size_t slot = (static_cast<size_t>(blk) * n_kv + h) * bs + pos % bs;
    float f[2][8], amax[2] = {0.0f, 0.0f};
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        f[0][2 * w] = __uint_as_float(kx[w] << 16);
        f[0][2 * w + 1] = __uint_as_float(kx[w] & 0xffff0000u);
        f[1][2 * w] = __uint_as_float(vx[w] << 16);
        f[1][2 * w + 1] = __uint_as_float(vx[w] & 0xffff0000u);
    }
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
        for (int e = 0; e < 8; ++e) amax[r] = fmaxf(amax[r], fabsf(f[r][e]));
#pragma unroll
    for (int o = 1; o < kLanes; o <<= 1) {                      // K and V reductions interleaved
        const float mk = __shfl_xor(amax[0], o, kWave);
        const float mv = __shfl_xor(amax[1], o, kWave);
        amax[0] = fmaxf(amax[0], mk);
        amax[1] = fmaxf(amax[1], mv);
    }
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        const float scale = fmaxf(amax[r], 1e-8f) / 127.0f;
        piece_u32x2 packed = {0u, 0u};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float q = fminf(fmaxf(rintf(f[r][e] / scale), -127.0f), 127.0f);
            packed[e >> 2] |= (static_cast<uint32_t>(static_cast<int>(q)) & 0xffu) << (8 * (e & 3));
        }
        *reinterpret_cast<piece_u32x2*>((r ? vc : kc) + slot * kD + 8 * c) = packed;
        if (c == 0) (r ? vs : ks)[slot] = scale;
    }
}

// The decode step's append: one token per sequence, at position
// seq_lens[s] - 1, rows of 16-byte units (bf16, head_dim 128, block_size 16:
// 16 units of K and of V per (sequence, kv head)). A sequence whose length
// the decode rejects, or whose table entry there is outside the pool, gets
// no write - the same tokens the decode pass with the append folded in
// writes.
__global__ __launch_bounds__(256) void kv_append_last_kernel(uint4* __restrict__ kc, uint4* __restrict__ vc,
                                                             const uint4* __restrict__ kn,
                                                             const uint4* __restrict__ vn,
                                                             const int32_t* __restrict__ table, int table_stride,
                                                             const int32_t* __restrict__ seq_lens, int num_seqs,
                                                             int max_seq_len, int num_blocks, int n_kv) {
    constexpr int kUnits = 16, kBS = 16;
    const long long idx = static_cast<long long>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (idx >= static_cast<long long>(num_seqs) * n_kv * kUnits) return;
    const int u = static_cast<int>(idx % kUnits);
    const long long th = idx / kUnits;
    const int h = static_cast<int>(th % n_kv);
    const int s = static_cast<int>(th / n_kv);
    const int L = seq_lens[s];
    if (!seq_len_ok(L, 1, max_seq_len, table_stride * kBS)) return;
    const int pos = L - 1;
    const int blk = table[static_cast<size_t>(s) * table_stride + pos / kBS];
    if (blk < 0 || blk >= num_blocks) return;
    const size_t dst = ((static_cast<size_t>(blk) * n_kv + h) * kBS + pos % kBS) * kUnits + u;
    const size_t src = static_cast<size_t>(th) * kUnits + u;
    kc[dst] = kn[src];
    vc[dst] = vn[src];
}

// The decode step's append into an 8-bit pool: one token per sequence at
// position seq_lens[s] - 1, bf16 input, quantised exactly as
// kv_append_q8_kernel does (head_dim 128, block_size 16): 16 lanes per
// (sequence, kv head), each holding 8 values of its K row and 8 of its V row
// (as kv_append_q8_d128_kernel). The same tokens as the decode pass with
// the append folded in.
__global__ __launch_bounds__(256) void kv_append_q8_last_kernel(int8_t* __restrict__ kc, int8_t* __restrict__ vc,
                                                                float* __restrict__ ks, float* __restrict__ vs,
                                                                const uint16_t* __restrict__ kn,
                                                                const uint16_t* __restrict__ vn,
                                                                const int32_t* __restrict__ table, int table_stride,
                                                                const int32_t* __restrict__ seq_lens, int num_seqs,
                                                                int max_seq_len, int num_blocks, int n_kv) {
    constexpr int kD = 128, kBS = 16, kLanes = 16;
    const int c = threadIdx.x & (kLanes - 1);
    const long long total = static_cast<long long>(num_seqs) * n_kv;
    const long long th = static_cast<long long>(blockIdx.x) * (blockDim.x / kLanes) + threadIdx.x / kLanes;
    if (th >= total) return;                                  // the 16 lanes of a row exit together
    const size_t src = static_cast<size_t>(th) * kD + 8 * c;
    const piece_u32x4 kx = *reinterpret_cast<const piece_u32x4*>(kn + src);
    const piece_u32x4 vx = *reinterpret_cast<const piece_u32x4*>(vn + src);
    const int h = static_cast<int>(th % n_kv);
    const int s = static_cast<int>(th / n_kv);
    const int L = seq_lens[s];
    if (!seq_len_ok(L, 1, max_seq_len, table_stride * kBS)) return;
    const int pos = L - 1;
    const int blk = table[static_cast<size_t>(s) * table_stride + pos / kBS];
    if (blk < 0 || blk >= num_blocks) return;
    const size_t slot = (static_cast<size_t>(blk) * n_kv + h) * kBS + pos % kBS;
    float f[2][8], amax[2] = {0.0f, 0.0f};
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        f[0][2 * w] = __uint_as_float(kx[w] << 16);
        f[0][2 * w + 1] = __uint_as_float(kx[w] & 0xffff0000u);
        f[1][2 * w] = __uint_as_float(vx[w] << 16);
        f[1][2 * w + 1] = __uint_as_float(vx[w] & 0xffff0000u);
    }
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
        for (int e = 0; e < 8; ++e) amax[r] = fmaxf(amax[r], fabsf(f[r][e]));
#pragma unroll
    for (int o = 1; o < kLanes; o <<= 1) {
        const float mk = __shfl_xor(amax[0], o, kWave);
        const float mv = __shfl_xor(amax[1], o, kWave);
        amax[0] = fmaxf(amax[0], mk);
        amax[1] = fmaxf(amax[1], mv);
    }
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        const float scale = fmaxf(amax[r], 1e-8f) / 127.0f;
        piece_u32x2 packed = {0u, 0u};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float q = fminf(fmaxf(rintf(f[r][e] / scale), -127.0f), 127.0f);
            packed[e >> 2] |= (static_cast<uint32_t>(static_cast<int>(q)) & 0xffu) << (8 * (e & 3));
        }
        *reinterpret_cast<piece_u32x2*>((r ? vc : kc) + slot * kD + 8 * c) = packed;
        if (c == 0) (r ? vs : ks)[slot] = scale;
    }
}

}  // namespace

hipError_t launch_kv_append_q8(int8_t* k_cache, int8_t* v_cache, float* k_scale, float* v_scale, const void* k_new,
                               const void* v_new, bool bf16_in, const int32_t* table, int table_stride,
                               const int32_t* start_pos, const int32_t* new_start, int num_seqs, int total_new,
                               int num_blocks, int n_kv, int head_dim, int block_size, hipStream_t stream,
                               const int32_t* seq_lens, int max_seq_len) {
    const long long rows = 2LL * total_new * n_kv;
    const unsigned grid = static_cast<unsigned>((rows + 3) / 4);     // four waves per workgroup
    const auto a16 = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; };
    const size_t lds = staged_bytes(num_seqs);
    if (bf16_in && head_dim == 128 && a16(k_new) && a16(v_new) && a16(k_cache) && a16(v_cache)) {
        const long long pairs = static_cast<long long>(total_new) * n_kv;   // 16 per workgroup
        hipLaunchKernelGGL(kv_append_q8_d128_kernel, dim3(static_cast<unsigned>((pairs + 15) / 16)), dim3(256), lds,
                           stream, k_cache, v_cache, k_scale, v_scale, static_cast<const uint16_t*>(k_new),
                           static_cast<const uint16_t*>(v_new), table, table_stride, start_pos, new_start, num_seqs,
                           total_new, num_blocks, n_kv, block_size, seq_lens, max_seq_len);
    } else if (bf16_in)
        hipLaunchKernelGGL(kv_append_q8_kernel<uint16_t>, dim3(grid), dim3(256), lds, stream, k_cache, v_cache,
                           k_scale, v_scale, static_cast<const uint16_t*>(k_new), static_cast<const uint16_t*>(v_new),
                           table, table_stride, start_pos, new_start, num_seqs, total_new, num_blocks, n_kv,
                           head_dim, block_size, seq_lens, max_seq_len);
    else
        hipLaunchKernelGGL(kv_append_q8_kernel<float>, dim3(grid), dim3(256), lds, stream, k_cache, v_cache, k_scale,
                           v_scale, static_cast<const float*>(k_new), static_cast<const float*>(v_new), table,
                           table_stride, start_pos, new_start, num_seqs, total_new, num_blocks, n_kv, head_dim,
                           block_size, seq_lens, max_seq_len);
    return hipGetLastError();
}

hipError_t launch_kv_append(void* k_cache, void* v_cache, const void* k_new, const void* v_new,
                            const int32_t* table, int table_stride, const int32_t* start_pos,
                            const int32_t* new_start, int num_seqs, int total_new, int num_blocks,
                            int n_kv, int row_bytes, int block_size, hipStream_t stream,
                            const int32_t* seq_lens, int max_seq_len) {
    const uintptr_t align = reinterpret_cast<uintptr_t>(k_cache) | reinterpret_cast<uintptr_t>(v_cache) |
                            reinterpret_cast<uintptr_t>(k_new) | reinterpret_cast<uintptr_t>(v_new);
#define PKV_APPEND(U)                                                                          \
    return launch_unit<U>(k_cache, v_cache, k_new, v_new, table, table_stride, start_pos,      \
                          new_start, num_seqs, total_new, num_blocks, n_kv, row_bytes,         \
                          block_size, stream, seq_lens, max_seq_len)
    if (row_bytes % 16 == 0 && align % 16 == 0) PKV_APPEND(16);
    if (row_bytes % 8 == 0 && align % 8 == 0) PKV_APPEND(8);
    if (row_bytes % 4 == 0 && align % 4 == 0) PKV_APPEND(4);
    PKV_APPEND(2);
#undef PKV_APPEND
}

hipError_t launch_kv_append_last(void* k_cache, void* v_cache, const void* k_new, const void* v_new,
                                 const int32_t* table, int table_stride, const int32_t* seq_lens, int num_seqs,
                                 int max_seq_len, int num_blocks, int n_kv, hipStream_t stream) {
    const long long work = static_cast<long long>(num_seqs) * n_kv * 16;
    hipLaunchKernelGGL(kv_append_last_kernel, dim3(static_cast<unsigned>((work + 255) / 256)), dim3(256), 0, stream,
                       static_cast<uint4*>(k_cache), static_cast<uint4*>(v_cache), static_cast<const uint4*>(k_new),
                       static_cast<const uint4*>(v_new), table, table_stride, seq_lens, num_seqs, max_seq_len,
                       num_blocks, n_kv);
    return hipGetLastError();
}

hipError_t launch_kv_append_q8_last(int8_t* k_codes, int8_t* v_codes, float* k_scale, float* v_scale,
                                    const void* k_new, const void* v_new, const int32_t* table, int table_stride,
                                    const int32_t* seq_lens, int num_seqs, int max_seq_len, int num_blocks, int n_kv,
                                    hipStream_t stream) {
    const long long pairs = static_cast<long long>(num_seqs) * n_kv;   // 16 per workgroup
    hipLaunchKernelGGL(kv_append_q8_last_kernel, dim3(static_cast<unsigned>((pairs + 15) / 16)), dim3(256), 0, stream,
                       k_codes, v_codes, k_scale, v_scale, static_cast<const uint16_t*>(k_new),
                       static_cast<const uint16_t*>(v_new), table, table_stride, seq_lens, num_seqs, max_seq_len,
                       num_blocks, n_kv);
    return hipGetLastError();
}

}  // namespace pkv
