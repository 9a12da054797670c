// C ABI entry points: argument validation, workspace layout and dispatch.
//
// Every check runs before the first launch, so an error return leaves the
// caller's buffers untouched. Kernels run asynchronously on the caller's
// stream.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "kernels.h"
#include "pagedkv.h"

namespace {

constexpr int kMaxHeadDim = 512;
constexpr int kMaxSplitTokens = 8192;
constexpr size_t kAlign = 256;

hipEvent_t g_prof_before = nullptr;
hipEvent_t g_prof_after = nullptr;

// The profiling pair, when both events are set: recorded by the timed
// kernel's own dispatch.
pkv::KernelEvents profile_events() {
    pkv::KernelEvents ev;
    if (g_prof_before && g_prof_after) {
        ev.start = g_prof_before;
        ev.stop = g_prof_after;
    }
    return ev;
}

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

int elem_bytes(int dtype) {
    if (dtype == PKV_F32) return 4;
    if (dtype == PKV_BF16) return 2;
    return 0;
}

// Auto split size: the largest of 1024/512/256 tokens (rounded to whole
// blocks) that still gives the launch enough (row, kv head, range)
// workgroups to cover the chip several times over.
int auto_split(int rows, int n_kv, int block_size, int max_seq_len) {
    const long long pairs = static_cast<long long>(rows) * n_kv;
    int chosen = 0;
    for (int cand : {1024, 512, 256}) {
        int sp = (cand + block_size - 1) / block_size * block_size;
        if (sp > kMaxSplitTokens) sp = kMaxSplitTokens / block_size * block_size;
        if (sp < block_size) sp = block_size;
        chosen = sp;
        const long long ranges = (max_seq_len + sp - 1) / sp;
        if (pairs * ranges >= 2048) break;
    }
    return chosen;
}

int resolve_split(int rows, int n_kv, int block_size, int max_seq_len, int requested, int* out) {
    if (requested < 0) return PKV_ERR_INVALID_ARGUMENT;
    if (requested == 0) {
        *out = auto_split(rows, n_kv, block_size, max_seq_len);
        return PKV_OK;
    }
    if (requested % block_size || requested > kMaxSplitTokens) return PKV_ERR_INVALID_ARGUMENT;
    *out = requested;
    return PKV_OK;
}

struct Layout {
    size_t ml_bytes;
    size_t o_offset;
    size_t prefix_offset;
    size_t total;
};

// Large chunks over an 8-bit pool: bf16 staging copies of the sequences'
// K and V blocks (maxb = ceil(max_seq_len / block_size) per sequence) and
// their compact table.
struct StagingLayout {
    int maxb;
    size_t v_offset;
    size_t table_offset;
    size_t total;
};
StagingLayout staging_layout(int num_seqs, int max_seq_len, int n_kv, int head_dim, int block_size) {
    StagingLayout l{};
    l.maxb = (max_seq_len + block_size - 1) / block_size;
    const size_t blocks = static_cast<size_t>(num_seqs) * l.maxb;
    const size_t pool = align_up(blocks * n_kv * block_size * head_dim * sizeof(uint16_t));
    l.v_offset = pool;
    l.table_offset = 2 * pool;
    l.total = 2 * pool + align_up(blocks * sizeof(int32_t));
    return l;
}

Layout ws_layout(int rows, int n_q, int head_dim, int max_splits) {
    const size_t parts = static_cast<size_t>(rows) * n_q * max_splits;
    Layout w;
    w.ml_bytes = parts * sizeof(pkv::PartialML);
    w.o_offset = align_up(w.ml_bytes);
    w.prefix_offset = align_up(w.o_offset + parts * head_dim * sizeof(float));
    w.total = w.prefix_offset;
    return w;
}

// Balanced pass: W + S*n_kv partial slots of `rows` rows (decode: the G
// heads; small chunks: kChunkSlotRows (query, head) rows), then the prefix.
Layout ws_layout_balanced(int num_seqs, int rows, int n_kv, int head_dim, int waves) {
    const size_t parts = (static_cast<size_t>(waves) + static_cast<size_t>(num_seqs) * n_kv) * rows;
    Layout w;
    w.ml_bytes = parts * sizeof(pkv::PartialML);
    w.o_offset = align_up(w.ml_bytes);
    w.prefix_offset = align_up(w.o_offset + parts * head_dim * sizeof(float));
    w.total = w.prefix_offset + align_up((static_cast<size_t>(num_seqs) + 1) * sizeof(int));
    return w;
}

// Grid size of the balanced pass for the current device (cached for the
// last shape asked about, per pass: bf16 decode, 8-bit decode, small chunks).
enum BalancedPass { kDecodeBf16 = 0, kDecodeInt8 = 1, kChunkBf16 = 2, kChunkInt8 = 3 };
int balanced_waves(int n_q, int n_kv, int num_seqs, BalancedPass f = kDecodeBf16) {
    static thread_local int last_dev[4] = {-1, -1, -1, -1}, last_g[4] = {}, last_s[4] = {}, last_w[4] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    const int g = n_q / n_kv;
    if (dev != last_dev[f] || g != last_g[f] || num_seqs != last_s[f]) {
        last_w[f] = f >= kChunkBf16 ? pkv::chunk_balanced_waves(n_q, n_kv, num_seqs, f == kChunkInt8)
                                    : pkv::decode_balanced_waves(n_q, n_kv, num_seqs, f == kDecodeInt8);
        last_dev[f] = dev;
        last_g[f] = g;
        last_s[f] = num_seqs;
    }
    return last_w[f];
}

int check_shape(int num_seqs, int max_seq_len, int num_blocks, int n_q, int n_kv, int head_dim,
                int block_size, int table_stride, int dtype, float scale) {
    if (num_seqs < 0 || max_seq_len < 1 || num_blocks < 1 || n_q < 1 || n_kv < 1 ||
        head_dim < 1 || block_size < 1 || table_stride < 1)
        return PKV_ERR_INVALID_ARGUMENT;
    if (n_q % n_kv) return PKV_ERR_INVALID_ARGUMENT;
    if (!elem_bytes(dtype)) return PKV_ERR_INVALID_ARGUMENT;
    if (!std::isfinite(scale)) return PKV_ERR_INVALID_ARGUMENT;
    if (head_dim > kMaxHeadDim) return PKV_ERR_UNSUPPORTED;
    return PKV_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// The workspace checks of run_attention, on their own, so that entry points
// that launch an append first can reject a bad workspace before it.
int check_workspace(const pkv::AttnArgs& a, bool balanced, const void* workspace, size_t workspace_bytes,
                    Layout* layout) {
    if (!workspace) return PKV_ERR_NULL_POINTER;
    if (reinterpret_cast<uintptr_t>(workspace) % kAlign) return PKV_ERR_INVALID_ARGUMENT;
    const Layout w = balanced ? ws_layout_balanced(a.num_seqs, a.n_q / a.n_kv, a.n_kv, a.head_dim, a.waves)
                              : ws_layout(a.num_rows, a.n_q, a.head_dim, a.max_splits);
    if (workspace_bytes < w.total) return PKV_ERR_WORKSPACE_TOO_SMALL;
    if (layout) *layout = w;
    return PKV_OK;
}

int run_attention(pkv::AttnArgs& a, void* out, float* lse, int dtype, bool decode, bool balanced,
                  void* workspace, size_t workspace_bytes, hipStream_t stream) {
    if (a.num_rows == 0) return PKV_OK;
    Layout w;
    const int rc = check_workspace(a, balanced, workspace, workspace_bytes, &w);
    if (rc != PKV_OK) return rc;
    char* ws = static_cast<char*>(workspace);
    a.ws_ml = reinterpret_cast<pkv::PartialML*>(ws);
    a.ws_o = reinterpret_cast<float*>(ws + w.o_offset);
    a.prefix = balanced ? reinterpret_cast<int*>(ws + w.prefix_offset) : nullptr;
    if (!balanced) a.waves = 0;
    const bool bf16 = dtype == PKV_BF16;
    const bool aligned = aligned16(a.q) && aligned16(a.k_cache) && aligned16(a.v_cache);

    hipError_t e;
    if (balanced) {
        e = pkv::launch_decode_balanced(a, stream, profile_events());
    } else if (decode && bf16 && aligned &&
               pkv::decode_fast_supported(a.n_q, a.n_kv, a.head_dim, a.block_size, a.split_tokens)) {
        e = pkv::launch_decode_fast(a, stream, profile_events());
    } else {
        e = pkv::launch_split_generic(a, bf16, stream);
    }
    if (e != hipSuccess) return PKV_ERR_HIP;
    e = pkv::launch_merge(a, out, lse, bf16, stream);
    return e == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

bool balanced_eligible(int dtype, int split_tokens, int num_seqs, int n_q, int n_kv, int head_dim,
                       int block_size) {
    return dtype == PKV_BF16 && split_tokens == 0 &&
           pkv::decode_balanced_supported(n_q, n_kv, head_dim, block_size, num_seqs);
}

}  // namespace

extern "C" const char* pkv_strerror(int status) {
    switch (status) {
        case PKV_OK: return "ok";
        case PKV_ERR_NULL_POINTER: return "null pointer";
        case PKV_ERR_INVALID_ARGUMENT: return "invalid argument";
        case PKV_ERR_UNSUPPORTED: return "unsupported shape or dtype";
        case PKV_ERR_OUT_OF_BLOCKS: return "out of KV blocks";
        case PKV_ERR_INVALID_FREE: return "invalid free (out of range, already free, or repeated)";
        case PKV_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
        case PKV_ERR_TABLE_FULL: return "block table row full";
        case PKV_ERR_HIP: return "HIP launch error";
        case PKV_ERR_NO_MEMORY: return "out of host memory";
        case PKV_ERR_INVALID_BLOCK: return "invalid block (out of range, not allocated, or repeated)";
        case PKV_ERR_SCRATCH_LIMIT: return "the batch needs more split-K workspace than the static scratch holds";
        default: return "unknown status";
    }
}

extern "C" int pkv_set_profile_events(void* before, void* after) {
    g_prof_before = static_cast<hipEvent_t>(before);
    g_prof_after = static_cast<hipEvent_t>(after);
    return PKV_OK;
}

extern "C" int kv_append(void* k_cache, void* v_cache, const void* k_new, const void* v_new,
                         const int32_t* block_table, int32_t table_stride,
                         const int32_t* start_pos, const int32_t* new_start,
                         int32_t num_seqs, int32_t total_new, int32_t num_blocks,
                         int32_t n_kv, int32_t head_dim, int32_t block_size, int32_t dtype,
                         void* stream) {
    if (num_seqs < 0 || total_new < 0 || num_blocks < 1 || n_kv < 1 || head_dim < 1 ||
        block_size < 1 || table_stride < 1)
        return PKV_ERR_INVALID_ARGUMENT;
    const int eb = elem_bytes(dtype);
    if (!eb) return PKV_ERR_INVALID_ARGUMENT;
    if (total_new == 0) return PKV_OK;
    if (num_seqs == 0) return PKV_ERR_INVALID_ARGUMENT;
    if (!k_cache || !v_cache || !k_new || !v_new || !block_table || !start_pos || !new_start)
        return PKV_ERR_NULL_POINTER;
    hipError_t e = pkv::launch_kv_append(k_cache, v_cache, k_new, v_new, block_table, table_stride,
                                         start_pos, new_start, num_seqs, total_new, num_blocks, n_kv,
                                         head_dim * eb, block_size, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

extern "C" int kv_copy_blocks(void* k_cache, void* v_cache, const int32_t* src_ids, const int32_t* dst_ids,
                              int32_t n, int32_t num_blocks, int32_t n_kv, int32_t head_dim,
                              int32_t block_size, int32_t dtype, void* stream) {
    if (n < 0 || num_blocks < 1 || n_kv < 1 || head_dim < 1 || block_size < 1) return PKV_ERR_INVALID_ARGUMENT;
    const int eb = elem_bytes(dtype);
    if (!eb) return PKV_ERR_INVALID_ARGUMENT;
    if (n == 0) return PKV_OK;
    if (!k_cache || !v_cache || !src_ids || !dst_ids) return PKV_ERR_NULL_POINTER;
    const size_t block_bytes = static_cast<size_t>(n_kv) * block_size * head_dim * eb;
    const hipError_t e = pkv::launch_copy_blocks(k_cache, v_cache, src_ids, dst_ids, n, num_blocks, block_bytes,
                                                 static_cast<hipStream_t>(stream));
    return e == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

extern "C" int kv_copy_blocks_q8(void* k_codes, void* v_codes, float* k_scale, float* v_scale, const int32_t* src_ids,
                                 const int32_t* dst_ids, int32_t n, int32_t num_blocks, int32_t n_kv, int32_t head_dim,
                                 int32_t block_size, void* stream) {
    if (n < 0 || num_blocks < 1 || n_kv < 1 || head_dim < 1 || block_size < 1) return PKV_ERR_INVALID_ARGUMENT;
    if (n == 0) return PKV_OK;
    if (!k_codes || !v_codes || !k_scale || !v_scale || !src_ids || !dst_ids) return PKV_ERR_NULL_POINTER;
    hipStream_t st = static_cast<hipStream_t>(stream);
    // codes: n_kv * B * head_dim bytes per block; scales: n_kv * B floats
    hipError_t e = pkv::launch_copy_blocks(k_codes, v_codes, src_ids, dst_ids, n, num_blocks,
                                           static_cast<size_t>(n_kv) * block_size * head_dim, st);
    if (e == hipSuccess)
        e = pkv::launch_copy_blocks(k_scale, v_scale, src_ids, dst_ids, n, num_blocks,
                                    static_cast<size_t>(n_kv) * block_size * sizeof(float), st);
    return e == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

extern "C" int sample_workspace_size(int32_t rows, int32_t vocab, size_t* bytes) {
    if (!bytes) return PKV_ERR_NULL_POINTER;
    if (rows < 0 || vocab < 1 || vocab > pkv::kSampleChunk * pkv::kSampleMaxCand) return PKV_ERR_INVALID_ARGUMENT;
    *bytes = pkv::sample_workspace_bytes(rows, vocab);
    return PKV_OK;
}

extern "C" int sample_tokens(int32_t* token, int32_t* kept, const float* logits, int32_t rows, int32_t vocab,
                             int64_t ld, const float* temperature, const int32_t* top_k, const float* top_p,
                             const float* u, void* workspace, size_t workspace_bytes, void* stream) {
    if (rows < 0 || vocab < 1 || ld < vocab) return PKV_ERR_INVALID_ARGUMENT;
    if (vocab > pkv::kSampleChunk * pkv::kSampleMaxCand) return PKV_ERR_INVALID_ARGUMENT;
    if (static_cast<int64_t>(rows) * pkv::sample_chunks(vocab) > INT32_MAX) return PKV_ERR_INVALID_ARGUMENT;
    if (rows == 0) return PKV_OK;
    if (!token || !logits || !temperature || !top_k || !top_p || !u || !workspace) return PKV_ERR_NULL_POINTER;
    if (workspace_bytes < pkv::sample_workspace_bytes(rows, vocab)) return PKV_ERR_WORKSPACE_TOO_SMALL;
    if (reinterpret_cast<uintptr_t>(workspace) % 8 != 0) return PKV_ERR_INVALID_ARGUMENT;
    pkv::SampleArgs a{logits, vocab, static_cast<size_t>(ld), temperature, top_k, top_p, u, token, kept,
                      static_cast<unsigned char*>(workspace), rows, pkv::sample_chunks(vocab),
                      pkv::sample_region_bytes(vocab)};
    const hipError_t e = pkv::launch_sample(a, rows, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

extern "C" int paged_attn_split_tokens(int32_t num_q_rows, int32_t n_kv, int32_t block_size,
                                       int32_t max_seq_len, int32_t requested, int32_t* out) {
    if (!out) return PKV_ERR_NULL_POINTER;
    if (num_q_rows < 0 || n_kv < 1 || block_size < 1 || max_seq_len < 1) return PKV_ERR_INVALID_ARGUMENT;
    return resolve_split(num_q_rows, n_kv, block_size, max_seq_len, requested, out);
}

extern "C" int paged_attn_workspace_size(int32_t num_q_rows, int32_t n_q, int32_t n_kv,
                                         int32_t head_dim, int32_t block_size, int32_t max_seq_len,
                                         int32_t split_tokens, size_t* bytes) {
    if (!bytes) return PKV_ERR_NULL_POINTER;
    if (num_q_rows < 0 || n_q < 1 || n_kv < 1 || head_dim < 1 || block_size < 1 || max_seq_len < 1)
        return PKV_ERR_INVALID_ARGUMENT;
    int split = 0;
    int rc = resolve_split(num_q_rows, n_kv, block_size, max_seq_len, split_tokens, &split);
    if (rc != PKV_OK) return rc;
    const int max_splits = (max_seq_len + split - 1) / split;
    size_t need = ws_layout(num_q_rows, n_q, head_dim, max_splits).total;
    if (n_q % n_kv == 0 && balanced_eligible(PKV_BF16, split_tokens, num_q_rows, n_q, n_kv, head_dim, block_size)) {
        for (BalancedPass f : {kDecodeBf16, kDecodeInt8}) {   // bf16 and 8-bit K/V (paged_attn_decode_q8)
            const int waves = balanced_waves(n_q, n_kv, num_q_rows, f);
            if (waves < 1) return PKV_ERR_HIP;
            const size_t b = ws_layout_balanced(num_q_rows, n_q / n_kv, n_kv, head_dim, waves).total;
            if (b > need) need = b;
        }
    }
    *bytes = need;
    return PKV_OK;
}

extern "C" int paged_attn_chunk_workspace_size(int32_t num_seqs, int32_t total_q, int32_t max_q_len, int32_t n_q,
                                               int32_t n_kv, int32_t head_dim, int32_t block_size,
                                               int32_t max_seq_len, int32_t split_tokens, size_t* bytes) {
    if (!bytes) return PKV_ERR_NULL_POINTER;
    if (num_seqs < 0 || max_q_len < 0) return PKV_ERR_INVALID_ARGUMENT;
    int rc = paged_attn_workspace_size(total_q, n_q, n_kv, head_dim, block_size, max_seq_len, split_tokens, bytes);
    if (rc != PKV_OK) return rc;
    if (split_tokens == 0 && n_q % n_kv == 0 &&
        pkv::chunk_balanced_supported(n_q, n_kv, head_dim, block_size, num_seqs, max_q_len)) {
        for (BalancedPass f : {kChunkBf16, kChunkInt8}) {   // bf16 and 8-bit K/V (paged_attn_chunk_q8)
            const int waves = balanced_waves(n_q, n_kv, num_seqs, f);
            if (waves < 1) return PKV_ERR_HIP;
            const size_t b = ws_layout_balanced(num_seqs, pkv::kChunkSlotRows, n_kv, head_dim, waves).total;
            if (b > *bytes) *bytes = b;
        }
    }
    return PKV_OK;
}

extern "C" int paged_attn_decode(void* out, float* lse, const void* q,
                                 const void* k_cache, const void* v_cache,
                                 const int32_t* block_table, int32_t table_stride,
                                 const int32_t* seq_lens,
                                 int32_t num_seqs, int32_t max_seq_len, int32_t num_blocks,
                                 int32_t n_q, int32_t n_kv, int32_t head_dim, int32_t block_size,
                                 float scale, int32_t dtype, int32_t split_tokens,
                                 void* workspace, size_t workspace_bytes, void* stream) {
    int rc = check_shape(num_seqs, max_seq_len, num_blocks, n_q, n_kv, head_dim, block_size,
                         table_stride, dtype, scale);
    if (rc != PKV_OK) return rc;
    if (num_seqs == 0) return PKV_OK;
    if (!out || !q || !k_cache || !v_cache || !block_table || !seq_lens) return PKV_ERR_NULL_POINTER;
    int split = 0;
    rc = resolve_split(num_seqs, n_kv, block_size, max_seq_len, split_tokens, &split);
    if (rc != PKV_OK) return rc;
    const bool balanced = balanced_eligible(dtype, split_tokens, num_seqs, n_q, n_kv, head_dim, block_size) &&
                          aligned16(q) && aligned16(k_cache) && aligned16(v_cache) && aligned16(out);
    pkv::AttnArgs a{};
    if (balanced) {
        a.waves = balanced_waves(n_q, n_kv, num_seqs);
        if (a.waves < 1) return PKV_ERR_HIP;
    }
    a.q = q;
    a.q_start = nullptr;
    a.k_cache = k_cache;
    a.v_cache = v_cache;
    a.table = block_table;
    a.seq_lens = seq_lens;
    a.table_stride = table_stride;
    a.num_seqs = num_seqs;
    a.num_rows = num_seqs;
    a.max_q_len = 1;
    a.max_seq_len = max_seq_len;
    a.num_blocks = num_blocks;
    a.n_q = n_q;
    a.n_kv = n_kv;
    a.head_dim = head_dim;
    a.block_size = block_size;
    a.split_tokens = split;
    a.max_splits = (max_seq_len + split - 1) / split;
    a.scale_log2 = scale * 1.44269504088896340736f;
    return run_attention(a, out, lse, dtype, true, balanced, workspace, workspace_bytes,
                         static_cast<hipStream_t>(stream));
}

extern "C" int paged_attn_decode_append(void* out, float* lse, const void* q, void* k_cache, void* v_cache,
                                        const void* k_new, const void* v_new, const int32_t* block_table,
                                        int32_t table_stride, const int32_t* seq_lens, int32_t num_seqs,
                                        int32_t max_seq_len, int32_t num_blocks, int32_t n_q, int32_t n_kv,
                                        int32_t head_dim, int32_t block_size, float scale, int32_t dtype,
                                        void* workspace, size_t workspace_bytes, void* stream) {
    int rc = check_shape(num_seqs, max_seq_len, num_blocks, n_q, n_kv, head_dim, block_size,
                         table_stride, dtype, scale);
    if (rc != PKV_OK) return rc;
    if (num_seqs == 0) return PKV_OK;
    if (!out || !q || !k_cache || !v_cache || !k_new || !v_new || !block_table || !seq_lens)
        return PKV_ERR_NULL_POINTER;
    if (!balanced_eligible(dtype, 0, num_seqs, n_q, n_kv, head_dim, block_size) || !aligned16(q) ||
        !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out) || !aligned16(k_new) || !aligned16(v_new))
        return PKV_ERR_UNSUPPORTED;
    pkv::AttnArgs a{};
    a.waves = balanced_waves(n_q, n_kv, num_seqs);
    if (a.waves < 1) return PKV_ERR_HIP;
    a.q = q;
    a.q_start = nullptr;
    a.k_cache = k_cache;
    a.v_cache = v_cache;
    a.table = block_table;
    a.seq_lens = seq_lens;
    a.table_stride = table_stride;
    a.num_seqs = num_seqs;
    a.num_rows = num_seqs;
    a.max_q_len = 1;
    a.max_seq_len = max_seq_len;
    a.num_blocks = num_blocks;
    a.n_q = n_q;
    a.n_kv = n_kv;
    a.head_dim = head_dim;
    a.block_size = block_size;
    int split = 0;
    rc = resolve_split(num_seqs, n_kv, block_size, max_seq_len, 0, &split);
    if (rc != PKV_OK) return rc;
    a.split_tokens = split;
    a.max_splits = (max_seq_len + split - 1) / split;
    a.scale_log2 = scale * 1.44269504088896340736f;
    // the workspace is checked before the append can write the pool
    rc = check_workspace(a, true, workspace, workspace_bytes, nullptr);
    if (rc != PKV_OK) return rc;
    // The append rides in the split pass while the batch has at most half
    // as many (sequence, kv head) segments as the pass has waves; with
    // more, many waves append rows, each a dependent round trip under full
    // load, and a launch of its own is faster (measured, bf16 and 8-bit:
    // 64 x 8 and 8 x 8 segments folded win, 256 x 8 folded loses).
    if (2LL * num_seqs * n_kv <= a.waves) {
        a.k_new = k_new;
        a.v_new = v_new;
        a.k_app = k_cache;
        a.v_app = v_cache;
    } else {
        const hipError_t e = pkv::launch_kv_append_last(k_cache, v_cache, k_new, v_new, block_table, table_stride,
                                                        seq_lens, num_seqs, max_seq_len, num_blocks, n_kv,
                                                        static_cast<hipStream_t>(stream));
        if (e != hipSuccess) return PKV_ERR_HIP;
    }
    return run_attention(a, out, lse, dtype, true, true, workspace, workspace_bytes,
                         static_cast<hipStream_t>(stream));
}

extern "C" int kv_append_q8(void* k_codes, void* v_codes, float* k_scale, float* v_scale, const void* k_new,
                            const void* v_new, int32_t new_dtype, const int32_t* block_table, int32_t table_stride,
                            const int32_t* start_pos, const int32_t* new_start, int32_t num_seqs, int32_t total_new,
                            int32_t num_blocks, int32_t n_kv, int32_t head_dim, int32_t block_size, void* stream) {
    if (num_seqs < 0 || total_new < 0 || num_blocks < 1 || n_kv < 1 || head_dim < 1 || block_size < 1 ||
        table_stride < 1)
        return PKV_ERR_INVALID_ARGUMENT;
    if (!elem_bytes(new_dtype)) return PKV_ERR_INVALID_ARGUMENT;
    if (total_new == 0) return PKV_OK;
    if (num_seqs == 0) return PKV_ERR_INVALID_ARGUMENT;
    if (!k_codes || !v_codes || !k_scale || !v_scale || !k_new || !v_new || !block_table || !start_pos ||
        !new_start)
        return PKV_ERR_NULL_POINTER;
    const hipError_t e = pkv::launch_kv_append_q8(
        static_cast<int8_t*>(k_codes), static_cast<int8_t*>(v_codes), k_scale, v_scale, k_new, v_new,
        new_dtype == PKV_BF16, block_table, table_stride, start_pos, new_start, num_seqs, total_new, num_blocks, n_kv,
        head_dim, block_size, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

extern "C" int paged_attn_decode_q8(void* out, float* lse, const void* q, const void* k_codes, const void* v_codes,
                                    const float* k_scale, const float* v_scale, const int32_t* block_table,
                                    int32_t table_stride, const int32_t* seq_lens, int32_t num_seqs,
                                    int32_t max_seq_len, int32_t num_blocks, int32_t n_q, int32_t n_kv,
                                    int32_t head_dim, int32_t block_size, float scale, void* workspace,
                                    size_t workspace_bytes, void* stream) {
    int rc = check_shape(num_seqs, max_seq_len, num_blocks, n_q, n_kv, head_dim, block_size, table_stride, PKV_BF16,
                         scale);
    if (rc != PKV_OK) return rc;
    if (num_seqs == 0) return PKV_OK;
    if (!out || !q || !k_codes || !v_codes || !k_scale || !v_scale || !block_table || !seq_lens)
        return PKV_ERR_NULL_POINTER;
    if (!pkv::decode_balanced_supported(n_q, n_kv, head_dim, block_size, num_seqs)) return PKV_ERR_UNSUPPORTED;
    if (!aligned16(q) || !aligned16(out) || !aligned16(k_codes) || !aligned16(v_codes) || !aligned16(k_scale) ||
        !aligned16(v_scale))
        return PKV_ERR_INVALID_ARGUMENT;
    pkv::AttnArgs a{};
    a.waves = balanced_waves(n_q, n_kv, num_seqs, kDecodeInt8);
    if (a.waves < 1) return PKV_ERR_HIP;
    a.q = q;
    a.q_start = nullptr;
    a.k_cache = k_codes;
    a.v_cache = v_codes;
    a.k_scale = k_scale;
    a.v_scale = v_scale;
    a.table = block_table;
    a.seq_lens = seq_lens;
    a.table_stride = table_stride;
    a.num_seqs = num_seqs;
    a.num_rows = num_seqs;
    a.max_q_len = 1;
    a.max_seq_len = max_seq_len;
    a.num_blocks = num_blocks;
    a.n_q = n_q;
    a.n_kv = n_kv;
    a.head_dim = head_dim;
    a.block_size = block_size;
    a.split_tokens = block_size;
    a.max_splits = 1;
    a.scale_log2 = scale * 1.44269504088896340736f;
    return run_attention(a, out, lse, PKV_BF16, true, true, workspace, workspace_bytes,
                         static_cast<hipStream_t>(stream));
}

extern "C" int paged_attn_decode_q8_append(void* out, float* lse, const void* q, void* k_codes, void* v_codes,
                                           float* k_scale, float* v_scale, const void* k_new, const void* v_new,
                                           const int32_t* block_table, int32_t table_stride, const int32_t* seq_lens,
                                           int32_t num_seqs, int32_t max_seq_len, int32_t num_blocks, int32_t n_q,
                                           int32_t n_kv, int32_t head_dim, int32_t block_size, float scale,
                                           void* workspace, size_t workspace_bytes, void* stream) {
    int rc = check_shape(num_seqs, max_seq_len, num_blocks, n_q, n_kv, head_dim, block_size, table_stride, PKV_BF16,
                         scale);
    if (rc != PKV_OK) return rc;
    if (num_seqs == 0) return PKV_OK;
    if (!out || !q || !k_codes || !v_codes || !k_scale || !v_scale || !k_new || !v_new || !block_table || !seq_lens)
        return PKV_ERR_NULL_POINTER;
    if (!pkv::decode_balanced_supported(n_q, n_kv, head_dim, block_size, num_seqs)) return PKV_ERR_UNSUPPORTED;
    if (!aligned16(q) || !aligned16(out) || !aligned16(k_new) || !aligned16(v_new) || !aligned16(k_codes) ||
        !aligned16(v_codes) || !aligned16(k_scale) || !aligned16(v_scale))
        return PKV_ERR_INVALID_ARGUMENT;
    pkv::AttnArgs a{};
    a.waves = balanced_waves(n_q, n_kv, num_seqs, kDecodeInt8);
    if (a.waves < 1) return PKV_ERR_HIP;
    a.q = q;
    a.q_start = nullptr;
    a.k_cache = k_codes;
    a.v_cache = v_codes;
    a.k_scale = k_scale;
    a.v_scale = v_scale;
    a.table = block_table;
    a.seq_lens = seq_lens;
    a.table_stride = table_stride;
    a.num_seqs = num_seqs;
    a.num_rows = num_seqs;
    a.max_q_len = 1;
    a.max_seq_len = max_seq_len;
    a.num_blocks = num_blocks;
    a.n_q = n_q;
    a.n_kv = n_kv;
    a.head_dim = head_dim;
    a.block_size = block_size;
    a.split_tokens = block_size;
    a.max_splits = 1;
    a.scale_log2 = scale * 1.44269504088896340736f;
    // the workspace is checked before the append can write the pool
    rc = check_workspace(a, true, workspace, workspace_bytes, nullptr);
    if (rc != PKV_OK) return rc;
    // folded while segments <= waves / 2, as for bf16 (paged_attn_decode_append)
    if (2LL * num_seqs * n_kv <= a.waves) {
        a.k_new = k_new;
        a.v_new = v_new;
        a.k_app = k_codes;
        a.v_app = v_codes;
        a.ks_app = k_scale;
        a.vs_app = v_scale;
    } else {
        const hipError_t e = pkv::launch_kv_append_q8_last(
            static_cast<int8_t*>(k_codes), static_cast<int8_t*>(v_codes), k_scale, v_scale, k_new, v_new, block_table,
            table_stride, seq_lens, num_seqs, max_seq_len, num_blocks, n_kv, static_cast<hipStream_t>(stream));
        if (e != hipSuccess) return PKV_ERR_HIP;
    }
    return run_attention(a, out, lse, PKV_BF16, true, true, workspace, workspace_bytes,
                         static_cast<hipStream_t>(stream));
}

namespace {

// paged_attn_chunk, and with k_new / v_new set its append as well
// (paged_attn_chunk_append), launched first. Folding it into the balanced
// small-chunk pass was measured slower (verification chunks of 5: 130.3 vs
// 126.9 us per step): a chunk's new rows span up to two tiles per segment,
// each with its own row lookups and stores ahead of that tile's loads.
int chunk_impl(void* out, float* lse, const void* q, const int32_t* q_start, void* k_cache, void* v_cache,
               const void* k_new, const void* v_new, const int32_t* block_table, int32_t table_stride,
               const int32_t* seq_lens, int32_t num_seqs, int32_t total_q, int32_t max_q_len, int32_t max_seq_len,
               int32_t num_blocks, int32_t n_q, int32_t n_kv, int32_t head_dim, int32_t block_size, float scale,
               int32_t dtype, int32_t split_tokens, void* workspace, size_t workspace_bytes, void* stream) {
    int rc = check_shape(num_seqs, max_seq_len, num_blocks, n_q, n_kv, head_dim, block_size,
                         table_stride, dtype, scale);
    if (rc != PKV_OK) return rc;
    if (total_q < 0 || max_q_len < 0 || max_q_len > max_seq_len) return PKV_ERR_INVALID_ARGUMENT;
    if (total_q == 0) return PKV_OK;
    if (num_seqs == 0 || max_q_len == 0) return PKV_ERR_INVALID_ARGUMENT;
    if (!out || !q || !q_start || !k_cache || !v_cache || !block_table || !seq_lens)
        return PKV_ERR_NULL_POINTER;
    const bool append = k_new || v_new;
    if (append && (!k_new || !v_new)) return PKV_ERR_NULL_POINTER;
    hipStream_t st = static_cast<hipStream_t>(stream);
    bool appended = false;
    auto append_first = [&]() -> int {   // the append as its own launch, before the attention
        if (!append || appended) return PKV_OK;
        appended = true;
        const hipError_t e = pkv::launch_kv_append(k_cache, v_cache, k_new, v_new, block_table, table_stride,
                                                   nullptr, q_start, num_seqs, total_q, num_blocks, n_kv,
                                                   head_dim * elem_bytes(dtype), block_size, st, seq_lens,
                                                   max_seq_len);
        return e == hipSuccess ? PKV_OK : PKV_ERR_HIP;
    };
    int split = 0;
    rc = resolve_split(total_q, n_kv, block_size, max_seq_len, split_tokens, &split);
    if (rc != PKV_OK) return rc;
    const bool mfma = dtype == PKV_BF16 && split_tokens == 0 &&
                      pkv::chunk_mfma_supported(n_q, n_kv, head_dim, block_size, max_seq_len) &&
                      aligned16(q) && aligned16(k_cache) && aligned16(v_cache) && aligned16(out);
    pkv::AttnArgs a{};
    a.q = q;
    a.q_start = q_start;
    a.k_cache = k_cache;
    a.v_cache = v_cache;
    a.table = block_table;
    a.seq_lens = seq_lens;
    a.table_stride = table_stride;
    a.num_seqs = num_seqs;
    a.num_rows = total_q;
    a.max_q_len = max_q_len;
    a.max_seq_len = max_seq_len;
    a.num_blocks = num_blocks;
    a.n_q = n_q;
    a.n_kv = n_kv;
    a.head_dim = head_dim;
    a.block_size = block_size;
    a.split_tokens = split;
    a.max_splits = (max_seq_len + split - 1) / split;
    a.scale_log2 = scale * 1.44269504088896340736f;
    // Small chunks (every C_s <= 32 / G rows' worth): the balanced partition
    // over all (sequence, kv head, block) tiles with both products on the
    // matrix cores, as decode, when the workspace holds its partials
    // (paged_attn_chunk_workspace_size); otherwise the chunk kernels below.
    if (dtype == PKV_BF16 && split_tokens == 0 && workspace &&
        reinterpret_cast<uintptr_t>(workspace) % kAlign == 0 && aligned16(q) && aligned16(k_cache) &&
        aligned16(v_cache) && pkv::chunk_balanced_supported(n_q, n_kv, head_dim, block_size, num_seqs, max_q_len)) {
        const int waves = balanced_waves(n_q, n_kv, num_seqs, kChunkBf16);
        const Layout w = ws_layout_balanced(num_seqs, pkv::kChunkSlotRows, n_kv, head_dim, waves);
        if (waves >= 1 && workspace_bytes >= w.total) {
            char* ws = static_cast<char*>(workspace);
            a.waves = waves;
            a.ws_ml = reinterpret_cast<pkv::PartialML*>(ws);
            a.ws_o = reinterpret_cast<float*>(ws + w.o_offset);
            a.prefix = reinterpret_cast<int*>(ws + w.prefix_offset);
            rc = append_first();
            if (rc != PKV_OK) return rc;
            hipError_t e = pkv::launch_chunk_balanced(a, st, profile_events());
            if (e == hipSuccess) e = pkv::launch_merge(a, out, lse, true, st);
            return e == hipSuccess ? PKV_OK : PKV_ERR_HIP;
        }
    }
    // the split path's workspace is checked before the append can write the pool
    if (!mfma) {
        rc = check_workspace(a, false, workspace, workspace_bytes, nullptr);
        if (rc != PKV_OK) return rc;
    }
    if (mfma && append && aligned16(k_new) && aligned16(v_new)) {
        // the append fused into the matrix-core chunk kernel
        a.k_new = k_new;
        a.v_new = v_new;
        a.k_app = k_cache;
        a.v_app = v_cache;
        const hipError_t e = pkv::launch_chunk_mfma(a, out, lse, st, profile_events());
        return e == hipSuccess ? PKV_OK : PKV_ERR_HIP;
    }
    rc = append_first();
    if (rc != PKV_OK) return rc;
    if (mfma) {
        const hipError_t e = pkv::launch_chunk_mfma(a, out, lse, st, profile_events());
        return e == hipSuccess ? PKV_OK : PKV_ERR_HIP;
    }
    return run_attention(a, out, lse, dtype, false, false, workspace, workspace_bytes, st);
}

}  // namespace

extern "C" int paged_attn_chunk(void* out, float* lse, const void* q, const int32_t* q_start,
                                const void* k_cache, const void* v_cache,
                                const int32_t* block_table, int32_t table_stride,
                                const int32_t* seq_lens,
                                int32_t num_seqs, int32_t total_q, int32_t max_q_len,
                                int32_t max_seq_len, int32_t num_blocks,
                                int32_t n_q, int32_t n_kv, int32_t head_dim, int32_t block_size,
                                float scale, int32_t dtype, int32_t split_tokens,
                                void* workspace, size_t workspace_bytes, void* stream) {
    return chunk_impl(out, lse, q, q_start, const_cast<void*>(k_cache), const_cast<void*>(v_cache), nullptr,
                      nullptr, block_table, table_stride, seq_lens, num_seqs, total_q, max_q_len, max_seq_len,
                      num_blocks, n_q, n_kv, head_dim, block_size, scale, dtype, split_tokens, workspace,
                      workspace_bytes, stream);
}

extern "C" int paged_attn_chunk_append(void* out, float* lse, const void* q, const int32_t* q_start,
                                       void* k_cache, void* v_cache, const void* k_new, const void* v_new,
                                       const int32_t* block_table, int32_t table_stride, const int32_t* seq_lens,
                                       int32_t num_seqs, int32_t total_q, int32_t max_q_len, int32_t max_seq_len,
                                       int32_t num_blocks, int32_t n_q, int32_t n_kv, int32_t head_dim,
                                       int32_t block_size, float scale, int32_t dtype, int32_t split_tokens,
                                       void* workspace, size_t workspace_bytes, void* stream) {
    if (total_q > 0 && (!k_new || !v_new)) return PKV_ERR_NULL_POINTER;
    return chunk_impl(out, lse, q, q_start, k_cache, v_cache, k_new, v_new, block_table, table_stride, seq_lens,
                      num_seqs, total_q, max_q_len, max_seq_len, num_blocks, n_q, n_kv, head_dim, block_size, scale,
                      dtype, split_tokens, workspace, workspace_bytes, stream);
}

namespace {

// paged_attn_chunk_q8 and paged_attn_chunk_q8_append: every argument and the
// workspace are checked before the first launch. Then either the balanced
// pass (verification-sized chunks; the quantising append of the chunk's
// rows at seq_lens - C_s launched first when k_new is set) or, past 32 rows
// per kv head, the sequences' blocks dequantised to bf16 into the workspace
// (the append fused into that pass) and the bf16 matrix-core chunk kernel
// over them.
int chunk_q8_impl(void* out, float* lse, const void* q, const int32_t* q_start, void* k_codes, void* v_codes,
                  float* k_scale, float* v_scale, const void* k_new, const void* v_new, const int32_t* block_table,
                  int32_t table_stride, const int32_t* seq_lens, int32_t num_seqs, int32_t total_q, int32_t max_q_len,
                  int32_t max_seq_len, int32_t num_blocks, int32_t n_q, int32_t n_kv, int32_t head_dim,
                  int32_t block_size, float scale, void* workspace, size_t workspace_bytes, void* stream) {
    int rc = check_shape(num_seqs, max_seq_len, num_blocks, n_q, n_kv, head_dim, block_size, table_stride, PKV_BF16,
                         scale);
    if (rc != PKV_OK) return rc;
    if (total_q < 0 || max_q_len < 0 || max_q_len > max_seq_len) return PKV_ERR_INVALID_ARGUMENT;
    if (total_q == 0) return PKV_OK;
    if (num_seqs == 0 || max_q_len == 0) return PKV_ERR_INVALID_ARGUMENT;
    if (!out || !q || !q_start || !k_codes || !v_codes || !k_scale || !v_scale || !block_table || !seq_lens)
        return PKV_ERR_NULL_POINTER;
    const bool append = k_new || v_new;
    if (append && (!k_new || !v_new)) return PKV_ERR_NULL_POINTER;
    const bool balanced = pkv::chunk_balanced_supported(n_q, n_kv, head_dim, block_size, num_seqs, max_q_len);
    if (!balanced && !pkv::chunk_mfma_supported(n_q, n_kv, head_dim, block_size, max_seq_len))
        return PKV_ERR_UNSUPPORTED;
    if (!aligned16(q) || !aligned16(out) || !aligned16(k_codes) || !aligned16(v_codes) || !aligned16(k_scale) ||
        !aligned16(v_scale))
        return PKV_ERR_INVALID_ARGUMENT;
    if (!workspace) return PKV_ERR_NULL_POINTER;
    if (reinterpret_cast<uintptr_t>(workspace) % kAlign) return PKV_ERR_INVALID_ARGUMENT;
    char* ws = static_cast<char*>(workspace);
    pkv::AttnArgs a{};
    a.q = q;
    a.q_start = q_start;
    a.seq_lens = seq_lens;
    a.num_seqs = num_seqs;
    a.num_rows = total_q;
    a.max_q_len = max_q_len;
    a.max_seq_len = max_seq_len;
    a.n_q = n_q;
    a.n_kv = n_kv;
    a.head_dim = head_dim;
    a.block_size = block_size;
    a.scale_log2 = scale * 1.44269504088896340736f;
    StagingLayout l{};
    if (balanced) {
        a.waves = balanced_waves(n_q, n_kv, num_seqs, kChunkInt8);
        if (a.waves < 1) return PKV_ERR_HIP;
        const Layout w = ws_layout_balanced(num_seqs, pkv::kChunkSlotRows, n_kv, head_dim, a.waves);
        if (workspace_bytes < w.total) return PKV_ERR_WORKSPACE_TOO_SMALL;
        a.k_cache = k_codes;
        a.v_cache = v_codes;
        a.k_scale = k_scale;
        a.v_scale = v_scale;
        a.table = block_table;
        a.table_stride = table_stride;
        a.num_blocks = num_blocks;
        a.split_tokens = block_size;
        a.max_splits = 1;
        a.ws_ml = reinterpret_cast<pkv::PartialML*>(ws);
        a.ws_o = reinterpret_cast<float*>(ws + w.o_offset);
        a.prefix = reinterpret_cast<int*>(ws + w.prefix_offset);
    } else {
        l = staging_layout(num_seqs, max_seq_len, n_kv, head_dim, block_size);
        if (static_cast<size_t>(num_seqs) * l.maxb > static_cast<size_t>(INT32_MAX)) return PKV_ERR_INVALID_ARGUMENT;
        if (workspace_bytes < l.total) return PKV_ERR_WORKSPACE_TOO_SMALL;
        a.k_cache = ws;                            // the chunk over the staged bf16 blocks
        a.v_cache = ws + l.v_offset;
        a.table = reinterpret_cast<int32_t*>(ws + l.table_offset);
        a.table_stride = l.maxb;
        a.num_blocks = num_seqs * l.maxb;
    }
    hipStream_t st = static_cast<hipStream_t>(stream);
    hipError_t e = hipSuccess;
    // large chunks: the append fused into the block expansion below
    const bool fused = append && !balanced && aligned16(k_new) && aligned16(v_new);
    if (append && !fused)
        e = pkv::launch_kv_append_q8(static_cast<int8_t*>(k_codes), static_cast<int8_t*>(v_codes), k_scale, v_scale,
                                     k_new, v_new, true, block_table, table_stride, nullptr, q_start, num_seqs,
                                     total_q, num_blocks, n_kv, head_dim, block_size, st, seq_lens, max_seq_len);
    if (e != hipSuccess) return PKV_ERR_HIP;
    if (balanced) {
        e = pkv::launch_chunk_balanced(a, st, profile_events());
        if (e == hipSuccess) e = pkv::launch_merge(a, out, lse, true, st);
        return e == hipSuccess ? PKV_OK : PKV_ERR_HIP;
    }
    pkv::AttnArgs d{};   // the 8-bit pool, for the staging copy
    d.k_cache = k_codes;
    d.v_cache = v_codes;
    d.k_scale = k_scale;
    d.v_scale = v_scale;
    d.table = block_table;
    d.table_stride = table_stride;
    d.seq_lens = seq_lens;
    d.num_seqs = num_seqs;
    d.max_seq_len = max_seq_len;
    d.num_blocks = num_blocks;
    d.n_kv = n_kv;
    d.head_dim = head_dim;
    d.block_size = block_size;
    if (fused) {
        d.q_start = q_start;
        d.k_new = k_new;
        d.v_new = v_new;
        d.k_app = k_codes;
        d.v_app = v_codes;
        d.ks_app = k_scale;
        d.vs_app = v_scale;
    }
    e = pkv::launch_dequant_blocks(d, static_cast<uint16_t*>(const_cast<void*>(a.k_cache)),
                                   static_cast<uint16_t*>(const_cast<void*>(a.v_cache)),
                                   const_cast<int32_t*>(a.table), l.maxb, st);
    if (e == hipSuccess) e = pkv::launch_chunk_mfma(a, out, lse, st, profile_events());
    return e == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

}  // namespace

extern "C" int paged_attn_chunk_q8_workspace_size(int32_t num_seqs, int32_t total_q, int32_t max_q_len, int32_t n_q,
                                                  int32_t n_kv, int32_t head_dim, int32_t block_size,
                                                  int32_t max_seq_len, size_t* bytes) {
    if (!bytes) return PKV_ERR_NULL_POINTER;
    if (num_seqs < 0 || total_q < 0 || max_q_len < 0 || n_q < 1 || n_kv < 1 || n_q % n_kv || head_dim < 1 ||
        block_size < 1 || max_seq_len < 1)
        return PKV_ERR_INVALID_ARGUMENT;
    *bytes = 0;
    if (pkv::chunk_balanced_supported(n_q, n_kv, head_dim, block_size, num_seqs, max_q_len)) {
        const int waves = balanced_waves(n_q, n_kv, num_seqs, kChunkInt8);
        if (waves < 1) return PKV_ERR_HIP;
        *bytes = ws_layout_balanced(num_seqs, pkv::kChunkSlotRows, n_kv, head_dim, waves).total;
    } else if (pkv::chunk_mfma_supported(n_q, n_kv, head_dim, block_size, max_seq_len)) {
        *bytes = staging_layout(num_seqs, max_seq_len, n_kv, head_dim, block_size).total;
    }
    return PKV_OK;
}

extern "C" int paged_attn_chunk_q8(void* out, float* lse, const void* q, const int32_t* q_start, const void* k_codes,
                                   const void* v_codes, const float* k_scale, const float* v_scale,
                                   const int32_t* block_table, int32_t table_stride, const int32_t* seq_lens,
                                   int32_t num_seqs, int32_t total_q, int32_t max_q_len, int32_t max_seq_len,
                                   int32_t num_blocks, int32_t n_q, int32_t n_kv, int32_t head_dim, int32_t block_size,
                                   float scale, void* workspace, size_t workspace_bytes, void* stream) {
    return chunk_q8_impl(out, lse, q, q_start, const_cast<void*>(k_codes), const_cast<void*>(v_codes),
                         const_cast<float*>(k_scale), const_cast<float*>(v_scale), nullptr, nullptr, block_table,
                         table_stride, seq_lens, num_seqs, total_q, max_q_len, max_seq_len, num_blocks, n_q, n_kv,
                         head_dim, block_size, scale, workspace, workspace_bytes, stream);
}

extern "C" int paged_attn_chunk_q8_append(void* out, float* lse, const void* q, const int32_t* q_start,
                                          void* k_codes, void* v_codes, float* k_scale, float* v_scale,
                                          const void* k_new, const void* v_new, const int32_t* block_table,
                                          int32_t table_stride, const int32_t* seq_lens, int32_t num_seqs,
                                          int32_t total_q, int32_t max_q_len, int32_t max_seq_len, int32_t num_blocks,
                                          int32_t n_q, int32_t n_kv, int32_t head_dim, int32_t block_size,
                                          float scale, void* workspace, size_t workspace_bytes, void* stream) {
    if (total_q > 0 && (!k_new || !v_new)) return PKV_ERR_NULL_POINTER;
    return chunk_q8_impl(out, lse, q, q_start, k_codes, v_codes, k_scale, v_scale, k_new, v_new, block_table,
                         table_stride, seq_lens, num_seqs, total_q, max_q_len, max_seq_len, num_blocks, n_q, n_kv,
                         head_dim, block_size, scale, workspace, workspace_bytes, stream);
}
