// Host-side launch wrappers for the paged-KV kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pkv {

// Partial softmax state of one (row, query head, key range): max of the
// scaled scores in log2 units, and the sum of 2^(score - max).
struct PartialML {
    float m;
    float l;
};

struct AttnArgs {
    const void* q;
    const int32_t* q_start;      // nullptr: one query row per sequence
    const void* k_cache;         // bf16 / fp32 elements, or 8-bit codes when k_scale is set
    const void* v_cache;
    const float* k_scale;        // 8-bit K/V: [num_blocks][n_kv][block_size] scales; nullptr otherwise
    const float* v_scale;
    const int32_t* table;
    const int32_t* seq_lens;
    int table_stride;
    int num_seqs;
    int num_rows;                // decode: num_seqs; chunk: total query rows
    int max_q_len;
    int max_seq_len;
    int num_blocks;
    int n_q, n_kv, head_dim, block_size;
    int split_tokens, max_splits;
    float scale_log2;            // scale * log2(e)
    float* ws_o;                 // fixed split: [rows][n_q][max_splits][head_dim]
                                 // balanced: [waves + S*n_kv][G][head_dim]
    PartialML* ws_ml;            // same slots as ws_o, without the head_dim axis
    int waves;                   // balanced decode: grid size W (0 = fixed split)
    int* prefix;                 // balanced decode: [S+1] block-count prefix sums
    // Balanced decode with the append folded in (else all null): the new
    // token of each sequence (bf16 [num_seqs][n_kv][head_dim]) is written
    // to position seq_lens[s] - 1 of k_app / v_app (the same pools as
    // k_cache / v_cache; 8-bit pools: quantised, scales to ks_app / vs_app)
    // before that tile is read.
    const void* k_new;
    const void* v_new;
    void* k_app;
    void* v_app;
    float* ks_app;               // 8-bit pools: where the appended rows' scales go (k_scale / v_scale)
    float* vs_app;
};

// Optional event pair recorded by the kernel's own dispatch (start and end
// of its execution), for timing one kernel without extra stream packets.
struct KernelEvents {
    hipEvent_t start = nullptr;
    hipEvent_t stop = nullptr;
    bool on() const { return start || stop; }
};

// start_pos null: a chunk step, whose sequence s's new tokens are the last
// new_start[s+1] - new_start[s] of seq_lens[s] keys (sequences the chunk
// pass rejects get no write).
hipError_t launch_kv_append(void* k_cache, void* v_cache, const void* k_new, const void* v_new,
                            const int32_t* table, int table_stride, const int32_t* start_pos,
                            const int32_t* new_start, int num_seqs, int total_new, int num_blocks,
                            int n_kv, int row_bytes, int block_size, hipStream_t stream,
                            const int32_t* seq_lens = nullptr, int max_seq_len = 0);

// The decode step's append on its own: one token per sequence at position
// seq_lens[s] - 1 (bf16, head_dim 128, block_size 16; 16-byte aligned).
hipError_t launch_kv_append_last(void* k_cache, void* v_cache, const void* k_new, const void* v_new,
                                 const int32_t* table, int table_stride, const int32_t* seq_lens, int num_seqs,
                                 int max_seq_len, int num_blocks, int n_kv, hipStream_t stream);

// The same for an 8-bit pool (bf16 input, quantised as kv_append_q8 does).
hipError_t launch_kv_append_q8_last(int8_t* k_codes, int8_t* v_codes, float* k_scale, float* v_scale,
                                    const void* k_new, const void* v_new, const int32_t* table, int table_stride,
                                    const int32_t* seq_lens, int num_seqs, int max_seq_len, int num_blocks, int n_kv,
                                    hipStream_t stream);

// Quantising append (8-bit codes + one fp32 scale per token and kv head);
// start_pos null: the chunk step's positions, as launch_kv_append.
hipError_t launch_kv_append_q8(int8_t* k_cache, int8_t* v_cache, float* k_scale, float* v_scale, const void* k_new,
                               const void* v_new, bool bf16_in, const int32_t* table, int table_stride,
                               const int32_t* start_pos, const int32_t* new_start, int num_seqs, int total_new,
                               int num_blocks, int n_kv, int head_dim, int block_size, hipStream_t stream,
                               const int32_t* seq_lens = nullptr, int max_seq_len = 0);

// Token sampling after the LM head. Rows whose top-k set is small go
// through a candidate pass (chunks of kSampleChunk logits, each keeping its
// own top-k) and are finished from those candidates; rows with top-k off
// (vocabularies of at most kSampleHistChunks chunks) through per-chunk mass
// histograms and per-chunk lists of the tokens near each chunk's own top-p
// boundary; the others by one workgroup over the whole row.
constexpr int kSampleChunk = 8192;      // logits per candidate-pass workgroup
constexpr int kSampleMaxK = 256;        // largest top-k on the candidate path
constexpr int kSampleMaxCand = 8192;    // candidates one finishing workgroup holds
constexpr int kSampleHistBins = 2048;   // mass histogram bins per chunk (top 11 bits of the order key)
constexpr int kSampleHistChunks = 64;   // widest row (in chunks) the histogram path merges
constexpr int kSampleListCap = 4096;    // tokens one chunk lists around its own top-p boundary
constexpr int kSampleWinBins = 5;       // the bins of that list: the chunk's boundary bin and two on each side
constexpr int kSampleBucketCap = 12288; // boundary-bin tokens of a row the finishing pass holds
inline int sample_chunks(int vocab) { return (vocab + kSampleChunk - 1) / kSampleChunk; }
inline bool sample_hist_rows(int vocab) { return sample_chunks(vocab) <= kSampleHistChunks; }
// Per (row, chunk): a region of kSampleMaxK (key, index) candidates or, when
// the row has at most kSampleHistChunks chunks, of kSampleHistBins fp64
// masses (the candidates fit in it). For such vocabularies the regions are
// followed by, per (row, chunk), a 16-byte header, 64 fp64 sums (every 32nd
// bin's), a list of kSampleListCap 8-byte entries and a SampleChunkTally.
inline size_t sample_region_bytes(int vocab) {
    return sample_hist_rows(vocab) ? static_cast<size_t>(kSampleHistBins) * 8u
                                   : static_cast<size_t>(kSampleMaxK) * 8u;
}
struct SampleChunkTally {  // histogram rows with top-p on, per chunk, written by the chunk pass
    uint32_t wlo, whi;     // the bins whose tokens the chunk listed (around its own top-p boundary)
    uint32_t listed[4];    // tokens listed by each wave (0xFFFFFFFF: more than its share)
    uint32_t up[4];        // tokens above the window, per wave
    uint32_t inbin[4][kSampleWinBins];  // tokens per wave and window bin (wlo + i)
};
inline size_t sample_workspace_bytes(int rows, int vocab) {
    const bool hist = sample_hist_rows(vocab);
    const size_t per = sample_region_bytes(vocab) + (hist ? 16u + 512u + kSampleListCap * 8u + sizeof(SampleChunkTally) : 0u);
    return static_cast<size_t>(rows) * sample_chunks(vocab) * per;
}
struct SampleChunkHead {
    float mc;          // largest z of the chunk
    float pad;
    double total;      // sum of exp(z - mc) over the chunk
};
struct SampleArgs {
    const float* logits;         // [rows][ld], the first vocab entries used
    int vocab;
    size_t ld;
    const float* temperature;    // [rows]
    const int32_t* top_k;        // [rows], 0 = off
    const float* top_p;          // [rows], >= 1 = off
    const float* u;              // [rows] uniform numbers in [0, 1)
    int32_t* token;              // [rows]
    int32_t* kept;               // [rows][2] tokens kept by top-k and by top-p, or nullptr
    unsigned char* ws;           // sample_workspace_bytes(rows, vocab), 8-byte aligned
    int rows;
    int chunks;                  // sample_chunks(vocab)
    size_t region;               // sample_region_bytes(vocab)
};
hipError_t launch_sample(const SampleArgs& a, int rows, hipStream_t stream);

// Whole-block copies (src_ids[i] -> dst_ids[i], both pools) for
// copy-on-write; block_bytes = n_kv * block_size * head_dim * element size.
hipError_t launch_copy_blocks(void* k_cache, void* v_cache, const int32_t* src_ids, const int32_t* dst_ids,
                              int n, int num_blocks, size_t block_bytes, hipStream_t stream);

// Large chunks over an 8-bit pool (head_dim 128): every block the sequences
// hold, as bf16 scale x code, into a staging pool (block i of sequence s at
// s * maxb + i, maxb = ceil(max_seq_len / block_size)) with a compact table
// [num_seqs][maxb] naming those blocks (-1: no block there); the bf16 chunk
// kernel then runs over them. a: the 8-bit call's arguments. With
// a.k_new / a.v_new set (bf16 [total_q][n_kv][128], 16-byte aligned, rows
// per sequence from a.q_start) the chunk's own tokens are quantised from
// them into the pool (a.k_app / a.v_app codes, a.ks_app / a.vs_app scales)
// on the way, as kv_append_q8 at seq_lens - C_s would.
hipError_t launch_dequant_blocks(const AttnArgs& a, uint16_t* k_out, uint16_t* v_out, int32_t* table_out, int maxb,
                                 hipStream_t stream);

// Split pass for any shape/dtype (one wave per row, head and key range).
hipError_t launch_split_generic(const AttnArgs& a, bool bf16, hipStream_t stream);

// Split pass tuned for decode with bf16, head_dim 128, block_size 16.
bool decode_fast_supported(int n_q, int n_kv, int head_dim, int block_size, int split_tokens);
hipError_t launch_decode_fast(const AttnArgs& a, hipStream_t stream, KernelEvents ev = {});

// Balanced decode pass (bf16, head_dim 128, block_size 16): equal tile
// ranges per wave across sequence boundaries.
bool decode_balanced_supported(int n_q, int n_kv, int head_dim, int block_size, int num_seqs);
int decode_balanced_waves(int n_q, int n_kv, int num_seqs, bool int8_kv = false);
hipError_t launch_decode_balanced(const AttnArgs& a, hipStream_t stream, KernelEvents ev = {});

// Small chunks through the same balanced partition (bf16, head_dim 128,
// block_size 16): every (query, head) row of a kv head, at most
// kChunkSlotRows of them (max_q_len * G), on the matrix cores; partial slots
// of kChunkSlotRows rows, merged by launch_merge (a.q_start set).
constexpr int kChunkSlotRows = 32;
bool chunk_balanced_supported(int n_q, int n_kv, int head_dim, int block_size, int num_seqs, int max_q_len);
int chunk_balanced_waves(int n_q, int n_kv, int num_seqs, bool int8_kv = false);
hipError_t launch_chunk_balanced(const AttnArgs& a, hipStream_t stream, KernelEvents ev = {});

// Chunk attention on MFMA (bf16, head_dim 128, block_size 16, sequences of
// at most 32768 keys): writes out and lse directly, no workspace. With
// a.k_new / a.v_new set (bf16 [total_q][n_kv][128], 16-byte aligned) it is
// the chunk step: the chunk's rows are also written to a.k_app / a.v_app
// (the pools) at positions seq_lens - C_s .. seq_lens - 1, and the chunk's
// own keys are read from the new rows.
bool chunk_mfma_supported(int n_q, int n_kv, int head_dim, int block_size, int max_seq_len);
hipError_t launch_chunk_mfma(const AttnArgs& a, void* out, float* lse, hipStream_t stream,
                             KernelEvents ev = {});

// Merge pass: combines each row's partial states into out (and lse).
hipError_t launch_merge(const AttnArgs& a, void* out, float* lse, bool bf16, hipStream_t stream);

}  // namespace pkv
