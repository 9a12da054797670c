// Host-side block pool: a rank-ordered free set of KV block ids.
//
// Lab page (Inference Engineering), class KVPool: blocks are handed out
// smallest-first from a sorted free list and returned (list re-sorted) when
// a sequence ends; chapter 5 section 3.2: blocks are taken on demand as a
// sequence grows; serving tutorial section 1.7: reclaim must never free a
// block twice or leak one.
//
// The free set is a bitmap over *ranks* (rank i <-> id order[i]), so the
// next block to hand out is the lowest set bit: O(num_blocks / 64) per
// call in the worst case, no allocation after creation.
//
// Blocks are reference counted (serving tutorial section 4.2: physical
// blocks shared between a common prefix or beam branches through their
// tables; section 1.7: a shared block goes back to the allocator only when
// its last holder releases it). A block is free exactly when its count is
// 0. A shared block that is about to be written is replaced, in the writing
// sequence's row only, by a fresh copy (copy-on-write, section 4.2).
#include <algorithm>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <new>
#include <vector>

#include "pagedkv.h"

struct kvpool {
    int32_t num_blocks;
    int32_t block_size;
    int32_t num_free;
    int32_t scan_from;             // no free rank below scan_from * 64
    std::vector<int32_t> order;    // rank -> id
    std::vector<int32_t> rank;     // id -> rank
    std::vector<uint64_t> free_bits;  // bit r set <=> rank r is free
    std::vector<int32_t> refs;     // id -> holders (0 <=> free)
};

namespace {

inline bool is_free(const kvpool* p, int32_t r) {
    return (p->free_bits[r >> 6] >> (r & 63)) & 1u;
}
inline void set_free(kvpool* p, int32_t r) {
    p->free_bits[r >> 6] |= (uint64_t(1) << (r & 63));
}
inline void clear_free(kvpool* p, int32_t r) {
    p->free_bits[r >> 6] &= ~(uint64_t(1) << (r & 63));
}

}  // namespace

extern "C" int kvpool_create(int32_t num_blocks, int32_t block_size,
                             const int32_t* alloc_order, kvpool_t** out) {
    if (!out) return PKV_ERR_NULL_POINTER;
    *out = nullptr;
    if (num_blocks < 1 || block_size < 1) return PKV_ERR_INVALID_ARGUMENT;
    kvpool* p = new (std::nothrow) kvpool();
    if (!p) return PKV_ERR_NO_MEMORY;
    try {
        p->num_blocks = num_blocks;
        p->block_size = block_size;
        p->order.resize(num_blocks);
        p->rank.assign(num_blocks, -1);
        for (int32_t r = 0; r < num_blocks; ++r) {
            int32_t id = alloc_order ? alloc_order[r] : r;
            if (id < 0 || id >= num_blocks || p->rank[id] != -1) {
                delete p;
                return PKV_ERR_INVALID_ARGUMENT;
            }
            p->order[r] = id;
            p->rank[id] = r;
        }
        p->refs.assign(num_blocks, 0);
        p->free_bits.assign((num_blocks + 63) / 64, 0);
        for (int32_t r = 0; r < num_blocks; ++r) set_free(p, r);
        p->num_free = num_blocks;
        p->scan_from = 0;
    } catch (...) {
        delete p;
        return PKV_ERR_NO_MEMORY;
    }
    *out = p;
    return PKV_OK;
}

extern "C" int kvpool_destroy(kvpool_t* pool) {
    delete pool;
    return PKV_OK;
}

extern "C" int kvpool_alloc(kvpool_t* p, int32_t n, int32_t* out_ids) {
    if (!p) return PKV_ERR_NULL_POINTER;
    if (n < 0) return PKV_ERR_INVALID_ARGUMENT;
    if (n == 0) return PKV_OK;
    if (!out_ids) return PKV_ERR_NULL_POINTER;
    if (n > p->num_free) return PKV_ERR_OUT_OF_BLOCKS;
    int32_t got = 0;
    const int32_t words = static_cast<int32_t>(p->free_bits.size());
    for (int32_t w = p->scan_from; w < words && got < n; ++w) {
        uint64_t bits = p->free_bits[w];
        while (bits && got < n) {
            int32_t r = w * 64 + __builtin_ctzll(bits);
            bits &= bits - 1;
            clear_free(p, r);
            p->refs[p->order[r]] = 1;
            out_ids[got++] = p->order[r];
        }
        if (p->free_bits[w] == 0) p->scan_from = w + 1;
    }
    p->num_free -= got;
    return PKV_OK;
}

namespace {

// True when ids[0..n) are in range, allocated and pairwise distinct. Uses
// the free bits of the listed ranks as scratch marks and restores them.
bool valid_held_ids(kvpool* p, int32_t n, const int32_t* ids) {
    int32_t i = 0;
    for (; i < n; ++i) {
        const int32_t id = ids[i];
        if (id < 0 || id >= p->num_blocks) break;
        const int32_t r = p->rank[id];
        if (is_free(p, r)) break;   // free, or listed earlier in this call
        set_free(p, r);
    }
    for (int32_t j = 0; j < i; ++j) clear_free(p, p->rank[ids[j]]);
    return i == n;
}

}  // namespace

extern "C" int kvpool_free(kvpool_t* p, int32_t n, const int32_t* ids) {
    if (!p) return PKV_ERR_NULL_POINTER;
    if (n < 0) return PKV_ERR_INVALID_ARGUMENT;
    if (n == 0) return PKV_OK;
    if (!ids) return PKV_ERR_NULL_POINTER;
    // Validate everything first so a failing call has no effect.
    if (!valid_held_ids(p, n, ids)) return PKV_ERR_INVALID_FREE;
    int32_t freed = 0;
    for (int32_t j = 0; j < n; ++j) {
        const int32_t id = ids[j];
        if (--p->refs[id] > 0) continue;   // other holders keep it
        const int32_t r = p->rank[id];
        set_free(p, r);
        if ((r >> 6) < p->scan_from) p->scan_from = r >> 6;
        ++freed;
    }
    p->num_free += freed;
    return PKV_OK;
}

extern "C" int kvpool_share(kvpool_t* p, int32_t n, const int32_t* ids) {
    if (!p) return PKV_ERR_NULL_POINTER;
    if (n < 0) return PKV_ERR_INVALID_ARGUMENT;
    if (n == 0) return PKV_OK;
    if (!ids) return PKV_ERR_NULL_POINTER;
    if (!valid_held_ids(p, n, ids)) return PKV_ERR_INVALID_BLOCK;
    for (int32_t j = 0; j < n; ++j) ++p->refs[ids[j]];
    return PKV_OK;
}

extern "C" int kvpool_refcount(const kvpool_t* p, int32_t id, int32_t* out) {
    if (!p || !out) return PKV_ERR_NULL_POINTER;
    if (id < 0 || id >= p->num_blocks) return PKV_ERR_INVALID_ARGUMENT;
    *out = p->refs[id];
    return PKV_OK;
}

extern "C" int kvpool_num_free(const kvpool_t* p, int32_t* out) {
    if (!p || !out) return PKV_ERR_NULL_POINTER;
    *out = p->num_free;
    return PKV_OK;
}

extern "C" int kvpool_free_ids(const kvpool_t* p, int32_t* out, int32_t* count) {
    if (!p || !out || !count) return PKV_ERR_NULL_POINTER;
    int32_t c = 0;
    for (int32_t r = 0; r < p->num_blocks; ++r)
        if (is_free(p, r)) out[c++] = p->order[r];
    *count = c;
    return PKV_OK;
}

extern "C" int kvpool_ensure(kvpool_t* p, int32_t* row, int32_t* num_held,
                             int32_t row_capacity, int32_t length) {
    if (!p || !row || !num_held) return PKV_ERR_NULL_POINTER;
    if (length < 0 || row_capacity < 0 || *num_held < 0 || *num_held > row_capacity)
        return PKV_ERR_INVALID_ARGUMENT;
    const int64_t need = (static_cast<int64_t>(length) + p->block_size - 1) / p->block_size;
    if (need <= *num_held) return PKV_OK;
    if (need > row_capacity) return PKV_ERR_TABLE_FULL;
    const int32_t more = static_cast<int32_t>(need - *num_held);
    int rc = kvpool_alloc(p, more, row + *num_held);
    if (rc != PKV_OK) return rc;
    *num_held = static_cast<int32_t>(need);
    return PKV_OK;
}

extern "C" int kvpool_release(kvpool_t* p, int32_t* row, int32_t* num_held) {
    if (!p || !num_held) return PKV_ERR_NULL_POINTER;
    if (*num_held == 0) return PKV_OK;
    if (!row) return PKV_ERR_NULL_POINTER;
    int rc = kvpool_free(p, *num_held, row);
    if (rc != PKV_OK) return rc;
    for (int32_t i = 0; i < *num_held; ++i) row[i] = -1;
    *num_held = 0;
    return PKV_OK;
}

extern "C" int kvpool_fork(kvpool_t* p, const int32_t* src_row, int32_t src_held, int32_t* dst_row,
                           int32_t* dst_held, int32_t row_capacity, int32_t length) {
    if (!p || !dst_held) return PKV_ERR_NULL_POINTER;
    if (length < 0 || src_held < 0 || row_capacity < 0 || *dst_held != 0) return PKV_ERR_INVALID_ARGUMENT;
    const int64_t need = (static_cast<int64_t>(length) + p->block_size - 1) / p->block_size;
    if (need > src_held) return PKV_ERR_INVALID_ARGUMENT;
    if (need > row_capacity) return PKV_ERR_TABLE_FULL;
    if (need == 0) return PKV_OK;
    if (!src_row || !dst_row) return PKV_ERR_NULL_POINTER;
    const int32_t n = static_cast<int32_t>(need);
    const int rc = kvpool_share(p, n, src_row);
    if (rc != PKV_OK) return rc;
    for (int32_t i = 0; i < n; ++i) dst_row[i] = src_row[i];
    *dst_held = n;
    return PKV_OK;
}

extern "C" int kvpool_cow(kvpool_t* p, int32_t* row, int32_t num_held, int32_t start, int32_t count,
                          int32_t* copy_src, int32_t* copy_dst, int32_t capacity, int32_t* num_copies) {
    if (!p || !num_copies) return PKV_ERR_NULL_POINTER;
    *num_copies = 0;
    if (num_held < 0 || start < 0 || count < 0 || capacity < 0) return PKV_ERR_INVALID_ARGUMENT;
    if (count == 0 || num_held == 0) return PKV_OK;
    if (!row) return PKV_ERR_NULL_POINTER;
    const int64_t first = start / p->block_size;
    const int64_t last = std::min<int64_t>((static_cast<int64_t>(start) + count - 1) / p->block_size,
                                           static_cast<int64_t>(num_held) - 1);
    // Check first: every id in range and allocated, enough copy slots and
    // enough free blocks; nothing changes on failure.
    int32_t shared = 0;
    for (int64_t i = first; i <= last; ++i) {
        const int32_t id = row[i];
        if (id < 0 || id >= p->num_blocks || p->refs[id] < 1) return PKV_ERR_INVALID_BLOCK;
        if (p->refs[id] > 1) ++shared;
    }
    if (shared == 0) return PKV_OK;
    if (!copy_src || !copy_dst) return PKV_ERR_NULL_POINTER;
    if (shared > capacity) return PKV_ERR_INVALID_ARGUMENT;
    if (shared > p->num_free) return PKV_ERR_OUT_OF_BLOCKS;
    int32_t c = 0;
    for (int64_t i = first; i <= last; ++i) {
        const int32_t id = row[i];
        if (p->refs[id] < 2) continue;
        int32_t fresh = -1;
        kvpool_alloc(p, 1, &fresh);
        --p->refs[id];
        copy_src[c] = id;
        copy_dst[c] = fresh;
        row[i] = fresh;
        ++c;
    }
    *num_copies = c;
    return PKV_OK;
}

extern "C" int kvpool_truncate(kvpool_t* p, int32_t* row, int32_t* num_held, int32_t length) {
    if (!p || !num_held) return PKV_ERR_NULL_POINTER;
    if (length < 0 || *num_held < 0) return PKV_ERR_INVALID_ARGUMENT;
    const int64_t keep = (static_cast<int64_t>(length) + p->block_size - 1) / p->block_size;
    if (keep >= *num_held) return PKV_OK;
    if (!row) return PKV_ERR_NULL_POINTER;
    const int32_t k = static_cast<int32_t>(keep);
    const int rc = kvpool_free(p, *num_held - k, row + k);
    if (rc != PKV_OK) return rc;
    for (int32_t i = k; i < *num_held; ++i) row[i] = -1;
    *num_held = k;
    return PKV_OK;
}
