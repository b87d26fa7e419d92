// Host block allocator behind the pa_alloc_* entry points.
//
// "vLLM PagedAttention 技术深度解析" (kwkr.cn) §1.2.2: a sequence starts with an empty
// table and takes a block from the pool whenever its last block is full; on exit its
// blocks go back.  §1.3.2: shared prefixes with copy-on-write and reference counts,
// a block is released only when nobody holds it.  "PagedAttention" concept report
// (compassingai.com) §6: a write into a block whose count exceeds one first moves the
// writer to a fresh copy; §11: free blocks live in one free list; §13: an exhausted
// pool is an explicit out-of-memory error that leaves running work untouched.
//
// Every operation is O(1) except fork/free/table export (O(table length)) and the
// statistics (O(blocks in use)).  One mutex per allocator serialises callers.  A batch
// of appends is all or nothing: each append records what it changed, and a failure
// part-way undoes the earlier ones in reverse order (free stack order included).
#include <algorithm>
#include <mutex>
#include <new>
#include <unordered_map>
#include <vector>

#include "internal.h"

struct pa_allocator {
    int num_blocks;
    int block_size;
    std::vector<int32_t> free_stack;  // back() is popped next
    std::vector<int32_t> refs;
    struct Seq {
        std::vector<int32_t> table;
        int32_t ctx = 0;
    };
    std::unordered_map<int64_t, Seq> seqs;
    int64_t next_id = 0;
    std::mutex mu;

    int32_t pop() {
        int32_t b = free_stack.back();
        free_stack.pop_back();
        refs[b] = 1;
        return b;
    }

    // What one append changed, enough to undo it: the sequence, whether it pushed a
    // fresh block onto its table, and the block a copy-on-write replaced (-1: none).
    struct Undo {
        Seq *seq;
        bool pushed;
        int32_t replaced;
    };

    // One append; caller holds the mutex.  With `undo`, records the change.
    int append(int64_t sid, int32_t *slot, int32_t *cow_src, int32_t *cow_dst, Undo *undo = nullptr) {
        auto it = seqs.find(sid);
        if (it == seqs.end()) return pa::fail(PA_ERR_INVALID, "unknown sequence %lld", (long long)sid);
        Seq &s = it->second;
        const int32_t B = block_size;
        const int32_t off = s.ctx % B;
        *cow_src = -1;
        *cow_dst = -1;
        if (undo) *undo = Undo{&s, false, -1};
        if (off == 0) {
            if (free_stack.empty()) return pa::fail(PA_ERR_OOM, "no free block for sequence %lld", (long long)sid);
            const int32_t b = pop();
            s.table.push_back(b);
            *slot = b * B;
            if (undo) undo->pushed = true;
        } else {
            const int32_t last = s.table.back();
            if (refs[last] > 1) {
                if (free_stack.empty()) return pa::fail(PA_ERR_OOM, "no free block to copy block %d", last);
                const int32_t b = pop();
                refs[last] -= 1;
                s.table.back() = b;
                *cow_src = last;
                *cow_dst = b;
                *slot = b * B + off;
                if (undo) undo->replaced = last;
            } else {
                *slot = last * B + off;
            }
        }
        s.ctx += 1;
        return PA_OK;
    }

    // Reverse one recorded append (appends are undone newest first, so every block
    // returns to the free stack at the position it was popped from).
    void revert(const Undo &u) {
        Seq &s = *u.seq;
        s.ctx -= 1;
        if (u.pushed) {
            const int32_t b = s.table.back();
            s.table.pop_back();
            refs[b] = 0;
            free_stack.push_back(b);
        } else if (u.replaced >= 0) {
            const int32_t b = s.table.back();
            s.table.back() = u.replaced;
            refs[u.replaced] += 1;
            refs[b] = 0;
            free_stack.push_back(b);
        }
    }
};

extern "C" {

int pa_alloc_create(int num_blocks, int block_size, pa_allocator **out) {
    if (!out) return pa::fail(PA_ERR_INVALID, "out is NULL");
    *out = nullptr;
    if (num_blocks <= 0 || block_size <= 0)
        return pa::fail(PA_ERR_INVALID, "num_blocks=%d block_size=%d", num_blocks, block_size);
    if ((int64_t)num_blocks * block_size > INT32_MAX)
        return pa::fail(PA_ERR_INVALID, "num_blocks * block_size overflows int32 slots");
    pa_allocator *a = new (std::nothrow) pa_allocator();
    if (!a) return pa::fail(PA_ERR_OOM, "host allocation failed");
    a->num_blocks = num_blocks;
    a->block_size = block_size;
    a->refs.assign(num_blocks, 0);
    a->free_stack.resize(num_blocks);
    for (int i = 0; i < num_blocks; ++i) a->free_stack[i] = num_blocks - 1 - i;
    *out = a;
    return PA_OK;
}

void pa_alloc_destroy(pa_allocator *a) { delete a; }

int pa_alloc_set_free_order(pa_allocator *a, const int32_t *ids, int n) {
    if (!a || (!ids && n)) return pa::fail(PA_ERR_INVALID, "NULL argument");
    std::lock_guard<std::mutex> g(a->mu);
    if (n != a->num_blocks) return pa::fail(PA_ERR_INVALID, "need all %d blocks, got %d", a->num_blocks, n);
    for (int32_t r : a->refs)
        if (r) return pa::fail(PA_ERR_INVALID, "blocks are in use");
    std::vector<char> seen(a->num_blocks, 0);
    for (int i = 0; i < n; ++i) {
        if (ids[i] < 0 || ids[i] >= a->num_blocks || seen[ids[i]])
            return pa::fail(PA_ERR_INVALID, "ids is not a permutation (position %d)", i);
        seen[ids[i]] = 1;
    }
    for (int i = 0; i < n; ++i) a->free_stack[i] = ids[n - 1 - i];
    return PA_OK;
}

int pa_alloc_new_seq(pa_allocator *a, int64_t *seq) {
    if (!a || !seq) return pa::fail(PA_ERR_INVALID, "NULL argument");
    std::lock_guard<std::mutex> g(a->mu);
    const int64_t id = a->next_id++;
    a->seqs.emplace(id, pa_allocator::Seq());
    *seq = id;
    return PA_OK;
}

int pa_alloc_append_slot(pa_allocator *a, int64_t seq, int32_t *slot, int32_t *cow_src,
                         int32_t *cow_dst) {
    if (!a || !slot || !cow_src || !cow_dst) return pa::fail(PA_ERR_INVALID, "NULL argument");
    std::lock_guard<std::mutex> g(a->mu);
    return a->append(seq, slot, cow_src, cow_dst);
}

int pa_alloc_append_slots(pa_allocator *a, const int64_t *seqs, int n, int32_t *slots,
                          int32_t *cow_src, int32_t *cow_dst, int *num_cow, int *num_done) {
    if (num_done) *num_done = 0;
    if (num_cow) *num_cow = 0;
    if (!a || n < 0 || (n && (!seqs || !slots || !cow_src || !cow_dst)) || !num_cow)
        return pa::fail(PA_ERR_INVALID, "NULL argument or n < 0");
    std::lock_guard<std::mutex> g(a->mu);
    std::vector<pa_allocator::Undo> undo;
    try {
        undo.resize((size_t)n);
    } catch (const std::bad_alloc &) {
        return pa::fail(PA_ERR_OOM, "host allocation failed");
    }
    int ncow = 0;
    for (int i = 0; i < n; ++i) {
        int32_t s, cs, cd;
        const int rc = a->append(seqs[i], &s, &cs, &cd, &undo[(size_t)i]);
        if (rc != PA_OK) {
            // all or nothing: take back appends 0 .. i-1, newest first
            for (int j = i - 1; j >= 0; --j) a->revert(undo[(size_t)j]);
            pa::fail(rc, "append %d of %d (sequence %lld): %s; no append kept", i, n, (long long)seqs[i],
                     rc == PA_ERR_OOM ? "no free block" : "unknown sequence");
            return rc;
        }
        slots[i] = s;
        if (cs >= 0) {
            cow_src[ncow] = cs;
            cow_dst[ncow] = cd;
            ++ncow;
        }
    }
    *num_cow = ncow;
    if (num_done) *num_done = n;
    return PA_OK;
}

int pa_alloc_adopt(pa_allocator *a, int num_tokens, int64_t *seq, int32_t *block_ids, int cap) {
    if (!a || !seq || num_tokens < 0 || cap < 0 || (cap > 0 && !block_ids))
        return pa::fail(PA_ERR_INVALID, "bad argument");
    std::lock_guard<std::mutex> g(a->mu);
    const int64_t n = ((int64_t)num_tokens + a->block_size - 1) / a->block_size;
    if (n > cap) return pa::fail(PA_ERR_BOUNDS, "%lld blocks exceed cap %d", (long long)n, cap);
    if (n > (int64_t)a->free_stack.size())
        return pa::fail(PA_ERR_OOM, "%lld blocks wanted, %zu free", (long long)n, a->free_stack.size());
    pa_allocator::Seq sq;
    sq.ctx = num_tokens;
    for (int64_t j = 0; j < n; ++j) {
        const int32_t b = a->pop();
        sq.table.push_back(b);
        block_ids[j] = b;
    }
    const int64_t id = a->next_id++;
    a->seqs.emplace(id, std::move(sq));
    *seq = id;
    return PA_OK;
}

int pa_alloc_fork(pa_allocator *a, int64_t parent, int64_t *child) {
    if (!a || !child) return pa::fail(PA_ERR_INVALID, "NULL argument");
    std::lock_guard<std::mutex> g(a->mu);
    auto it = a->seqs.find(parent);
    if (it == a->seqs.end()) return pa::fail(PA_ERR_INVALID, "unknown sequence %lld", (long long)parent);
    pa_allocator::Seq c = it->second;  // copy before emplace may rehash
    for (int32_t b : c.table) a->refs[b] += 1;
    const int64_t id = a->next_id++;
    a->seqs.emplace(id, std::move(c));
    *child = id;
    return PA_OK;
}

int pa_alloc_free_seq(pa_allocator *a, int64_t seq) {
    if (!a) return pa::fail(PA_ERR_INVALID, "NULL argument");
    std::lock_guard<std::mutex> g(a->mu);
    auto it = a->seqs.find(seq);
    if (it == a->seqs.end()) return pa::fail(PA_ERR_INVALID, "unknown sequence %lld", (long long)seq);
    for (int32_t b : it->second.table)
        if (--a->refs[b] == 0) a->free_stack.push_back(b);
    a->seqs.erase(it);
    return PA_OK;
}

int pa_alloc_block_table(pa_allocator *a, int64_t seq, int32_t *out, int cap, int *num_blocks,
                         int *context_len) {
    if (!a || (cap > 0 && !out) || cap < 0) return pa::fail(PA_ERR_INVALID, "bad argument");
    std::lock_guard<std::mutex> g(a->mu);
    auto it = a->seqs.find(seq);
    if (it == a->seqs.end()) return pa::fail(PA_ERR_INVALID, "unknown sequence %lld", (long long)seq);
    const auto &t = it->second.table;
    const int n = (int)t.size();
    std::copy(t.begin(), t.begin() + std::min(n, cap), out);
    if (num_blocks) *num_blocks = n;
    if (context_len) *context_len = it->second.ctx;
    if (n > cap) return pa::fail(PA_ERR_BOUNDS, "table of %d blocks exceeds cap %d", n, cap);
    return PA_OK;
}

int pa_alloc_block_tables(pa_allocator *a, const int64_t *seqs, int n, int32_t *out,
                          int max_blocks_per_seq, int32_t *context_lens) {
    if (!a || n < 0 || max_blocks_per_seq <= 0 || (n && (!seqs || !out || !context_lens)))
        return pa::fail(PA_ERR_INVALID, "bad argument");
    std::lock_guard<std::mutex> g(a->mu);
    for (int i = 0; i < n; ++i) {
        auto it = a->seqs.find(seqs[i]);
        if (it == a->seqs.end()) return pa::fail(PA_ERR_INVALID, "unknown sequence %lld", (long long)seqs[i]);
        const auto &t = it->second.table;
        if ((int)t.size() > max_blocks_per_seq)
            return pa::fail(PA_ERR_BOUNDS, "sequence %lld has %zu blocks > %d", (long long)seqs[i],
                            t.size(), max_blocks_per_seq);
        int32_t *row = out + (int64_t)i * max_blocks_per_seq;
        std::copy(t.begin(), t.end(), row);
        std::fill(row + t.size(), row + max_blocks_per_seq, -1);
        context_lens[i] = it->second.ctx;
    }
    return PA_OK;
}

int pa_alloc_refcount(pa_allocator *a, int32_t block, int *refcount) {
    if (!a || !refcount) return pa::fail(PA_ERR_INVALID, "NULL argument");
    std::lock_guard<std::mutex> g(a->mu);
    if (block < 0 || block >= a->num_blocks) return pa::fail(PA_ERR_BOUNDS, "block %d", block);
    *refcount = a->refs[block];
    return PA_OK;
}

int pa_alloc_get_stats(pa_allocator *a, pa_alloc_stats *out) {
    if (!a || !out) return pa::fail(PA_ERR_INVALID, "NULL argument");
    std::lock_guard<std::mutex> g(a->mu);
    pa_alloc_stats s{};
    s.total_blocks = a->num_blocks;
    s.free_blocks = (int64_t)a->free_stack.size();
    for (int32_t r : a->refs) {
        s.used_blocks += r > 0;
        s.shared_blocks += r > 1;
    }
    s.num_seqs = (int64_t)a->seqs.size();
    // filled slots per block: the largest fill any holder sees (a shared block counts once)
    std::unordered_map<int32_t, int32_t> fill;
    const int32_t B = a->block_size;
    for (const auto &kv : a->seqs) {
        const auto &sq = kv.second;
        s.logical_tokens += sq.ctx;
        for (size_t j = 0; j < sq.table.size(); ++j) {
            const int32_t f = std::min<int32_t>(B, sq.ctx - (int32_t)j * B);
            int32_t &cur = fill[sq.table[j]];
            cur = std::max(cur, f);
        }
    }
    for (const auto &kv : fill) s.stored_tokens += kv.second;
    s.wasted_slots = s.used_blocks * B - s.stored_tokens;
    // kwkr.cn §1.4.1 monitoring figures and compassingai.com §7 EMU (ratios of the
    // counts above, each 0 when its denominator is)
    const double slots_total = (double)s.total_blocks * B;
    const double slots_used = (double)s.used_blocks * B;
    s.block_utilisation = (double)s.used_blocks / (double)s.total_blocks;
    s.sharing_rate = (double)s.shared_blocks / (double)s.total_blocks;
    s.fragmentation_rate = (double)s.wasted_slots / slots_total;
    s.emu = s.used_blocks > 0 ? (double)s.stored_tokens / slots_used : 0.0;
    *out = s;
    return PA_OK;
}

}  // extern "C"
