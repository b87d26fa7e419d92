#pragma once
// Which sequences a shared-prefix group serves (pa_decode_grouped).
//
// Groups are given as consecutive ranges of sequences (group_start, read as an ascending
// array) with the number of leading spans their members share (group_parts); which blocks
// a batch shares is the allocator's knowledge ("PagedAttention" concept report
// (compassingai.com) §6: blocks shared by reference count).  The device checks every
// member before its shared spans are read once for the whole group, so a group described
// wrongly costs speed, never results: a sequence the check rejects attends to its whole
// context itself.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

struct GroupPlanArgs {
    const int32_t *block_tables;
    const int32_t *context_lens;
    const int32_t *group_start;  // [num_groups + 1]
    const int32_t *group_parts;  // [num_groups]
    int num_seqs;
    int num_groups;
    int max_blocks_per_seq;
    int log2_block;
    int num_blocks;
    int span;             // tokens per shared span (a multiple of the block size)
    int group_rows;       // most members a group may have
    int max_group_parts;  // bound on group_parts[j]
};

// Called by a whole wave with the same s (lookups spread over the lanes); the result is
// uniform.  Sequence s belongs to group j = (number of group starts <= s) - 1; it is
// served when that group is well formed (0 <= start <= s < next start <= num_seqs, at
// most group_rows members, 1 <= parts <= max_group_parts), its shared tokens end before
// its newest one (parts * span <= ctx - 1), and its table reaches every shared block
// through the same entry as the group's first sequence, inside the pool.  j and parts are
// set whether or not s is served.
__device__ inline bool group_serves(const GroupPlanArgs &p, int s, int lane, int &j, int &parts) {
    int count = 0;
    for (int base = 0; base < p.num_groups; base += 64) {
        const int i = base + lane;
        count += __popcll(__ballot(i < p.num_groups && p.group_start[i] <= s));
    }
    j = count - 1;
    bool ok = j >= 0;
    int s0 = 0;
    parts = 0;
    if (ok) {
        s0 = p.group_start[j];
        const int s1 = p.group_start[j + 1];
        parts = p.group_parts[j];
        ok = s0 >= 0 && s0 <= s && s < s1 && s1 <= p.num_seqs && s1 - s0 <= p.group_rows && parts >= 1 &&
             parts <= p.max_group_parts;
    }
    const int ctx = p.context_lens[s];
    const int64_t shared = (int64_t)parts * p.span;
    ok = ok && ctx >= 1 && shared <= (int64_t)ctx - 1;
    const int64_t nblk = shared >> p.log2_block;
    ok = ok && nblk <= p.max_blocks_per_seq;
    if (ok) {
        const int32_t *ts = p.block_tables + (int64_t)s * p.max_blocks_per_seq;
        const int32_t *t0 = p.block_tables + (int64_t)s0 * p.max_blocks_per_seq;
        bool bad = false;
        for (int k = lane; k < (int)nblk; k += 64) {
            const int32_t b = ts[k];
            bad |= b != t0[k] || b < 0 || b >= p.num_blocks;
        }
        ok = !__any(bad);
    }
    return ok;
}

// The same decision for a sequence s that the caller already places in group j (the
// group's start s0, next start s1 and parts read by the caller): true exactly when
// group_serves(p, s, ...) holds with that j and parts.  Every load it needs is known up
// front (the group starts, s's length, both tables' shared entries), so they are issued
// together: one memory round trip instead of three dependent ones.  The caller
// guarantees 0 <= s0, s < num_seqs (the loads are made with clamped indices, without a
// branch, and their results ignored where out of range).
__device__ inline bool group_serves_in(const GroupPlanArgs &p, int s, int j, int s0, int s1, int parts,
                                       int lane) {
    const int64_t shared = (int64_t)parts * p.span;
    const int64_t nblk = shared >> p.log2_block;
    const bool shape_ok = s0 >= 0 && s0 <= s && s < s1 && s1 <= p.num_seqs && s1 - s0 <= p.group_rows &&
                          parts >= 1 && parts <= p.max_group_parts && nblk <= p.max_blocks_per_seq;
    if (p.num_groups <= 64 && nblk <= 64) {
        // one lookup of each kind per lane, all issued before any is used
        const int32_t *ts = p.block_tables + (int64_t)s * p.max_blocks_per_seq;
        const int32_t *t0 = p.block_tables + (int64_t)s0 * p.max_blocks_per_seq;
        const bool lk = shape_ok && lane < (int)nblk;
        const int kl = lk ? lane : 0;  // index 0 lies in every table row and group array
        const int32_t b = ts[kl];
        const int32_t b0 = t0[kl];
        const int gs = p.group_start[lane < p.num_groups ? lane : 0];
        const int ctx = p.context_lens[s];
        // every term evaluated (no short circuit, which would sink the table loads behind
        // the group-start comparison)
        const bool bad = __any(lk & ((b != b0) | (b < 0) | (b >= p.num_blocks)));
        const int count = __popcll(__ballot((lane < p.num_groups) & (gs <= s)));
        return shape_ok & (count - 1 == j) & (ctx >= 1) & (shared <= (int64_t)ctx - 1) & !bad;
    }
    bool bad = !shape_ok;
    if (shape_ok) {
        const int32_t *ts = p.block_tables + (int64_t)s * p.max_blocks_per_seq;
        const int32_t *t0 = p.block_tables + (int64_t)s0 * p.max_blocks_per_seq;
        for (int k = lane; k < (int)nblk; k += 64) {
            const int32_t b = ts[k];
            bad |= b != t0[k] || b < 0 || b >= p.num_blocks;
        }
    }
    const int ctx = shape_ok ? p.context_lens[s] : 0;
    int count = 0;
    for (int base = 0; base < p.num_groups; base += 64) {
        const int i = base + lane;
        count += __popcll(__ballot(i < p.num_groups && p.group_start[i] <= s));
    }
    return shape_ok && count - 1 == j && ctx >= 1 && shared <= (int64_t)ctx - 1 && !__any(bad);
}

}  // namespace pa
