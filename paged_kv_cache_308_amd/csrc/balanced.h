#pragma once
// Balanced split, shared by the vector and the matrix-core decode kernels.
//
// The batch's work is one ordered list of fixed-size chunks (KV head, then sequence,
// then chunk of the sequence), optionally with a few units ahead of each item's chunks
// that stand for the cost of starting it.  Each of W workers (waves of the vector
// kernel, workgroups of the matrix-core one) takes an equal contiguous range of it;
// when a worker finishes the chunks of a (sequence, KV head) item that lie in its
// range it writes that item's partial (running max, sum and weighted value sums per
// query head) to slot `worker + item`; a range holding none of an item's chunks
// writes nothing for it.  Ranges and items are both ordered, so two
// (worker, item) pairs that share a slot would need a later worker on an earlier item,
// which cannot happen.  balanced_merge_kernel combines each item's partials with
// log-sum-exp weights ("PagedAttention" concept report (compassingai.com) §8 defines
// the attention; the split changes only the order of the sums).
//
// Workspace header (int32), written by workgroup 0 of the decode launch: [0] units per
// KV head, [1] units per worker, [2] workers, [3] units ahead of each non-empty item's
// chunks (a share of the list that stands for the cost of starting an item; no worker
// reads anything for them), [4 + s] units of the sequences before s (s = 0..S).
#include <hip/hip_runtime.h>

#include "internal.h"
#include "kernel_common.h"

namespace pa {

constexpr int BAL_MAX_SEQS = kBalancedMaxSeqs;  // sequences per batch in balanced mode
constexpr int BAL_HDR = 4;          // header ints before the prefix

// Combine the partials of one (sequence, query head) written by the workers whose
// ranges cover it: out = sum_w 2^(m_w - M) acc_w / sum_w 2^(m_w - M) l_w.
template <typename T, int D, int G>
__global__ __launch_bounds__(64) void balanced_merge_kernel(
    void *__restrict__ out, const int32_t *__restrict__ ws_hdr, const float *__restrict__ ws_max,
    const float *__restrict__ ws_sum, const float *__restrict__ ws_acc,
    const int32_t *__restrict__ context_lens, int num_seqs, int num_kv_heads) {
    const int num_q_heads = num_kv_heads * G;
    const int sh = blockIdx.x;
    const int s = sh / num_q_heads;
    const int h = sh - s * num_q_heads;
    const int kvh = h / G;
    const int gg = h - kvh * G;
    const int64_t obase = (int64_t)sh * D;
    const int ctx = context_lens[s];
    const int per_head = ws_hdr[0];
    const int per = ws_hdr[1];
    const int ov = ws_hdr[3];
    const int first = ws_hdr[BAL_HDR + s];
    const int units = ws_hdr[BAL_HDR + s + 1] - first;
    const int n = units > ov ? units - ov : 0;  // chunks after the item's start units
    if (ctx < 0 || n == 0) {
        for (int j = threadIdx.x; j < D; j += 64) store_out<T>(out, obase + j, ctx < 0 ? NAN : 0.f);
        return;
    }
    const int g0 = kvh * per_head + first + ov;
    const int w0 = g0 / per, w1 = (g0 + n - 1) / per;
    const int64_t item = (int64_t)kvh * num_seqs + s;
    // Partials in groups of four, every load of a group issued together, folded into a
    // running (max, sum, weighted sums) with log-sum-exp rescaling.
    constexpr int JP = D / 64;  // output elements per thread
    constexpr int NB = 4;
    float M = -INFINITY, Lsum = 0.f, A[JP];
#pragma unroll
    for (int jj = 0; jj < JP; ++jj) A[jj] = 0.f;
    bool bad = false;
    for (int w = w0; w <= w1; w += NB) {
        float mw[NB], lw[NB], aw[NB][JP];
#pragma unroll
        for (int i = 0; i < NB; ++i) {
            const bool ok = w + i <= w1;
            const int64_t slot = ((int64_t)(ok ? w + i : w0) + item) * G + gg;  // always a written slot
            const float x = ws_max[slot];
            bad |= ok && x != x;
            mw[i] = ok ? x : -INFINITY;
            lw[i] = ok ? ws_sum[slot] : 0.f;
#pragma unroll
            for (int jj = 0; jj < JP; ++jj) aw[i][jj] = ok ? ws_acc[slot * D + threadIdx.x + 64 * jj] : 0.f;
        }
        float Mn = M;
#pragma unroll
        for (int i = 0; i < NB; ++i) Mn = fmaxf(Mn, mw[i]);
        const float Ms = Mn == -INFINITY ? 0.f : Mn;
        const float r = fast_exp2(M - Ms);
        Lsum *= r;
#pragma unroll
        for (int jj = 0; jj < JP; ++jj) A[jj] *= r;
#pragma unroll
        for (int i = 0; i < NB; ++i) {
            const float f = fast_exp2(mw[i] - Ms);
            Lsum += lw[i] * f;
#pragma unroll
            for (int jj = 0; jj < JP; ++jj) A[jj] += aw[i][jj] * f;
        }
        M = Mn;
    }
#pragma unroll
    for (int jj = 0; jj < JP; ++jj) {
        float o = Lsum > 0.f ? A[jj] / Lsum : 0.f;
        if (bad) o = NAN;
        store_out<T>(out, obase + threadIdx.x + 64 * jj, o);
    }
}

template <typename T, int D, int G>
int launch_balanced_merge(const DecodeArgs &a) {
    hipLaunchKernelGGL((balanced_merge_kernel<T, D, G>), dim3(a.num_seqs * a.num_q_heads), dim3(64), 0,
                       (hipStream_t)a.stream, a.out, a.ws_hdr, a.ws_max, a.ws_sum, a.ws_acc, a.context_lens,
                       a.num_seqs, a.num_kv_heads);
    return check_launch("balanced_merge");
}

}  // namespace pa
