#pragma once
// Several causal query tokens per sequence over the paged cache, on the matrix cores
// (gfx950 MFMA): the chunked-prefill / prefix-cache-hit case ("PagedAttention 深度解析"
// (5ulink.com) §六 item 5) of the same attention through the block table ("PagedAttention"
// concept report (compassingai.com) §5 and §8).  Sequence s has n_s query tokens, the
// last n_s positions of its context (their K/V already cached); the token at position
// p attends to the cached tokens t <= p.
//
// A workgroup takes one (KV head, sequence, tile of 128 query rows), a row being one
// (query token, query head of the group) pair: 128 / g tokens times the g heads that
// share the KV head.  Each of its four waves owns 32 rows (two 16-row fragments that
// share every operand read).  The workgroup walks the keys its rows can see ([0, last
// row's position]) in tiles of 32 keys (64 at d = 64, the same bytes); every tile is
// loaded once, through the block table, straight from HBM into one of three LDS buffers
// (global_load_lds, 1 KiB per load, no register staging) two tiles ahead of use, and all
// four waves read it there.  In LDS a row's 16-byte pieces are permuted (an XOR of the
// piece index with a function of the row), which keeps both operand reads below free
// of bank conflicts without padding.  Per tile and wave:
//
//   S^T[t][r]  = sum_d K[t][d] Q[r][d]          A = K rows (16 keys x 32 d), B = Q^T
//   O^T[d][r] += sum_t V[t][d] P[r][t]          A = V^T (16 d x 32 keys),   B = P^T
//
// on v_mfma_f32_16x16x32_{f16,bf16}.  Lane l supplies A[l%16][8(l/16)..+8] and
// B[8(l/16)..+8][l%16] and receives D[4(l/16)..+4][l%16], so the score fragment holds,
// per lane, one row's scores for keys 4q..4q+3 and 16+4q..16+4q+3: exactly a P^T
// operand once the V^T operand uses the same k order (two LDS transpose reads,
// ds_read_b64_tr_b16, of the V rows).  The causal mask compares each key's position with
// its row's.  Softmax is fp32 online in the exp2 domain;
// P enters the second product rounded to the storage type and the normaliser sums the
// rounded weights (on the matrix cores, P against a ones operand).  Rows are written by
// the wave that owns them (no merge).
//
// Workgroups are spread over the XCDs in contiguous ranges with the row tiles numbered
// fastest, so the row tiles that read the same sequence's blocks share an XCD's L2 (K and V
// are read with cacheable loads); within a range the sequences run longest first.
#include <hip/hip_runtime.h>

#include "decode_mfma.h"
#include "internal.h"
#include "kernel_common.h"

namespace pa {
namespace mq {

using mfma::Mma;
using mfma::f32x4;
#ifndef PA_MQ_WAVES
#define PA_MQ_WAVES 4
#endif
constexpr int MW = PA_MQ_WAVES;  // waves per workgroup
#ifndef PA_MQ_FRAGS
#define PA_MQ_FRAGS 2
#endif
#ifndef PA_MQ_KEYS
#define PA_MQ_KEYS 32
#endif
#ifndef PA_MQ_LPT
#define PA_MQ_LPT 1
#endif
#ifndef PA_MQ_WAVES_PER_EU
#define PA_MQ_WAVES_PER_EU 3  // waves per SIMD the register allocation must allow
#endif
// 16-row query fragments per wave.  Four halve the LDS reads per product but need more
// than 256 registers (one wave per SIMD), which measured 1.4x slower than two; one (8
// waves of 16 rows, 4 waves per SIMD) measured 0.239 of the matrix-core peak against
// 0.277 with two.
constexpr int RF = PA_MQ_FRAGS;
constexpr int ROWS = 16 * RF * MW;   // query rows per workgroup
static_assert(PA_MQ_KEYS % 32 == 0 && (RF == 1 || RF == 2 || RF == 4), "tile shape");

// Two fp32 weights rounded to T (to nearest even) and packed, the first in the low half
// (one v_cvt_pk_{f16,bf16}_f32 on gfx950).
template <typename T>
__device__ inline uint32_t round2(float a, float b);
template <>
__device__ inline uint32_t round2<F16>(float a, float b) {
    typedef float f2 __attribute__((ext_vector_type(2)));
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f2{a, b}), h2));
}
template <>
__device__ inline uint32_t round2<BF16>(float a, float b) {
    typedef float f2 __attribute__((ext_vector_type(2)));
    typedef __bf16 b2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f2{a, b}), b2));
}

template <typename T, int D, int G>
__global__ __launch_bounds__(MW * 64) __attribute__((amdgpu_waves_per_eu(PA_MQ_WAVES_PER_EU))) void multi_query_kernel(
    void *__restrict__ out, const uint8_t *__restrict__ query, const uint8_t *__restrict__ key_cache,
    const uint8_t *__restrict__ value_cache, const int32_t *__restrict__ block_tables,
    const int32_t *__restrict__ context_lens, const int32_t *__restrict__ query_start,
    int max_blocks_per_seq, int num_seqs, int num_kv_heads, int num_query_tokens, int tiles_per_seq,
    int max_query_len, int log2_block, int num_blocks, float scale_log2) {
    constexpr int ROW = D * 2;             // bytes per token row
    constexpr int KT = PA_MQ_KEYS * (D == 64 ? 2 : 1);  // keys per tile: the same bytes at d = 64
    constexpr int NKK = D / 32;            // 32-wide d steps of the score product
    constexpr int NN = D / 16;             // 16-row d fragments of the output
    constexpr int NT = KT / 16;            // 16-key score operands per tile
    constexpr int NH = KT / 32;            // 32-key value products per tile
    // rows unpadded, their 16-byte pieces permuted (swz): every 1 KiB of a tile is one
    // direct load of the workgroup
    constexpr int KBYTES = KT * ROW;
    constexpr int BUF = 2 * KBYTES;  // one tile: K rows, then V rows

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int n = lane & 15;  // query row of a fragment / key row within a 16-key operand
    const int q = lane >> 4;  // k group

    // Contiguous ranges of workgroups per XCD; within an XCD's range the row tiles run
    // fastest, then its KV heads, then the sequences longest first (the last workgroups
    // dispatched are the shortest).  Batches of up to MW * 64 sequences are sorted.
    const int L = xcd_remap(blockIdx.x, gridDim.x);
    const int tile = L % tiles_per_seq;
    const int rest = L / tiles_per_seq;
    int rank, kvh;
    if (PA_MQ_LPT && num_kv_heads % 8 == 0) {
        const int hx = num_kv_heads / 8;  // KV heads per XCD
        const int per_xcd = num_seqs * hx;
        const int r = rest % per_xcd;
        rank = r / hx;
        kvh = (rest / per_xcd) * hx + r % hx;
    } else {
        rank = rest % num_seqs;
        kvh = rest / num_seqs;
    }
    __shared__ uint32_t sm_order[MW * 64];
    int s = PA_MQ_LPT && num_seqs <= MW * 64 ? longest_first<MW * 64>(context_lens, num_seqs, rank, sm_order) : rank;
    s = __builtin_amdgcn_readfirstlane(s);
    const int num_q_heads = num_kv_heads * G;

    const int ctx = context_lens[s];
    const int q0 = query_start[s];
    const int nq = query_start[s + 1] - q0;
    const int rows = nq * G;  // flattened (token, head) rows of the sequence
    if (nq <= 0 || ROWS * tile >= rows) return;
    const bool bad_len = ctx < 0 || nq > ctx || nq > max_query_len;

    // this lane's rows (one per fragment f: token ti, head g) and their positions; the
    // wave's and the workgroup's last positions bound the keys they read
    const int wrow0 = ROWS * tile + 16 * RF * wave;  // first row of the wave
    // this lane's row of fragment f: its query-token row of query / out (-1: none) and
    // query head, computed where needed (not held through the key loop)
    auto row_io = [&](int f, int &gh) -> int64_t {
        const int r = wrow0 + 16 * f + n;
        const bool ok = r < rows;
        const int ti = (ok ? r : rows - 1) / G;
        gh = (ok ? r : rows - 1) % G;
        const int64_t orow = (int64_t)q0 + ti;
        return ok && orow >= 0 && orow < num_query_tokens ? orow : -1;
    };
    int pos[RF];
#pragma unroll
    for (int f = 0; f < RF; ++f) pos[f] = ctx - nq + (min(wrow0 + 16 * f + n, rows - 1)) / G;
    const int wg_last = min(rows, ROWS * tile + ROWS) - 1;
    const int end = bad_len ? 0 : ctx - nq + wg_last / G + 1;  // keys the workgroup reads

    // three buffers, each its own variable: the compiler then tells a buffer's LDS reads
    // from direct loads into another and does not wait for those
    __shared__ __attribute__((aligned(1024))) uint8_t lds0[BUF];
    __shared__ __attribute__((aligned(1024))) uint8_t lds1[BUF];
    __shared__ __attribute__((aligned(1024))) uint8_t lds2[BUF];

    const int block_size = 1 << log2_block;
    const int32_t *table = block_tables + (int64_t)s * max_blocks_per_seq;
    const int64_t head_off = (int64_t)kvh * block_size * ROW;
    const int64_t block_bytes = (int64_t)num_kv_heads * block_size * ROW;

    // Q^T operands: lane holds Q[row n of fragment f][32 kk + 8 q .. +8]; rows past the
    // sequence are zero
    u32x4 qb[RF][NKK];
#pragma unroll
    for (int f = 0; f < RF; ++f) {
        int gh;
        const int64_t orow = row_io(f, gh);
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) {
            qb[f][kk] = u32x4{0, 0, 0, 0};
            if (orow >= 0)
                qb[f][kk] = *(const u32x4 *)(query + ((orow * num_q_heads + kvh * G + gh) * D + 32 * kk + 8 * q) * 2);
        }
    }

    // Scores stay unscaled until the exponent: exp2(s * x - m) with s = |scale * log2 e| > 0,
    // so the running max can be taken on raw products (a negative scale flips the sign
    // of q instead, which is exact).
    const float sl = fabsf(scale_log2);
    if (scale_log2 < 0.f) {
#pragma unroll
        for (int f = 0; f < RF; ++f)
#pragma unroll
            for (int kk = 0; kk < NKK; ++kk) qb[f][kk] ^= u32x4{0x80008000u, 0x80008000u, 0x80008000u, 0x80008000u};
    }
    // first key position any of the wave's rows cannot see: tiles below it need no mask
    const int wave_first_pos = ctx - nq + min(wrow0, rows - 1) / G;

    // Per row: m, the reference max the weights are taken against (scaled; the same in a
    // column's 4 lanes); o, the weighted value sums; osum, the sum of the rounded weights,
    // formed on the matrix cores as the product of P with a ones operand (every element
    // of a lane's fragment holds its row's sum).  The reference only moves, and o and
    // osum are only rescaled, when a row's max exceeds it by more than 2^RESCALE_LOG2,
    // so the weights stay in (0, 2^RESCALE_LOG2]: the result is the same up to rounding.
    constexpr float RESCALE_LOG2 = 8.f;
    const uint32_t one2 = std::is_same<T, F16>::value ? 0x3C003C00u : 0x3F803F80u;  // two 1.0s
    const u32x4 ones = u32x4{one2, one2, one2, one2};
    float m[RF];
    f32x4 o[RF][NN], osum[RF];
#pragma unroll
    for (int f = 0; f < RF; ++f) {
        m[f] = -INFINITY;
        osum[f] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < NN; ++i) o[f][i] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    bool bad = bad_len;
    // per fragment: the raw product above which a row's reference must move
    const float inv_sl = 1.f / sl;
    float bound[RF];
#pragma unroll
    for (int f = 0; f < RF; ++f) bound[f] = -INFINITY;

    const int ntiles = (end + KT - 1) / KT;

    typedef short s16x4 __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) uint8_t lds_u8;
    // Piece permutation: piece c of row r (16 bytes) sits at piece c ^ swz(r % 16) of the
    // row.  The 16 rows one K operand read touches (same piece), and the 8 rows half a V
    // transpose read touches (32 bytes each), then lie in different banks.
    auto swz = [](int r) -> int {
        r &= 15;
        return D == 128 ? 2 * (r & 7) + ((r >> 3) & 1) : 2 * ((r >> 1) & 3) + ((r >> 3) & 1);
    };
    // Direct loads: a tile's K (then V) is KBYTES / 1024 loads of 1 KiB, NI per wave; load j
    // fills rows j * RPL .. + RPL (one 16-key group); lane l writes LDS bytes 16 l of it, so
    // it fetches the global piece that the permutation puts there.
    constexpr int RPL = 1024 / ROW;           // rows per load
    constexpr int NI = KBYTES / 1024 / MW;    // loads of K (and of V) per wave and tile
    static_assert(NI * MW * 1024 == KBYTES && RPL <= 16, "a tile must divide into 1 KiB loads per wave");
    uint32_t gofs[NI];                        // lane's byte offset in its 16-key group
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        const int j = wave * NI + i;
        const int r = j * RPL + (16 * lane) / ROW;
        const int p = ((16 * lane) % ROW) / 16;
        gofs[i] = (uint32_t)((r & 15) * ROW + 16 * (p ^ swz(r)));
    }
    // The table entry of this wave's 16-key group of the next tile to issue (a wave's
    // loads of a tile lie in one group), looked up one tile ahead so that no issue waits
    // for it: the entry, -1 (no data) or -2 (past the table row).
    static_assert(NI * RPL <= 16 && 16 % (NI * RPL) == 0, "a wave's loads of a tile share one 16-key group");
    const int wgrp = __builtin_amdgcn_readfirstlane((wave * NI * RPL) >> 4);
    int32_t ent = -1;
    auto lookup = [&](int t) {
        const int kj = t * KT + 16 * wgrp;
        ent = -1;
        if (kj < end) {
            const int lb = kj >> log2_block;
            ent = lb < max_blocks_per_seq ? table[lb] : -2;
        }
    };
    // issue tile t's loads into buf (block 0's rows where a group has no data: inside the
    // pool; masked, and V rows past the end zeroed once landed), then look up tile t + 1
    auto issue = [&](uint8_t *buf, int t) {
        const int kj = t * KT + 16 * wgrp;
#pragma unroll
        for (int i = 0; i < NI; ++i) asm volatile("" : "+v"(gofs[i]));
        int64_t b = 0;
        if (ent != -1) {
            if (ent >= 0 && ent < num_blocks)
                b = (int64_t)ent * block_bytes + head_off + (int64_t)(kj & (block_size - 1)) * ROW;
            else
                bad = true;
        }
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const int j = wave * NI + i;
            __builtin_amdgcn_global_load_lds((const void *)(key_cache + b + gofs[i]),
                                             (__attribute__((address_space(3))) void *)(buf + j * 1024), 16, 0, 0);
            __builtin_amdgcn_global_load_lds((const void *)(value_cache + b + gofs[i]),
                                             (__attribute__((address_space(3))) void *)(buf + KBYTES + j * 1024), 16,
                                             0, 0);
        }
        lookup(t + 1);
    };
    // this wave's loads of every tile but the newest issued have landed (2 NI loads per
    // tile in flight at most: s_waitcnt vmcnt(2 NI), gfx9 encoding with expcnt 7, lgkmcnt 15)
    auto wait_previous = [&]() {
        constexpr int V = 2 * NI;
        __builtin_amdgcn_s_waitcnt((V & 15) | ((V >> 4) << 14) | (7 << 4) | (15 << 8));
    };
    // Workgroup barrier that leaves the newest tile's loads in flight: __syncthreads()
    // would wait for every load (its release fence covers loads into LDS).  Each wave has
    // already waited for its own loads of the tile the others read next (wait_previous);
    // it waits for its own LDS operations (zeroing, reads of the buffer about to be
    // refilled), then meets the others.  The signal fences keep the compiler from moving
    // memory operations across.
    auto barrier = [&]() {
        __builtin_amdgcn_s_waitcnt((63 & 15) | ((63 >> 4) << 14) | (7 << 4) | (0 << 8));  // lgkmcnt(0)
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        __builtin_amdgcn_s_barrier();
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
    };
    // V rows of tile t at or past `end` as zeros (this wave's pieces, once landed): their
    // weight is 0, and 0 * NaN would poison the product
    auto zero_tail = [&](uint8_t *buf, int t) {
        const int k0 = t * KT;
        if (k0 + KT > end) {
#pragma unroll
            for (int i = 0; i < NI; ++i) {
                const int j = wave * NI + i;
                const int r = j * RPL + (16 * lane) / ROW;
                if (k0 + r >= end) *(u32x4 *)(buf + KBYTES + j * 1024 + 16 * lane) = u32x4{0, 0, 0, 0};
            }
        }
    };
    // operand read offsets of the lane (constant over tiles): K piece 4 kk + q of row n;
    // V 8 bytes of row 4 q + n / 4 at byte 32 nn + 8 (n % 4) (the rows 16 and 32 further
    // share the permutation)
    uint32_t kofs[NKK], vofs[NN];
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) kofs[kk] = (uint32_t)(n * ROW + 16 * ((4 * kk + q) ^ swz(n)));
#pragma unroll
    for (int nn = 0; nn < NN; ++nn) {
        const int r = 4 * q + (n >> 2);
        vofs[nn] = (uint32_t)(KBYTES + r * ROW + 16 * ((2 * nn + ((n & 3) >> 1)) ^ swz(r)) + 8 * (n & 1));
    }
    auto k_at = [&](const uint8_t *buf, int tt, int kk) -> u32x4 {
        return *(const u32x4 *)(buf + 16 * tt * ROW + kofs[kk]);
    };
    auto v_base = [&](const uint8_t *buf) -> const uint8_t * { return buf; };
    auto read_v = [&](const uint8_t *vb, int nn, int h) -> u32x4 {
        const lds_u8 *r0 = (const lds_u8 *)vb + vofs[nn] + 32 * h * ROW;
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4 *)(r0));
        const s16x4 hi =
            __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4 *)(r0 + 16 * ROW));
        const uint2 lw = __builtin_bit_cast(uint2, lo), hw = __builtin_bit_cast(uint2, hi);
        return u32x4{lw.x, lw.y, hw.x, hw.y};
    };
    typedef float Scores[RF][NT][4];
    // scores S^T of the tile in buf: lane holds keys 16 tt + 4 q + i of row n of each
    // fragment (raw products; the scale enters at the exponent)
    auto scores = [&](const uint8_t *buf, Scores &sc) {
#pragma unroll
        for (int tt = 0; tt < NT; ++tt) {
            f32x4 acc[RF];
#pragma unroll
            for (int f = 0; f < RF; ++f) acc[f] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < NKK; ++kk) {
                const u32x4 ka = k_at(buf, tt, kk);
#pragma unroll
                for (int f = 0; f < RF; ++f) acc[f] = Mma<T>::run(ka, qb[f][kk], acc[f]);
            }
#pragma unroll
            for (int f = 0; f < RF; ++f)
#pragma unroll
                for (int i = 0; i < 4; ++i) sc[f][tt][i] = acc[f][i];
        }
    };
    // causal mask of tile t: keys past each row's position (only tiles that reach past the
    // wave's first row need it)
    auto mask = [&](Scores &sc, int t) {
        const int k0 = t * KT;
        if (k0 + KT - 1 > wave_first_pos) {
#pragma unroll
            for (int tt = 0; tt < NT; ++tt)
#pragma unroll
                for (int f = 0; f < RF; ++f)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        if (k0 + 16 * tt + 4 * q + i > pos[f]) sc[f][tt][i] = -INFINITY;
        }
    };
    auto rescale = [&](const float (&alpha)[RF]) {
#pragma unroll
        for (int f = 0; f < RF; ++f) {
            osum[f] *= alpha[f];
#pragma unroll
            for (int nn = 0; nn < NN; ++nn) o[f][nn] *= alpha[f];
        }
    };
    // online softmax of a tile's (masked) scores, first half: the reference a row's weights
    // are taken against only moves when the row's scores pass it by more than
    // 2^RESCALE_LOG2.  Each lane compares its own scores with that bound (raw products
    // against (m + RESCALE_LOG2) / sl); only when some lane's pass does the wave take the
    // rows' maxima over their 4 lanes and move the references (alpha: the factor for the
    // sums so far).  ms: the reference the weights are taken against.
    auto row_max = [&](const Scores &sc, float (&alpha)[RF], float (&ms)[RF]) {
        bool pass = false;
        float lm[RF];
#pragma unroll
        for (int f = 0; f < RF; ++f) {
            float cm = sc[f][0][0];
#pragma unroll
            for (int tt = 0; tt < NT; ++tt)
#pragma unroll
                for (int i = 0; i < 4; ++i) cm = fmaxf(cm, sc[f][tt][i]);
            lm[f] = cm;
            pass |= cm > bound[f];
            alpha[f] = 1.f;
        }
        if (__any(pass)) {
#pragma unroll
            for (int f = 0; f < RF; ++f) {
                const float mt = max_over_column(lm[f]) * sl;  // the tile's max of the row
                const bool g = mt > m[f] + RESCALE_LOG2;
                alpha[f] = g ? fast_exp2(m[f] - mt) : 1.f;
                m[f] = g ? mt : m[f];
                bound[f] = (m[f] + RESCALE_LOG2) * inv_sl;
            }
            rescale(alpha);
        }
#pragma unroll
        for (int f = 0; f < RF; ++f) ms[f] = m[f] == -INFINITY ? 0.f : m[f];
    };
    // second half: the weights, as P^T operands per 32-key half h (k slot j < 4 -> key
    // 32h + 4q + j, j >= 4 -> key 32h + 16 + 4q + j - 4)
    auto weights = [&](const Scores &sc, const float (&ms)[RF], u32x4 (&pb)[RF][NH]) {
#pragma unroll
        for (int f = 0; f < RF; ++f)
#pragma unroll
            for (int h = 0; h < NH; ++h) {
                uint32_t pk[4];
#pragma unroll
                for (int u = 0; u < 2; ++u)
#pragma unroll
                    for (int i = 0; i < 4; i += 2)
                        pk[2 * u + i / 2] = round2<T>(fast_exp2(fmaf(sc[f][2 * h + u][i], sl, -ms[f])),
                                                      fast_exp2(fmaf(sc[f][2 * h + u][i + 1], sl, -ms[f])));
                pb[f][h] = u32x4{pk[0], pk[1], pk[2], pk[3]};
            }
    };
    // the normaliser (P against a ones operand) and the value product of the tile in buf
    auto values = [&](const uint8_t *buf, const u32x4 (&pb)[RF][NH]) {
        const auto vb = v_base(buf);
#pragma unroll
        for (int h = 0; h < NH; ++h)
#pragma unroll
            for (int f = 0; f < RF; ++f) osum[f] = Mma<T>::run(ones, pb[f][h], osum[f]);
#pragma unroll
        for (int nn = 0; nn < NN; ++nn) {
#pragma unroll
            for (int h = 0; h < NH; ++h) {
                // keys 32h + 4q .. +3, then 32h + 16 + 4q .. +3, of d = 16 nn + n
                const u32x4 va = read_v(vb, nn, h);
#pragma unroll
                for (int f = 0; f < RF; ++f) o[f][nn] = Mma<T>::run(va, pb[f][h], o[f][nn]);
            }
        }
    };

    // a wave skips the tiles past its own last row
    const int wave_end = wrow0 < rows ? ctx - nq + (min(rows, wrow0 + 16 * RF) - 1) / G + 1 : 0;
    auto compute = [&](const uint8_t *buf, int t) {
        if (t * KT >= wave_end) return;
        // The operand offsets are opaque at each step (an empty asm): the compiler then folds
        // the buffer's constant LDS address into each read's offset field instead of keeping
        // offset + address copies per buffer live through the loop.
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) asm volatile("" : "+v"(kofs[kk]));
#pragma unroll
        for (int nn = 0; nn < NN; ++nn) asm volatile("" : "+v"(vofs[nn]));
        Scores sc;
        scores(buf, sc);
        mask(sc, t);
        float alpha[RF], ms[RF];
        row_max(sc, alpha, ms);
        u32x4 pb[RF][NH];
        weights(sc, ms, pb);
        values(buf, pb);
    };
    // Three buffers, tile t in buffer t % 3, loaded directly from HBM into LDS two tiles
    // ahead of use.  Step t: tile t + 2's loads are issued into the buffer tile t - 1 left,
    // tile t is used, the wave waits for its own loads of tile t + 1 (zeroing V rows past
    // the end), and one barrier makes every wave's loads of tile t + 1 visible and frees
    // buffer t % 3.  Loads past the last tile read block 0's rows and are never used.
    if (ntiles > 0) {
        lookup(0);
        issue(lds0, 0);
        issue(lds1, 1);
        wait_previous();
        zero_tail(lds0, 0);
        barrier();
        auto step = [&](uint8_t *cur, uint8_t *nxt, uint8_t *fre, int t) {
            issue(fre, t + 2);
            compute(cur, t);
            wait_previous();
            zero_tail(nxt, t + 1);
            barrier();
        };
        // whole rounds of three steps, then the last one or two: no path back into the loop
        // skips a step, so the compiler's wait before each buffer's reads stays exact (a
        // skipped step would leave that buffer's loads apparently in flight)
        int t = 0;
        for (; t + 2 < ntiles; t += 3) {
            step(lds0, lds1, lds2, t);
            step(lds1, lds2, lds0, t + 1);
            step(lds2, lds0, lds1, t + 2);
        }
        if (t < ntiles) step(lds0, lds1, lds2, t);
        if (t + 1 < ntiles) step(lds1, lds2, lds0, t + 1);
    }

    __shared__ int sm_bad;
    if (threadIdx.x == 0) sm_bad = 0;
    __syncthreads();
    if (bad) sm_bad = 1;
    __syncthreads();
    const bool any_bad = sm_bad != 0;
    // each wave writes its own rows; the normaliser of a row sums its column's 4 lanes
#pragma unroll
    for (int f = 0; f < RF; ++f) {
        const float l = osum[f][0];
        int gh;
        const int64_t orow = row_io(f, gh);
        if (orow < 0) continue;
        const float inv = l > 0.f ? 1.f / l : 0.f;
        const int64_t obase = (orow * num_q_heads + kvh * G + gh) * D;
#pragma unroll
        for (int nn = 0; nn < NN; ++nn)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float ov = any_bad ? NAN : o[f][nn][i] * inv;
                store_out<T>(out, obase + 16 * nn + 4 * q + i, ov);
            }
    }
}

template <typename T, int D, int G>
int launch_t(const DecodeArgs &a) {
    const int tiles = (a.max_query_len * G + ROWS - 1) / ROWS;
    const int64_t grid = (int64_t)a.num_kv_heads * a.num_seqs * tiles;
    if (grid > 0x7fffffff) return fail(PA_ERR_UNSUPPORTED, "grid of %lld workgroups", (long long)grid);
    hipLaunchKernelGGL((multi_query_kernel<T, D, G>), dim3((unsigned)grid), dim3(MW * 64), 0,
                       (hipStream_t)a.stream, a.out, (const uint8_t *)a.query, (const uint8_t *)a.key_cache,
                       (const uint8_t *)a.value_cache, a.block_tables, a.context_lens, a.query_start,
                       a.max_blocks_per_seq, a.num_seqs, a.num_kv_heads, a.num_query_tokens, tiles,
                       a.max_query_len, __builtin_ctz(a.block_size), a.num_blocks, a.scale_log2);
    return check_launch("multi_query");
}

template <typename T, int D>
int by_group(const DecodeArgs &a) {
    switch (a.num_q_heads / a.num_kv_heads) {
        case 1: return launch_t<T, D, 1>(a);
        case 2: return launch_t<T, D, 2>(a);
        case 4: return launch_t<T, D, 4>(a);
        case 8: return launch_t<T, D, 8>(a);
        case 16: return launch_t<T, D, 16>(a);
    }
    return fail(PA_ERR_UNSUPPORTED, "group %d", a.num_q_heads / a.num_kv_heads);
}

template <typename T>
int by_dim(const DecodeArgs &a) {
    if (a.head_dim == 64) return by_group<T, 64>(a);
    if (a.head_dim == 128) return by_group<T, 128>(a);
    return fail(PA_ERR_UNSUPPORTED, "head_dim %d", a.head_dim);
}

}  // namespace mq
}  // namespace pa
