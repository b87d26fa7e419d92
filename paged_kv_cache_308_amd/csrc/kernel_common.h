// Device helpers shared by the decode kernels (gfx950 / wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Storage element types.
struct F32 {
    static constexpr int bytes = 4;
};
struct F16 {
    static constexpr int bytes = 2;
};
struct BF16 {
    static constexpr int bytes = 2;
};

// 16 stored bytes -> fp32 values.
template <typename T>
__device__ inline void to_f32(const u32x4 &w, float (&f)[16 / T::bytes]);

template <>
__device__ inline void to_f32<F32>(const u32x4 &w, float (&f)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) f[i] = __uint_as_float(w[i]);
}
template <>
__device__ inline void to_f32<F16>(const u32x4 &w, float (&f)[8]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t x = w[i];  // bit_cast of a vector element would read element 0
        const f16x2 h = __builtin_bit_cast(f16x2, x);
        f[2 * i] = (float)h[0];
        f[2 * i + 1] = (float)h[1];
    }
}
template <>
__device__ inline void to_f32<BF16>(const u32x4 &w, float (&f)[8]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f[2 * i] = __uint_as_float(w[i] << 16);
        f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
}

// Dot product of two 16-byte slices, fp32 result.  16-bit types use the packed
// dot instructions (two products summed into an fp32 accumulator per op).
template <typename T>
__device__ inline float dot16(const u32x4 &a, const u32x4 &b);

template <>
__device__ inline float dot16<F32>(const u32x4 &a, const u32x4 &b) {
    float s = __uint_as_float(a[0]) * __uint_as_float(b[0]);
#pragma unroll
    for (int i = 1; i < 4; ++i) s = fmaf(__uint_as_float(a[i]), __uint_as_float(b[i]), s);
    return s;
}
template <>
__device__ inline float dot16<F16>(const u32x4 &a, const u32x4 &b) {
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t x = a[i], y = b[i];  // scalar copies: see to_f32<F16>
        s = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, x), __builtin_bit_cast(f16x2, y), s, false);
    }
    return s;
}
template <>
__device__ inline float dot16<BF16>(const u32x4 &a, const u32x4 &b) {
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t x = a[i], y = b[i];  // scalar copies: see to_f32<F16>
        s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, x), __builtin_bit_cast(bf16x2, y), s,
                                            false);
    }
    return s;
}

// K/V rows are read once per decode step unless blocks are shared between sequences:
// non-temporal loads keep them from displacing reusable lines (measured +8-10% on
// streaming batches); plain loads let sequences that share prefix blocks hit in L2.
template <bool NT, typename W>
__device__ inline W kv_load(const W *p) {
    if constexpr (NT)
        return __builtin_nontemporal_load(p);
    else
        return *p;
}

// DPP lane exchange inside 16-lane rows.
template <int CTRL>
__device__ inline float dpp(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// Sum over groups of N adjacent lanes (N = 4, 8, 16, 32); every lane of a group gets
// the same bits (each step adds a value to its mirror image, which commutes exactly).
template <int N>
__device__ inline float row_sum(float v) {
    static_assert(N == 4 || N == 8 || N == 16 || N == 32, "group size");
    v += dpp<0xB1>(v);   // quad_perm [1,0,3,2]: lane ^ 1
    v += dpp<0x4E>(v);   // quad_perm [2,3,0,1]: lane ^ 2
    if (N >= 8) v += dpp<0x141>(v);  // row_half_mirror: the other quad of each 8
    if (N >= 16) v += dpp<0x140>(v);  // row_mirror: the other half of each 16
    if (N >= 32) v += __shfl_xor(v, 16);
    return v;
}

// ---------------------------------------------------------------- E4M3 codes
// OCP E4M3 (bias 7, 3 fraction bits, no infinities, 0x7F / 0xFF NaN).  The gfx950
// conversion instructions widen two codes at a time, exactly (every E4M3 value is an
// f16, bf16 and f32 value); the scale operand is 1.

// Codes 2h, 2h+1 of a 4-code word (h = 0, 1) widened to a 16-bit pair.
template <typename T>
__device__ inline uint32_t e4m3_pair(uint32_t w, bool hi);
template <>
__device__ inline uint32_t e4m3_pair<F16>(uint32_t w, bool hi) {
    return __builtin_bit_cast(uint32_t, hi ? __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)w, 1.0f, true)
                                           : __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)w, 1.0f, false));
}
template <>
__device__ inline uint32_t e4m3_pair<BF16>(uint32_t w, bool hi) {
    return __builtin_bit_cast(uint32_t, hi ? __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w, 1.0f, true)
                                           : __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w, 1.0f, false));
}

// 4 * N codes (N = 4: u32x4, N = 2: u32x2) -> fp32.
template <int N, typename W>
__device__ inline void e4m3_to_f32(const W &w, float (&f)[4 * N]) {
    typedef float f32x2 __attribute__((ext_vector_type(2)));
#pragma unroll
    for (int i = 0; i < N; ++i) {
        const uint32_t x = w[i];  // scalar copy: see to_f32<F16>
        const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)x, false);
        const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)x, true);
        f[4 * i] = lo[0];
        f[4 * i + 1] = lo[1];
        f[4 * i + 2] = hi[0];
        f[4 * i + 3] = hi[1];
    }
}

// The E4M3 code nearest to y: round to nearest, ties to the even code; |y| >= 448 and
// infinities saturate to the largest finite code of y's sign; NaN gives 0x7F.
__device__ inline uint32_t e4m3_encode(float y) {
    const uint32_t u = __float_as_uint(y);
    const uint32_t sign = (u >> 24) & 0x80u;
    const uint32_t a = u & 0x7fffffffu;
    if (a > 0x7f800000u) return 0x7fu;        // NaN
    if (a >= 0x43e00000u) return sign | 0x7eu; // 448 = 1.75 * 2^8 and above
    if (a < 0x3c800000u) {                      // below 2^-6: multiples of 2^-9
        const float q = rintf(__uint_as_float(a) * 512.f);  // exact product, ties to even
        return sign | (uint32_t)q;              // 8 -> 0x08 = 2^-6, the first normal
    }
    // normal: keep 3 of the 23 fraction bits, ties to even (a carry bumps the exponent)
    const uint32_t r = a + 0x7ffffu + ((a >> 20) & 1u);
    const uint32_t e = (r >> 23) - 120u;        // rebias 127 -> 7
    return sign | (e << 3) | ((r >> 20) & 7u);
}

// Max and sum over the four lanes l, l ^ 16, l ^ 32, l ^ 48 of a wave (the 4 lanes of a
// matrix-core fragment column), every lane receiving the same value.  gfx950's
// v_permlane32_swap pairs each lane with lane ^ 32 and v_permlane16_swap with lane ^ 16,
// on the vector unit (no LDS round trip).
__device__ inline float max_over_column(float x) {
    const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ inline float sum_over_column(float x) {
    const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// 2^x on the hardware transcendental unit (exact 1 at 0, 0 at -inf).
__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Workgroup w is dispatched to XCD w % 8.  Number work items so that each XCD runs
// a contiguous range of them.
__device__ inline int xcd_remap(int w, int n) {
    constexpr int NX = 8;
    const int x = w % NX, k = w / NX;
    const int q = n / NX, r = n % NX;
    return x * q + (x < r ? x : r) + k;
}

// Longest-first order of a batch: the index of the sequence whose context is the
// rank-th longest (ties: lower index first; negative lengths count as 0), for batches
// of at most NTH sequences (NTH = threads of the calling workgroup, a power of two).
// Every workgroup computes the same order: a bitonic sort of (length, index) keys,
// one key per lane; a batch that fits one wave is sorted by every wave on its own
// with lane exchanges only, a larger one by the whole workgroup, the exchanges
// between waves going through LDS (`sm`, NTH words).  The caller guarantees
// num_seqs <= NTH and rank < num_seqs; uniform control flow (the barriers).
template <int NTH>
__device__ inline int longest_first(const int32_t *__restrict__ context_lens, int num_seqs, int rank,
                                    uint32_t *sm) {
    static_assert(NTH <= 1024 && (NTH & (NTH - 1)) == 0, "one key per thread, 10 index bits");
    constexpr uint32_t LEN_MAX = (1u << 22) - 1;  // 22 length bits above 10 index bits
    const int ns = num_seqs <= 1 ? 1 : 1 << (32 - __builtin_clz(num_seqs - 1));  // power of two >= S
    const bool wide = ns > 64;
    const int t = wide ? (int)threadIdx.x : (int)(threadIdx.x & 63);
    uint32_t key = 0;  // slots past the batch sort last
    if (t < num_seqs) {
        const int c = context_lens[t];
        const uint32_t len = c <= 0 ? 0u : ((uint32_t)c > LEN_MAX ? LEN_MAX : (uint32_t)c);
        key = (len << 10) | (1023u - (uint32_t)t);
    }
    for (int k = 2; k <= ns; k <<= 1) {
        for (int j = k >> 1; j > 0; j >>= 1) {
            uint32_t other;
            if (j >= 64) {
                sm[t] = key;
                __syncthreads();
                other = sm[t ^ j];
                __syncthreads();
            } else {
                other = (uint32_t)__shfl_xor((int)key, j);
            }
            // blocks of k alternate direction; the last (k = ns) runs descending
            const bool keep_max = ((t & j) == 0) == ((t & k) == 0);
            key = keep_max ? (key > other ? key : other) : (key < other ? key : other);
        }
    }
    uint32_t kr;
    if (wide) {
        sm[t] = key;
        __syncthreads();
        kr = sm[rank];
    } else {
        kr = (uint32_t)__shfl((int)key, rank);
    }
    return 1023 - (int)(kr & 1023u);
}

// Round fp32 to the output type (round to nearest even) and store element i.
template <typename T>
__device__ inline void store_out(void *out, int64_t i, float v);

template <>
__device__ inline void store_out<F32>(void *out, int64_t i, float v) {
    ((float *)out)[i] = v;
}
template <>
__device__ inline void store_out<F16>(void *out, int64_t i, float v) {
    ((_Float16 *)out)[i] = (_Float16)v;
}
template <>
__device__ inline void store_out<BF16>(void *out, int64_t i, float v) {
    uint32_t u = __float_as_uint(v);
    uint16_t r;
    if ((u & 0x7fffffffu) > 0x7f800000u)
        r = 0x7fc0;  // NaN
    else
        r = (uint16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
    ((uint16_t *)out)[i] = r;
}

}  // namespace pa
