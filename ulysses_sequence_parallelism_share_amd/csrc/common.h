// Shared device-side definitions for the gfx950 kernels of the Ulysses
// attention share: vector types, the MFMA wrapper and its accumulator
// layout, and fast division by run-time constants.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

#define SP_LOG2E 1.4426950408889634f
#define SP_LN2 0.6931471805599453f

// ---------------------------------------------------------------------------
// Division of non-negative 31-bit integers by a run-time constant d >= 1
// (Granlund & Montgomery, "Division by invariant integers using
// multiplication", PLDI 1994, round-up variant): with s = ceil(log2 d) and
// m = floor(2^32 (2^s - d) / d) + 1, n / d = (umulhi(n, m) + n) >> s for
// every n < 2^31.
// ---------------------------------------------------------------------------
struct FastDiv {
    uint32_t d, m, s;
};

static inline FastDiv make_fastdiv(uint32_t d) {
    FastDiv f;
    f.d = d;
    uint32_t s = 0;
    while ((1ull << s) < d) ++s;
    f.s = s;
    f.m = (uint32_t)((((1ull << s) - d) << 32) / d + 1);
    return f;
}

__device__ __forceinline__ uint32_t fdiv(uint32_t n, const FastDiv &f) {
    return (__umulhi(n, f.m) + n) >> f.s;
}

// ---------------------------------------------------------------------------
// MFMA 32x32x16, bf16 inputs, fp32 accumulate (v_mfma_f32_32x32x16_bf16).
// Lane l supplies row (A) / column (B) l % 32 and, for half l / 32, 8 of the
// 16 k-values; A and B pair the same (half, element) slots, so any fixed
// assignment of k-indices to slots that both operands share is valid.
// Result: lane l holds column l % 32; register r holds row
// (r / 4) * 8 + (l / 32) * 4 + r % 4.
// ---------------------------------------------------------------------------
__device__ __forceinline__ f32x16 mfma32(const bf16x8 &a, const bf16x8 &b, const f32x16 &c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Row of accumulator register r for lane half `half`.
__device__ __forceinline__ constexpr int acc_row(int r, int half) {
    return (r >> 2) * 8 + half * 4 + (r & 3);
}

__device__ __forceinline__ bf16x8 pack8(const f32x16 &a, int base) {
    bf16x8 r;
#pragma unroll
    for (int i = 0; i < 8; ++i) r[i] = (bf16)a[base + i];
    return r;
}

__device__ __forceinline__ float wave_max_pair(float x) {
    // lanes l and l ^ 32 hold the two halves of one column; v_permlane32_swap
    // exchanges the upper half of one copy with the lower half of the other,
    // so every lane sees both values without an LDS round trip
    const uint32_t u = __float_as_uint(x);
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
