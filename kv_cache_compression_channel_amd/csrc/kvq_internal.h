// kvq_internal.h -- shared host/device plumbing of libkvq (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <string>

#include "../../include/kvq.h"

namespace kvq {

// ----------------------------------------------------------------- errors --

int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
void clear_error();

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Checks the launch status of the kernels just enqueued.
int launch_status(const char* what);

inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

#define KVQ_REQUIRE(cond, ...)                               \
    do {                                                     \
        if (!(cond)) return ::kvq::fail(KVQ_EINVAL, __VA_ARGS__); \
    } while (0)

#define KVQ_REQUIRE_ALIGNED(p, name)                                              \
    do {                                                                          \
        if ((p) && !::kvq::aligned16(p))                                          \
            return ::kvq::fail(KVQ_EALIGN, "%s must be 16-byte aligned", name);   \
    } while (0)

// ------------------------------------------------------------ device side --

// bf16 <-> fp32.  Widening is exact (the 16 bits become the top half).
__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf_to_f(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }

// Streaming 16-byte loads and stores with the non-temporal hint: data touched exactly once should
// not displace what the caches hold for other waves (measured: 6.2 -> 6.9 TB/s on a 2 GB one-pass
// read, and 8% off the INT4 dequantizer, whose output stream is 4x its code stream).
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ float4 ld_stream_f4(const float* p) {
    const f32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(p));
    return make_float4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint4 ld_stream_u4(const void* p) {
    const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint2 ld_stream_u2(const void* p) {
    const u32x2_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(p));
    return make_uint2(v.x, v.y);
}
__device__ __forceinline__ void st_stream_f4(float* p, float4 v) {
    __builtin_nontemporal_store(f32x4_t{v.x, v.y, v.z, v.w}, reinterpret_cast<f32x4_t*>(p));
}
__device__ __forceinline__ void st_stream_u4(void* p, uint4 v) {
    __builtin_nontemporal_store(u32x4_t{v.x, v.y, v.z, v.w}, reinterpret_cast<u32x4_t*>(p));
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// Two fp32 -> two bf16 (round to nearest even, one v_cvt_pk_bf16_f32), low half = a.
__device__ __forceinline__ uint32_t pack_bf2(float a, float b) {
    bf16x2_t v;
    v[0] = (__bf16)a;
    v[1] = (__bf16)b;
    return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ uint16_t f_to_bf(float a) { return (uint16_t)(pack_bf2(a, 0.0f) & 0xffffu); }

// Smallest bf16 >= f for finite f > 0: adding 0xffff carries into the kept half
// exactly when any dropped bit is set.
__device__ __forceinline__ uint16_t bf_ceil_pos(float f) {
    return (uint16_t)((__float_as_uint(f) + 0xffffu) >> 16);
}

// min / max / clamp on finite values.  fminf/fmaxf follow IEEE-754 NaN rules, for which the
// compiler quiets every operand it cannot prove canonical with an extra v_max_f32 x, x, x;
// the inputs here are finite by contract, so the hardware min3/max3/med3 are used directly.
__device__ __forceinline__ float vmin3(float a, float b, float c) {
    float r;
    asm("v_min3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
    return r;
}
__device__ __forceinline__ float vmax3(float a, float b, float c) {
    float r;
    asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
    return r;
}
// max(a, |b|, |c|): the absolute values as source modifiers of the one instruction
__device__ __forceinline__ float vmax3_abs(float a, float b, float c) {
    float r;
    asm("v_max3_f32 %0, %1, |%2|, |%3|" : "=v"(r) : "v"(a), "v"(b), "v"(c));
    return r;
}
__device__ __forceinline__ float vmin2(float a, float b) {
    float r;
    asm("v_min_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
    return r;
}
__device__ __forceinline__ float vmax2(float a, float b) {
    float r;
    asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
    return r;
}
__device__ __forceinline__ float vclamp(float x, float lo, float hi) { return __builtin_amdgcn_fmed3f(x, lo, hi); }

// Butterfly exchange across lanes at xor distances below 32: ds_swizzle's bit mode.
template <int OFF>
__device__ __forceinline__ float xor_lane(float x) {
    static_assert(OFF >= 1 && OFF < 32, "xor distance below 32");
    return __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, x), 0x1f | (OFF << 10)));
}
// x[lane] + x[lane ^ 32] and max(x[lane], x[lane ^ 32]) in every lane: v_permlane32_swap trades
// the upper half of one copy of x for the lower half of another, after which each lane holds
// both operands (which of the two registers holds which does not change a sum or a maximum).
__device__ __forceinline__ float add_halves(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float max_halves(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return vmax2(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
// Sum over the lanes lane ^ j for j in [0, 2 * END) stepping by OFF, OFF ... END powers of two
// below 32 (every lane ends with the sum of its group)
template <int OFF, int END>
__device__ __forceinline__ float add_lanes(float x) {
    if constexpr (OFF < END) return add_lanes<2 * OFF, END>(x + xor_lane<OFF>(x));
    else return x;
}
template <int OFF, int END>
__device__ __forceinline__ float max_lanes(float x) {
    if constexpr (OFF < END) return max_lanes<2 * OFF, END>(vmax2(x, xor_lane<OFF>(x)));
    else return x;
}
// The same reductions with the distances in descending order (32 first, then OFF, OFF/2, ... 1):
// the order of a plain xor-shuffle loop from 32 down to 1, so sums keep its rounding.
template <int OFF>
__device__ __forceinline__ float add_lanes_desc(float x) {
    if constexpr (OFF >= 1) return add_lanes_desc<OFF / 2>(x + xor_lane<OFF>(x));
    else return x;
}
template <int OFF>
__device__ __forceinline__ float max_lanes_desc(float x) {
    if constexpr (OFF >= 1) return max_lanes_desc<OFF / 2>(vmax2(x, xor_lane<OFF>(x)));
    else return x;
}
// v[src] of a wave-uniform lane index src, in every lane (one v_readlane_b32, no LDS)
__device__ __forceinline__ float lane_value(float v, int src) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), src));
}

// min and max of 8 values folded into running (mn, mx).
__device__ __forceinline__ void minmax8(const float (&v)[8], float& mn, float& mx) {
    mn = vmin3(vmin3(vmin3(mn, v[0], v[1]), v[2], v[3]), vmin3(v[4], v[5], v[6]), v[7]);
    mx = vmax3(vmax3(vmax3(mx, v[0], v[1]), v[2], v[3]), vmax3(v[4], v[5], v[6]), v[7]);
}

// round(x / s) with IEEE division semantics (round-half-to-even of the correctly
// rounded quotient).  Fast path: y = x * r with r = fl(1/s) (correctly rounded),
// valid while |x / s| < 256: then |y - x/s| < 2^-14.9 and |fl(x/s) - x/s| < 2^-16, so
// unless x/s lies within 2^-14 of a half-integer, y, fl(x/s) and x/s all round to
// the same integer; otherwise |y - rint(y)| > 0.4999 and the true division decides.
__device__ __forceinline__ float rint_div(float x, float s, float r) {
    const float y = x * r;
    float n = __builtin_rintf(y);
    if (__builtin_fabsf(y - n) > 0.4999f) n = __builtin_rintf(x / s);
    return n;
}

// rint_div for 8 values, with the exact-division fallback taken behind one branch.
template <int N>
__device__ __forceinline__ void rint_div_n(const float (&x)[N], const float (&s)[N], const float (&r)[N],
                                           float (&n)[N]) {
    bool slow = false;
#pragma unroll
    for (int k = 0; k < N; ++k) {
        const float y = x[k] * r[k];
        n[k] = __builtin_rintf(y);
        slow |= __builtin_fabsf(y - n[k]) > 0.4999f;
    }
    if (slow) {
#pragma unroll
        for (int k = 0; k < N; ++k) {
            const float y = x[k] * r[k];
            if (__builtin_fabsf(y - __builtin_rintf(y)) > 0.4999f) n[k] = __builtin_rintf(x[k] / s[k]);
        }
    }
}

}  // namespace kvq
