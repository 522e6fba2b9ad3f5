// int4_common.h -- device helpers shared by the 4-bit kernels (quantizer, dequantizer,
// streaming append, eviction): cache geometry, the per-group parameter and code steps, and
// nibble packing.  The arithmetic follows the Explainer (KV cache 压缩：把历史装得更小),
// quantization section, with the integer steps of the Walkthrough (KV Compression
// 公式到源码对照) §1.2 at qmin = 0, qmax = 15.
#pragma once

#include <cfloat>

#include "kvq_internal.h"

namespace kvq {

// Min or max over aligned groups of L lanes (L a power of two up to 64).  Within a row of 16 lanes
// each step is one VALU instruction with a DPP source operand, v_min/v_max(permuted v, v): quad
// permutations [1,0,3,2] and [2,3,0,1], then the half-row mirror (lane i <-> 7 - i) and the row
// mirror (i <-> 15 - i); after each step every lane holds the value of its 2, 4, 8, 16 lanes.  The
// two wait states a DPP read needs after a VALU write of its source are issued with the step.
// Across rows, lane exchanges.  Every lane of a group ends with the group's value.
#define KVQ_DPP_STEP(OP, PAT)                                                                        \
    __device__ __forceinline__ float dpp_##OP##_##PAT(float v) {                                     \
        float r;                                                                                     \
        asm("s_nop 1\n\tv_" #OP "_f32_dpp %0, %1, %1 " KVQ_DPP_PAT_##PAT " row_mask:0xf bank_mask:0xf" \
            : "=v"(r)                                                                                \
            : "v"(v));                                                                               \
        return r;                                                                                    \
    }
#define KVQ_DPP_PAT_q1032 "quad_perm:[1,0,3,2]"
#define KVQ_DPP_PAT_q2301 "quad_perm:[2,3,0,1]"
#define KVQ_DPP_PAT_hmir "row_half_mirror"
#define KVQ_DPP_PAT_mir "row_mirror"
KVQ_DPP_STEP(min, q1032)
KVQ_DPP_STEP(min, q2301)
KVQ_DPP_STEP(min, hmir)
KVQ_DPP_STEP(min, mir)
KVQ_DPP_STEP(max, q1032)
KVQ_DPP_STEP(max, q2301)
KVQ_DPP_STEP(max, hmir)
KVQ_DPP_STEP(max, mir)
#undef KVQ_DPP_STEP

template <int L, bool MAX>
__device__ __forceinline__ float lane_group_reduce(float v) {
    static_assert(L >= 1 && L <= 64 && (L & (L - 1)) == 0, "group of 1 to 64 lanes");
    if constexpr (L >= 2) v = MAX ? dpp_max_q1032(v) : dpp_min_q1032(v);
    if constexpr (L >= 4) v = MAX ? dpp_max_q2301(v) : dpp_min_q2301(v);
    if constexpr (L >= 8) v = MAX ? dpp_max_hmir(v) : dpp_min_hmir(v);
    if constexpr (L >= 16) v = MAX ? dpp_max_mir(v) : dpp_min_mir(v);
    if constexpr (L >= 32) v = MAX ? vmax2(v, __shfl_xor(v, 16)) : vmin2(v, __shfl_xor(v, 16));
    if constexpr (L >= 64) v = MAX ? vmax2(v, __shfl_xor(v, 32)) : vmin2(v, __shfl_xor(v, 32));
    return v;
}

struct I4Geom {
    int64_t B, T, H, d, g, R, Tq;
    int64_t nKg;   // K groups per (b, h) = ceil(Tq / g)
    int64_t nVt;   // V tiles per (b, h) = ceil(Tq / 64)
    int64_t nRt;   // residual tiles per (b, h) = ceil(R / 64)
    int64_t ldq;   // quantized-token rows per (b, h) in the sections (cap, or Tq)
    int64_t ldk;   // K group rows per (b, h) in the sections = ceil(ldq / g)
    int64_t ldr;   // residual rows per (b, h) in the sections (rcap, or R)
    int64_t sb, st, sh;   // element strides of the quantizer's input over b, token, h ([B][T][H][d]: T*H*d, H*d, d)
};

struct I4Ptrs {
    uint8_t* k_codes;
    uint16_t* k_scale;
    uint16_t* k_zero;
    uint8_t* v_codes;
    uint16_t* v_scale;
    uint16_t* v_zero;
    uint16_t* k_res;
    uint16_t* v_res;
};

// (b, j, h) of block index u in a [B][n][H] ordering with h fastest, in 32-bit arithmetic
// (block counts fit 31 bits; 64-bit division costs several times more instructions)
struct Bjh {
    int64_t b, j, h;
};
__device__ __forceinline__ Bjh split_bjh(uint32_t u, uint32_t H, uint32_t n) {
    const uint32_t q = u / H;
    return Bjh{(int64_t)(q / n), (int64_t)(q % n), (int64_t)(u - q * H)};
}

__device__ __forceinline__ void unpack8(const uint4 a, float (&v)[8]) {
    v[0] = bf_lo(a.x); v[1] = bf_hi(a.x); v[2] = bf_lo(a.y); v[3] = bf_hi(a.y);
    v[4] = bf_lo(a.z); v[5] = bf_hi(a.z); v[6] = bf_lo(a.w); v[7] = bf_hi(a.w);
}

// Per-group parameters from the group's min and max:
//   s = smallest bf16 >= max(max(max - min, 1e-8) / 15, |min| / 256),
//   z = bf16(round(0 - min / s)).
// bf16 holds every integer of magnitude <= 256 exactly; with s >= |min| / 256 the zero
// point is one of them, so the levels (k - z) s cover [min, max] and every value of the
// group lies within s / 2 of its level.  A group that straddles zero has range >= |min|,
// so only groups far from zero relative to their range take the second bound.
struct GroupParams {
    float s, r, z;
    uint16_t sb, zb;
};

__device__ __forceinline__ GroupParams group_params(float mn, float mx) {
    GroupParams p;
    float range = mx - mn;
    range = vmax2(range, 1e-8f);
    // |min| / 256 is exact (a power-of-two scaling) except below the normal range, where the
    // product by 2^-8 rounds exactly as the division does
    p.sb = bf_ceil_pos(vmax2(range / 15.0f, __builtin_fabsf(mn) * 0.00390625f));
    p.s = bf_to_f(p.sb);
    // r only feeds the fast code path, whose tolerance covers the 1-ulp hardware reciprocal (see
    // codes8); the stored values come from IEEE operations.
    p.r = __builtin_amdgcn_rcpf(p.s);
    // z = round(0 - fl(mn / s)), |mn / s| <= 256.  y = mn * r lies within 8e-5 of the quotient, as
    // does fl(mn / s), so unless -y is within 1e-3 of a half-integer both round alike (and to
    // zeros of the same sign while |y| is far above the subnormal range); otherwise the IEEE
    // division decides.  0 - m: the backend lowers a subtraction from +0 to a negation, which
    // turns m = +0 into -0; IEEE gives 0 - (+-0) = +0, so the zero quotient is explicit.
    const float y = mn * p.r;
    float zr = __builtin_rintf(-y);
    if (__builtin_fabsf(-y - zr) > 0.499f || __builtin_fabsf(y) < 1e-30f) {
        const float m = mn / p.s;
        zr = (m == 0.0f) ? 0.0f : __builtin_rintf(-m);
    }
    p.zb = f_to_bf(zr);
    p.z = bf_to_f(p.zb);
    return p;
}

// q = clip(round(x / s) + z, 0, 15) with IEEE-division semantics, for 8 elements.
// Fast path (z in [0, 15], so |x / s| <= 31 for every x of the group):
// w = fma(x, 1/s, z) lies within 4e-6 of x/s + z and fl(x/s) within 2e-6 of x/s, so
// unless x/s + z is within 1e-5 of a half-integer, rint(w) = rint(fl(x/s)) + z;
// otherwise |w - rint(w)| > 0.4999 and the true division decides (this also settles
// exact ties, which round half to even on x/s before z is added).  The fallback sits
// behind one branch per 8 elements; groups with z outside [0, 15] always take it:
// rint(x/s) + z is then an fp32 sum of two integers, exact whenever the result can
// fall in [0, 15] (Sterbenz) and far outside otherwise.
// The clip is needed on the fallback only: for x in [min, max] of the group, x/s + z lies in
// [-0.5 - 2e-5, 15.5 + 2e-5] (s >= range / 15 up to rounding, |min/s + z| <= 0.5 + 2e-5), so a
// w that rounds outside [0, 15] lies within 1e-4 of -0.5 or 15.5 and has taken the fallback.
template <bool UNIFORM>
__device__ __forceinline__ void codes8(const float (&x)[8], const float (&s)[8], const float (&r)[8],
                                       const float (&z)[8], bool fast, float (&q)[8]) {
    float n[8];
    bool slow = !fast;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const float w = __builtin_fmaf(x[k], r[k], z[k]);
        n[k] = __builtin_rintf(w);
        slow |= __builtin_fabsf(w - n[k]) > 0.4999f;
    }
    if (slow) {
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const float w = __builtin_fmaf(x[k], r[k], z[k]);
            if (!fast || __builtin_fabsf(w - __builtin_rintf(w)) > 0.4999f)
                n[k] = __builtin_rintf(x[k] / s[k]) + z[k];
            n[k] = vclamp(n[k], 0.0f, 15.0f);
        }
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) q[k] = n[k];
}

// 8 codes (as floats in [0, 15]) -> one dword, byte j = code(2j) | code(2j+1) << 4.
__device__ __forceinline__ uint32_t pack_codes(const float (&q)[8]) {
    uint32_t even = 0, odd = 0;
    even = __builtin_amdgcn_cvt_pk_u8_f32(q[0], 0, even);
    even = __builtin_amdgcn_cvt_pk_u8_f32(q[2], 1, even);
    even = __builtin_amdgcn_cvt_pk_u8_f32(q[4], 2, even);
    even = __builtin_amdgcn_cvt_pk_u8_f32(q[6], 3, even);
    odd = __builtin_amdgcn_cvt_pk_u8_f32(q[1], 0, odd);
    odd = __builtin_amdgcn_cvt_pk_u8_f32(q[3], 1, odd);
    odd = __builtin_amdgcn_cvt_pk_u8_f32(q[5], 2, odd);
    odd = __builtin_amdgcn_cvt_pk_u8_f32(q[7], 3, odd);
    return even | (odd << 4);
}

// Shape checks of a cache descriptor (quant_int4.hip); KVQ_OK or KVQ_EINVAL / KVQ_EALIGN.
int check_cache_shape(const kvq_int4_cache* c, const char* name);

}  // namespace kvq

// FN<d, g>(...) for the supported (d, g) pairs (validated before dispatch).
#define KVQ_DISPATCH_DG(d, g, FN, ...)                                        \
    do {                                                                      \
        if (d == 64 && g == 32) FN<64, 32>(__VA_ARGS__);                      \
        else if (d == 64 && g == 64) FN<64, 64>(__VA_ARGS__);                 \
        else if (d == 128 && g == 32) FN<128, 32>(__VA_ARGS__);               \
        else if (d == 128 && g == 64) FN<128, 64>(__VA_ARGS__);               \
        else if (d == 128 && g == 128) FN<128, 128>(__VA_ARGS__);             \
        else if (d == 256 && g == 32) FN<256, 32>(__VA_ARGS__);               \
        else if (d == 256 && g == 64) FN<256, 64>(__VA_ARGS__);               \
        else FN<256, 128>(__VA_ARGS__);                                       \
    } while (0)
