// attn_int4.hip -- GQA decode attention that reads the INT4 cache and dequantizes it in
// registers (Explainer (KV cache 压缩：把历史装得更小): the attention kernel reads the
// low-bit cache and dequantizes it; fusing the dequantization is what turns fewer bytes
// into bandwidth savings; GQA: consecutive query heads share one KV head).
//
// out[b][hq] = softmax_t(sm_scale * q . k_hat_t) . v_hat_t over all T tokens of KV head
// h = hq / (Hq / H); INT4 tokens dequantize as x_hat = (code - z) * s, residual tokens
// are bf16.  Split-K: one block per (b, h, token split) handles all Hq/H query heads
// that share the KV head (each KV byte is read once), then a combine kernel merges the
// splits with log-sum-exp weights.
//
// Dequantization is folded into the arithmetic instead of materialised:
//   K (scale per channel over a token group):  q . k_hat = sum_c (q_c s_c) code_c - sum_c q_c s_c z_c
//   V (scale per token per channel group):     p v_hat = (p s) code - (p s) z
// so each element costs one fused multiply-add on its 4-bit code.  Softmax runs in the
// base-2 domain (q pre-multiplied by sm_scale * log2 e), fp32 throughout.
//
// Lane layout (VALU path): d/8 lanes per token, 8 channels per lane; a wave takes
// 512/d tokens per step; dot products are finished with butterfly shuffles.
#include <cmath>
#include <mutex>

#include "kvq_internal.h"

namespace kvq {
int check_cache_shape(const kvq_int4_cache* c, const char* name);
void launch_attn_mfma(const kvq_int4_cache* c, const void* q, int64_t Hq, float qscale, float* ws, int nsplit,
                      int64_t split_len, int nslot, float* lgw, int64_t ldl, hipStream_t st);
int res_splits(int64_t R);
int mfma_waves(int64_t g, int64_t nq, bool lg);

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr float kNegBig = -3.0e38f;

struct AttnArgs {
    const uint8_t* k_codes;
    const uint16_t* k_scale;
    const uint16_t* k_zero;
    const uint8_t* v_codes;
    const uint16_t* v_scale;
    const uint16_t* v_zero;
    const uint16_t* k_res;
    const uint16_t* v_res;
    const uint16_t* q;
    void* out;
    int ot;
    float* ws;
    float* lgw;                   // base-2 logits [B][Hq][ldl], or NULL
    float* ml;                    // per (b, hq): final max logit and sum of 2^(logit - max), or NULL
    int64_t ldl;
    int64_t B, T, H, R, Tq, nKg, Hq;
    int64_t ldq, ldk, ldr;        // rows per (b, h) of the code / V-scale, K-group and residual sections
    int64_t range_lo, range_hi;   // token range this launch covers
    int64_t split_len;
    int nsplit;                   // splits of this launch per (b, h)
    int nslot, slot_off;          // ws slots per (b, hq) and this launch's first slot
    float qscale;   // sm_scale * log2(e)
};

__device__ __forceinline__ void unpack8(const uint4 a, float (&v)[8]) {
    v[0] = bf_lo(a.x); v[1] = bf_hi(a.x); v[2] = bf_lo(a.y); v[3] = bf_hi(a.y);
    v[4] = bf_lo(a.z); v[5] = bf_hi(a.z); v[6] = bf_lo(a.w); v[7] = bf_hi(a.w);
}

template <int D, int GS, int NQ>
__global__ void __launch_bounds__(kThreads) attn_split_kernel(const AttnArgs a) {
    constexpr int LPT = D / 8;        // lanes per token
    constexpr int TPW = 64 / LPT;     // tokens per wave step
    constexpr int TPS = TPW * kWaves; // tokens per block step
    constexpr int NGD = D / GS;
    __shared__ float s_m[kWaves][NQ], s_l[kWaves][NQ];
    __shared__ float s_acc[kWaves][NQ][D];

    const int tid = threadIdx.x, lane = tid % 64, wv = tid / 64;
    const int li = lane % LPT, tg = lane / LPT;
    const int64_t bh = blockIdx.x / a.nsplit;
    const int split = (int)(blockIdx.x % a.nsplit);
    const int64_t b = bh / a.H, h = bh % a.H;
    const int64_t t_begin = a.range_lo + (int64_t)split * a.split_len;
    const int64_t t_end = min(a.range_hi, t_begin + a.split_len);
    const int64_t Tq = a.Tq;

    float qv[NQ][8];
#pragma unroll
    for (int qi = 0; qi < NQ; ++qi) {
        const uint4 raw = *reinterpret_cast<const uint4*>(a.q + ((b * a.Hq + h * NQ + qi) * D + 8 * li));
        unpack8(raw, qv[qi]);
#pragma unroll
        for (int c = 0; c < 8; ++c) qv[qi][c] *= a.qscale;
    }
    float m[NQ], l[NQ], acc[NQ][8], zacc[NQ];
#pragma unroll
    for (int qi = 0; qi < NQ; ++qi) {
        m[qi] = kNegBig; l[qi] = 0.0f; zacc[qi] = 0.0f;
#pragma unroll
        for (int c = 0; c < 8; ++c) acc[qi][c] = 0.0f;
    }
    float qk[NQ][8], zb[NQ];
    int64_t cur_grp = -1;
    const uint8_t* kc = a.k_codes + (b * a.H + h) * a.ldq * (D / 2) + 4 * li;
    const uint8_t* vc = a.v_codes + (b * a.H + h) * a.ldq * (D / 2) + 4 * li;
    const int vgrp = (8 * li) / GS;

    for (int64_t t0 = t_begin; t0 < t_end; t0 += TPS) {
        const int64_t t = t0 + wv * TPW + tg;
        const bool valid = t < t_end;
        float logit[NQ];
        if (valid && t < Tq) {
            const int64_t grp = t / GS;
            if (grp != cur_grp) {
                const int64_t mi = ((b * a.H + h) * a.ldk + grp) * D + 8 * li;
                float s[8], z[8];
                unpack8(*reinterpret_cast<const uint4*>(a.k_scale + mi), s);
                unpack8(*reinterpret_cast<const uint4*>(a.k_zero + mi), z);
#pragma unroll
                for (int qi = 0; qi < NQ; ++qi) {
                    float zz = 0.0f;
#pragma unroll
                    for (int c = 0; c < 8; ++c) {
                        qk[qi][c] = qv[qi][c] * s[c];
                        zz = __builtin_fmaf(qk[qi][c], z[c], zz);
                    }
                    zb[qi] = zz;
                }
                cur_grp = grp;
            }
            const uint32_t w = *reinterpret_cast<const uint32_t*>(kc + t * (D / 2));
            float code[8];
#pragma unroll
            for (int c = 0; c < 8; ++c) code[c] = (float)((w >> (4 * c)) & 15u);
#pragma unroll
            for (int qi = 0; qi < NQ; ++qi) {
                float p = -zb[qi];
#pragma unroll
                for (int c = 0; c < 8; ++c) p = __builtin_fmaf(qk[qi][c], code[c], p);
                logit[qi] = p;
            }
        } else if (valid) {
            float kv[8];
            unpack8(*reinterpret_cast<const uint4*>(a.k_res + ((b * a.H + h) * a.ldr + (t - Tq)) * D + 8 * li), kv);
#pragma unroll
            for (int qi = 0; qi < NQ; ++qi) {
                float p = 0.0f;
#pragma unroll
                for (int c = 0; c < 8; ++c) p = __builtin_fmaf(qv[qi][c], kv[c], p);
                logit[qi] = p;
            }
        } else {
#pragma unroll
            for (int qi = 0; qi < NQ; ++qi) logit[qi] = 0.0f;
        }
        // finish the dot products across the LPT lanes of the token
#pragma unroll
        for (int off = 1; off < LPT; off *= 2)
#pragma unroll
            for (int qi = 0; qi < NQ; ++qi) logit[qi] += __shfl_xor(logit[qi], off);
        if (a.lgw && valid && li == 0) {
#pragma unroll
            for (int qi = 0; qi < NQ; ++qi) a.lgw[(b * a.Hq + h * NQ + qi) * a.ldl + t] = logit[qi];
        }

        float p[NQ];
#pragma unroll
        for (int qi = 0; qi < NQ; ++qi) {
            if (valid && logit[qi] > m[qi]) {
                const float alpha = exp2f(m[qi] - logit[qi]);
                l[qi] *= alpha;
                zacc[qi] *= alpha;
#pragma unroll
                for (int c = 0; c < 8; ++c) acc[qi][c] *= alpha;
                m[qi] = logit[qi];
            }
            p[qi] = valid ? exp2f(logit[qi] - m[qi]) : 0.0f;
            l[qi] += p[qi];
        }
        if (valid && t < Tq) {
            const uint32_t w = *reinterpret_cast<const uint32_t*>(vc + t * (D / 2));
            const int64_t mi = ((b * a.H + h) * a.ldq + t) * NGD + vgrp;
            const float vs = bf_to_f(a.v_scale[mi]), vz = bf_to_f(a.v_zero[mi]);
            float code[8];
#pragma unroll
            for (int c = 0; c < 8; ++c) code[c] = (float)((w >> (4 * c)) & 15u);
#pragma unroll
            for (int qi = 0; qi < NQ; ++qi) {
                const float pv = p[qi] * vs;
                zacc[qi] = __builtin_fmaf(pv, vz, zacc[qi]);
#pragma unroll
                for (int c = 0; c < 8; ++c) acc[qi][c] = __builtin_fmaf(pv, code[c], acc[qi][c]);
            }
        } else if (valid) {
            float vv[8];
            unpack8(*reinterpret_cast<const uint4*>(a.v_res + ((b * a.H + h) * a.ldr + (t - Tq)) * D + 8 * li), vv);
#pragma unroll
            for (int qi = 0; qi < NQ; ++qi)
#pragma unroll
                for (int c = 0; c < 8; ++c) acc[qi][c] = __builtin_fmaf(p[qi], vv[c], acc[qi][c]);
        }
    }

    // acc - zacc: the V zero points (this lane's 8 channels share one V group)
#pragma unroll
    for (int qi = 0; qi < NQ; ++qi)
#pragma unroll
        for (int c = 0; c < 8; ++c) acc[qi][c] -= zacc[qi];

    // merge the token groups of the wave (same channels, different tokens)
#pragma unroll
    for (int off = LPT; off < 64; off *= 2) {
#pragma unroll
        for (int qi = 0; qi < NQ; ++qi) {
            const float mo = __shfl_xor(m[qi], off), lo = __shfl_xor(l[qi], off);
            const float M = fmaxf(m[qi], mo);
            const float sa = exp2f(m[qi] - M), sb = exp2f(mo - M);
            l[qi] = l[qi] * sa + lo * sb;
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                const float ao = __shfl_xor(acc[qi][c], off);
                acc[qi][c] = acc[qi][c] * sa + ao * sb;
            }
            m[qi] = M;
        }
    }
    if (tg == 0) {
#pragma unroll
        for (int qi = 0; qi < NQ; ++qi) {
            if (li == 0) { s_m[wv][qi] = m[qi]; s_l[wv][qi] = l[qi]; }
#pragma unroll
            for (int c = 0; c < 8; ++c) s_acc[wv][qi][8 * li + c] = acc[qi][c];
        }
    }
    __syncthreads();
    // merge the waves and write this split's (m, l, acc[D]) for every query head
    for (int e = tid; e < NQ * D; e += kThreads) {
        const int qi = e / D, c = e % D;
        float M = s_m[0][qi];
#pragma unroll
        for (int w = 1; w < kWaves; ++w) M = fmaxf(M, s_m[w][qi]);
        float L = 0.0f, A = 0.0f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const float f = exp2f(s_m[w][qi] - M);
            L += s_l[w][qi] * f;
            A += s_acc[w][qi][c] * f;
        }
        float* dst = a.ws + ((b * a.Hq + h * NQ + qi) * a.nslot + a.slot_off + split) * (D + 2);
        if (c == 0) { dst[0] = M; dst[1] = L; }
        dst[2 + c] = A;
    }
}

// (M, L) of a merged row and its normalised output.
template <int D, int OT>
__device__ __forceinline__ void combine_store(int64_t row, int lane, float M, float L, const float (&A)[D / 64],
                                              void* __restrict__ out, float* __restrict__ ml) {
    if (ml && lane == 0) *reinterpret_cast<float2*>(ml + 2 * row) = make_float2(M, L);
#pragma unroll
    for (int j = 0; j < D / 64; ++j) {
        const int c = lane + 64 * j;
        const float o = A[j] / L;
        if constexpr (OT == KVQ_FP32)
            static_cast<float*>(out)[row * D + c] = o;
        else
            static_cast<uint16_t*>(out)[row * D + c] = f_to_bf(o);
    }
}

constexpr int kFewSlots = 16;   // slot counts merged with all loads in flight at once

// Log-sum-exp merge of the split partials (m, l, acc[D]) of one (b, hq) row per wave: lanes
// read the slots' maxima and sums in parallel, then each lane sums its D/64 channels over the
// slots with every slot's weight taken from the lane that holds it.
template <int D, int OT>
__global__ void __launch_bounds__(256) attn_combine_kernel(const float* __restrict__ ws, int nslot, int64_t rows,
                                                          void* __restrict__ out, float* __restrict__ ml) {
    constexpr int CPL = D / 64;     // channels per lane
    const int lane = threadIdx.x % 64;
    const int64_t row = (int64_t)blockIdx.x * 4 + threadIdx.x / 64;   // b * Hq + hq
    if (row >= rows) return;
    const float* base = ws + row * nslot * (D + 2);
    if (nslot <= kFewSlots) {
        // every load issued before any reduction: one round trip to memory instead of two; the
        // sums run in the same order as below, so the result is the same to the bit
        float ms = kNegBig, ls = 0.0f, x[kFewSlots][CPL];
        if (lane < nslot) { ms = base[(int64_t)lane * (D + 2)]; ls = base[(int64_t)lane * (D + 2) + 1]; }
#pragma unroll
        for (int s = 0; s < kFewSlots; ++s) {
#pragma unroll
            for (int j = 0; j < CPL; ++j) x[s][j] = s < nslot ? base[(int64_t)s * (D + 2) + 2 + lane + 64 * j] : 0.0f;
        }
        const float M = max_lanes_desc<16>(max_halves(ms));
        const float f = lane < nslot ? exp2f(ms - M) : 0.0f;
        float L = lane < nslot ? __builtin_fmaf(ls, f, 0.0f) : 0.0f, A[CPL];
#pragma unroll
        for (int j = 0; j < CPL; ++j) A[j] = 0.0f;
#pragma unroll
        for (int s = 0; s < kFewSlots; ++s) {
            if (s < nslot) {
                const float fk = lane_value(f, s);
#pragma unroll
                for (int j = 0; j < CPL; ++j) A[j] = __builtin_fmaf(x[s][j], fk, A[j]);
            }
        }
        L = add_lanes_desc<16>(add_halves(L));
        combine_store<D, OT>(row, lane, M, L, A, out, ml);
        return;
    }
    float M = kNegBig;
    for (int s = lane; s < nslot; s += 64) M = fmaxf(M, base[(int64_t)s * (D + 2)]);
    M = max_lanes_desc<16>(max_halves(M));
    float L = 0.0f, A[CPL];
#pragma unroll
    for (int j = 0; j < CPL; ++j) A[j] = 0.0f;
    for (int s0 = 0; s0 < nslot; s0 += 64) {
        const int s = s0 + lane;
        float f = 0.0f;
        if (s < nslot) {
            const float* sp = base + (int64_t)s * (D + 2);
            f = exp2f(sp[0] - M);
            L = __builtin_fmaf(sp[1], f, L);
        }
        const int ns = min(64, nslot - s0);
        int k = 0;
        for (; k + 4 <= ns; k += 4) {   // four slots' loads in flight
            float x[4][CPL];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const float* sp = base + (int64_t)(s0 + k + u) * (D + 2) + 2;
#pragma unroll
                for (int j = 0; j < CPL; ++j) x[u][j] = sp[lane + 64 * j];
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const float fk = __shfl(f, k + u);
#pragma unroll
                for (int j = 0; j < CPL; ++j) A[j] = __builtin_fmaf(x[u][j], fk, A[j]);
            }
        }
        for (; k < ns; ++k) {
            const float fk = __shfl(f, k);
            const float* sp = base + (int64_t)(s0 + k) * (D + 2) + 2;
#pragma unroll
            for (int j = 0; j < CPL; ++j) A[j] = __builtin_fmaf(sp[lane + 64 * j], fk, A[j]);
        }
    }
    L = add_lanes_desc<16>(add_halves(L));
    combine_store<D, OT>(row, lane, M, L, A, out, ml);
}

// Decode-time H2O scores: acc[b][h][t] += sum over the NQ query heads n of KV head h of
// 2^(lgw[b][h*NQ+n][t] - M_n) / L_n, the attention weight of token t in this step (summed over n in
// order, in fp32, then added to acc once).  Four consecutive tokens per thread; the logit rows
// are 16-byte aligned (ldl % 4 == 0).
template <int NQ>
__global__ void __launch_bounds__(256) h2o_accum_kernel(const float* __restrict__ lgw, const float* __restrict__ ml,
                                                       float* __restrict__ acc, int64_t ldl, int64_t ld_acc, int64_t H,
                                                       int64_t Hq, int64_t T, int nchunk) {
    const int64_t bh = blockIdx.x / nchunk;
    const int64_t b = bh / H, h = bh % H;
    const int64_t t = ((int64_t)(blockIdx.x % nchunk) * 256 + threadIdx.x) * 4;
    if (t >= T) return;
    float M[NQ], L[NQ];
#pragma unroll
    for (int n = 0; n < NQ; ++n) {
        const float2 v = *reinterpret_cast<const float2*>(ml + 2 * (b * Hq + h * NQ + n));
        M[n] = v.x;
        L[n] = v.y;
    }
    float s[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int n = 0; n < NQ; ++n) {
        const float4 x = *reinterpret_cast<const float4*>(lgw + (b * Hq + h * NQ + n) * ldl + t);
        s[0] += exp2f(x.x - M[n]) / L[n];
        s[1] += exp2f(x.y - M[n]) / L[n];
        s[2] += exp2f(x.z - M[n]) / L[n];
        s[3] += exp2f(x.w - M[n]) / L[n];
    }
    float* ar = acc + bh * ld_acc + t;
    const int nt = (int)min<int64_t>(4, T - t);
#pragma unroll
    for (int i = 0; i < 4; ++i)
        if (i < nt) ar[i] += s[i];
}

void launch_h2o_accum(const AttnArgs& a, float* acc, int64_t ld_acc, int nq, hipStream_t st) {
    const int nchunk = (int)cdiv(a.T, 1024);
    const dim3 grid((unsigned)(a.B * a.H * nchunk)), blk(256);
#define KVQ_ACC(NQ_) hipLaunchKernelGGL((h2o_accum_kernel<NQ_>), grid, blk, 0, st, a.lgw, a.ml, acc, a.ldl, ld_acc, \
                                        a.H, a.Hq, a.T, nchunk)
    switch (nq) {
        case 1: KVQ_ACC(1); break;
        case 2: KVQ_ACC(2); break;
        case 4: KVQ_ACC(4); break;
        case 8: KVQ_ACC(8); break;
        default: KVQ_ACC(16); break;
    }
#undef KVQ_ACC
}

// How the token axis is cut.  d = 128: the INT4 tokens [0, Tq) go to the matrix-core kernel
// (splits on multiples of 512 tokens, so every wave's range starts on a 128-token boundary) and
// the residual to blocks of the same launch (64 tokens each).  Otherwise everything goes to the
// VALU kernel (splits on multiples of max(g, 64) tokens).  Each split writes one partial slot
// per (b, hq); the combine merges them.
struct SplitPlan {
    bool mfma;
    int nsplit_q;           // matrix-core splits over [0, Tq)
    int64_t len_q;
    int nres;               // residual splits inside the matrix-core launch
    int nsplit_v;           // VALU splits over [0, T)
    int64_t len_v;
    int nslot;
};


int64_t split_len_for(int64_t n, int64_t want, int64_t unit) {
    int64_t len = cdiv(cdiv(n, want), unit) * unit;
    return len < unit ? unit : len;
}

// Workgroups to aim for: the plain matrix-core kernel at 3 waves per SIMD holds 3 workgroups per
// CU, and 768 of them fill the 256 CUs once; otherwise 1024 (2 rounds at 2 per CU; one round
// measured the same).  The plan depends on the cache and the heads only, so the variant that also
// writes logits (2 waves per SIMD) cuts the tokens the same way and its output is the plain
// kernel's, bit for bit.
SplitPlan plan_splits(int64_t B, int64_t H, int64_t T, int64_t R, int64_t d, int64_t g, int64_t nq) {
    SplitPlan p{};
    const int64_t Tq = T - R;
    p.mfma = (d == 128) && Tq > 0;
    const int64_t blocks = (p.mfma && mfma_waves(g, nq, false) == 3) ? 768 : 1024;
    const int64_t want = cdiv(blocks, B * H);
    if (p.mfma) {
        p.len_q = split_len_for(Tq, want, 512);
        p.nsplit_q = (int)cdiv(Tq, p.len_q);
        p.nres = res_splits(R);
        p.nslot = p.nsplit_q + p.nres;
        return p;
    }
    p.len_v = split_len_for(T, want, g > 64 ? g : 64);
    p.nsplit_v = (int)cdiv(T, p.len_v);
    p.nslot = p.nsplit_v;
    return p;
}

template <int D, int GS, int NQ>
void launch_attn(const AttnArgs& a, hipStream_t st) {
    hipLaunchKernelGGL((attn_split_kernel<D, GS, NQ>), dim3((unsigned)(a.B * a.H * a.nsplit)), dim3(kThreads), 0, st,
                       a);
}

template <int D>
void launch_combine(const AttnArgs& a, hipStream_t st) {
    const int64_t rows = a.B * a.Hq;
    const dim3 grid((unsigned)cdiv(rows, 4)), blk(256);
    if (a.ot == KVQ_FP32)
        hipLaunchKernelGGL((attn_combine_kernel<D, KVQ_FP32>), grid, blk, 0, st, a.ws, a.nslot, rows, a.out, a.ml);
    else
        hipLaunchKernelGGL((attn_combine_kernel<D, KVQ_BF16>), grid, blk, 0, st, a.ws, a.nslot, rows, a.out, a.ml);
}

template <int D, int GS>
void dispatch_nq(const AttnArgs& a, int nq, hipStream_t st) {
    switch (nq) {
        case 1: launch_attn<D, GS, 1>(a, st); break;
        case 2: launch_attn<D, GS, 2>(a, st); break;
        case 4: launch_attn<D, GS, 4>(a, st); break;
        case 8: launch_attn<D, GS, 8>(a, st); break;
        default: launch_attn<D, GS, 16>(a, st); break;
    }
}

void dispatch_combine(const AttnArgs& a, int64_t d, hipStream_t st) {
    if (d == 64) launch_combine<64>(a, st);
    else if (d == 128) launch_combine<128>(a, st);
    else launch_combine<256>(a, st);
}

void dispatch(const AttnArgs& a, int64_t d, int64_t g, int nq, hipStream_t st) {
    if (d == 64 && g == 32) dispatch_nq<64, 32>(a, nq, st);
    else if (d == 64) dispatch_nq<64, 64>(a, nq, st);
    else if (d == 128 && g == 32) dispatch_nq<128, 32>(a, nq, st);
    else if (d == 128 && g == 64) dispatch_nq<128, 64>(a, nq, st);
    else if (d == 128) dispatch_nq<128, 128>(a, nq, st);
    else if (g == 32) dispatch_nq<256, 32>(a, nq, st);
    else if (g == 64) dispatch_nq<256, 64>(a, nq, st);
    else dispatch_nq<256, 128>(a, nq, st);
}

}  // namespace
}  // namespace kvq

extern "C" {

size_t kvq_decode_attn_int4_ws(const kvq_int4_cache* c, int64_t Hq) {
    if (!c || c->B < 1 || c->H < 1 || c->T < 1 || c->g < 1 || Hq < 1 || c->R < 0 || c->R > c->T) return 0;
    const kvq::SplitPlan p = kvq::plan_splits(c->B, c->H, c->T, c->R, c->d, c->g, Hq / c->H);
    return (size_t)(c->B * Hq * p.nslot * (c->d + 2)) * sizeof(float);
}

}  // extern "C"

namespace kvq {
namespace {

// Logit rows of the H2O variant: 16-byte aligned, after the split partials in the workspace.
int64_t logit_ld(int64_t T) { return cdiv(T, 4) * 4; }
size_t h2o_ws_offset(const kvq_int4_cache* c, int64_t Hq) {
    return (size_t)cdiv((int64_t)kvq_decode_attn_int4_ws(c, Hq), 256) * 256;
}

// Shared body of the two decode-attention entry points; acc == NULL: plain attention.
int decode_attn(const char* name, const kvq_int4_cache* c, const void* q, int64_t Hq, float sm_scale, void* out,
                int ot, float* acc, int64_t ld_acc, void* ws, size_t ws_bytes, size_t ws_need, hipStream_t st) {
    const int rc = check_cache_shape(c, name);
    if (rc) return rc;
    KVQ_REQUIRE(q && out, "%s: NULL q or out", name);
    KVQ_REQUIRE(ot == KVQ_FP32 || ot == KVQ_BF16, "%s: ot must be KVQ_FP32 or KVQ_BF16", name);
    KVQ_REQUIRE(Hq >= 1 && Hq % c->H == 0, "%s: Hq (%lld) must be a multiple of H (%lld)", name, (long long)Hq,
                (long long)c->H);
    const int64_t nq = Hq / c->H;
    KVQ_REQUIRE(nq == 1 || nq == 2 || nq == 4 || nq == 8 || nq == 16,
                "%s: Hq / H must be 1, 2, 4, 8 or 16 (got %lld)", name, (long long)nq);
    KVQ_REQUIRE(ws && ws_bytes >= ws_need, "%s: workspace of %zu bytes needed", name, ws_need);
    KVQ_REQUIRE(c->T <= ((int64_t)1 << 30), "%s: T must be at most 2^30 tokens", name);
    KVQ_REQUIRE_ALIGNED(q, "q");
    KVQ_REQUIRE_ALIGNED(out, "out");
    KVQ_REQUIRE_ALIGNED(ws, "ws");
    const SplitPlan p = plan_splits(c->B, c->H, c->T, c->R, c->d, c->g, nq);
    KVQ_REQUIRE(c->B * c->H * p.nslot < ((int64_t)1 << 31) && c->B * Hq * p.nslot < ((int64_t)1 << 31),
                "%s: grid too large", name);
    AttnArgs a;
    a.k_codes = c->k_codes; a.k_scale = c->k_scale; a.k_zero = c->k_zero;
    a.v_codes = c->v_codes; a.v_scale = c->v_scale; a.v_zero = c->v_zero;
    a.k_res = c->k_res; a.v_res = c->v_res;
    a.q = static_cast<const uint16_t*>(q);
    a.out = out;
    a.ot = ot;
    a.ws = static_cast<float*>(ws);
    a.lgw = nullptr;
    a.ml = nullptr;
    a.ldl = logit_ld(c->T);
    if (acc) {
        a.lgw = reinterpret_cast<float*>(static_cast<char*>(ws) + h2o_ws_offset(c, Hq));
        a.ml = a.lgw + c->B * Hq * a.ldl;
    }
    a.B = c->B; a.T = c->T; a.H = c->H; a.R = c->R; a.Tq = c->T - c->R;
    a.nKg = cdiv(a.Tq, c->g);
    a.ldq = c->cap ? c->cap : a.Tq;
    a.ldk = cdiv(a.ldq, c->g);
    a.ldr = c->rcap ? c->rcap : c->R;
    a.Hq = Hq;
    a.nslot = p.nslot;
    a.qscale = sm_scale * 1.4426950408889634f;
    if (p.mfma) {
        launch_attn_mfma(c, q, Hq, a.qscale, a.ws, p.nsplit_q, p.len_q, p.nslot, a.lgw, a.ldl, st);
    } else {
        a.range_lo = 0;
        a.range_hi = c->T;
        a.split_len = p.len_v;
        a.nsplit = p.nsplit_v;
        a.slot_off = 0;
        dispatch(a, c->d, c->g, (int)nq, st);
    }
    dispatch_combine(a, c->d, st);
    if (acc) launch_h2o_accum(a, acc, ld_acc, (int)nq, st);
    return launch_status(name);
}

}  // namespace
}  // namespace kvq

extern "C" {

int kvq_decode_attn_int4(const kvq_int4_cache* c, const void* q, int64_t Hq, float sm_scale, void* out, int ot,
                         void* ws, size_t ws_bytes, kvq_stream stream) {
    return kvq::decode_attn("kvq_decode_attn_int4", c, q, Hq, sm_scale, out, ot, nullptr, 0, ws, ws_bytes,
                            kvq_decode_attn_int4_ws(c, Hq), static_cast<hipStream_t>(stream));
}

// Scratch of the allocation-free entry point: the split partials, in a fixed array each GPU holds
// from the library's load until the process ends.  In host code the name is a stand-in, not a
// device address: the address is taken once per device with hipGetSymbolAddress.
static __device__ __attribute__((aligned(256))) uint8_t scratch[KVQ_ATTN_SCRATCH_BYTES];

}  // extern "C"

namespace kvq {
namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's copy of the scratch array (its address taken on the first call on that
// device, with the device current).
int scratch_of_current_device(const char* name, void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(KVQ_EHIP, "%s: hipGetDevice: %s", name, hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices) return fail(KVQ_EINVAL, "%s: device %d out of range", name, dev);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return fail(KVQ_EHIP, "%s: hipGetSymbolAddress(scratch): %s", name, hipGetErrorString(e));
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return KVQ_OK;
}

}  // namespace
}  // namespace kvq

extern "C" {

int kvq_decode_attn_int4_noalloc(const kvq_int4_cache* c, const void* q, int64_t Hq, float sm_scale, void* out,
                                 int ot, kvq_stream stream) {
    const char* name = "kvq_decode_attn_int4_noalloc";
    const size_t need = kvq_decode_attn_int4_ws(c, Hq);
    KVQ_REQUIRE(need <= (size_t)KVQ_ATTN_SCRATCH_BYTES,
                "%s: the split partials need %zu bytes, more than the %u-byte scratch (use kvq_decode_attn_int4 "
                "with a workspace)", name, need, (unsigned)KVQ_ATTN_SCRATCH_BYTES);
    void* ws = nullptr;
    const int rc = kvq::scratch_of_current_device(name, &ws);
    if (rc) return rc;
    return kvq::decode_attn(name, c, q, Hq, sm_scale, out, ot, nullptr, 0, ws, (size_t)KVQ_ATTN_SCRATCH_BYTES, need,
                            static_cast<hipStream_t>(stream));
}

size_t kvq_decode_attn_int4_h2o_ws(const kvq_int4_cache* c, int64_t Hq) {
    const size_t base = kvq_decode_attn_int4_ws(c, Hq);
    if (!base) return 0;
    return kvq::h2o_ws_offset(c, Hq) + (size_t)(c->B * Hq * (kvq::logit_ld(c->T) + 2)) * sizeof(float);
}

int kvq_decode_attn_int4_h2o(const kvq_int4_cache* c, const void* q, int64_t Hq, float sm_scale, void* out, int ot,
                             float* acc, int64_t ld_acc, void* ws, size_t ws_bytes, kvq_stream stream) {
    KVQ_REQUIRE(acc, "kvq_decode_attn_int4_h2o: NULL acc");
    KVQ_REQUIRE(c && ld_acc >= c->T, "kvq_decode_attn_int4_h2o: ld_acc must be >= T");
    KVQ_REQUIRE_ALIGNED(acc, "acc");
    return kvq::decode_attn("kvq_decode_attn_int4_h2o", c, q, Hq, sm_scale, out, ot, acc, ld_acc, ws, ws_bytes,
                            kvq_decode_attn_int4_h2o_ws(c, Hq), static_cast<hipStream_t>(stream));
}

}  // extern "C"
