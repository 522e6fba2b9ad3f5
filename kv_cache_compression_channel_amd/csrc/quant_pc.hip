// quant_pc.hip -- per-channel symmetric / asymmetric quantization and its dequantization.
//
// Walkthrough (KV Compression 公式到源码对照) §1.1 and §1.2: one scale (and zero point)
// per channel, reduced over the token rows of each slice; §1.3 for the dequantization.
//
// Layout: x is nb slices of [R][C]; each thread owns VEC (8 or 1) consecutive channels
// and walks rows, so a wave reads whole rows with 16-byte (bf16) / 32-byte (fp32) loads.
// Three launches: (1) per (slice, row chunk, channel) min/max into the workspace,
// (2) per (slice, channel) parameters, (3) codes.  Each launch reads x once; pass (3)
// follows pass (1) on the same stream, so slices small enough to stay in the MALL are
// read from HBM once.
#include <cfloat>

#include "kvq_internal.h"

namespace kvq {
namespace {

constexpr int kThreads = 256;
// Rows per min/max chunk: at least kRowsPerChunk (the workspace is sized for that), grown by
// doubling while the grid keeps at least kMinMaxBlocks workgroups (4 per CU).  On the full-model
// cache ([128][8192][4096] bf16) whole 8192-row slices per chunk took the quantizer from 7.34 to
// 7.03 ms against 256-row chunks: fewer, longer workgroups and 32x fewer partials.
constexpr int kRowsPerChunk = 256;
constexpr int64_t kMinMaxBlocks = 1024;
// The code and dequantization passes need no partials, so they take short row chunks: a
// workgroup then issues one batch of loads and then its stores (8 stores per thread in the code
// pass, 4 in the dequantizer) instead of 64, and the workgroups in flight write a compact window
// of the output.  On MI355X that made the code pass 5% faster (256-row chunks against 32), and
// the dequantizer 3-5% (256 against 64), then 10% (64 against 32, once its loads no longer
// waited behind store branches) and 1% more (32 against 16).
constexpr int kCodeRows = 32;
constexpr int kDqRows = 16;
// Row loads a thread issues before it uses any: every pass waits on memory once per batch.
constexpr int kBatch = 8;
constexpr int kDqBatch = 4;   // the dequantizer's batch: its 16-row chunk at 4 rows per pass

struct PcParams {
    float s;     // scale
    float r;     // fl(1 / s)
    float zf;    // zero point as float (0 for sym)
    float fast;  // 1 when every |x / s| of the channel is < 256
};

struct PcGeom {
    int64_t nb, R, C, ldx, bsx;
    int lpr;   // lanes per row (power of two, <= 64)
    int rpp;   // rows per pass = kThreads / lpr
    int64_t ncb, nrc;  // column blocks, row chunks
    int64_t rpc;       // rows per chunk of the min/max pass
};

// The raw bits of VEC consecutive values of x (fp32 or bf16) and their conversion to fp32, kept
// apart so that a thread can issue every row's load before it converts any.
struct XRaw {
    uint4 a, b;
};
template <int XT, int VEC>
__device__ __forceinline__ XRaw load_raw(const void* x, int64_t off) {
    XRaw r;
    if constexpr (XT == KVQ_FP32) {
        const float* p = static_cast<const float*>(x) + off;
        if constexpr (VEC == 8) {
            r.a = *reinterpret_cast<const uint4*>(p);
            r.b = *reinterpret_cast<const uint4*>(p + 4);
        } else {
            r.a.x = __float_as_uint(*p);
        }
    } else {
        const uint16_t* p = static_cast<const uint16_t*>(x) + off;
        if constexpr (VEC == 8) r.a = *reinterpret_cast<const uint4*>(p);
        else r.a.x = *p;
    }
    return r;
}
template <int XT, int VEC>
__device__ __forceinline__ void unpack_raw(const XRaw& r, float (&v)[VEC]) {
    if constexpr (XT == KVQ_FP32) {
        if constexpr (VEC == 8) {
            v[0] = __uint_as_float(r.a.x); v[1] = __uint_as_float(r.a.y);
            v[2] = __uint_as_float(r.a.z); v[3] = __uint_as_float(r.a.w);
            v[4] = __uint_as_float(r.b.x); v[5] = __uint_as_float(r.b.y);
            v[6] = __uint_as_float(r.b.z); v[7] = __uint_as_float(r.b.w);
        } else {
            v[0] = __uint_as_float(r.a.x);
        }
    } else {
        if constexpr (VEC == 8) {
            v[0] = bf_lo(r.a.x); v[1] = bf_hi(r.a.x); v[2] = bf_lo(r.a.y); v[3] = bf_hi(r.a.y);
            v[4] = bf_lo(r.a.z); v[5] = bf_hi(r.a.z); v[6] = bf_lo(r.a.w); v[7] = bf_hi(r.a.w);
        } else {
            v[0] = bf_to_f((uint16_t)r.a.x);
        }
    }
}

// Pass 1: min and max of every channel over one chunk of rows.
template <int XT, int VEC>
__global__ void __launch_bounds__(kThreads) pc_minmax_kernel(const void* __restrict__ x, PcGeom g,
                                                             float2* __restrict__ part) {
    __shared__ float smn[kThreads * VEC];
    __shared__ float smx[kThreads * VEC];
    // block counts fit 31 bits (the host checks): 32-bit division
    const uint32_t bid = blockIdx.x, q1 = bid / (uint32_t)g.ncb;
    const int64_t cb = bid - q1 * (uint32_t)g.ncb;
    const int64_t rc = q1 % (uint32_t)g.nrc;
    const int64_t s = q1 / (uint32_t)g.nrc;
    const int lane = threadIdx.x % g.lpr, rl = threadIdx.x / g.lpr;
    const int64_t c0 = (cb * g.lpr + lane) * VEC;
    float mn[VEC], mx[VEC];
#pragma unroll
    for (int k = 0; k < VEC; ++k) { mn[k] = FLT_MAX; mx[k] = -FLT_MAX; }
    if (c0 < g.C) {
        // kBatch rows' loads in flight per step; rows past the chunk's end repeat its last row,
        // which leaves min and max as they are
        const int64_t r_end = min(g.R, (rc + 1) * g.rpc);
        for (int64_t r0 = rc * g.rpc + rl; r0 < r_end; r0 += kBatch * g.rpp) {
            XRaw raw[kBatch];
#pragma unroll
            for (int u = 0; u < kBatch; ++u) {
                const int64_t r = min(r0 + u * g.rpp, r_end - 1);
                raw[u] = load_raw<XT, VEC>(x, s * g.bsx + r * g.ldx + c0);
            }
            __builtin_amdgcn_sched_barrier(0);   // the batch's loads all issued before the first use
#pragma unroll
            for (int u = 0; u < kBatch; u += 2) {
                float v0[VEC], v1[VEC];
                unpack_raw<XT, VEC>(raw[u], v0);
                unpack_raw<XT, VEC>(raw[u + 1], v1);
#pragma unroll
                for (int k = 0; k < VEC; ++k) {
                    mn[k] = vmin3(mn[k], v0[k], v1[k]);
                    mx[k] = vmax3(mx[k], v0[k], v1[k]);
                }
            }
        }
    }
#pragma unroll
    for (int k = 0; k < VEC; ++k) {
        smn[threadIdx.x * VEC + k] = mn[k];
        smx[threadIdx.x * VEC + k] = mx[k];
    }
    __syncthreads();
    // column j of the block (lane = j / VEC, element = j % VEC) reduced over the row lanes
    const int ncol = g.lpr * VEC;
    for (int j = threadIdx.x; j < ncol; j += kThreads) {
        const int ln = j / VEC, k = j % VEC;
        float a = FLT_MAX, b = -FLT_MAX;
        for (int q = 0; q < g.rpp; ++q) {
            a = vmin2(a, smn[(q * g.lpr + ln) * VEC + k]);
            b = vmax2(b, smx[(q * g.lpr + ln) * VEC + k]);
        }
        const int64_t c = cb * ncol + j;
        if (c < g.C) part[(s * g.nrc + rc) * g.C + c] = make_float2(a, b);
    }
}

// Scale and zero point of one channel from its min and max (Walkthrough §1.1, §1.2).
template <bool SYM>
__device__ __forceinline__ PcParams pc_param_of(float mn, float mx, int qmin, int qmax) {
    PcParams P;
    int z = 0;
    if constexpr (SYM) {
        float a = vmax2(mx, -mn);           // max |x|
        a = vmax2(a, 1e-8f);
        P.s = a / (float)qmax;
    } else {
        float range = mx - mn;
        range = vmax2(range, 1e-8f);
        P.s = range / (float)(qmax - qmin);
        const float m = mn / P.s;   // qmin - m with an explicit zero case (see group_params of the INT4 path)
        const float zr = (qmin == 0 && m == 0.0f) ? 0.0f : __builtin_rintf((float)qmin - m);
        z = (int)vclamp(zr, -128.0f, 127.0f);
    }
    P.r = 1.0f / P.s;
    P.zf = (float)z;
    P.fast = (vmax2(fabsf(mn), fabsf(mx)) * P.r <= 250.0f) ? 1.0f : 0.0f;
    return P;
}

// Codes of 8 values of one row: q = clip(round(x / s) + zp, qmin, qmax), packed low byte first.
template <int VEC>
__device__ __forceinline__ void pc_codes(const float (&v)[VEC], const float (&ps)[VEC], const float (&pr)[VEC],
                                         const float (&pz)[VEC], bool fast, float lo, float hi,
                                         int8_t (&o)[VEC]) {
    float n[VEC];
    if (fast) {
        rint_div_n<VEC>(v, ps, pr, n);
    } else {
#pragma unroll
        for (int k = 0; k < VEC; ++k) n[k] = __builtin_rintf(v[k] / ps[k]);
    }
#pragma unroll
    for (int k = 0; k < VEC; ++k) {
        // n and zf are integers: the fp32 sum is exact whenever the result can land in
        // [qmin, qmax] (Sterbenz), and far outside otherwise, so the clip is exact.
        o[k] = (int8_t)(int)vclamp(n[k] + pz[k], lo, hi);
    }
}

__device__ __forceinline__ uint2 pack8_i8(const int8_t (&o)[8]) {
    uint2 w;
    w.x = (uint32_t)(uint8_t)o[0] | ((uint32_t)(uint8_t)o[1] << 8) | ((uint32_t)(uint8_t)o[2] << 16) |
          ((uint32_t)(uint8_t)o[3] << 24);
    w.y = (uint32_t)(uint8_t)o[4] | ((uint32_t)(uint8_t)o[5] << 8) | ((uint32_t)(uint8_t)o[6] << 16) |
          ((uint32_t)(uint8_t)o[7] << 24);
    return w;
}

// Pass 2: per (slice, channel) scale / zero point (Walkthrough §1.1, §1.2).
template <bool SYM>
__global__ void __launch_bounds__(kThreads) pc_params_kernel(const float2* __restrict__ part, int64_t nb,
                                                             int64_t nrc, int64_t C, int qmin, int qmax,
                                                             float* __restrict__ scale, int8_t* __restrict__ zp,
                                                             PcParams* __restrict__ prm) {
    const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (i >= nb * C) return;
    const int64_t s = i / C, c = i % C;
    float mn = FLT_MAX, mx = -FLT_MAX;
    for (int64_t k = 0; k < nrc; ++k) {
        const float2 p = part[(s * nrc + k) * C + c];
        mn = vmin2(mn, p.x);
        mx = vmax2(mx, p.y);
    }
    const PcParams P = pc_param_of<SYM>(mn, mx, qmin, qmax);
    scale[i] = P.s;
    if (zp) zp[i] = (int8_t)P.zf;
    prm[i] = P;
}

// Pass 3: codes q = clip(round(x / s) + zp, qmin, qmax).
template <int XT, int VEC>
__global__ void __launch_bounds__(kThreads) pc_code_kernel(const void* __restrict__ x, PcGeom g,
                                                           const PcParams* __restrict__ prm, int qmin, int qmax,
                                                           int8_t* __restrict__ q) {
    // block counts fit 31 bits (the host checks): 32-bit division
    const uint32_t bid = blockIdx.x, q1 = bid / (uint32_t)g.ncb;
    const int64_t cb = bid - q1 * (uint32_t)g.ncb;
    const int64_t rc = q1 % (uint32_t)g.nrc;
    const int64_t s = q1 / (uint32_t)g.nrc;
    const int lane = threadIdx.x % g.lpr, rl = threadIdx.x / g.lpr;
    const int64_t c0 = (cb * g.lpr + lane) * VEC;
    if (c0 >= g.C) return;
    PcParams P[VEC];
#pragma unroll
    for (int k = 0; k < VEC; ++k) P[k] = prm[s * g.C + c0 + k];
    const float lo = (float)qmin, hi = (float)qmax;
    const int64_t r_end = min(g.R, (rc + 1) * kCodeRows);
    // every row of the chunk (at most kCodeRows / 4: rpp >= 4) loaded before any is coded.  A row
    // past the end takes the last row for its load and its store alike (the same codes to the same
    // bytes), so no load or store sits behind a branch.
    constexpr int NRT = kCodeRows / 4;
    XRaw raw[NRT];
    int64_t rr[NRT];
#pragma unroll
    for (int u = 0; u < NRT; ++u) {
        rr[u] = min(rc * kCodeRows + rl + u * g.rpp, r_end - 1);
        raw[u] = load_raw<XT, VEC>(x, s * g.bsx + rr[u] * g.ldx + c0);
    }
    __builtin_amdgcn_sched_barrier(0);   // every load issued before the first use
    float ps[VEC], pr[VEC], pz[VEC];
    bool fast = true;
#pragma unroll
    for (int k = 0; k < VEC; ++k) {
        ps[k] = P[k].s; pr[k] = P[k].r; pz[k] = P[k].zf;
        fast = fast && (P[k].fast != 0.0f);
    }
#pragma unroll
    for (int u = 0; u < NRT; ++u) {
        float v[VEC];
        unpack_raw<XT, VEC>(raw[u], v);
        int8_t o[VEC];
        pc_codes<VEC>(v, ps, pr, pz, fast, lo, hi, o);
        int8_t* dst = q + (s * g.R + rr[u]) * g.C + c0;
        if constexpr (VEC == 8) {
            *reinterpret_cast<uint2*>(dst) = pack8_i8(o);
        } else {
            dst[0] = o[0];
        }
    }
}

// Dequantization x_hat = ((float)(q - zp)) * s (Walkthrough §1.3).  Same geometry as the
// code pass: each thread owns VEC channels (scales loaded once) and walks rows.
template <int OT, int VEC>
__global__ void __launch_bounds__(kThreads) pc_dequant_kernel(const int8_t* __restrict__ q,
                                                              const float* __restrict__ scale,
                                                              const int8_t* __restrict__ zp, PcGeom g,
                                                              void* __restrict__ out) {
    // block counts fit 31 bits (the host checks): 32-bit division
    const uint32_t bid = blockIdx.x, q1 = bid / (uint32_t)g.ncb;
    const int64_t cb = bid - q1 * (uint32_t)g.ncb;
    const int64_t rc = q1 % (uint32_t)g.nrc;
    const int64_t s = q1 / (uint32_t)g.nrc;
    const int lane = threadIdx.x % g.lpr, rl = threadIdx.x / g.lpr;
    const int64_t c0 = (cb * g.lpr + lane) * VEC;
    if (c0 >= g.C) return;
    // the channel parameters as two 16-byte and one 8-byte load (one branch on zp, uniform)
    float sc[VEC], zf[VEC];
    if constexpr (VEC == 8) {
        const float4 a = *reinterpret_cast<const float4*>(scale + s * g.C + c0);
        const float4 b = *reinterpret_cast<const float4*>(scale + s * g.C + c0 + 4);
        sc[0] = a.x; sc[1] = a.y; sc[2] = a.z; sc[3] = a.w; sc[4] = b.x; sc[5] = b.y; sc[6] = b.z; sc[7] = b.w;
        uint2 z = make_uint2(0u, 0u);
        if (zp) z = *reinterpret_cast<const uint2*>(zp + s * g.C + c0);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            zf[k] = (float)(int8_t)(z.x >> (8 * k));
            zf[k + 4] = (float)(int8_t)(z.y >> (8 * k));
        }
    } else {
        sc[0] = scale[s * g.C + c0];
        zf[0] = zp ? (float)zp[s * g.C + c0] : 0.0f;
    }
    const int64_t r_end = min(g.R, (rc + 1) * kDqRows);
    for (int64_t r0 = rc * kDqRows + rl; r0 < r_end; r0 += kDqBatch * g.rpp) {
    // kDqBatch rows' codes loaded before any is used.  A row past the end takes the last row, for
    // its load and its store alike: it writes that row's values to that row again (the same
    // bytes), so no load or store sits behind a branch (a conditional store lets the compiler
    // sink the row's load into the branch, where it waits on its own).
    int64_t e[kDqBatch];
    uint2 wq[kDqBatch];
    int8_t wq1[kDqBatch];
#pragma unroll
    for (int u = 0; u < kDqBatch; ++u) {
        e[u] = (s * g.R + min(r0 + u * g.rpp, r_end - 1)) * g.C + c0;
        if constexpr (VEC == 8) wq[u] = *reinterpret_cast<const uint2*>(q + e[u]);
        else wq1[u] = q[e[u]];
    }
    __builtin_amdgcn_sched_barrier(0);   // every load of the batch issued before the first store
#pragma unroll
    for (int u = 0; u < kDqBatch; ++u) {
        float v[VEC];
        if constexpr (VEC == 8) {
            const uint2 w = wq[u];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                v[k] = ((float)(int8_t)(w.x >> (8 * k)) - zf[k]) * sc[k];
                v[k + 4] = ((float)(int8_t)(w.y >> (8 * k)) - zf[k + 4]) * sc[k + 4];
            }
        } else {
            v[0] = ((float)wq1[u] - zf[0]) * sc[0];
        }
        if constexpr (OT == KVQ_FP32) {
            float* o = static_cast<float*>(out) + e[u];
            if constexpr (VEC == 8) {
                st_stream_f4(o, make_float4(v[0], v[1], v[2], v[3]));
                st_stream_f4(o + 4, make_float4(v[4], v[5], v[6], v[7]));
            } else {
                o[0] = v[0];
            }
        } else {
            uint16_t* o = static_cast<uint16_t*>(out) + e[u];
            if constexpr (VEC == 8) {
                st_stream_u4(o, make_uint4(pack_bf2(v[0], v[1]), pack_bf2(v[2], v[3]), pack_bf2(v[4], v[5]),
                                           pack_bf2(v[6], v[7])));
            } else {
                o[0] = f_to_bf(v[0]);
            }
        }
    }
    }
}

PcGeom geom_of(int64_t nb, int64_t R, int64_t C, int64_t ldx, int64_t bsx, bool vec8);

int64_t nrc_of(int64_t R) { return cdiv(R, kRowsPerChunk); }

PcGeom geom_of(int64_t nb, int64_t R, int64_t C, int64_t ldx, int64_t bsx, bool vec8) {
    const int64_t cols = vec8 ? C / 8 : C;
    int lpr = 1;
    while (lpr < 64 && lpr < cols) lpr *= 2;
    return PcGeom{nb, R, C, ldx, nb == 1 ? 0 : bsx, lpr, kThreads / lpr, cdiv(cols, lpr), nrc_of(R), kRowsPerChunk};
}

size_t ws_bytes_for(int64_t nb, int64_t R, int64_t C) {
    const size_t part = (size_t)(nb * nrc_of(R) * C) * sizeof(float2);
    const size_t prm = (size_t)(nb * C) * sizeof(PcParams);
    return ((part + 255) / 256) * 256 + prm;
}

template <int XT>
int launch_pc(const void* x, PcGeom g, bool vec8, bool sym, int qmin, int qmax, int8_t* q, float* scale,
              int8_t* zp, void* ws, hipStream_t st) {
    float2* part = static_cast<float2*>(ws);
    const size_t part_bytes = (size_t)(g.nb * g.nrc * g.C) * sizeof(float2);
    PcParams* prm = reinterpret_cast<PcParams*>(static_cast<char*>(ws) + ((part_bytes + 255) / 256) * 256);
    const int64_t nblk = g.nb * g.nrc * g.ncb;
    if (vec8)
        hipLaunchKernelGGL((pc_minmax_kernel<XT, 8>), dim3((unsigned)nblk), dim3(kThreads), 0, st, x, g, part);
    else
        hipLaunchKernelGGL((pc_minmax_kernel<XT, 1>), dim3((unsigned)nblk), dim3(kThreads), 0, st, x, g, part);
    const unsigned pblk = (unsigned)cdiv(g.nb * g.C, kThreads);
    if (sym)
        hipLaunchKernelGGL((pc_params_kernel<true>), dim3(pblk), dim3(kThreads), 0, st, part, g.nb, g.nrc, g.C,
                           qmin, qmax, scale, zp, prm);
    else
        hipLaunchKernelGGL((pc_params_kernel<false>), dim3(pblk), dim3(kThreads), 0, st, part, g.nb, g.nrc, g.C,
                           qmin, qmax, scale, zp, prm);
    PcGeom gc = g;
    gc.nrc = cdiv(g.R, (int64_t)kCodeRows);
    const int64_t nblk_c = gc.nb * gc.nrc * gc.ncb;
    if (vec8)
        hipLaunchKernelGGL((pc_code_kernel<XT, 8>), dim3((unsigned)nblk_c), dim3(kThreads), 0, st, x, gc, prm, qmin,
                           qmax, q);
    else
        hipLaunchKernelGGL((pc_code_kernel<XT, 1>), dim3((unsigned)nblk_c), dim3(kThreads), 0, st, x, gc, prm, qmin,
                           qmax, q);
    return launch_status("per-channel quantization");
}

int quant_pc(const void* x, int xt, int64_t nb, int64_t R, int64_t C, int64_t ldx, int64_t bsx, bool sym,
             int qmin, int qmax, int8_t* q, float* scale, int8_t* zp, void* ws, size_t ws_bytes,
             kvq_stream stream, const char* name) {
    KVQ_REQUIRE(x && q && scale, "%s: NULL x, q or scale", name);
    KVQ_REQUIRE(sym || zp, "%s: zp is required", name);
    KVQ_REQUIRE(xt == KVQ_FP32 || xt == KVQ_BF16, "%s: xt must be KVQ_FP32 or KVQ_BF16", name);
    KVQ_REQUIRE(nb >= 1 && R >= 1 && C >= 1, "%s: nb, R, C must be >= 1", name);
    KVQ_REQUIRE(ldx >= C, "%s: ldx (%lld) < C (%lld)", name, (long long)ldx, (long long)C);
    KVQ_REQUIRE(nb == 1 || bsx >= R * ldx, "%s: bsx < R*ldx", name);
    KVQ_REQUIRE(nb * R * C < ((int64_t)1 << 40), "%s: tensor too large", name);
    KVQ_REQUIRE(ws != nullptr && ws_bytes >= ws_bytes_for(nb, R, C), "%s: workspace of %zu bytes needed", name,
                ws_bytes_for(nb, R, C));
    KVQ_REQUIRE_ALIGNED(x, "x");
    KVQ_REQUIRE_ALIGNED(q, "q");
    KVQ_REQUIRE_ALIGNED(scale, "scale");
    KVQ_REQUIRE_ALIGNED(zp, "zp");
    KVQ_REQUIRE_ALIGNED(ws, "ws");
    const bool vec8 = (C % 8 == 0) && (ldx % 8 == 0) && (nb == 1 || bsx % 8 == 0);
    PcGeom g = geom_of(nb, R, C, ldx, bsx, vec8);
    while (g.rpc < R && g.nb * cdiv(R, 2 * g.rpc) * g.ncb >= kMinMaxBlocks) {
        g.rpc *= 2;
        g.nrc = cdiv(R, g.rpc);
    }
    KVQ_REQUIRE(g.nb * g.nrc * g.ncb < ((int64_t)1 << 31), "%s: grid too large", name);
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (xt == KVQ_FP32) return launch_pc<KVQ_FP32>(x, g, vec8, sym, qmin, qmax, q, scale, zp, ws, st);
    return launch_pc<KVQ_BF16>(x, g, vec8, sym, qmin, qmax, q, scale, zp, ws, st);
}

}  // namespace

int dequant_pc(const kvq_pc_tensor* t, void* out, int ot, hipStream_t st) {
    KVQ_REQUIRE(t && t->q && t->scale && out, "kvq_dequant: NULL pointer");
    KVQ_REQUIRE(t->nb >= 1 && t->R >= 1 && t->C >= 1, "kvq_dequant: nb, R, C must be >= 1");
    KVQ_REQUIRE(ot == KVQ_FP32 || ot == KVQ_BF16, "kvq_dequant: ot must be KVQ_FP32 or KVQ_BF16");
    KVQ_REQUIRE_ALIGNED(t->q, "q");
    KVQ_REQUIRE_ALIGNED(t->scale, "scale");
    KVQ_REQUIRE_ALIGNED(out, "out");
    const bool vec8 = t->C % 8 == 0;
    PcGeom g = geom_of(t->nb, t->R, t->C, t->C, t->R * t->C, vec8);
    g.nrc = cdiv(t->R, (int64_t)kDqRows);
    const int64_t nblk = g.nb * g.nrc * g.ncb;
    KVQ_REQUIRE(nblk < ((int64_t)1 << 31), "kvq_dequant: grid too large");
    const dim3 grid((unsigned)nblk), blk(kThreads);
    if (ot == KVQ_FP32) {
        if (vec8)
            hipLaunchKernelGGL((pc_dequant_kernel<KVQ_FP32, 8>), grid, blk, 0, st, t->q, t->scale, t->zp, g, out);
        else
            hipLaunchKernelGGL((pc_dequant_kernel<KVQ_FP32, 1>), grid, blk, 0, st, t->q, t->scale, t->zp, g, out);
    } else {
        if (vec8)
            hipLaunchKernelGGL((pc_dequant_kernel<KVQ_BF16, 8>), grid, blk, 0, st, t->q, t->scale, t->zp, g, out);
        else
            hipLaunchKernelGGL((pc_dequant_kernel<KVQ_BF16, 1>), grid, blk, 0, st, t->q, t->scale, t->zp, g, out);
    }
    return launch_status("per-channel dequantization");
}

}  // namespace kvq

extern "C" {

size_t kvq_quant_pc_ws(int64_t nb, int64_t R, int64_t C) {
    if (nb < 1 || R < 1 || C < 1) return 0;
    return kvq::ws_bytes_for(nb, R, C);
}

int kvq_quant_sym(const void* x, int xt, int64_t nb, int64_t R, int64_t C, int64_t ldx, int64_t bsx, int bits,
                  int8_t* q, float* scale, int8_t* zp_or_null, void* ws, size_t ws_bytes, kvq_stream stream) {
    KVQ_REQUIRE(bits >= 2 && bits <= 8, "kvq_quant_sym: bits must be in [2, 8] (got %d)", bits);
    const int qmax = (1 << (bits - 1)) - 1;
    return kvq::quant_pc(x, xt, nb, R, C, ldx, bsx, true, -qmax, qmax, q, scale, zp_or_null, ws, ws_bytes, stream,
                         "kvq_quant_sym");
}

int kvq_quant_asym(const void* x, int xt, int64_t nb, int64_t R, int64_t C, int64_t ldx, int64_t bsx, int qmin,
                   int qmax, int8_t* q, float* scale, int8_t* zp, void* ws, size_t ws_bytes, kvq_stream stream) {
    KVQ_REQUIRE(qmin >= -128 && qmax <= 127 && qmin < qmax,
                "kvq_quant_asym: need -128 <= qmin < qmax <= 127 (got %d, %d)", qmin, qmax);
    return kvq::quant_pc(x, xt, nb, R, C, ldx, bsx, false, qmin, qmax, q, scale, zp, ws, ws_bytes, stream,
                         "kvq_quant_asym");
}

}  // extern "C"
